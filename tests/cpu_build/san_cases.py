"""Every C ABI entry point of the sanitized CPU build (libvdn_vda_sim_san.so)
on small cases, in a process that preloads the sanitizer runtime:

    LD_PRELOAD=<libclang_rt.asan> python tests/cpu_build/san_cases.py <library> [--full] [--tsan] [--shard=i/n]
    LD_PRELOAD=<libclang_rt.asan> python tests/cpu_build/san_cases.py <library> --heavy

(tests/test_cpu_build.py starts it so, with one case per kernel variant and
mode; --full runs every forward edge case, every backward case and every
adjacent-map case, about eight minutes in one process; --tsan, for the
ThreadSanitizer build, leaves out the arbitrary bit patterns: they send the
statistics kernel down its range recovery, where every consumer wave whose sums
are not finite writes the same 1 to the shared flag before the barrier that
orders its readers, a race only in form, and the 768p-frame case, whose races
do not depend on the frame size; --shard=i/n runs the i-th of n shares of the
cases, balanced by their rough cost, so that n processes share the sweep;
--heavy runs only the heavy cases instead, all 24 heads of the 768p clip). Any
AddressSanitizer or UndefinedBehaviorSanitizer report ends the process with a
nonzero status; the results themselves are compared with the oracle by the
unsanitized tests, so here they are only checked to be finite.
"""

import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [os.path.dirname(HERE), os.path.dirname(os.path.dirname(HERE))]

import numpy as np  # noqa: E402

import test_gpu_adjacent as GA  # noqa: E402
import test_gpu_backward as GB  # noqa: E402
import test_gpu_parity as P  # noqa: E402
import test_gpu_widths as GW  # noqa: E402
import test_gpu_training_f32 as GT  # noqa: E402
from cpu_build import sim as S  # noqa: E402
from frame_wise_delta_02_amd import synth  # noqa: E402


def finite(*arrays):
    for a in arrays:
        if a is not None:
            assert np.isfinite(S.to_f64(a)).all()


FORWARD = ("d32_bf16", "d16_bf16", "d32_f32", "ragged_f32_128", "no_text_bf16", "T1_bf16", "T2_f32",
           "chunk3_bf16", "batch2_bf16", "U1_bf16_128", "U2_f32_16", "ragged_bf16_128")
FORWARD_QUICK = ("d32_bf16", "d16_bf16", "d32_f32", "no_text_bf16", "T1_bf16", "U1_bf16_128", "U2_f32_16")
BACKWARD_QUICK = ("bwd_64_ragged", "bwd_32_bridge", "bwd_16_chunk3", "bwd_64_no_text", "bwd_16_ql2", "bwd_T1",
                  "bwd_16", "bwd_128_gain")
ADJACENT_QUICK = ("adj_small", "adj_d16", "adj_tiny", "adj_d48")
PADDED = ("d48_bf16", "d80_bf16", "d96_bf16_chunk3", "d112_bf16", "d48_f32", "d112_f32", "d80_no_text_bf16",
          "d48_T1_bf16", "d96_batch2_bf16")
PADDED_QUICK = ("d48_f32", "d80_no_text_bf16", "d48_T1_bf16")


def cases(full, tsan=False):
    """The sweep as a list of (label, run(L)) pairs, in a fixed order."""
    out = []

    def forward(name, mode):
        def run(L):
            w = P.EDGE[name]
            x = synth.make_inputs(w)
            if mode == "bridge":
                o, _, _ = S.run_forward(L, x, w, epilogue=False, bridge=True)
            else:
                o, _, _ = S.run_forward(L, x, w, epilogue=True, scan=mode,
                                        rms_weight=np.linspace(0.5, 1.5, w.d) if w.d == 128 else None)
            finite(o)
        return run

    for name in FORWARD if full else FORWARD_QUICK:
        for mode in ("frames", "chunks", "bridge"):
            out.append((f"forward {name} {mode}", forward(name, mode)))

    # widths between the built ones: the zero-padded copies in, the output's
    # channels back; with the gain, the raw readout, the bridge
    def padded(name, mode):
        def run(L):
            w = GW.CASES[name]
            x = synth.make_inputs(w)
            if mode == "bridge":
                o, _, _ = S.run_forward(L, x, w, epilogue=False, bridge=True)
            else:
                o, _, _ = S.run_forward(L, x, w, epilogue=True, scan=mode, rms_weight=np.linspace(0.5, 1.5, w.d))
            finite(o)
        return run

    for name in (PADDED if full else PADDED_QUICK):
        for mode in ("frames", "chunks", "bridge"):
            out.append((f"forward {name} {mode}", padded(name, mode)))

    def noalloc(L):
        w = P.EDGE["ragged_bf16_128" if full else "d32_bf16"]
        finite(S.run_forward_noalloc(L, synth.make_inputs(w), w))

    out.append(("forward_noalloc", noalloc))

    def noalloc_padded(L):
        w = GW.CASES["d48_T1_bf16"]
        finite(S.run_forward_noalloc(L, synth.make_inputs(w), w))

    out.append(("forward_noalloc d48_T1_bf16", noalloc_padded))

    # arbitrary bit patterns in every input (negative, infinite and NaN beta and
    # alpha included): the results are meaningless, but no access may leave its
    # buffer and no operation may be undefined, whatever the data
    def bit_patterns(name, seed, mode):
        def run(L):
            rng = np.random.default_rng(seed)
            w = P.EDGE[name]
            x = synth.make_inputs(w)
            for k, a in x.items():
                if a.dtype == np.uint16:
                    x[k] = rng.integers(0, 1 << 16, a.shape, dtype=np.uint16)
                elif a.dtype == np.float32:
                    x[k] = rng.integers(0, 1 << 32, a.shape, dtype=np.uint32).view(np.float32)
            if mode == "noalloc":
                S.run_forward_noalloc(L, x, w)
            elif mode == "bridge":
                S.run_forward(L, x, w, epilogue=False, bridge=True)
            else:
                S.run_forward(L, x, w, epilogue=True, scan=mode)
        return run

    names = () if tsan else ("ragged_bf16_128", "d32_bf16", "ragged_f32_128") if full else ("ragged_bf16_128",
                                                                                            "d32_f32")
    for i, name in enumerate(names):
        for mode in ("frames", "chunks", "bridge", "noalloc"):
            out.append((f"forward on arbitrary bit patterns {name} {mode}", bit_patterns(name, 99 + i, mode)))

    def prepare(name, kw):
        def run(L):
            w = synth.WORKLOADS["long_prep_bf16"].scaled(name=name, **kw)
            x = synth.make_inputs(w)
            qh, kh, vh = S.run_prepare(L, x, w)
            finite(qh, kh, vh)
            _, kf, vf = S.run_prepare(L, x, w, query_l2=True)
            o, _, _ = S.run_forward(L, x, w, epilogue=True, query_l2=True, inputs={"k": kf, "v": vf})
            finite(o)
        return run

    for name, kw in (("prep_small_bf16", dict(H=2, T=5, grid_h=6, grid_w=10, L=8)),
                     ("prep_small_f32", dict(H=2, T=5, grid_h=6, grid_w=10, L=8, dtype="f32")),
                     ("prep_T1_ragged", P.PREP_EDGE["prep_T1_ragged"]),
                     ("prep_d64", dict(H=2, T=6, grid_h=5, grid_w=7, L=4, d=64)),
                     ("prep_d48", GW.PREP_CASES["prep_d48_bf16"]), ("prep_d80_f32", GW.PREP_CASES["prep_d80_f32"])):
        out.append((f"prepare + fused query {name}", prepare(name, kw)))

    def backward(name):
        def run(L):
            case = GB.CASES[name]
            w, epi = case["w"], case.get("epilogue", True)
            bridge, ql2 = case.get("bridge", False), case.get("query_l2", False)
            x = synth.make_inputs(w)
            if ql2:
                GB._raw_queries(x, w)
            rw = np.linspace(0.5, 1.5, w.d) if case.get("gain") else None
            _, fws, _ = S.run_forward(L, x, w, epilogue=epi, rms_weight=rw, bridge=bridge, query_l2=ql2)
            # the gain's gradient on the cases that give a gain: both readout
            # variants run across the cases
            got, _, _ = S.run_backward(L, x, w, GB._dy(w), fws, epilogue=epi, rms_weight=rw, bridge=bridge,
                                       query_l2=ql2, gain=epi and case.get("gain", False))
            finite(*(v for v in got.values() if v is not None))
        return run

    for name in GB.CASES if full else BACKWARD_QUICK:
        out.append((f"backward {name}", backward(name)))

    # widths between the built ones: the forward's padded copies, dy, k, v in,
    # every gradient out
    def backward_padded(name):
        def run(L):
            case = GW.BWD_CASES[name]
            w, epi, bridge = case["w"], case.get("epilogue", True), case.get("bridge", False)
            x = synth.make_inputs(w)
            rw = np.linspace(0.5, 1.5, w.d) if case.get("gain") else None
            _, fws, _ = S.run_forward(L, x, w, epilogue=epi, rms_weight=rw, bridge=bridge)
            got, _, _ = S.run_backward(L, x, w, GB._dy(w), fws, epilogue=epi, rms_weight=rw, bridge=bridge,
                                       gain=epi)
            finite(*(v for v in got.values() if v is not None))
        return run

    for name in GW.BWD_CASES if full else ("bwd_d48_gain", "bwd_d80_raw_bridge"):
        out.append((f"backward {name}", backward_padded(name)))

    # float32 inputs: the float32 first and third stages
    def backward_f32(name):
        def run(L):
            case = GT.CASES[name]
            w, epi, bridge = case["w"], case.get("epilogue", True), case.get("bridge", False)
            ql2 = case.get("query_l2", False)
            x = synth.make_inputs(w)
            if ql2:
                GT.raw_queries(x, w)
            rw = np.linspace(0.5, 1.5, w.d) if case.get("gain") else None
            _, fws, _ = S.run_forward(L, x, w, epilogue=epi, rms_weight=rw, bridge=bridge, query_l2=ql2)
            got, _, _ = S.run_backward(L, x, w, GT._dy(w), fws, epilogue=epi, rms_weight=rw, bridge=bridge,
                                       query_l2=ql2, gain=epi)
            finite(*(v for v in got.values() if v is not None))
        return run

    for name in GT.CASES if full else ("tiny_f32_gain", "d64_raw_chunk3", "d32_query_l2", "d48_gain"):
        out.append((f"backward {name}", backward_f32(name)))

    # forward and backward at the 768p clip's frame size (48 x 84 tokens,
    # d = 128, 256 text tokens), where the kernels' 32-bit row offsets are
    # largest
    def frame_768p(L):
        w = synth.WORKLOADS["768p_bf16"].scaled(name="bwd_768p_frame", H=1, T=4, L=256)
        x = synth.make_inputs(w)
        o, fws, _ = S.run_forward(L, x, w, epilogue=True)
        finite(o)
        got, _, _ = S.run_backward(L, x, w, GB._dy(w), fws, epilogue=True, gain=True)
        finite(*(v for v in got.values()))

    if not tsan:
        out.append(("forward + backward at the 768p frame size", frame_768p))

    adj_cases = dict(GA.CASES, **GW.ADJ_CASES)

    def adjacent(name):
        def run(L):
            w, dm = adj_cases[name]
            p = synth.make_adjacent_inputs(w, dm)
            finite(*S.run_gates(L, p, w, dm))
            for mode in ("y_in", "in_place", "no_y_in"):
                finite(S.run_out_proj(L, p, w, mode))
        return run

    for name in adj_cases if full else ADJACENT_QUICK:
        out.append((f"gates + out_proj {name}", adjacent(name)))
    return out


# rough cost of the slow cases in seconds under AddressSanitizer (the rest
# take about one), for sharing the sweep evenly between processes
COST = (("768p frame", 24.0), ("bit patterns ragged_bf16_128", 10.0), ("no_text_bf16", 6.5),
        ("U1_bf16_128", 3.8), ("ragged_bf16_128", 3.0), ("bwd_64_ragged", 3.4), ("bwd_B2", 10.0),
        ("ragged_f32_128", 2.0), ("bwd_d80", 12.0), ("bwd_128_gain", 8.0), ("bwd_d112", 8.0), ("bwd_d96", 6.0))


def _cost(label):
    return next((c for key, c in COST if key in label), 1.0)


def share(all_cases, shard, shards):
    """The cases of process ``shard`` of ``shards``: each case, the costliest
    first, goes to the process with the least work so far (ties to the lowest
    index); the same split in every process."""
    load = [0.0] * shards
    mine = {i: [] for i in range(shards)}
    order = sorted(range(len(all_cases)), key=lambda i: (-_cost(all_cases[i][0]), i))
    for i in order:
        j = min(range(shards), key=lambda k: (load[k], k))
        load[j] += _cost(all_cases[i][0])
        mine[j].append(i)
    return [all_cases[i] for i in sorted(mine[shard])]


def heavy_cases():
    """Forward and backward with all 24 heads of the 768p clip at its frame size
    (48 x 84 tokens, d = 128, 256 text tokens), four frames: every per-frame
    32-bit offset and row stride of the full clip (frame bases are 64-bit, so
    the frame count changes none of them).  About 13 minutes."""
    def run(L):
        w = synth.WORKLOADS["768p_bf16"].scaled(name="768p_frames4", T=4)
        x = synth.make_inputs(w)
        for scan in ("frames", "chunks"):
            o, fws, _ = S.run_forward(L, x, w, epilogue=True, scan=scan)
            finite(o)
        got, _, _ = S.run_backward(L, x, w, GB._dy(w), fws, epilogue=True)
        finite(*(v for v in got.values()))
    return [("forward + backward, 24 heads at the 768p frame size", run)]


def main(path, full, tsan=False, shard=0, shards=1, heavy=False):
    L = S.load(path)
    mine = heavy_cases() if heavy else share(cases(full, tsan), shard, shards)
    for label, run in mine:
        t0 = time.time()
        run(L)
        print(f"ran {label} ({time.time() - t0:.1f} s)", flush=True)
    print(f"all entry points ran: {len(mine)} cases")


if __name__ == "__main__":
    args = sys.argv[2:]
    shard, shards = 0, 1
    for a in args:
        if a.startswith("--shard="):
            shard, shards = (int(v) for v in a[len("--shard="):].split("/"))
    main(sys.argv[1], "--full" in args, "--tsan" in args, shard, shards, "--heavy" in args)
