"""The library's own HIP sources compiled for the host and run on the CPU
(tests/cpu_build: every lane a fiber, cross-lane operations and barriers as
rendezvous points, buffer descriptors with their range checks).

* Under AddressSanitizer and UndefinedBehaviorSanitizer (check.cpp): the
  forward pass on exact-size host allocations, every kernel variant the
  forward launches (both dtypes, d = 16 .. 128, one token per frame, no text,
  T = 1 and 2); A_t, B_t and (I + A_t)^{-1} against a float64 reference, and no
  out-of-range access, undefined behaviour, divergent cross-lane operation or
  unequal barrier count.
* The forward's statistics launch alone (gram_launch.cpp) at the 768p frame
  size on arbitrary bit patterns and on data; the whole 768p launch on request.
* Through the C ABI from Python (libvdn_vda_sim.so): outputs and every
  intermediate against the oracle with the tolerances of the GPU parity tests,
  both scans, the decay bridge, the prep kernels, the fused query norm, the
  backward stages, the adjacent maps and seeded random shapes.
* Every entry point of the sanitized library (tests/cpu_build/san_cases.py,
  shared between processes), arbitrary bit patterns included; all 24 heads of
  the 768p clip at its frame size on request.
* ThreadSanitizer over the emulator's schedule, a fiber per lane: no data race
  between waves and no unsynchronised exchange between the lanes of a wave in
  any entry point.
* The emulator's own checks (selftest.cpp).

These run the kernels' code, not a model of it, but not the gfx950 binary:
they check indexing, bounds, synchronisation counts and arithmetic, not the
compiler's output or the hardware.  Parity proper is the GPU suite's.  Tests
marked as needing VDA_CPU_BUILD_FULL=1 take five to fifteen minutes each.
"""

import os
import subprocess

import numpy as np
import pytest

import oracle
import gpu_harness as G
import test_gpu_parity as P
import test_gpu_widths as GW
from cpu_build import build as CB
from cpu_build import sim as S
from frame_wise_delta_02_amd import synth

pytestmark = pytest.mark.skipif(CB.compiler() is None, reason="no host clang++ for the CPU build")


@pytest.fixture(scope="module")
def check_exe():
    return CB.build(S.OUT, "check")


@pytest.fixture(scope="module")
def lib():
    return S.load(CB.build(S.OUT, "lib"))


# H, T, grid_h, grid_w, d, L, dtype
SAN_SHAPES = [
    (2, 6, 6, 11, 128, 12, "bf16"),
    (3, 7, 5, 9, 64, 37, "bf16"),
    (2, 6, 6, 11, 32, 12, "bf16"),
    (2, 6, 6, 11, 16, 12, "bf16"),
    (2, 6, 6, 11, 128, 12, "f32"),
    (2, 6, 4, 4, 64, 8, "f32"),
    (2, 6, 4, 4, 32, 8, "f32"),
    (2, 6, 4, 4, 16, 8, "f32"),
    (1, 3, 1, 1, 128, 3, "bf16"),
    (2, 5, 4, 5, 128, 0, "bf16"),
    (2, 1, 4, 8, 128, 16, "bf16"),
    (2, 2, 4, 8, 128, 16, "f32"),
]


@pytest.mark.parametrize("shape", SAN_SHAPES, ids=["x".join(map(str, s)) for s in SAN_SHAPES])
def test_forward_under_sanitizers(check_exe, shape):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_stack_use_after_return=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([check_exe, *map(str, shape)], capture_output=True, text=True, timeout=900, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "Sanitizer" not in out and "[simt]" not in out, out[-4000:]


def _gram_launches(args_list):
    """gram_launch (the forward's statistics launch alone, sanitized) once per
    argument list, all at once; asserts that each run is clean and returns
    their report lines."""
    exe = CB.build(S.OUT, "gram_launch")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_stack_use_after_return=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    procs = [subprocess.Popen([exe, *map(str, a)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                              env=env) for a in args_list]
    lines = []
    for p in procs:
        try:
            out, _ = p.communicate(timeout=3600)
        except subprocess.TimeoutExpired:
            p.kill()
            out, _ = p.communicate()
        assert p.returncode == 0, out[-4000:]
        assert "runtime error" not in out and "Sanitizer" not in out and "[simt]" not in out, out[-4000:]
        lines.append(out.strip().splitlines()[-1])
    return lines


def _written(line):
    return int(line.split("slots written ")[1].split(",")[0]), int(line.split("workgroups ")[1].split(",")[0])


def test_statistics_launch_at_the_768p_frame_size():
    """The statistics launch as the forward makes it, at the 768p clip's frame
    (48 x 84 tokens, d = 128, 256 text tokens) on two heads and two absorbed
    frames, with exact-size inputs: on arbitrary bit patterns nothing leaves its
    buffer and nothing is undefined; on data the statistics agree with float64;
    every formed slot is written whole, by one workgroup."""
    shape = (1, 2, 4, 48, 84, 128, 256)
    for line in _gram_launches([(*shape, "bits"), (*shape, "data")]):
        assert _written(line) == (2 * 3, 2 * 3), line


@pytest.mark.skipif(os.environ.get("VDA_CPU_BUILD_FULL") != "1",
                    reason="the whole 768p statistics launch, about 8 minutes on 8 cores: set VDA_CPU_BUILD_FULL=1")
@pytest.mark.parametrize("fill", ["bits", "data"])
def test_statistics_launch_of_the_768p_clip(fill):
    """The whole statistics launch of the 768p clip (1 x 24 heads x 60 frames,
    48 x 84 tokens, d = 128, 256 text tokens: 1392 video and 24 text
    workgroups), as the forward makes it, on exact-size inputs, its workgroups
    shared by up to seven processes: every one of the 1416 slots written whole
    by one workgroup, no sanitizer or emulator report (on arbitrary bit
    patterns too), sampled statistics within float64 tolerance."""
    n = max(1, min(7, os.cpu_count() or 1))
    lines = _gram_launches([(1, 24, 60, 48, 84, 128, 256, fill, i, n) for i in range(n)])
    written = [_written(line) for line in lines]
    assert sum(w for w, _ in written) == 24 * 59 and sum(g for _, g in written) == 24 * 59, lines


PARITY = {n: P.EDGE[n] for n in ("d32_bf16", "d64_bf16", "d16_bf16", "d32_f32", "ragged_f32_128", "no_text_bf16",
                                  "T1_bf16", "T2_f32", "chunk3_bf16", "batch2_bf16", "U1_bf16_128", "U2_f32_16")}
PARITY["tiny_f32"] = synth.WORKLOADS["tiny_f32"]
PARITY["ragged_bf16_128"] = P.EDGE["ragged_bf16_128"]


def _case(lib, w, scan=None, bridge=False, rms=False):
    x = synth.make_inputs(w)
    rw = np.random.default_rng(5).uniform(0.5, 1.5, w.d) if rms else None
    tol = G.TOL[w.dtype]
    out, ws, desc = S.run_forward(lib, x, w, epilogue=False, bridge=bridge, scan=scan)
    inter = S.intermediates(lib, ws, desc, w)
    out2, _, _ = S.run_forward(lib, x, w, epilogue=True, rms_weight=rw, bridge=bridge, scan=scan)
    heads = list(range(w.H))
    ref = P._oracle_heads(x, w, heads, gate=True, rms_weight=rw, bridge=bridge)
    err_o = G.slice_rel_err(S.to_f64(out), ref["o"])
    err_y = G.slice_rel_err(S.to_f64(out2), ref["y"])
    P._check_intermediates(inter, ref, w, heads, tol)
    assert err_o <= tol, err_o
    assert err_y <= tol, err_y


# both scans on every case but the two-batch one (the slowest; the frame scan)
PARITY_RUNS = [(n, s) for n in PARITY for s in P.SCANS if not (n == "batch2_bf16" and s == "chunks")]


@pytest.mark.parametrize("name,scan", PARITY_RUNS, ids=[f"{n}-{s}" for n, s in PARITY_RUNS])
def test_forward_matches_oracle(lib, name, scan):
    _case(lib, PARITY[name], scan=scan, rms=name.endswith("128") or name == "d32_bf16")


@pytest.mark.parametrize("name", ["bridge_chunk3_bf16", "bridge_d16_f32"])
def test_decay_bridge_matches_oracle(lib, name):
    _case(lib, P.BRIDGE[name], bridge=True)


def _prep_refs(x, w, b, h):
    sl = lambda a: a[b, :, :, h:h + 1]
    f = G.oracle_view({"q": sl(x["q"]), "k": sl(x["k"]), "v": sl(x["v"])}, w)
    wsl = lambda n: x[n][h * w.d:(h + 1) * w.d].astype(np.float64)
    return oracle.prep(f["q"], f["k"], f["v"], wsl("wk_s"), wsl("wk_t"), wsl("wv_s"), wsl("wv_t"),
                       w.grid_h, w.grid_w, l2_eps=1e-6)


PREP = {
    "prep_small_bf16": dict(H=2, T=9, grid_h=6, grid_w=10, L=8),
    "prep_small_f32": dict(H=2, T=9, grid_h=6, grid_w=10, L=8, dtype="f32"),
    "prep_T2_ragged": P.PREP_EDGE["prep_T2_ragged"],
    "prep_H8_tiles": dict(H=8, T=4, grid_h=9, grid_w=13, L=4),
}
PREP.update(GW.PREP_CASES)  # widths between the built ones


@pytest.mark.parametrize("name", list(PREP))
def test_prepare_matches_oracle(lib, name):
    w = synth.WORKLOADS["long_prep_bf16"].scaled(name=name, **PREP[name])
    x = synth.make_inputs(w)
    qh, kh, vh = S.run_prepare(lib, x, w)
    tol = 1e-2 if w.dtype == "bf16" else 1e-5
    for b in range(w.B):
        for h in range(w.H):
            rq, rk, rv = _prep_refs(x, w, b, h)
            for n, ref, got in (("q", rq, qh), ("k", rk, kh), ("v", rv, vh)):
                e = G.slice_rel_err(S.to_f64(got[b:b + 1, :, :, h:h + 1]), ref[None])
                assert e <= tol, (n, b, h, e)
    # the prepare that leaves the query to the readout writes the same K^, V^
    qn, kf, vf = S.run_prepare(lib, x, w, query_l2=True)
    assert qn is None and np.array_equal(kf, kh) and np.array_equal(vf, vh)


@pytest.mark.parametrize("name", ["ql2_bf16_128", "ql2_bf16_32", "ql2_f32_128"])
def test_query_l2_matches_oracle(lib, name):
    """Prepare under VDN_VDA_QUERY_L2, then the raw query into the forward pass,
    against the oracle on the prepared features."""
    w = synth.WORKLOADS["long_prep_bf16"].scaled(name=name, **P.QL2[name])
    x = synth.make_inputs(w)
    heads = list(range(w.H))
    _, kf, vf = S.run_prepare(lib, x, w, query_l2=True)
    refs = [_prep_refs(x, w, 0, h) for h in heads]
    prepared = {n: np.concatenate([r[i] for r in refs], axis=2)[None] for i, n in enumerate(("q", "k", "v"))}
    rw = np.random.default_rng(11).uniform(0.5, 1.5, w.d)
    for epi, gain in ((False, None), (True, rw)):
        out, _, _ = S.run_forward(lib, x, w, epilogue=epi, rms_weight=gain, query_l2=True, inputs={"k": kf, "v": vf})
        ref = P._oracle_heads(x, w, heads, gate=True, rms_weight=gain, prepared=prepared)
        assert G.slice_rel_err(S.to_f64(out), ref["y" if epi else "o"]) <= G.TOL[w.dtype], (epi,)


def test_values_beyond_the_half_range(lib):
    """|sqrt(beta) v| far above 65504 in two video frames and the text frame:
    the statistics kernel's recovery path (the unit contracted again on
    power-of-two scaled operands) against the oracle."""
    w = P.EDGE["ragged_bf16_128"]
    x = synth.make_inputs(w)
    v = oracle.widen_bf16_bits(x["v"])
    v[:, 3, :30, 1] *= 1.0e5
    v[:, 7, 50:, 0] *= 3.0e4
    x["v"] = synth.f64_to_bf16_bits(v)
    vt = oracle.widen_bf16_bits(x["v_text"])
    vt[:, :5, 2] *= 2.0e5
    x["v_text"] = synth.f64_to_bf16_bits(vt)
    out, ws, desc = S.run_forward(lib, x, w, epilogue=True)
    inter = S.intermediates(lib, ws, desc, w)
    ref = P._oracle_heads(x, w, list(range(w.H)), gate=True)
    tol = G.TOL[w.dtype]
    assert np.isfinite(S.to_f64(out)).all()
    assert G.slice_rel_err(S.to_f64(out), ref["y"]) <= tol
    assert G.mat_rel_err(inter["B"][:, :, 1:w.T - 1], ref["B"][:, :, 1:w.T - 1]) <= tol
    assert G.mat_rel_err(inter["S_T"], ref["S_T"]) <= tol


# ---------------------------------------------------------------------------
# head widths between the built ones (zero-padded to the next), with the
# checks of the GPU width tests
# ---------------------------------------------------------------------------
WIDTHS = [n for n in GW.CASES if n != "d112_768p_frame"]


@pytest.mark.parametrize("name", WIDTHS)
def test_padded_widths_match_oracle(lib, name):
    w = GW.CASES[name]
    x = synth.make_inputs(w)
    heads = list(range(w.H))
    rw = np.random.default_rng(5).uniform(0.5, 1.5, w.d)
    tol = G.TOL[w.dtype]
    scan = "chunks" if name.endswith("chunk3") else "frames"
    out, _, _ = S.run_forward(lib, x, w, epilogue=False, scan=scan)
    assert G.slice_rel_err(S.to_f64(out), P._oracle_heads(x, w, heads, gate=False)["o"]) <= tol
    for gain in (None, rw):
        y, _, _ = S.run_forward(lib, x, w, epilogue=True, rms_weight=gain, scan=scan,
                                bridge=name == "d48_f32")
        ref = P._oracle_heads(x, w, heads, gate=True, rms_weight=gain, bridge=name == "d48_f32")
        assert G.slice_rel_err(S.to_f64(y), ref["y"]) <= tol, gain is not None


@pytest.mark.parametrize("name", list(GW.BWD_CASES))
def test_padded_width_backward_matches_oracle(lib, name):
    import test_gpu_backward as GB
    case = GW.BWD_CASES[name]
    w, epi, bridge = case["w"], case.get("epilogue", True), case.get("bridge", False)
    x = synth.make_inputs(w)
    dy = GB._dy(w)
    gain = np.random.default_rng(5).uniform(0.5, 1.5, w.d) if case.get("gain") else None
    _, fws, _ = S.run_forward(lib, x, w, epilogue=epi, rms_weight=gain, bridge=bridge)
    got, _, _ = S.run_backward(lib, x, w, dy, fws, epilogue=epi, rms_weight=gain, bridge=bridge, gain=epi)
    got = {k: S.to_f64(v) for k, v in got.items() if v is not None}
    errs = GW.backward_errors(got, GW.backward_reference(x, w, dy, epi, gain, bridge), w, epi)
    bad = {k: v for k, v in errs.items() if not v <= G.TOL[w.dtype]}
    assert not bad, bad


import test_gpu_training_f32 as GT  # noqa: E402


@pytest.mark.parametrize("name", list(GT.CASES))
def test_f32_backward_matches_oracle(lib, name):
    case = GT.CASES[name]
    w, epi, bridge, ql2 = case["w"], case.get("epilogue", True), case.get("bridge", False), case.get("query_l2", False)
    x = synth.make_inputs(w)
    if ql2:
        GT.raw_queries(x, w)
    dy = GT._dy(w)
    gain = np.random.default_rng(5).uniform(0.5, 1.5, w.d) if case.get("gain") else None
    _, fws, _ = S.run_forward(lib, x, w, epilogue=epi, rms_weight=gain, bridge=bridge, query_l2=ql2)
    got, _, _ = S.run_backward(lib, x, w, dy, fws, epilogue=epi, rms_weight=gain, bridge=bridge, query_l2=ql2,
                               gain=epi)
    got = {k: S.to_f64(v) for k, v in got.items() if v is not None}
    errs = GW.backward_errors(got, GT.reference(x, w, dy, epi, gain, bridge, ql2), w, epi)
    bad = {k: v for k, v in errs.items() if not v <= G.TOL["f32"]}
    assert not bad, bad
    # records are read in every case, so the frames' keys reach the output
    assert np.abs(got["dk"]).max() > 0


# ---------------------------------------------------------------------------
# the backward pass: the three stages against the oracle's gradients, with the
# checks of the GPU backward tests
# ---------------------------------------------------------------------------
import test_gpu_backward as GB  # noqa: E402
from oracle import vda_grad  # noqa: E402

BWD = ["bwd_128", "bwd_128_raw", "bwd_64_ragged", "bwd_32_bridge", "bwd_64_bridge", "bwd_16_chunk3",
       "bwd_64_no_text", "bwd_128_ql2", "bwd_16_ql2", "bwd_T1", "bwd_T2", "bwd_B2_chunk3", "bwd_128_gain", "bwd_16"]


@pytest.mark.parametrize("name", BWD)
def test_backward_matches_oracle(lib, name):
    case = GB.CASES[name]
    w, epi, bridge, ql2 = case["w"], case.get("epilogue", True), case.get("bridge", False), case.get("query_l2", False)
    x = synth.make_inputs(w)
    if ql2:
        GB._raw_queries(x, w)
    dy = GB._dy(w)
    rw = np.random.default_rng(5).uniform(0.5, 1.5, w.d) if case.get("gain") else None
    _, fws, _ = S.run_forward(lib, x, w, epilogue=epi, rms_weight=rw, bridge=bridge, query_l2=ql2)
    got, bws, lay = S.run_backward(lib, x, w, dy, fws, epilogue=epi, rms_weight=rw, bridge=bridge, query_l2=ql2,
                                   l2_eps=GB.L2_EPS, gain=epi)
    f = G.oracle_view({k: x[k] for k in ("q", "k", "v", "beta", "k_text", "v_text", "beta_text", "gate")}, w)
    # the gain's gradient is formed with the epilogue, at a gain of ones when none is given
    gain = rw if rw is not None else (np.ones(w.d) if epi else None)
    ref = vda_grad.backward(f["q"], f["k"], f["v"], x["alpha"].astype(np.float64), f["beta"], f["k_text"],
                            f["v_text"], f["beta_text"], G.oracle_view({"dy": dy}, w)["dy"],
                            gate=f["gate"] if epi else None, rms_weight=gain, chunk=w.chunk, bridge=bridge,
                            query_l2=GB.L2_EPS if ql2 else None)
    B, H, T, U, d, L = w.B, w.H, w.T, w.U, w.d, w.L
    nc = -(-T // w.chunk)
    do_want = np.moveaxis(ref["do"], 1, 3)
    if ql2:
        do_want = do_want / np.sqrt(np.sum(f["q"] ** 2, axis=-1, keepdims=True) + GB.L2_EPS)
    fr = slice(1, max(T - 1, 1))
    sym = lambda a: a + np.swapaxes(a, -1, -2)
    sec = lambda off, shape, dt="f32": S.section(bws, off, shape, dt)
    dA, dB = sec(lay.d_a, (B, H, T + 1, d, d)), sec(lay.d_b, (B, H, T + 1, d, d))
    lam_f, lam_r = sec(lay.lam_f, (B, H, T + 1, d, d)), sec(lay.lam_r, (B, H, T + 1, d, d))
    errs = {
        "dq": G.slice_rel_err(S.to_f64(got["dq"]), ref["dq"]),
        "do": G.slice_rel_err(sec(lay.d_out, (B, T, U, H, d), "bf16") if epi else G.oracle_view({"dy": dy}, w)["dy"],
                              do_want),
        "dS_q": G.mat_rel_err(sec(lay.d_state_q, (B, H, T, d, d)), ref["dS_q"]),
        "dF": GB._rel(sec(lay.d_record_f, (B, H, nc, d, d))[:, :, :max(nc - 2, 0)], ref["dF"][:, :, :max(nc - 2, 0)]),
        "dR": GB._rel(sec(lay.d_record_r, (B, H, nc, d, d))[:, :, 2:], ref["dR"][:, :, 2:]),
        "lam_f": GB._rel(lam_f[:, :, fr], ref["dfwd"][:, :, fr]),
        "lam_r": GB._rel(lam_r[:, :, fr], ref["drev"][:, :, fr]),
        "dS_T": GB._rel(lam_f[:, :, T], ref["dS_T"]),
        "dA": GB._rel(sym(dA[:, :, fr]), sym(ref["dA"][:, :, fr])),
        "dB": GB._rel(dB[:, :, fr], ref["dB"][:, :, fr]),
        "dA_T": GB._rel(sym(dA[:, :, T]), sym(ref["dA_T"])) if L else 0.0,
        "dB_T": GB._rel(dB[:, :, T], ref["dB_T"]) if L else 0.0,
        "dalpha": GB._rel(got["dalpha"].astype(np.float64), ref["dalpha"]),
        "dk": G.slice_rel_err(S.to_f64(got["dk"]), ref["dk"]),
        "dv": G.slice_rel_err(S.to_f64(got["dv"]), ref["dv"]),
        "dbeta": G.slice_rel_err(S.to_f64(got["dbeta"])[..., None], ref["dbeta"][..., None]),
    }
    if epi:
        errs["dgate"] = G.slice_rel_err(S.to_f64(got["dgate"]), ref["dgate"])
        errs["dgamma"] = GB._rel(got["dgamma"].astype(np.float64), ref["dgamma"])
    if L:
        txt = lambda a: a.reshape((B, 1) + a.shape[1:] + ((1,) if a.ndim == 3 else ()))
        errs.update({"dk_text": G.slice_rel_err(txt(S.to_f64(got["dk_text"])), txt(ref["dk_txt"])),
                     "dv_text": G.slice_rel_err(txt(S.to_f64(got["dv_text"])), txt(ref["dv_txt"])),
                     "dbeta_text": G.slice_rel_err(txt(S.to_f64(got["dbeta_text"])), txt(ref["dbeta_txt"]))})
    bad = {k: v for k, v in errs.items() if not v <= G.TOL[w.dtype]}
    assert not bad, bad
    # the anchors take no part in any scan, and their tokens reach no state
    assert np.abs(dA[:, :, [0, T - 1]]).max() == 0 and np.abs(dB[:, :, [0, T - 1]]).max() == 0
    for k in ("dk", "dv", "dbeta"):
        assert np.abs(S.to_f64(got[k])[:, [0, T - 1]]).max() == 0, k


@pytest.mark.parametrize("name", ["bwd_128_gain", "bwd_16", "bwd_64_ql2_gain"])
def test_gain_gradient_changes_nothing_else(lib, name):
    """The readout variant that also forms the gain's gradient leaves dq, dgate
    and every later gradient bit for bit as the variant without, and gives the
    same gradient on a second call."""
    case = GB.CASES[name]
    w, bridge, ql2 = case["w"], case.get("bridge", False), case.get("query_l2", False)
    x = synth.make_inputs(w)
    if ql2:
        GB._raw_queries(x, w)
    dy = GB._dy(w)
    rw = np.random.default_rng(5).uniform(0.5, 1.5, w.d)
    _, fws, _ = S.run_forward(lib, x, w, epilogue=True, rms_weight=rw, bridge=bridge, query_l2=ql2)
    runs = [S.run_backward(lib, x, w, dy, fws, epilogue=True, rms_weight=rw, bridge=bridge, query_l2=ql2,
                           l2_eps=GB.L2_EPS, gain=g)[0] for g in (False, True, True)]
    for k, v in runs[0].items():
        if v is not None:
            assert np.array_equal(v.view(np.uint8), runs[1][k].view(np.uint8)), k
    assert np.array_equal(runs[1]["dgamma"], runs[2]["dgamma"])
    assert np.isfinite(runs[1]["dgamma"]).all()


# ---------------------------------------------------------------------------
# the adjacent linear maps, with the checks of the GPU adjacent-map tests
# ---------------------------------------------------------------------------
import test_gpu_adjacent as GA  # noqa: E402
from oracle import vda_adjacent as adj  # noqa: E402


ADJ = dict(GA.CASES, **GW.ADJ_CASES)


@pytest.mark.parametrize("name", list(ADJ))
def test_gates_match_oracle(lib, name):
    w, dm = ADJ[name]
    p = synth.make_adjacent_inputs(w, dm)
    gate, beta, alpha = S.run_gates(lib, p, w, dm)
    wg = GA._f64(p["w_gb"])
    g_ref, b_ref, a_ref = adj.gate_proj(GA._f64(p["x"]), wg[: w.H * w.d], wg[w.H * w.d:], GA._f64(p["w_alpha"]),
                                        w.H, w.d)
    assert G.slice_rel_err(S.to_f64(gate), g_ref) <= 2e-2
    assert G.slice_rel_err(GA._slices(S.to_f64(beta)), GA._slices(b_ref)) <= 2e-2
    assert np.abs(alpha.astype(np.float64) - a_ref).max() <= 1e-5


@pytest.mark.parametrize("mode", ["y_in", "in_place", "no_y_in"])
@pytest.mark.parametrize("name", list(ADJ))
def test_out_proj_matches_oracle(lib, name, mode):
    w, dm = ADJ[name]
    p = synth.make_adjacent_inputs(w, dm)
    y = S.run_out_proj(lib, p, w, mode)
    ref = adj.out_proj(GA._f64(p["o"]), GA._f64(p["w_o"]), None if mode == "no_y_in" else GA._f64(p["y_in"]))
    assert G.slice_rel_err(GA._slices(S.to_f64(y)), GA._slices(ref)) <= 2e-2


def _sweep(path, args, env, shards=max(1, min(6, os.cpu_count() or 1))):
    """tests/cpu_build/san_cases.py on the library at ``path``, its cases split
    over ``shards`` processes run at once; (exit status, stdout + stderr) of
    each."""
    import sys
    script = os.path.join(os.path.dirname(CB.__file__), "san_cases.py")
    procs = [subprocess.Popen([sys.executable, script, path, *args, f"--shard={i}/{shards}"], stdout=subprocess.PIPE,
                              stderr=subprocess.STDOUT, text=True, env=env) for i in range(shards)]
    results = []
    for p in procs:
        try:
            out, _ = p.communicate(timeout=1800)
        except subprocess.TimeoutExpired:
            p.kill()
            out, _ = p.communicate()
        results.append((p.returncode, out))
    return results


def test_every_entry_point_under_sanitizers():
    """tests/cpu_build/san_cases.py on the sanitized library: every entry point
    (forward in both scans, with the bridge and the fused query norm, the
    no-allocation forward, prepare, the three backward stages, the gates and
    the output projection) with AddressSanitizer and UndefinedBehaviorSanitizer."""
    path = CB.build(S.OUT, "lib_san")
    env = dict(os.environ, LD_PRELOAD=CB.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_stack_use_after_return=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    for rc, out in _sweep(path, [], env):
        assert rc == 0 and "all entry points ran" in out, out[-6000:]
        assert "runtime error" not in out and "Sanitizer" not in out and "[simt]" not in out, out[-6000:]


@pytest.mark.skipif(os.environ.get("VDA_CPU_BUILD_FULL") != "1",
                    reason="all 24 heads of the 768p clip through the sanitized build, about 13 minutes: "
                           "set VDA_CPU_BUILD_FULL=1")
def test_every_768p_head_under_sanitizers():
    """tests/cpu_build/san_cases.py --heavy: the forward (both scans) and the
    backward with all 24 heads of the 768p clip at its frame size, under
    AddressSanitizer and UndefinedBehaviorSanitizer."""
    import sys
    path = CB.build(S.OUT, "lib_san")
    env = dict(os.environ, LD_PRELOAD=CB.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_stack_use_after_return=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(CB.__file__), "san_cases.py"), path, "--heavy"],
                       capture_output=True, text=True, timeout=3600, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "all entry points ran: 1 cases" in r.stdout, out[-6000:]
    assert "runtime error" not in out and "Sanitizer" not in out and "[simt]" not in out, out[-6000:]


# ---------------------------------------------------------------------------
# seeded random shapes and flags, forward and backward against the oracle
# ---------------------------------------------------------------------------
def _random_case(seed):
    rng = np.random.default_rng(seed)
    dtype = str(rng.choice(["bf16", "f32"]))
    base = synth.WORKLOADS["768p_bf16" if dtype == "bf16" else "stress_f32"]
    # no single-token text frame: with one text token S_T has rank one, every
    # output of the frames that read it points along that token's value, the
    # RMSNorm output depends on q there only through its epsilon and the true
    # dq is proportional to epsilon, so a per-slice relative error measures
    # rounding against a near-zero reference
    w = base.scaled(name=f"random_{seed}", dtype=dtype, d=int(rng.choice([16, 32, 64, 128])),
                    B=int(rng.choice([1, 1, 2])), H=int(rng.integers(1, 5)), T=int(rng.integers(1, 14)),
                    grid_h=int(rng.integers(1, 9)), grid_w=int(rng.integers(1, 12)),
                    L=int(rng.choice([0, 3, 17, 40])), chunk=int(rng.integers(1, 7)))
    fl = dict(bridge=bool(rng.random() < 0.3), scan=[None, "frames", "chunks"][int(rng.integers(3))],
              epilogue=bool(rng.random() < 0.7), gain=bool(rng.random() < 0.3),
              backward=bool(dtype == "bf16" and rng.random() < 0.6))
    return w, fl


@pytest.mark.parametrize("seed", range(40))
def test_random_shapes_match_oracle(lib, seed):
    w, fl = _random_case(4000 + seed)
    x = synth.make_inputs(w)
    rw = np.random.default_rng(5).uniform(0.5, 1.5, w.d) if fl["gain"] else None
    out, ws, desc = S.run_forward(lib, x, w, epilogue=fl["epilogue"], rms_weight=rw, bridge=fl["bridge"],
                                  scan=fl["scan"])
    heads = list(range(w.H))
    ref = P._oracle_heads(x, w, heads, gate=True, rms_weight=rw, bridge=fl["bridge"])
    tol = G.TOL[w.dtype]
    P._check_intermediates(S.intermediates(lib, ws, desc, w), ref, w, heads, tol)
    assert G.slice_rel_err(S.to_f64(out), ref["y" if fl["epilogue"] else "o"]) <= tol, (w, fl)
    if not fl["backward"]:
        return
    dy = GB._dy(w)
    got, _, _ = S.run_backward(lib, x, w, dy, ws, epilogue=fl["epilogue"], rms_weight=rw, bridge=fl["bridge"])
    f = G.oracle_view({k: x[k] for k in ("q", "k", "v", "beta", "k_text", "v_text", "beta_text", "gate")}, w)
    gref = vda_grad.backward(f["q"], f["k"], f["v"], x["alpha"].astype(np.float64), f["beta"], f["k_text"],
                             f["v_text"], f["beta_text"], G.oracle_view({"dy": dy}, w)["dy"],
                             gate=f["gate"] if fl["epilogue"] else None, rms_weight=rw, chunk=w.chunk,
                             bridge=fl["bridge"])
    errs = {k: G.slice_rel_err(S.to_f64(got[k]), gref[k]) for k in ("dq", "dk", "dv")}
    errs["dalpha"] = GB._rel(got["dalpha"].astype(np.float64), gref["dalpha"])
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, (w, fl, bad)


# ---------------------------------------------------------------------------
# the emulator's own checks fire (tests/cpu_build/selftest.cpp)
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def selftest_exe():
    return CB.build(S.OUT, "selftest")


def _selftest(exe, case):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:detect_stack_use_after_return=0")
    return subprocess.run([exe, case], capture_output=True, text=True, timeout=300, env=env)


def test_emulated_mfma_layouts(selftest_exe):
    """Every matrix-core shape against a float64 product of its operands in
    the layout the emulator states (the library's kernels, built against the
    same layouts, match the oracle through the emulator and on the GPU)."""
    r = _selftest(selftest_exe, "mfma")
    assert r.returncode == 0 and "0 mismatches" in r.stdout, r.stdout + r.stderr


def test_emulator_reports_planted_faults(selftest_exe):
    """A buffer offset that wraps 2^32, unequal barrier counts and a cross-lane
    operation reached by half a wave are reported; loads past num_records read
    zero and stores there are dropped."""
    r = _selftest(selftest_exe, "wrap")
    assert r.returncode == 0 and "wraps 2^32" in r.stderr, r.stdout + r.stderr
    r = _selftest(selftest_exe, "range")
    assert r.returncode == 0, r.stdout + r.stderr
    r = _selftest(selftest_exe, "barriers")
    assert r.returncode == 0 and "barriers" in r.stderr, r.stdout + r.stderr
    r = _selftest(selftest_exe, "diverge")
    assert r.returncode != 0 and "deadlock" in r.stderr, r.stdout + r.stderr


def test_emulator_poisons_lds_between_workgroups():
    """In the library the parity tests run (built with SIMT_LDS_POISON), a
    workgroup that reads LDS it did not write gets all-ones bytes, not the
    previous workgroup's values (the first eight workgroups of a launch and
    every 32nd after start poisoned): the parity tests then also check that no
    kernel reads LDS it has not written."""
    exe = CB.build(S.OUT, "selftest_poison")
    r = subprocess.run([exe, "poison"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "reads ffffffff" in r.stdout, r.stdout + r.stderr


def test_emulator_splits_a_launch(selftest_exe):
    """A launch split over processes runs, in each, exactly its share of the
    workgroups (every third from the second), and all of them once undone."""
    r = _selftest(selftest_exe, "shard")
    assert r.returncode == 0 and "shard: ok" in r.stdout, r.stdout + r.stderr


# ---------------------------------------------------------------------------
# data races (ThreadSanitizer over the emulator's schedule): every lane a fiber
# of its own, ordered with the other lanes of its wave only by the wave's
# cross-lane operations and wave barriers and with the rest of the workgroup
# only by its barriers -- so both a race between waves and an exchange between
# lanes of one wave through memory with nothing between write and read (which
# on the hardware relies on the compiler keeping program order) are reported
# ---------------------------------------------------------------------------
def _tsan_run(exe, args, lanes=True):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=0:exitcode=66", SIMT_TSAN_LANES="1" if lanes else "0")
    return subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=900, env=env)


def test_race_detector_reports_planted_race():
    exe = CB.build(S.OUT, "selftest_tsan")
    r = _tsan_run(exe, ["race"])
    assert r.returncode == 66 and "data race" in r.stderr, r.stdout + r.stderr[-3000:]
    r = _tsan_run(exe, ["norace"])
    assert r.returncode == 0 and "ThreadSanitizer" not in r.stderr, r.stdout + r.stderr[-3000:]


def test_race_detector_reports_an_unsynchronised_exchange_between_lanes():
    """Lane 0 writes a word that lane 1 of the same wave reads: reported with a
    fiber per lane unless a wave barrier separates them; one fiber per wave (the
    lockstep view) sees no race either way."""
    exe = CB.build(S.OUT, "selftest_tsan")
    r = _tsan_run(exe, ["lanerace"])
    assert r.returncode == 66 and "data race" in r.stderr, r.stdout + r.stderr[-3000:]
    r = _tsan_run(exe, ["lanesync"])
    assert r.returncode == 0 and "ThreadSanitizer" not in r.stderr, r.stdout + r.stderr[-3000:]
    r = _tsan_run(exe, ["lanerace"], lanes=False)
    assert r.returncode == 0 and "ThreadSanitizer" not in r.stderr, r.stdout + r.stderr[-3000:]


TSAN_SHAPES = [(2, 6, 6, 11, 128, 12, "bf16"), (3, 7, 5, 9, 64, 37, "bf16"), (2, 6, 6, 11, 16, 12, "bf16"),
               (2, 6, 6, 11, 128, 12, "f32")]


@pytest.mark.parametrize("shape", TSAN_SHAPES, ids=["x".join(map(str, s)) for s in TSAN_SHAPES])
def test_forward_has_no_race(shape):
    exe = CB.build(S.OUT, "check_tsan")
    r = _tsan_run(exe, shape)
    assert r.returncode == 0 and "ThreadSanitizer" not in r.stderr, r.stdout + r.stderr[-4000:]


def test_every_entry_point_has_no_race():
    """tests/cpu_build/san_cases.py --tsan on the ThreadSanitizer build, a fiber
    per lane: every entry point, no data race between waves and no exchange
    between lanes of a wave without a wave-level synchronisation."""
    path = CB.build(S.OUT, "lib_tsan")
    env = dict(os.environ, LD_PRELOAD=CB.sanitizer_runtime("tsan"), TSAN_OPTIONS="halt_on_error=0:exitcode=66",
               SIMT_TSAN_LANES="1", OPENBLAS_NUM_THREADS="1")
    for rc, out in _sweep(path, ["--tsan"], env):
        assert rc == 0 and "all entry points ran" in out, out[-6000:]
        assert "ThreadSanitizer" not in out, out[-6000:]


# ---------------------------------------------------------------------------
# the GPU suite's own Python on the host library (tests/cpu_build/gpu_suite_on_host.py)
# ---------------------------------------------------------------------------
ON_HOST = ["tests/test_gpu_rms_gain.py::test_gain_gradient[bwd_16]",
           "tests/test_gpu_widths.py::test_padded_width_forward[d48_T1_bf16-frames]",
           "tests/test_gpu_widths.py::test_padded_width_backward[bwd_d80_raw_bridge]",
           "tests/test_gpu_widths.py::test_padded_width_gates[adj_d48]",
           "tests/test_gpu_training_f32.py::test_backward_f32[tiny_f32_gain]",
           "tests/test_gpu_backward.py::test_backward_readout[bwd_16]"]


def test_gpu_test_code_runs_on_the_host_library():
    """A few cases of each GPU test file run on the CPU build (the full
    selection with VDA_CPU_BUILD_FULL=1: every case but the full-size ones)."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if os.environ.get("VDA_CPU_BUILD_FULL"):
        args = ["tests/test_gpu_parity.py", "tests/test_gpu_backward.py", "tests/test_gpu_adjacent.py",
                "tests/test_gpu_rms_gain.py", "tests/test_gpu_widths.py", "tests/test_gpu_training_f32.py",
                "tests/test_zz_no_alloc.py", "-k", "not 768p and not long_prep and not stress and not workload_full"]
    else:
        args = ON_HOST
    r = subprocess.run([sys.executable, "tests/cpu_build/gpu_suite_on_host.py", *args, "-m", "gpu"], cwd=root,
                       capture_output=True, text=True, timeout=3600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
