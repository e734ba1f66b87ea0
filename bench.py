#!/usr/bin/env python3
"""Benchmark of the VDA forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 768p_bf16]

A step is one whole forward pass (frame statistics, text state, solve,
bidirectional scan, gather, readout with RMSNorm and the sigmoid gate; plus
prep for the long-clip workload) over one batch of seeded synthetic input
already resident in HBM.  Prints one JSON line.  Per-stage kernel times come
from HIP events that the library records on the launch stream between its
kernels; the dominant stage is priced against the HBM roofline with its
algorithmic bytes.  The oracle's time on a bounded sample of the same workload
is reported as the CPU baseline.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "VDA fwd+rev scan+readout frames/s & tokens/s per GPU; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
STAGE_SOURCES = {"gram": "vda_gram.hip", "solve": "vda_solve.hip",
                 "scan": "vda_scan.hip", "gather": "vda_scan.hip", "readout": "vda_readout.hip",
                 "prep": "vda_prep.hip"}


class Hip:
    """The few HIP runtime calls the timing needs (events on the launch stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, ctypes.c_void_p(stream)) == 0

    def elapsed(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventSynchronize(b) == 0
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


# kernel launches per stage and step (the prep kernel runs once on K, once on V)
LAUNCHES_PER_STAGE = {"prep": 2}


def algorithmic_bytes(w, stage: str) -> int:
    """Bytes a stage must move at minimum per step (inputs read once, outputs written once)."""
    esz = 2 if w.dtype == "bf16" else 4
    tok = w.B * w.T * w.U * w.H          # token-heads
    if stage == "gram":                  # K_t, V_t and beta_t of frames 1..T-2
        n = w.B * max(w.T - 2, 0) * w.U * w.H
        return n * (2 * w.d + 1) * esz
    if stage == "readout":               # Q and the gate logits in, O out
        return tok * 3 * w.d * esz
    if stage == "prep":                  # K, V in; K^, V^ out (Q's L2 is fused into the readout)
        return tok * 4 * w.d * esz
    return 0


# the prep's arithmetic per output element: a 5 x 5 spatial and a 5-tap temporal
# depthwise filter, 30 fp32 multiply-adds
PREP_FLOP_PER_OUTPUT = 60
# fp32 FMA without packed instructions (packed fp32 is off in every HIP build
# here): 256 CUs x 4 SIMDs x 16 lanes x 2 FLOP x 2.4 GHz; with packed
# instructions the chip's figure is twice this, 157.3 TFLOP/s
VALU_F32_PEAK_TFLOPS = 78.6


def prep_flops(w) -> int:
    """fp32 FLOP of one prep launch (one of K, V)."""
    return w.B * w.T * w.U * w.H * w.d * PREP_FLOP_PER_OUTPUT


def dominant_roofline(w, dom: str, dom_ms: float, dom_bytes: int, traffic, launches: int) -> dict:
    """The bench line's roofline object for the dominant kernel: one launch's
    algorithmic bytes over its average duration against the HBM peak, or for
    the prep, its fp32 FLOP against the ALU peak with the HBM rate beside it."""
    ach = dom_bytes / (dom_ms * 1e-3) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": traffic, "algorithmic_bytes": dom_bytes,
                "launch_ms": round(dom_ms, 4), "launches_per_step": launches}
    if dom == "prep":
        # the filter's fp32 arithmetic binds before its bytes do: 60 FLOP per
        # 4 bytes moved (one bfloat16 in, one out) is above the 9.8 FLOP/B
        # ridge of 78.6 TFLOP/s over 8 TB/s
        tf = prep_flops(w) / (dom_ms * 1e-3) / 1e12
        roofline.update({"bound": "alu", "achieved": round(tf, 2), "peak": VALU_F32_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / VALU_F32_PEAK_TFLOPS, 4),
                         "flops": prep_flops(w),
                         "hbm": {"achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(ach / HBM_PEAK_GBS, 4)}})
    return roofline


def job_bytes(w) -> int:
    """Whole-job algorithmic bytes, each byte the method needs moved once: Q and
    the gate logits of every frame in, O out; K, V, beta and alpha of the
    frames the scans absorb (1..T-2: the anchors are never absorbed); the text
    tokens' K, V, beta.  With the prep, K and V of every frame are read (the
    temporal taps reach the anchors).  The prepared K^, V^ are intermediates
    and are not counted."""
    esz = 2 if w.dtype == "bf16" else 4
    tok = w.B * w.T * w.U * w.H
    inner = w.B * max(w.T - 2, 0) * w.U * w.H
    kv_tok = tok if w.prep else inner
    n = tok * 3 * w.d * esz + kv_tok * 2 * w.d * esz + inner * esz
    n += w.B * max(w.T - 2, 0) * w.H * w.d * 4 + w.B * w.L * w.H * (2 * w.d + 1) * esz
    return n


# algorithmic matrix-core FLOP per launch: the statistics [A; B] = [Z | W]^T Z
# (2d x d outputs over U tokens) and the readout o = S q (d x d per token); the
# readout's hi + lo split of S doubles the executed products, not the
# algorithmic ones
def mfma_flops(w, stage: str) -> int:
    if stage == "gram":
        return 2 * (w.B * max(w.T - 2, 0) * w.H * w.U + w.B * w.H * w.L) * 2 * w.d * w.d
    if stage == "readout":
        return 2 * w.B * w.T * w.U * w.H * w.d * w.d
    return 0


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense: bf16/fp16, fp32 matrix
# the whole job's goal on the 768p workload: 60 % of the HBM roofline
JOB_TARGET_FRAC = 0.6


def mfma_record(w, stage: str, ms: float) -> dict:
    """Matrix-core work of a stage against the dense peak of its operand type,
    and the committed counter's busy fraction (MfmaUtil) when still current."""
    f = mfma_flops(w, stage)
    tf = f / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    busy = counters_for(stage, w.name).get("mfma_util")
    return {"algorithmic_flops": f, "achieved_TFLOPs": round(tf, 1), "peak_TFLOPs": peak,
            "frac": round(tf / peak, 4), "busy_counter": busy}


def copy_peak_gbs(torch, hip, stream, gib: float = 2.0, reps: int = 5) -> float:
    """Bytes read plus written per second by a plain device-to-device copy."""
    n = int(gib * (1 << 30))
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, stream)
    for _ in range(reps):
        dst.copy_(src)
    hip.record(e1, stream)
    ms = hip.elapsed(e0, e1) / reps
    del src, dst
    return 2 * n / (ms * 1e-3) / 1e9


def _sha(stage):
    p = os.path.join(ROOT, "frame_wise_delta_02_amd", "csrc", STAGE_SOURCES[stage])
    return hashlib.sha1(open(p, "rb").read()).hexdigest()[:12]


def counters_for(stage: str, workload: str):
    """The committed counter record of a kernel (HBM bytes per launch, matrix-core
    busy fraction), if its source is unchanged since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return {}
    rec = json.load(open(p)).get(f"{workload}:{stage}")
    if not rec or rec.get("source_sha") != _sha(stage):
        return {}
    return rec


def traffic_for(stage: str, workload: str):
    """Measured HBM bytes per launch from the committed counter summary, if still current."""
    return counters_for(stage, workload).get("bytes_per_launch")


def host_info() -> dict:
    """The host CPU model and the BLAS the oracle's numpy calls."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        import numpy as np
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": model, "blas": blas}


def cpu_baseline(x, w, budget_s: float):
    """The oracle, as it stands, on whole heads of the same inputs until the budget is spent."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    wid = lambda a: oracle.widen_bf16_bits(a) if a.dtype == np.uint16 else a.astype(np.float64)
    t0 = time.perf_counter()
    heads = 0
    for h in range(w.H):
        sl = [h]
        f = {k: wid(x[k][:, :, :, sl]) for k in ("q", "k", "v", "gate")}
        if w.prep:
            ws = lambda n: x[n][h * w.d:(h + 1) * w.d].astype(np.float64)
            f["q"][0], f["k"][0], f["v"][0] = oracle.prep(f["q"][0], f["k"][0], f["v"][0], ws("wk_s"), ws("wk_t"),
                                                          ws("wv_s"), ws("wv_t"), w.grid_h, w.grid_w)
        oracle.forward(f["q"], f["k"], f["v"], x["alpha"][:, :, sl].astype(np.float64),
                       wid(x["beta"][:, :, :, sl]), wid(x["k_text"][:, :, sl]), wid(x["v_text"][:, :, sl]),
                       wid(x["beta_text"][:, :, sl]), gate=f["gate"], chunk=w.chunk)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    full = el * w.H / heads
    return {"value": round(w.B * w.T / full, 4), "unit": "frames/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} of {w.H} heads, all {w.T} frames x {w.U} tokens, {el:.1f} s; "
                      f"scaled to the whole {w.H}-head job ({full:.1f} s)", **host_info()}


BWD_STAGES = ("bwd_readout", "bwd_scan", "bwd_gram")
BWD_SOURCES = {"bwd_readout": "vda_backward.hip", "bwd_scan": "vda_backward.hip", "bwd_gram": "vda_backward.hip"}


def bwd_algorithmic_bytes(w, stage: str) -> int:
    """Bytes a backward stage must move at minimum per step."""
    tok = w.B * w.T * w.U * w.H
    ttok = w.B * w.L * w.H
    dd = w.B * w.H * (w.T + 1) * w.d * w.d * 4
    if stage == "bwd_readout":   # q, gate, dy in; dq, dgate out; dS_q (float32 per frame) out
        return tok * 5 * w.d * 2 + w.B * w.H * w.T * w.d * w.d * 4
    if stage == "bwd_scan":      # dS_q, the statistics A, B and P in; dA, dB, dalpha out
        return dd * 6 + w.B * w.T * w.H * w.d * 4
    if stage == "bwd_gram":      # k, v, beta in; dk, dv, dbeta out (frames and text); dA, dB in
        return (tok + ttok) * (4 * w.d + 2) * 2 + 2 * dd
    return 0


def bench_backward(args, w, x, d, fwd, stream, hip, t_gen) -> int:
    """A training step of the layer: the forward pass, then the three backward
    stages; one JSON line with per-stage times (HIP events around each entry
    point) and the roofline of the slowest backward stage."""
    import numpy as np
    import torch

    from frame_wise_delta_02_amd import binding as bd
    if w.prep or w.dtype != "bf16":
        print("--backward runs bfloat16 workloads without prep", file=sys.stderr)
        return 2
    rng = np.random.default_rng(2024)
    dy = torch.from_numpy(rng.standard_normal(d["q"].shape).astype(np.float32)).to("cuda").to(torch.bfloat16)
    grid = (w.grid_h, w.grid_w)
    desc = bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, w.L, w.chunk, w.dtype, True)
    fws = fwd.workspace  # the forward's workspace, which every fwd() call rewrites
    bws = torch.empty(bd.backward_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    dq, dgate = torch.empty_like(d["q"]), torch.empty_like(d["gate"])
    dalpha = torch.empty((w.B, w.T, w.H, w.d), dtype=torch.float32, device="cuda")
    gout = tuple(torch.empty_like(d[k]) for k in ("k", "v", "beta", "k_text", "v_text", "beta_text"))

    def bwd(evs=None):
        if evs:
            hip.record(evs[0], stream)
        bd.backward_readout(d["q"], d["gate"], None, d["alpha"], dy, fws, grid=grid, n_text=w.L, chunk=w.chunk,
                            dq=dq, dgate=dgate, workspace=bws)
        if evs:
            hip.record(evs[1], stream)
        bd.backward_scan(d["alpha"], fws, bws, shape=(w.B, w.T, w.H, w.d), grid=grid, n_text=w.L,
                         chunk=w.chunk, dalpha=dalpha)
        if evs:
            hip.record(evs[2], stream)
        bd.backward_gram(d["k"], d["v"], d["beta"], d["k_text"], d["v_text"], d["beta_text"], bws, grid=grid,
                         chunk=w.chunk, out=gout)
        if evs:
            hip.record(evs[3], stream)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    wall0 = time.perf_counter()
    hip.record(e0, stream)
    for _ in range(args.steps):
        fwd()
        bwd()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = hip.elapsed(e0, e1) / args.steps
    # per-stage times: forward, then each backward stage
    sets = [[hip.event() for _ in range(5)] for _ in range(args.steps)]
    for evs in sets:
        hip.record(evs[0], stream)
        fwd()
        bwd(evs[1:])
    torch.cuda.synchronize()
    st = {"forward": 0.0, **{k: 0.0 for k in BWD_STAGES}}
    for evs in sets:
        st["forward"] += hip.elapsed(evs[0], evs[1]) / args.steps
        for i, k in enumerate(BWD_STAGES):
            st[k] += hip.elapsed(evs[i + 1], evs[i + 2]) / args.steps
    dom = max(BWD_STAGES, key=lambda k: st[k])
    dom_bytes = bwd_algorithmic_bytes(w, dom)
    ach = dom_bytes / (st[dom] * 1e-3) / 1e9
    frames = w.B * w.T
    rec = {
        "metric": "VDA forward + backward (training step of the layer) frames/s per GPU",
        "value": round(frames / (ms * 1e-3), 2), "unit": "frames/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "U": w.U, "grid": f"{w.grid_h}x{w.grid_w}",
                   "d": w.d, "text_tokens": w.L, "chunk": w.chunk, "state": "f32", "pass": "forward+backward"},
        "tokens_per_s": round(frames * w.U / (ms * 1e-3), 1),
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": dom_bytes,
                     "launch_ms": round(st[dom], 4), "note": "stage window: every launch of the entry point"},
        "stages_ms": {k: round(v, 4) for k, v in st.items()},
        "wall_s_timed": round(wall, 3), "input_gen_s": round(t_gen, 1), "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bfloat16


def bench_adjacent(args, w, d, stream, hip, t_gen) -> int:
    """The path with its adjacent maps: gate logits, beta and alpha from the
    block input x (d_model = H d), the forward pass reading them, then the
    output projection adding Y_in; one JSON line with per-stage times (HIP
    events around each entry point) and the matrix-core roofline of the larger
    GEMM."""
    import numpy as np
    import torch

    from frame_wise_delta_02_amd import binding as bd
    from frame_wise_delta_02_amd import synth
    if w.prep or w.dtype != "bf16":
        print("--adjacent runs bfloat16 workloads without prep", file=sys.stderr)
        return 2
    dm = w.H * w.d
    t0 = time.perf_counter()
    a = synth.make_adjacent_inputs(w, dm)
    t_gen += time.perf_counter() - t0

    def dev(arr):
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16) if arr.dtype == np.uint16 else torch.from_numpy(arr)
        return t.to("cuda")

    xa, wgb, wal, wo, yin = (dev(a[k]) for k in ("x", "w_gb", "w_alpha", "w_o", "y_in"))
    del a
    grid = (w.grid_h, w.grid_w)
    gate, beta, alpha = torch.empty_like(d["gate"]), torch.empty_like(d["beta"]), torch.empty_like(d["alpha"])
    gdesc = bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, 0, w.chunk, "bf16", False)
    gws = torch.empty(bd.lib().vdn_vda_gates_workspace_bytes(ctypes.byref(gdesc), dm), dtype=torch.uint8,
                      device="cuda")
    desc = bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, w.L, w.chunk, w.dtype, True)
    fws = torch.empty(bd.workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(d["q"])
    y = torch.empty_like(yin)

    def step(evs=None):
        rec = (lambda i: hip.record(evs[i], stream)) if evs else (lambda i: None)
        rec(0)
        bd.gates(xa, wgb, wal, heads=w.H, d=w.d, grid=grid, chunk=w.chunk, out=(gate, beta, alpha), workspace=gws)
        rec(1)
        bd.forward(d["q"], d["k"], d["v"], alpha, beta, d["k_text"], d["v_text"], d["beta_text"], gate, None,
                   grid=grid, chunk=w.chunk, epilogue=True, out=o, workspace=fws)
        rec(2)
        bd.out_proj(o, wo, yin, grid=grid, chunk=w.chunk, out=y)
        rec(3)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    wall0 = time.perf_counter()
    hip.record(e0, stream)
    for _ in range(args.steps):
        step()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = hip.elapsed(e0, e1) / args.steps
    sets = [[hip.event() for _ in range(4)] for _ in range(args.steps)]
    for evs in sets:
        step(evs)
    torch.cuda.synchronize()
    names = ("gates", "forward", "out_proj")
    st = {k: 0.0 for k in names}
    for evs in sets:
        for i, k in enumerate(names):
            st[k] += hip.elapsed(evs[i], evs[i + 1]) / args.steps
    M = w.B * w.T * w.U
    flops = {"gates": 2.0 * M * (dm + w.H) * dm, "out_proj": 2.0 * M * dm * dm}
    dom = max(flops, key=lambda k: st[k])
    ach = flops[dom] / (st[dom] * 1e-3) / 1e12
    frames = w.B * w.T
    rec = {
        "metric": "VDA forward with its adjacent linear maps (gates before, output projection after) frames/s per GPU",
        "value": round(frames / (ms * 1e-3), 2), "unit": "frames/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "U": w.U, "grid": f"{w.grid_h}x{w.grid_w}",
                   "d": w.d, "d_model": dm, "text_tokens": w.L, "chunk": w.chunk, "pass": "gates+forward+out_proj"},
        "tokens_per_s": round(frames * w.U / (ms * 1e-3), 1),
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops": flops[dom], "launch_ms": round(st[dom], 4),
                     "note": "stage window: every launch of the entry point"},
        "stages_ms": {k: round(v, 4) for k, v in st.items()},
        "wall_s_timed": round(wall, 3), "input_gen_s": round(t_gen, 1), "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="768p_bf16")
    ap.add_argument("--heads", type=int, default=0,
                    help="run the workload with this many heads instead (0: as defined)")
    ap.add_argument("--scan", choices=["auto", "frames", "chunks"], default="auto",
                    help="force the frame-by-frame or the chunk-composed scan (auto: the library picks)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle budget; 0 skips it")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step of the layer instead: the forward pass, then the three "
                         "backward stages (bfloat16 workloads without prep)")
    ap.add_argument("--adjacent", action="store_true",
                    help="time the path with the linear maps either side of it: gates from the block "
                         "input, the forward pass on them, the output projection (bfloat16 workloads without prep)")
    ap.add_argument("--copy-gib", type=float, default=0.0,
                    help="instead of the forward pass, time a plain device copy of this many GiB "
                         "(the reference for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (VDA heads never "
              f"interact, so a multi-GPU run is head-sharded with no communication inside VDA).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_gib > 0:
        n = int(args.copy_gib * (1 << 30))
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": round(el * 1e3, 4),
                          "GBs": round(2 * n / el / 1e9, 1)}), flush=True)
        return 0

    from frame_wise_delta_02_amd import binding as bd
    from frame_wise_delta_02_amd import synth

    w = synth.WORKLOADS[args.workload]
    if args.heads > 0:
        w = w.scaled(name=f"{w.name}_h{args.heads}", H=args.heads)
    t_gen = time.perf_counter()
    x = synth.make_inputs(w)
    t_gen = time.perf_counter() - t_gen
    torch.cuda.set_device(0)

    def dev(a):
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        return t.to("cuda")

    d = {k: dev(v) for k, v in x.items()}
    desc = bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, w.L, w.chunk, w.dtype, True)
    ws = torch.empty(bd.workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(d["q"])
    if w.prep:
        kh, vh = torch.empty_like(d["k"]), torch.empty_like(d["v"])
    grid = (w.grid_h, w.grid_w)
    stream = torch.cuda.current_stream().cuda_stream
    hip = Hip()

    # the long clip: conv + SiLU (+ L2 for K) in the prep kernels; the query's L2
    # normalisation is fused into the readout (VDN_VDA_QUERY_L2), q goes in raw
    pdesc = bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, w.L, w.chunk, w.dtype, False,
                         flags=bd.VDN_VDA_QUERY_L2)

    def prep_call():
        ptr = lambda t: ctypes.c_void_p(t.data_ptr())
        st = bd.lib().vdn_vda_prepare(ctypes.byref(pdesc), None, ptr(d["k"]), ptr(d["v"]), ptr(d["wk_s"]),
                                      ptr(d["wk_t"]), ptr(d["wv_s"]), ptr(d["wv_t"]), None, ptr(kh), ptr(vh),
                                      ctypes.c_void_p(stream))
        if st != bd.VDN_OK:
            raise bd.VdaError(st, "vdn_vda_prepare")

    step_q = (d["q"], kh, vh) if w.prep else (d["q"], d["k"], d["v"])

    def fwd(events=None):
        bd.forward(*step_q, d["alpha"], d["beta"], d["k_text"], d["v_text"], d["beta_text"], d["gate"], None,
                   grid=grid, chunk=w.chunk, epilogue=True, out=out, workspace=ws, query_l2=w.prep,
                   scan=None if args.scan == "auto" else args.scan, events=events)
    fwd.workspace = ws

    def step():
        if w.prep:
            prep_call()
        fwd()

    if args.backward:
        return bench_backward(args, w, x, d, fwd, stream, hip, t_gen)
    if args.adjacent:
        return bench_adjacent(args, w, d, stream, hip, t_gen)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps -----------------------------------
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    hip.record(e0, stream)
    for _ in range(args.steps):
        step()
    hip.record(e1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = hip.elapsed(e0, e1) / args.steps

    # ---- per-stage kernel times (HIP events between the library's kernels) --
    n_st = len(bd.STAGES)
    sets = [[hip.event() for _ in range(n_st + 1)] for _ in range(args.steps)]
    pe0, pe1 = hip.event(), hip.event()
    prep_ms = []
    for evs in sets:
        if w.prep:
            hip.record(pe0, stream)
            prep_call()
            hip.record(pe1, stream)
        fwd(events=[e.value for e in evs])
        if w.prep:
            prep_ms.append(hip.elapsed(pe0, pe1))
    torch.cuda.synchronize()
    stages = {name: 0.0 for name in bd.STAGES}
    for evs in sets:
        for i, name in enumerate(bd.STAGES):
            stages[name] += hip.elapsed(evs[i], evs[i + 1]) / args.steps
    if w.prep:
        stages["prep"] = sum(prep_ms) / len(prep_ms)

    dom = max(("gram", "readout", "prep") if w.prep else ("gram", "readout"), key=lambda s: stages[s])
    # per launch: the prep stage is two launches of one kernel (K, then V)
    launches = LAUNCHES_PER_STAGE.get(dom, 1)
    dom_bytes = algorithmic_bytes(w, dom) // launches
    dom_ms = stages[dom] / launches
    traffic = traffic_for(dom, w.name)
    roofline = dominant_roofline(w, dom, dom_ms, dom_bytes, traffic, launches)
    # what a plain device copy reaches on this GPU: the ceiling a streaming
    # kernel meets in practice, beside the 8 TB/s datasheet figure
    copy_gbs = copy_peak_gbs(torch, hip, stream)
    if roofline["unit"] == "GB/s":
        roofline["frac_of_copy"] = round(roofline["achieved"] / copy_gbs, 4)
    job_gbs = job_bytes(w) / (ms * 1e-3) / 1e9
    frames = w.B * w.T
    rec = {
        "metric": METRIC,
        "value": round(frames / (ms * 1e-3), 2),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "U": w.U,
                   "grid": f"{w.grid_h}x{w.grid_w}", "d": w.d, "text_tokens": w.L, "chunk": w.chunk,
                   "state": "f32", "prep": w.prep, "scan": args.scan},
        "tokens_per_s": round(frames * w.U / (ms * 1e-3), 1),
        "job_roofline": {"bound": "hbm", "algorithmic_bytes": job_bytes(w), "achieved_GBs": round(job_gbs, 1),
                         "peak": HBM_PEAK_GBS, "frac": round(job_gbs / HBM_PEAK_GBS, 4),
                         "copy_GBs": round(copy_gbs, 1), "frac_of_copy": round(job_gbs / copy_gbs, 4),
                         "target_frac": JOB_TARGET_FRAC,
                         "target_met": job_gbs / HBM_PEAK_GBS >= JOB_TARGET_FRAC},
        "roofline": roofline,
        "mfma": {st: mfma_record(w, st, stages[st]) for st in ("gram", "readout")},
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "wall_s_timed": round(wall, 3),
        "input_gen_s": round(t_gen, 1),
    }
    if args.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(x, w, args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
