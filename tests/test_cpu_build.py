"""The library's own HIP sources compiled for the host and run on the CPU
(tests/cpu_build: every lane a fiber, cross-lane operations and barriers as
rendezvous points, buffer descriptors with their range checks).

* Under AddressSanitizer and UndefinedBehaviorSanitizer (check.cpp): the
  forward pass on exact-size host allocations, every kernel variant the
  forward launches (both dtypes, d = 16 .. 128, one token per frame, no text,
  T = 1 and 2); A_t, B_t and (I + A_t)^{-1} against a float64 reference, and no
  out-of-range access, undefined behaviour, divergent cross-lane operation or
  unequal barrier count.
* Through the C ABI from Python (libvdn_vda_sim.so): outputs and every
  intermediate against the oracle with the tolerances of the GPU parity tests,
  both scans, the decay bridge, the prep kernels and the fused query norm.

These run the kernels' code, not a model of it, but not the gfx950 binary:
they check indexing, bounds, synchronisation counts and arithmetic, not the
compiler's output or the hardware.  Parity proper is the GPU suite's.
"""

import os
import subprocess

import numpy as np
import pytest

import oracle
import gpu_harness as G
import test_gpu_parity as P
from cpu_build import build as CB
from cpu_build import sim as S
from frame_wise_delta_02_amd import synth

pytestmark = pytest.mark.skipif(CB.compiler() is None, reason="no host clang++ for the CPU build")


@pytest.fixture(scope="module")
def check_exe():
    return CB.build(S.OUT, sanitize=True)


@pytest.fixture(scope="module")
def lib():
    return S.load(CB.build(S.OUT, sanitize=False))


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
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([check_exe, *map(str, shape)], capture_output=True, text=True, timeout=900, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "Sanitizer" not in out and "[simt]" not in out, out[-4000:]


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


@pytest.mark.parametrize("scan", P.SCANS)
@pytest.mark.parametrize("name", list(PARITY))
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
