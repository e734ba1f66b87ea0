"""GPU parity of the backward pass for float32 inputs (the dtype of the tiny
and conditioning-stress workloads) against the oracle's float64 gradients
(oracle/vda_grad.py), every input gradient, with the float32 tolerance of the
forward's parity tests: max relative error per (frame, head) slice (per vector
for dalpha and dgamma) <= 1e-3.  The first and third stages run float32
kernels of their own; the second, on the float32 workspace, is the bfloat16
path's."""

import numpy as np
import pytest

from frame_wise_delta_02_amd import synth
import gpu_harness as G
import test_gpu_widths as GW

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    G.say(request.node.nodeid)
    yield


_TINY = synth.WORKLOADS["tiny_f32"]
_STRESS = synth.WORKLOADS["stress_f32"]
# the tiny workload itself (records in use: T = 20, four chunks), the stress
# workload's keys and beta on fewer heads and frames, every head width, with
# and without the epilogue and a gain, the bridge, the raw query, three-frame
# chunks, two batches, a width between the built ones
CASES = {
    "tiny_f32_gain": dict(w=_TINY, gain=True),
    "stress_d128_bridge": dict(w=_STRESS.scaled(name="stress_d128_bridge", H=2, T=16, grid_h=4, grid_w=8, L=8),
                               bridge=True),
    "d64_raw_chunk3": dict(w=_TINY.scaled(name="d64_raw_chunk3", d=64, H=2, T=14, grid_h=5, grid_w=7, L=8, chunk=3),
                           epilogue=False),
    "d32_query_l2": dict(w=_TINY.scaled(name="d32_query_l2", d=32, H=2, T=16, grid_h=4, grid_w=9, L=4),
                         query_l2=True, gain=True),
    "d16_batch2": dict(w=_TINY.scaled(name="d16_batch2", B=2, T=17, chunk=3)),
    "d48_gain": dict(w=_TINY.scaled(name="d48_gain", d=48, H=2, T=15, grid_h=3, grid_w=5, L=4), gain=True),
}


def _dy(w):
    return np.random.default_rng(12345).standard_normal((w.B, w.T, w.U, w.H, w.d)).astype(np.float32)


def raw_queries(x, w):
    """Replace the unit queries by raw ones of per-token length 0.3 .. 3."""
    rng = np.random.default_rng(77)
    x["q"] = (x["q"] * rng.uniform(0.3, 3.0, x["q"].shape[:-1] + (1,))).astype(np.float32)


def reference(x, w, dy, epi, gain, bridge, ql2):
    if not ql2:
        return GW.backward_reference(x, w, dy, epi, gain, bridge)
    from oracle import vda_grad
    f = G.oracle_view({k: x[k] for k in ("q", "k", "v", "beta", "k_text", "v_text", "beta_text", "gate")}, w)
    g = gain if gain is not None else np.ones(w.d)
    return vda_grad.backward(f["q"], f["k"], f["v"], x["alpha"].astype(np.float64), f["beta"], f["k_text"],
                             f["v_text"], f["beta_text"], dy.astype(np.float64), gate=f["gate"], rms_weight=g,
                             chunk=w.chunk, bridge=bridge, query_l2=1e-6)


@pytest.mark.parametrize("name", list(CASES))
def test_backward_f32(name):
    """The whole backward (binding.backward, with the gain's gradient under the
    epilogue) after the forward, every input gradient against the oracle's."""
    import torch
    from frame_wise_delta_02_amd import binding as bd
    case = CASES[name]
    w, epi, bridge, ql2 = case["w"], case.get("epilogue", True), case.get("bridge", False), case.get("query_l2", False)
    x = synth.make_inputs(w)
    if ql2:
        raw_queries(x, w)
    dy = _dy(w)
    gain = np.random.default_rng(5).uniform(0.5, 1.5, w.d) if case.get("gain") else None
    _, ws, _, dev = G.run_forward(x, w, epilogue=epi, rms_weight=gain, bridge=bridge, query_l2=ql2)
    rw = None if gain is None else torch.from_numpy(gain.astype(np.float32)).cuda()
    G.say(f"backward {name}")
    r = bd.backward(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["k_text"] if w.L else None,
                    dev["v_text"] if w.L else None, dev["beta_text"] if w.L else None, dev["gate"] if epi else None,
                    rw, G.to_device(dy, w.dtype), ws, grid=(w.grid_h, w.grid_w), chunk=w.chunk, epilogue=epi,
                    bridge=bridge, query_l2=ql2, gain_grad=epi)
    torch.cuda.synchronize()
    got = {k: G.to_host_f64(v) for k, v in r.items() if v is not None and k != "workspace"}
    if epi:
        got["dgamma"] = got.pop("drms_weight")
    errs = GW.backward_errors(got, reference(x, w, dy, epi, gain, bridge, ql2), w, epi)
    G.say(f"{name}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= G.TOL["f32"]}
    assert not bad, bad
