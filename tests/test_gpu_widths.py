"""GPU parity at the head widths between the built ones (d = 48, 80, 96, 112):
the library runs its kernels at the next built width on zero-padded copies of
the inputs and copies the results' d channels back.  The forward's outputs
(the raw readout o and y after RMSNorm and the gate, with and without a gain)
and the backward's input gradients (the gain's included) against the oracle,
which runs at the caller's width, with the tolerances of the other parity
tests: max relative error per (frame, head) slice (per vector for dalpha and
dgamma) <= 2e-2 for bfloat16 inputs, <= 1e-3 for float32.  The adjacent maps,
plain products over a token's H d channels, run at the caller's width itself
and are checked as at the built widths; so does the prep (vdn_vda_prepare),
whose convolution is per channel: its lanes past the caller's channels idle."""

import numpy as np
import pytest

from frame_wise_delta_02_amd import synth
import gpu_harness as G
import test_gpu_parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    G.say(request.node.nodeid)
    yield


_BF = synth.WORKLOADS["768p_bf16"]
_F32 = synth.WORKLOADS["stress_f32"]
# every width, both dtypes, ragged grids and several tiles, no text tokens,
# T = 1, three-frame chunks, two batches, and the 768p frame size
CASES = {
    "d48_bf16": _BF.scaled(name="d48_bf16", d=48, H=3, T=13, grid_h=7, grid_w=9, L=8),
    "d80_bf16": _BF.scaled(name="d80_bf16", d=80, H=2, T=12, grid_h=10, grid_w=10, L=37),
    "d96_bf16_chunk3": _BF.scaled(name="d96_bf16_chunk3", d=96, H=2, T=20, grid_h=4, grid_w=10, chunk=3, L=8),
    "d112_bf16": _BF.scaled(name="d112_bf16", d=112, H=2, T=11, grid_h=6, grid_w=11, L=12),
    "d48_f32": _F32.scaled(name="d48_f32", d=48, H=2, T=10, grid_h=4, grid_w=8, L=8),
    "d112_f32": _F32.scaled(name="d112_f32", d=112, H=2, T=13, grid_h=7, grid_w=11, L=5),
    "d80_no_text_bf16": _BF.scaled(name="d80_no_text_bf16", d=80, H=2, T=15, grid_h=4, grid_w=9, L=0),
    "d48_T1_bf16": _BF.scaled(name="d48_T1_bf16", d=48, H=2, T=1, grid_h=4, grid_w=8, L=16),
    "d96_batch2_bf16": _BF.scaled(name="d96_batch2_bf16", d=96, B=2, H=2, T=16, grid_h=6, grid_w=11, L=12),
    "d112_768p_frame": _BF.scaled(name="d112_768p_frame", d=112, H=2, T=6, L=256),
}

SCANS = ["frames", "chunks"]


def _check(x, w, scan=None, bridge=False, query_l2=False):
    heads = list(range(w.H))
    rw = np.random.default_rng(5).uniform(0.5, 1.5, w.d)
    tol = G.TOL[w.dtype]
    out, _, _, dev = G.run_forward(x, w, epilogue=False, scan=scan, bridge=bridge, query_l2=query_l2)
    err_o = G.slice_rel_err(G.to_host_f64(out), P._oracle_heads(x, w, heads, gate=False, bridge=bridge,
                                                                  prepared=_normalised(x, w) if query_l2 else None)["o"])
    del out
    for gain in (None, rw):
        y, _, _, _ = G.run_forward(x, w, epilogue=True, rms_weight=gain, dev_inputs=dev, scan=scan, bridge=bridge,
                                   query_l2=query_l2)
        ref = P._oracle_heads(x, w, heads, gate=True, rms_weight=gain, bridge=bridge,
                              prepared=_normalised(x, w) if query_l2 else None)
        err_y = G.slice_rel_err(G.to_host_f64(y), ref["y"])
        G.say(f"{w.name}: o {err_o:.2e}, y {err_y:.2e} ({'gain' if gain is not None else 'no gain'})")
        assert err_y <= tol, err_y
    assert err_o <= tol, err_o


def _normalised(x, w):
    """The raw queries normalised in float64, as the oracle takes them."""
    q = G.oracle_view({"q": x["q"]}, w)["q"]
    return {"q": q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + 1e-6)}


@pytest.mark.parametrize("scan", SCANS)
@pytest.mark.parametrize("name", list(CASES))
def test_padded_width_forward(name, scan):
    w = CASES[name]
    _check(synth.make_inputs(w), w, scan=scan)


@pytest.mark.parametrize("name", ["d48_bf16", "d112_f32"])
def test_padded_width_decay_bridge(name):
    w = CASES[name]
    _check(synth.make_inputs(w), w, bridge=True)


def test_padded_width_raw_query():
    """VDN_VDA_QUERY_L2 at d = 80: the readout normalises raw queries of
    per-token length 0.3 .. 3 (the zero channels change no norm)."""
    w = CASES["d80_bf16"]
    x = synth.make_inputs(w)
    rng = np.random.default_rng(77)
    x["q"] = synth.f64_to_bf16_bits(synth.to_f64(x["q"], w.dtype) * rng.uniform(0.3, 3.0, x["q"].shape[:-1] + (1,)))
    _check(x, w, query_l2=True)


# the backward (bfloat16): with the epilogue and a gain, raw, the bridge, a
# clip without text tokens
BWD_CASES = {
    "bwd_d48_gain": dict(w=_BF.scaled(name="bwd_d48_gain", d=48, H=2, T=12, grid_h=5, grid_w=7, L=8), gain=True),
    "bwd_d80_raw_bridge": dict(w=_BF.scaled(name="bwd_d80_raw_bridge", d=80, H=2, T=16, grid_h=4, grid_w=9, L=4),
                               epilogue=False, bridge=True),
    "bwd_d96_chunk3": dict(w=_BF.scaled(name="bwd_d96_chunk3", d=96, H=2, T=14, grid_h=4, grid_w=6, L=4, chunk=3)),
    "bwd_d112_bridge_no_text": dict(w=_BF.scaled(name="bwd_d112_bridge_no_text", d=112, H=2, T=12, grid_h=5, grid_w=7,
                                                 L=0), bridge=True, gain=True),
}


def backward_errors(got, ref, w, epi):
    """Max relative errors of every input gradient (host float64 arrays in got)."""
    import test_gpu_backward as GB
    errs = {k: G.slice_rel_err(got[k], ref[k]) for k in ("dq", "dk", "dv")}
    errs["dbeta"] = G.slice_rel_err(got["dbeta"][..., None], ref["dbeta"][..., None])
    errs["dalpha"] = GB._rel(got["dalpha"], ref["dalpha"])
    if epi:
        errs["dgate"] = G.slice_rel_err(got["dgate"], ref["dgate"])
        errs["dgamma"] = GB._rel(got["dgamma"], ref["dgamma"])
    if w.L:
        txt = lambda a: a.reshape((w.B, 1) + a.shape[1:] + ((1,) if a.ndim == 3 else ()))
        for k, r in (("dk_text", "dk_txt"), ("dv_text", "dv_txt"), ("dbeta_text", "dbeta_txt")):
            errs[k] = G.slice_rel_err(txt(got[k]), txt(ref[r]))
    return errs


def backward_reference(x, w, dy, epi, gain, bridge):
    from oracle import vda_grad
    f = G.oracle_view({k: x[k] for k in ("q", "k", "v", "beta", "k_text", "v_text", "beta_text", "gate")}, w)
    g = gain if gain is not None else (np.ones(w.d) if epi else None)
    return vda_grad.backward(f["q"], f["k"], f["v"], x["alpha"].astype(np.float64), f["beta"], f["k_text"],
                             f["v_text"], f["beta_text"], G.oracle_view({"dy": dy}, w)["dy"],
                             gate=f["gate"] if epi else None, rms_weight=g, chunk=w.chunk, bridge=bridge)


@pytest.mark.parametrize("name", list(BWD_CASES))
def test_padded_width_backward(name):
    """The whole backward (binding.backward: the three stages, the gain's
    gradient with the epilogue) after the forward, every input gradient
    against the oracle's."""
    import torch
    from frame_wise_delta_02_amd import binding as bd
    import test_gpu_backward as GB
    case = BWD_CASES[name]
    w, epi, bridge = case["w"], case.get("epilogue", True), case.get("bridge", False)
    x = synth.make_inputs(w)
    dy = GB._dy(w)
    gain = np.random.default_rng(5).uniform(0.5, 1.5, w.d) if case.get("gain") else None
    _, ws, _, dev = G.run_forward(x, w, epilogue=epi, rms_weight=gain, bridge=bridge)
    rw = None if gain is None else torch.from_numpy(gain.astype(np.float32)).cuda()
    G.say(f"backward {name}")
    r = bd.backward(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["k_text"] if w.L else None,
                    dev["v_text"] if w.L else None, dev["beta_text"] if w.L else None, dev["gate"] if epi else None,
                    rw, G.to_device(dy, w.dtype), ws, grid=(w.grid_h, w.grid_w), chunk=w.chunk, epilogue=epi,
                    bridge=bridge, gain_grad=epi)
    torch.cuda.synchronize()
    got = {k: G.to_host_f64(v) for k, v in r.items() if v is not None and k != "workspace"}
    if epi:
        got["dgamma"] = got.pop("drms_weight")
    errs = backward_errors(got, backward_reference(x, w, dy, epi, gain, bridge), w, epi)
    G.say(f"{name}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= G.TOL[w.dtype]}
    assert not bad, bad


# the adjacent maps: (workload, model width)
ADJ_CASES = {
    "adj_d48": (_BF.scaled(name="adj_d48", B=1, T=3, grid_h=5, grid_w=7, H=3, d=48, L=0), 200),
    "adj_d112": (_BF.scaled(name="adj_d112", B=2, T=4, grid_h=6, grid_w=11, H=2, d=112, L=0), 320),
}


@pytest.mark.parametrize("name", list(ADJ_CASES))
def test_padded_width_gates(name):
    import test_gpu_adjacent as GA
    GA.check_gates(*ADJ_CASES[name], name)


@pytest.mark.parametrize("name", list(ADJ_CASES))
def test_padded_width_out_proj(name):
    import test_gpu_adjacent as GA
    GA.check_out_proj(*ADJ_CASES[name], "y_in", name)


# the prep (depthwise convolutions, SiLU, L2 norms) at the caller's width
PREP_CASES = {
    "prep_d48_bf16": dict(d=48, H=2, T=7, grid_h=6, grid_w=10, L=4),
    "prep_d112_bf16": dict(d=112, H=2, T=6, grid_h=9, grid_w=13, L=4),
    "prep_d80_f32": dict(d=80, H=2, T=5, grid_h=5, grid_w=7, L=4, dtype="f32"),
}


@pytest.mark.parametrize("name", list(PREP_CASES))
def test_padded_width_prepare(name):
    w = synth.WORKLOADS["long_prep_bf16"].scaled(name=name, **PREP_CASES[name])
    P._prep_case(w, heads=list(range(w.H)))
