"""GPU parity of the linear maps either side of the path (vdn_vda_gates,
vdn_vda_out_proj) against the oracle (oracle/vda_adjacent.py), on seeded
synthetic inputs: several tiles with ragged edges in every dimension, a model
width that is not a multiple of the K-panel, narrow heads, the output written
over Y_in, no Y_in, and the 768p shape checked on sampled tokens and frames.

Tolerances: the bfloat16 outputs (gate logits, beta, Y) as the forward's
(max relative error per slice <= 2e-2); alpha (float32 throughout) to 1e-5
absolute."""

import numpy as np
import pytest

from oracle import vda_adjacent as adj
from frame_wise_delta_02_amd import synth
import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    G.say(request.node.nodeid)
    yield


BASE = synth.WORKLOADS["768p_bf16"]
CASES = {
    # one ragged M-tile, two N-tiles (the second holds the beta columns), K = 200
    "adj_small": (BASE.scaled(name="adj_small", B=1, T=3, grid_h=5, grid_w=7, H=3, L=0), 200),
    # three M-tiles, a ragged N on the output side, K = 320
    "adj_ragged": (BASE.scaled(name="adj_ragged", B=2, T=5, grid_h=6, grid_w=11, H=2, d=64, L=0), 320),
    # narrow heads, beta columns inside the first tile
    "adj_d16": (BASE.scaled(name="adj_d16", B=1, T=4, grid_h=4, grid_w=4, H=3, d=16, L=0), 64),
    # one token per frame, the smallest model width (a single partial K-panel)
    "adj_tiny": (BASE.scaled(name="adj_tiny", B=1, T=2, grid_h=1, grid_w=1, H=1, d=16, L=0), 8),
}


def _dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _f64(a):
    return synth.to_f64(a, "bf16") if a.dtype == np.uint16 else a.astype(np.float64)


def _slices(a):
    """[B, T, U, ...] -> [B, T, U, 1, n] for the per-frame slice error."""
    return a.reshape(a.shape[0], a.shape[1], a.shape[2], 1, -1)


def check_gates(w, dm, name):
    """vdn_vda_gates on the case's seeded inputs against the oracle."""
    import torch
    from frame_wise_delta_02_amd import binding as bd
    p = synth.make_adjacent_inputs(w, dm)
    gate, beta, alpha = bd.gates(_dev(p["x"]), _dev(p["w_gb"]), _dev(p["w_alpha"]), heads=w.H, d=w.d,
                                 grid=(w.grid_h, w.grid_w))
    torch.cuda.synchronize()
    wg = _f64(p["w_gb"])
    g_ref, b_ref, a_ref = adj.gate_proj(_f64(p["x"]), wg[: w.H * w.d], wg[w.H * w.d:], _f64(p["w_alpha"]), w.H, w.d)
    errs = {"gate": G.slice_rel_err(G.to_host_f64(gate), g_ref),
            "beta": G.slice_rel_err(_slices(G.to_host_f64(beta)), _slices(b_ref)),
            "alpha_abs": float(np.abs(alpha.double().cpu().numpy() - a_ref).max())}
    G.say(f"{name}: " + " ".join(f"err({k})={v:.3e}" for k, v in errs.items()))
    assert errs["gate"] <= 2e-2 and errs["beta"] <= 2e-2 and errs["alpha_abs"] <= 1e-5, errs


@pytest.mark.parametrize("name", list(CASES))
def test_gates(name):
    check_gates(*CASES[name], name)


def check_out_proj(w, dm, mode, name):
    """vdn_vda_out_proj on the case's seeded inputs against the oracle."""
    import torch
    from frame_wise_delta_02_amd import binding as bd
    p = synth.make_adjacent_inputs(w, dm)
    o, wo, yin = _dev(p["o"]), _dev(p["w_o"]), _dev(p["y_in"])
    if mode == "y_in":
        y = bd.out_proj(o, wo, yin, grid=(w.grid_h, w.grid_w))
    elif mode == "in_place":
        y = bd.out_proj(o, wo, yin, grid=(w.grid_h, w.grid_w), out=yin)
        assert y.data_ptr() == yin.data_ptr()
    else:
        y = bd.out_proj(o, wo, None, grid=(w.grid_h, w.grid_w))
    torch.cuda.synchronize()
    ref = adj.out_proj(_f64(p["o"]), _f64(p["w_o"]), None if mode == "no_y_in" else _f64(p["y_in"]))
    err = G.slice_rel_err(_slices(G.to_host_f64(y)), _slices(ref))
    G.say(f"{name} {mode}: err(y)={err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mode", ["y_in", "in_place", "no_y_in"])
def test_out_proj(name, mode):
    check_out_proj(*CASES[name], mode, name)


def test_768p_sampled():
    """The 768p shape (B=1, T=60, 48 x 84 tokens, 24 heads of 128, d_model 3072):
    gate logits, beta and Y on 96 sampled tokens, alpha on 6 sampled frames."""
    import torch
    from frame_wise_delta_02_amd import binding as bd
    w, dm = BASE, BASE.H * BASE.d
    p = synth.make_adjacent_inputs(w, dm)
    G.say("768p gates")
    gate, beta, alpha = bd.gates(_dev(p["x"]), _dev(p["w_gb"]), _dev(p["w_alpha"]), heads=w.H, d=w.d,
                                 grid=(w.grid_h, w.grid_w))
    G.say("768p out_proj")
    y = bd.out_proj(_dev(p["o"]), _dev(p["w_o"]), _dev(p["y_in"]), grid=(w.grid_h, w.grid_w))
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    ts = rng.integers(0, w.T, 96)
    us = rng.integers(0, w.U, 96)
    us[:4] = [0, w.U - 1, 255, 256]          # tile edges
    wg = _f64(p["w_gb"])
    HD = w.H * w.d
    x_s = _f64(p["x"][0, ts, us])             # [96, dm]
    g_s = G.to_host_f64(gate[0, ts, us]).reshape(96, HD)
    b_s = G.to_host_f64(beta[0, ts, us])
    y_s = G.to_host_f64(y[0, ts, us])
    g_ref = x_s @ wg[:HD].T
    b_ref = adj.sigmoid(x_s @ wg[HD:].T)
    y_ref = _f64(p["y_in"][0, ts, us]) + _f64(p["o"][0, ts, us]).reshape(96, HD) @ _f64(p["w_o"]).T
    rel = lambda a, r: float(np.max(np.abs(a - r).max(axis=1) / np.abs(r).max(axis=1)))
    errs = {"gate": rel(g_s, g_ref), "beta": rel(b_s, b_ref), "y": rel(y_s, y_ref)}
    fr = [0, 1, 29, 58, 59, int(rng.integers(2, 58))]
    a_gpu = alpha.double().cpu().numpy()[0, fr].reshape(len(fr), HD)
    xbar = np.stack([_f64(p["x"][0, t]).mean(axis=0) for t in fr])
    a_ref = adj.sigmoid(xbar @ p["w_alpha"].astype(np.float64).T)
    errs["alpha_abs"] = float(np.abs(a_gpu - a_ref).max())
    G.say("768p: " + " ".join(f"err({k})={v:.3e}" for k, v in errs.items()))
    assert errs["gate"] <= 2e-2 and errs["beta"] <= 2e-2 and errs["y"] <= 2e-2 and errs["alpha_abs"] <= 1e-5, errs


def test_layer_chain():
    """The three entry points composed as a layer uses them: gates from x, the
    forward pass on those gates (with the epilogue), then the output projection
    adding Y_in, against the oracle's chain in float64 (the GPU's gates enter
    its forward rounded to bfloat16, so the tolerance covers that too)."""
    import torch
    import oracle
    from frame_wise_delta_02_amd import binding as bd
    w = BASE.scaled(name="layer", B=1, T=11, grid_h=4, grid_w=6, H=2, d=64, L=8)
    dm = 160
    x = synth.make_inputs(w)
    p = synth.make_adjacent_inputs(w, dm)
    grid = (w.grid_h, w.grid_w)
    gate, beta, alpha = bd.gates(_dev(p["x"]), _dev(p["w_gb"]), _dev(p["w_alpha"]), heads=w.H, d=w.d, grid=grid,
                                 chunk=w.chunk)
    d = {k: _dev(x[k]) for k in ("q", "k", "v", "k_text", "v_text", "beta_text")}
    o = bd.forward(d["q"], d["k"], d["v"], alpha, beta, d["k_text"], d["v_text"], d["beta_text"], gate, None,
                   grid=grid, chunk=w.chunk, epilogue=True)
    y = bd.out_proj(o, _dev(p["w_o"]), _dev(p["y_in"]), grid=grid, chunk=w.chunk)
    torch.cuda.synchronize()
    wg = _f64(p["w_gb"])
    HD = w.H * w.d
    g_ref, b_ref, a_ref = adj.gate_proj(_f64(p["x"]), wg[:HD], wg[HD:], _f64(p["w_alpha"]), w.H, w.d)
    f = {k: _f64(x[k]) for k in ("q", "k", "v", "k_text", "v_text", "beta_text")}
    fw = oracle.forward(f["q"], f["k"], f["v"], a_ref, b_ref, f["k_text"], f["v_text"], f["beta_text"], gate=g_ref,
                        chunk=w.chunk)
    y_ref = adj.out_proj(fw["y"], _f64(p["w_o"]), _f64(p["y_in"]))
    errs = {"o": G.slice_rel_err(G.to_host_f64(o), fw["y"]),
            "y": G.slice_rel_err(_slices(G.to_host_f64(y)), _slices(y_ref))}
    G.say("layer chain: " + " ".join(f"err({k})={v:.3e}" for k, v in errs.items()))
    assert errs["o"] <= 2e-2 and errs["y"] <= 2e-2, errs
