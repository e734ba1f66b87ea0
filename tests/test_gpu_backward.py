"""GPU parity of the backward pass against the oracle's gradients
(oracle/vda_grad.py), stage by stage: the first (vdn_vda_backward_readout: dq,
dgate, and do and dS_q in its workspace), the second (vdn_vda_backward_scan:
record and scan adjoints, dA, dB, dalpha) and the third
(vdn_vda_backward_gram: dk, dv, dbeta and the text gradients).  Tolerance as
for the forward's bfloat16 outputs: max relative error per (frame, head)
slice (per matrix for the d x d intermediates) <= 2e-2."""

import numpy as np
import pytest

from oracle import vda_grad
from frame_wise_delta_02_amd import synth
import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    G.say(request.node.nodeid)
    yield


BASE = synth.WORKLOADS["768p_bf16"]
CASES = {
    "bwd_128": dict(w=BASE.scaled(name="bwd_128", H=2, T=12, grid_h=5, grid_w=7, L=8)),
    "bwd_128_gain": dict(w=BASE.scaled(name="bwd_128_gain", H=2, T=11, grid_h=6, grid_w=11, L=8), gain=True),
    "bwd_128_raw": dict(w=BASE.scaled(name="bwd_128_raw", H=2, T=12, grid_h=5, grid_w=7, L=8), epilogue=False),
    "bwd_64_ragged": dict(w=BASE.scaled(name="bwd_64_ragged", d=64, H=3, T=13, grid_h=7, grid_w=9, L=4)),
    "bwd_32_bridge": dict(w=BASE.scaled(name="bwd_32_bridge", d=32, H=2, T=16, grid_h=4, grid_w=9, L=4),
                          bridge=True),
    # the decay bridge with records in use on both sides (7 chunks of 3)
    "bwd_64_bridge": dict(w=BASE.scaled(name="bwd_64_bridge", d=64, H=2, T=20, grid_h=4, grid_w=6, L=4, chunk=3),
                          bridge=True, gain=True),
    "bwd_16": dict(w=BASE.scaled(name="bwd_16", d=16, H=2, T=9, grid_h=4, grid_w=4, L=4), gain=True),
    "bwd_B2_chunk3": dict(w=BASE.scaled(name="bwd_B2_chunk3", B=2, H=2, T=14, grid_h=4, grid_w=6, L=4, chunk=3)),
    "bwd_T2": dict(w=BASE.scaled(name="bwd_T2", H=2, T=2, grid_h=4, grid_w=8, L=16)),
    "bwd_T1": dict(w=BASE.scaled(name="bwd_T1", d=64, H=2, T=1, grid_h=3, grid_w=5, L=8)),
    # narrow heads with records in use (bwd_16 and bwd_128_gain have too few
    # chunks for any record to be read), and a clip without text tokens
    "bwd_16_chunk3": dict(w=BASE.scaled(name="bwd_16_chunk3", d=16, H=2, T=17, grid_h=4, grid_w=5, L=4, chunk=3)),
    "bwd_32": dict(w=BASE.scaled(name="bwd_32", d=32, H=2, T=16, grid_h=4, grid_w=9, L=4)),
    "bwd_64_no_text": dict(w=BASE.scaled(name="bwd_64_no_text", d=64, H=1, T=12, grid_h=3, grid_w=5, L=0, chunk=3)),
    # raw queries (the forward normalises them, VDN_VDA_QUERY_L2): per-token lengths 0.3 .. 3
    "bwd_128_ql2": dict(w=BASE.scaled(name="bwd_128_ql2", H=2, T=12, grid_h=5, grid_w=7, L=8), query_l2=True),
    "bwd_64_ql2_gain": dict(w=BASE.scaled(name="bwd_64_ql2_gain", d=64, H=3, T=13, grid_h=7, grid_w=9, L=4),
                            query_l2=True, gain=True),
    "bwd_16_ql2": dict(w=BASE.scaled(name="bwd_16_ql2", d=16, H=2, T=17, grid_h=4, grid_w=5, L=4, chunk=3),
                       query_l2=True),
}

L2_EPS = 1e-6


def _raw_queries(x, w):
    """Replace the unit queries by raw ones of per-token length 0.3 .. 3."""
    rng = np.random.default_rng(77)
    scale = rng.uniform(0.3, 3.0, x["q"].shape[:-1] + (1,))
    x["q"] = synth.f64_to_bf16_bits(synth.to_f64(x["q"], w.dtype) * scale)


def _dy(w):
    rng = np.random.default_rng(12345)
    return synth.f64_to_bf16_bits(rng.standard_normal((w.B, w.T, w.U, w.H, w.d)))


def _run(name, stage2=False, stage3=False):
    """Forward, then the backward stages, on the case's seeded inputs; returns
    the GPU results, the oracle's gradients and the case's description."""
    import torch
    from frame_wise_delta_02_amd import binding as bd
    case = CASES[name]
    w, epi, bridge = case["w"], case.get("epilogue", True), case.get("bridge", False)
    ql2 = case.get("query_l2", False)
    x = synth.make_inputs(w)
    if ql2:
        _raw_queries(x, w)
    dy = _dy(w)
    rw = np.random.default_rng(5).uniform(0.5, 1.5, w.d) if case.get("gain") else None
    out, ws, desc, dev = G.run_forward(x, w, epilogue=epi, rms_weight=rw, bridge=bridge, query_l2=ql2)
    dy_d = G.to_device(dy, w.dtype)
    rw_d = None if rw is None else torch.from_numpy(rw.astype(np.float32)).cuda()
    G.say(f"backward_readout {name}")
    dq, dgate, bws = bd.backward_readout(dev["q"], dev["gate"], rw_d, dev["alpha"], dy_d, ws,
                                         grid=(w.grid_h, w.grid_w), n_text=w.L, chunk=w.chunk, epilogue=epi,
                                         bridge=bridge, query_l2=ql2, l2_eps=L2_EPS)
    torch.cuda.synchronize()
    gpu = {"dq": dq, "dgate": dgate, "bws": bws}
    if stage2:
        G.say(f"backward_scan {name}")
        gpu["dalpha"] = bd.backward_scan(dev["alpha"], ws, bws, shape=(w.B, w.T, w.H, w.d),
                                         grid=(w.grid_h, w.grid_w), n_text=w.L, chunk=w.chunk, epilogue=epi,
                                         bridge=bridge)
        torch.cuda.synchronize()
    if stage3:
        G.say(f"backward_gram {name}")
        gpu["gram"] = bd.backward_gram(dev["k"], dev["v"], dev["beta"], dev["k_text"], dev["v_text"],
                                       dev["beta_text"], bws, grid=(w.grid_h, w.grid_w), chunk=w.chunk,
                                       epilogue=epi)
        torch.cuda.synchronize()
    f = G.oracle_view({k: x[k] for k in ("q", "k", "v", "beta", "k_text", "v_text", "beta_text", "gate")}, w)
    ref = vda_grad.backward(f["q"], f["k"], f["v"], x["alpha"].astype(np.float64), f["beta"], f["k_text"],
                            f["v_text"], f["beta_text"], G.oracle_view({"dy": dy}, w)["dy"],
                            gate=f["gate"] if epi else None, rms_weight=rw, chunk=w.chunk, bridge=bridge,
                            query_l2=L2_EPS if ql2 else None)
    L = bd.backward_layout(bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, w.L, w.chunk, w.dtype, epi))
    if ql2:  # the first stage's d_out holds do / |q| per token
        q = f["q"]
        ref["do_written"] = np.moveaxis(ref["do"], 1, 3) / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + L2_EPS)
    return gpu, ref, L, w, epi, dy


def _section(bws, off, shape, dtype="f32"):
    import torch
    n = int(np.prod(shape))
    if dtype == "bf16":
        return bws[off:off + 2 * n].view(torch.int16).view(torch.bfloat16).reshape(shape).to(torch.float64).cpu().numpy()
    return bws[off:off + 4 * n].view(torch.float32).reshape(shape).to(torch.float64).cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_backward_readout(name):
    gpu, ref, L, w, epi, dy = _run(name)
    dq, dgate, bws = gpu["dq"], gpu["dgate"], gpu["bws"]
    do = _section(bws, L.d_out, (w.B, w.T, w.U, w.H, w.d), "bf16")
    dsq = _section(bws, L.d_state_q, (w.B, w.H, w.T, w.d, w.d))
    tol = G.TOL[w.dtype]
    # without the epilogue do is dy itself (the workspace copy is not written)
    do_want = ref["do_written"] if "do_written" in ref else np.moveaxis(ref["do"], 1, 3)
    errs = {"dq": G.slice_rel_err(G.to_host_f64(dq), ref["dq"]),
            "do": G.slice_rel_err(do if epi else G.oracle_view({"dy": dy}, w)["dy"], do_want),
            "dS_q": G.mat_rel_err(dsq, ref["dS_q"])}
    if epi:
        errs["dgate"] = G.slice_rel_err(G.to_host_f64(dgate), ref["dgate"])
    G.say(f"{name}: " + " ".join(f"err({k})={v:.3e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= tol, (k, v)


def _rel(got, ref):
    """max over leading axes of ||got - ref||_inf / ||ref||_inf of each trailing matrix
    (or vector); slices where the reference is zero must be zero too."""
    if got.size == 0:
        return 0.0
    axes = tuple(range(got.ndim - (2 if got.ndim >= 2 else 1), got.ndim))
    diff = np.abs(got - ref).max(axis=axes)
    scale = np.abs(ref).max(axis=axes)
    return float(np.max(np.where(scale > 0, diff / np.maximum(scale, 1e-300), diff)))


@pytest.mark.parametrize("name", list(CASES))
def test_backward_scan(name):
    """Second stage: record adjoints, the scans' adjoints, dA, dB (frames and
    text) and dalpha against the oracle."""
    gpu, ref, L, w, epi, dy = _run(name, stage2=True)
    B, H, T, d = w.B, w.H, w.T, w.d
    nc = -(-T // w.chunk)
    bws = gpu["bws"]
    dF = _section(bws, L.d_record_f, (B, H, nc, d, d))
    dR = _section(bws, L.d_record_r, (B, H, nc, d, d))
    lam_f = _section(bws, L.lam_f, (B, H, T + 1, d, d))
    lam_r = _section(bws, L.lam_r, (B, H, T + 1, d, d))
    dA = _section(bws, L.d_a, (B, H, T + 1, d, d))
    dB = _section(bws, L.d_b, (B, H, T + 1, d, d))
    dalpha = gpu["dalpha"].to(dtype=__import__("torch").float64).cpu().numpy()
    fr = slice(1, max(T - 1, 1))
    sym = lambda a: a + np.swapaxes(a, -1, -2)
    errs = {
        "dF": _rel(dF[:, :, : max(nc - 2, 0)], ref["dF"][:, :, : max(nc - 2, 0)]),
        "dR": _rel(dR[:, :, 2:], ref["dR"][:, :, 2:]),
        "lam_f": _rel(lam_f[:, :, fr], ref["dfwd"][:, :, fr]),
        "lam_r": _rel(lam_r[:, :, fr], ref["drev"][:, :, fr]),
        "dS_T": _rel(lam_f[:, :, T], ref["dS_T"]),
        # A_t is symmetric, so only dA + dA^T reaches an input: compare that
        # (the oracle's text frame, S_T = solve(P, B^T)^T, gives the transpose)
        "dA": _rel(sym(dA[:, :, fr]), sym(ref["dA"][:, :, fr])),
        "dB": _rel(dB[:, :, fr], ref["dB"][:, :, fr]),
        # (the text frame exists only with text tokens)
        "dA_T": _rel(sym(dA[:, :, T]), sym(ref["dA_T"])) if w.L else 0.0,
        "dB_T": _rel(dB[:, :, T], ref["dB_T"]) if w.L else 0.0,
        # every frame: under the decay bridge the anchors' alpha has a gradient too
        "dalpha": _rel(dalpha, ref["dalpha"]),
    }
    # the anchors take no part in any scan
    assert np.abs(dA[:, :, [0, T - 1]]).max() == 0 and np.abs(dB[:, :, [0, T - 1]]).max() == 0
    if not CASES[name].get("bridge"):
        assert np.abs(dalpha[:, [0, T - 1]]).max() == 0
    G.say(f"{name}: " + " ".join(f"err({k})={v:.3e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= G.TOL[w.dtype], (k, v)


@pytest.mark.parametrize("name", list(CASES))
def test_backward_gram(name):
    """Third stage: dk, dv, dbeta of every frame and of the text tokens."""
    gpu, ref, L, w, epi, dy = _run(name, stage2=True, stage3=True)
    dk, dv, dbeta, dkt, dvt, dbt = (None if t is None else G.to_host_f64(t) for t in gpu["gram"])
    B, T, H = w.B, w.T, w.H
    errs = {"dk": G.slice_rel_err(dk, ref["dk"]), "dv": G.slice_rel_err(dv, ref["dv"]),
            "dbeta": G.slice_rel_err(dbeta[..., None], ref["dbeta"][..., None])}
    if w.L:
        txt = lambda a: a.reshape((B, 1) + a.shape[1:] + ((1,) if a.ndim == 3 else ()))
        errs.update({"dk_text": G.slice_rel_err(txt(dkt), txt(ref["dk_txt"])),
                     "dv_text": G.slice_rel_err(txt(dvt), txt(ref["dv_txt"])),
                     "dbeta_text": G.slice_rel_err(txt(dbt), txt(ref["dbeta_txt"]))})
    # the anchors' tokens reach no state
    for a in (dk, dv, dbeta):
        assert np.abs(a[:, [0, T - 1]]).max() == 0
    G.say(f"{name}: " + " ".join(f"err({k})={v:.3e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= G.TOL[w.dtype], (k, v)


def test_backward_whole_matches_the_stages():
    """binding.backward (the three entry points in order) gives the stages' results."""
    import torch
    from frame_wise_delta_02_amd import binding as bd
    name = "bwd_64_ragged"
    gpu, ref, L, w, epi, dy = _run(name, stage2=True, stage3=True)
    x = synth.make_inputs(w)
    out, ws, desc, dev = G.run_forward(x, w, epilogue=epi)
    G.say(f"backward {name}")
    r = bd.backward(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["k_text"], dev["v_text"],
                    dev["beta_text"], dev["gate"], None, G.to_device(dy, w.dtype), ws, grid=(w.grid_h, w.grid_w),
                    chunk=w.chunk, epilogue=epi)
    torch.cuda.synchronize()
    pairs = {"dq": gpu["dq"], "dgate": gpu["dgate"], "dalpha": gpu["dalpha"]}
    pairs.update(zip(("dk", "dv", "dbeta", "dk_text", "dv_text", "dbeta_text"), gpu["gram"]))
    for k, t in pairs.items():
        assert torch.equal(r[k], t), k



def test_backward_768p_two_heads():
    """The 768p clip (B=1, T=60, 48 x 84 tokens, 24 heads of 128, 256 text
    tokens) in the configuration bench.py --backward times: the whole backward
    (binding.backward) on every head, checked against the oracle on heads 0
    and 13 for every input gradient."""
    import torch
    from frame_wise_delta_02_amd import binding as bd
    w = BASE
    hs = [0, 13]
    x = synth.make_inputs(w)
    dy = _dy(w)
    G.say("768p forward")
    out, ws, desc, dev = G.run_forward(x, w, epilogue=True)
    G.say("768p backward")
    r = bd.backward(dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["k_text"], dev["v_text"],
                    dev["beta_text"], dev["gate"], None, G.to_device(dy, w.dtype), ws, grid=(w.grid_h, w.grid_w),
                    chunk=w.chunk, epilogue=True)
    torch.cuda.synchronize()
    got = {k: r[k][..., hs, :] if r[k].dim() == 5 or k in ("dalpha", "dk_text", "dv_text") else r[k][..., hs]
           for k in ("dq", "dk", "dv", "dgate", "dalpha", "dbeta", "dk_text", "dv_text", "dbeta_text")}
    got = {k: v.to(torch.float64).cpu().numpy() for k, v in got.items()}
    del r, out, ws, dev
    G.say("768p oracle, heads 0 and 13")
    wide = lambda a: synth.to_f64(a, w.dtype)
    sub = {"q": wide(x["q"][:, :, :, hs]), "k": wide(x["k"][:, :, :, hs]), "v": wide(x["v"][:, :, :, hs]),
           "gate": wide(x["gate"][:, :, :, hs]), "beta": wide(x["beta"][:, :, :, hs]),
           "k_text": wide(x["k_text"][:, :, hs]), "v_text": wide(x["v_text"][:, :, hs]),
           "beta_text": wide(x["beta_text"][:, :, hs]), "alpha": x["alpha"][:, :, hs].astype(np.float64),
           "dy": wide(dy[:, :, :, hs])}
    ref = vda_grad.backward(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"], sub["k_text"], sub["v_text"],
                            sub["beta_text"], sub["dy"], gate=sub["gate"], chunk=w.chunk)
    txt = lambda a: a.reshape((a.shape[0], 1) + a.shape[1:] + ((1,) if a.ndim == 3 else ()))
    fr = slice(1, w.T - 1)
    errs = {"dq": G.slice_rel_err(got["dq"], ref["dq"]), "dgate": G.slice_rel_err(got["dgate"], ref["dgate"]),
            "dk": G.slice_rel_err(got["dk"][:, fr], ref["dk"][:, fr]),
            "dv": G.slice_rel_err(got["dv"][:, fr], ref["dv"][:, fr]),
            "dbeta": G.slice_rel_err(got["dbeta"][:, fr, ..., None], ref["dbeta"][:, fr, ..., None]),
            "dalpha": _rel(got["dalpha"][:, fr], ref["dalpha"][:, fr]),
            "dk_text": G.slice_rel_err(txt(got["dk_text"]), txt(ref["dk_txt"])),
            "dv_text": G.slice_rel_err(txt(got["dv_text"]), txt(ref["dv_txt"])),
            "dbeta_text": G.slice_rel_err(txt(got["dbeta_text"]), txt(ref["dbeta_txt"]))}
    # the anchors' tokens reach no state
    for k in ("dk", "dv", "dbeta"):
        assert np.abs(got[k][:, [0, w.T - 1]]).max() == 0, k
    G.say("768p heads 0, 13: " + " ".join(f"err({k})={v:.3e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= G.TOL[w.dtype], (k, v)
