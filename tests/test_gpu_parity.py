"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Every case draws seeded inputs, runs vdn_vda_forward (and vdn_vda_prepare for
the prep workload), and compares element by element with the oracle computed on
the same arrays.  Tolerance on the output: max relative error per (frame, head)
slice <= 1e-3 for float32 inputs and <= 2e-2 for bfloat16 inputs (fp32 state).
"""

import numpy as np
import pytest

import oracle
from frame_wise_delta_02_amd import synth
import gpu_harness as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name_case(request):
    G.say(request.node.nodeid)
    yield


def _oracle_heads(x, w, heads, gate=True, rms_weight=None, prepared=None, bridge=False):
    """Oracle forward on the listed heads only (inputs sliced before widening)."""
    sl = lambda a: a[:, :, :, heads] if a.ndim == 5 else a
    f = {}
    for k in ("q", "k", "v", "gate"):
        src = prepared[k] if (prepared is not None and k in prepared) else sl(x[k])
        f[k] = src if src.dtype == np.float64 else G.oracle_view({k: src}, w)[k]
    f["beta"] = G.oracle_view({"b": x["beta"][:, :, :, heads]}, w)["b"]
    f["alpha"] = x["alpha"][:, :, heads].astype(np.float64)
    for k in ("k_text", "v_text"):
        f[k] = G.oracle_view({k: x[k][:, :, heads]}, w)[k]
    f["beta_text"] = G.oracle_view({"b": x["beta_text"][:, :, heads]}, w)["b"]
    return oracle.forward(f["q"], f["k"], f["v"], f["alpha"], f["beta"], f["k_text"], f["v_text"],
                          f["beta_text"], gate=f["gate"] if gate else None, rms_weight=rms_weight,
                          chunk=w.chunk, bridge=bridge)


def _check_intermediates(inter, ref, w, heads, tol):
    T, nc = w.T, -(-w.T // w.chunk)
    hs = list(heads)
    if T > 2:
        fr = slice(1, T - 1)
        assert G.mat_rel_err(inter["A"][:, hs, fr], ref["A"][:, :, fr]) <= tol, "A"
        assert G.mat_rel_err(inter["B"][:, hs, fr], ref["B"][:, :, fr]) <= tol, "B"
        assert G.mat_rel_err(inter["Pinv"][:, hs, fr], ref["Pinv"][:, :, fr]) <= tol, "Pinv"
    if w.L:
        assert G.mat_rel_err(inter["S_T"][:, hs], ref["S_T"]) <= tol, "S_T"
    if nc >= 3:
        assert G.mat_rel_err(inter["F"][:, hs, : nc - 2], ref["F"][:, :, : nc - 2]) <= tol, "F"
        assert G.mat_rel_err(inter["R"][:, hs, 2:], ref["R"][:, :, 2:]) <= tol, "R"


def _run_case(w, heads=None, rms=False, check_inter=True, bridge=False, scan=None, group=None):
    """Forward (raw readout with intermediates, then with RMSNorm + gate) against
    the oracle on ``heads`` (all by default), the oracle called on ``group``
    heads at a time to bound host memory."""
    x = synth.make_inputs(w)
    heads = list(range(w.H)) if heads is None else heads
    groups = [heads] if group is None else [heads[i:i + group] for i in range(0, len(heads), group)]
    rw = np.random.default_rng(5).uniform(0.5, 1.5, w.d) if rms else None
    tol = G.TOL[w.dtype]
    out, ws, desc, dev = G.run_forward(x, w, epilogue=False, bridge=bridge, scan=scan)
    inter = G.intermediates(ws, desc, w) if check_inter else None
    del ws
    out2, _, _, _ = G.run_forward(x, w, epilogue=True, rms_weight=rw, dev_inputs=dev, bridge=bridge, scan=scan)
    err_o = err_y = 0.0
    for grp in groups:
        ref = _oracle_heads(x, w, grp, gate=True, rms_weight=rw, bridge=bridge)
        err_o = max(err_o, G.slice_rel_err(G.to_host_f64(out[:, :, :, grp]), ref["o"]))
        err_y = max(err_y, G.slice_rel_err(G.to_host_f64(out2[:, :, :, grp]), ref["y"]))
        if check_inter:
            _check_intermediates(inter, ref, w, grp, tol)
        del ref
    G.say(f"{w.name} T={w.T} U={w.U} H={w.H} d={w.d} scan={scan} heads={len(heads)}: "
          f"err(o)={err_o:.3e} err(y)={err_y:.3e} tol={tol}")
    assert err_o <= tol, err_o
    assert err_y <= tol, err_y
    return err_o, err_y


# Both scans (VDN_VDA_SCAN_FRAMES, VDN_VDA_SCAN_CHUNKS) on every workload and
# edge case: without a flag the library picks by the number of (batch, head)
# pairs, which would leave one of them untested on small shapes.
SCANS = ["frames", "chunks"]


@pytest.mark.parametrize("scan", SCANS)
@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16", "stress_f32", "stress_tight_f32"])
def test_workload_full_oracle(name, scan):
    _run_case(synth.WORKLOADS[name], rms=(name == "small_bf16"), scan=scan)


def test_768p_full_size_every_head():
    """The benchmarked workload at full size, in the launch configuration the
    benchmark times (the library's own scan choice): every one of the 24 heads
    against the oracle, the output and every intermediate."""
    _run_case(synth.WORKLOADS["768p_bf16"], group=4)


@pytest.mark.parametrize("scan", SCANS)
def test_768p_share8_full_size(scan):
    """One GPU's share of the 768p clip under an 8-way head split (3 heads), the
    regime the chunk-composed scan is for; the oracle checks every head."""
    _run_case(synth.WORKLOADS["768p_share8_bf16"], scan=scan)


EDGE = {
    # several tiles and ragged tails: U = 100 (64 + 36 gram tile, 3x32 + 4 readout tile), T = 17
    "ragged_bf16_128": synth.WORKLOADS["768p_bf16"].scaled(name="ragged_bf16_128", H=3, T=17, grid_h=10, grid_w=10, L=37),
    "ragged_f32_128": synth.WORKLOADS["stress_f32"].scaled(name="ragged_f32_128", H=2, T=13, grid_h=7, grid_w=11, L=5),
    "d64_bf16": synth.WORKLOADS["small_bf16"].scaled(name="d64_bf16", H=3, T=12, grid_h=5, grid_w=13, L=9),
    "d32_bf16": synth.WORKLOADS["small_bf16"].scaled(name="d32_bf16", d=32, H=2, T=16, grid_h=6, grid_w=6, L=4),
    "d32_f32": synth.WORKLOADS["tiny_f32"].scaled(name="d32_f32", d=32, H=2, T=11, grid_h=3, grid_w=7, L=3),
    "d16_bf16": synth.WORKLOADS["tiny_f32"].scaled(name="d16_bf16", dtype="bf16", H=3, T=14, L=2),
    "no_text_bf16": synth.WORKLOADS["768p_bf16"].scaled(name="no_text_bf16", H=2, T=15, grid_h=4, grid_w=9, L=0),
    "T1_bf16": synth.WORKLOADS["768p_bf16"].scaled(name="T1_bf16", H=2, T=1, grid_h=4, grid_w=8, L=16),
    "T2_f32": synth.WORKLOADS["stress_f32"].scaled(name="T2_f32", H=2, T=2, grid_h=4, grid_w=8, L=16),
    "T7_f32": synth.WORKLOADS["tiny_f32"].scaled(name="T7_f32", T=7),
    "chunk3_bf16": synth.WORKLOADS["small_bf16"].scaled(name="chunk3_bf16", H=2, T=20, grid_h=4, grid_w=10, chunk=3, L=8),
    "chunk1_f32": synth.WORKLOADS["tiny_f32"].scaled(name="chunk1_f32", T=9, chunk=1),
    "batch2_bf16": synth.WORKLOADS["768p_bf16"].scaled(name="batch2_bf16", B=2, H=2, T=16, grid_h=6, grid_w=11, L=12),
    # one and two tokens per frame: the one-token regime where a frame update is
    # the token delta rule with beta / (1 + beta) ([VDN-summary] "어떻게 쓰나"),
    # each a single valid row in a 64-token statistics tile and a 32-token readout tile
    "U1_bf16_128": synth.WORKLOADS["768p_bf16"].scaled(name="U1_bf16_128", H=2, T=12, grid_h=1, grid_w=1, L=3),
    "U2_bf16_128": synth.WORKLOADS["768p_bf16"].scaled(name="U2_bf16_128", H=2, T=13, grid_h=1, grid_w=2, L=3),
    "U1_f32_16": synth.WORKLOADS["tiny_f32"].scaled(name="U1_f32_16", T=12, grid_h=1, grid_w=1, L=2),
    "U2_f32_16": synth.WORKLOADS["tiny_f32"].scaled(name="U2_f32_16", T=11, grid_h=2, grid_w=1, L=2),
}


@pytest.mark.parametrize("scan", SCANS)
@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases(name, scan):
    _run_case(EDGE[name], rms=name.endswith("128") or name in ("d16_bf16", "d32_bf16"), scan=scan)


# VDA-Gather's decay bridge (VDN_VDA_DECAY_BRIDGE): every chunk position,
# a short last chunk, both dtypes and the narrow widths.
BRIDGE = {
    "bridge_bf16_128": EDGE["ragged_bf16_128"],
    "bridge_f32_128": EDGE["ragged_f32_128"],
    "bridge_chunk3_bf16": EDGE["chunk3_bf16"],
    "bridge_d16_f32": EDGE["T7_f32"].scaled(name="bridge_d16_f32", T=23),
    "bridge_768p": synth.WORKLOADS["768p_bf16"],
}


@pytest.mark.parametrize("name", list(BRIDGE))
def test_decay_bridge(name):
    w = BRIDGE[name]
    _run_case(w, bridge=True, group=4)


def test_zero_writes_give_text_only_readout():
    """beta = 0 on every video token and alpha = 1: every frame reads S_T q, with
    S_T the oracle's text state (the frame update from a zero state over the
    text tokens, [VDN-summary] "어떻게 동작하나")."""
    w = EDGE["ragged_bf16_128"]
    x = synth.make_inputs(w)
    x["beta"][:] = 0
    x["alpha"][:] = 1.0
    out, _, _, _ = G.run_forward(x, w, epilogue=False)
    f = G.oracle_view({k: x[k] for k in ("q", "k_text", "v_text", "beta_text")}, w)
    ST = np.stack([np.stack([oracle.text_state(f["k_text"][b, :, h], f["v_text"][b, :, h], f["beta_text"][b, :, h])
                             for h in range(w.H)]) for b in range(w.B)])
    want = np.einsum("btuhk,bhvk->btuhv", f["q"], ST)
    got = G.to_host_f64(out)
    err = G.slice_rel_err(got, want)
    G.say(f"zero writes: err={err:.3e}")
    assert err <= G.TOL[w.dtype]


def test_deterministic_rerun():
    w = EDGE["ragged_bf16_128"]
    x = synth.make_inputs(w)
    import torch
    o1, _, _, dev = G.run_forward(x, w, epilogue=True)
    o2, _, _, _ = G.run_forward(x, w, epilogue=True, dev_inputs=dev)
    assert torch.equal(o1, o2)


# ---------------------------------------------------------------------------
# prep (conv, SiLU, L2) and the fused long clip
# ---------------------------------------------------------------------------


def _prep_case(w, heads):
    import torch
    from frame_wise_delta_02_amd import binding as bd
    x = synth.make_inputs(w)
    dev = {k: G.to_device(v, w.dtype) for k, v in x.items()}
    G.say(f"prepare {w.name} T={w.T} grid={w.grid_h}x{w.grid_w} H={w.H}")
    qh, kh, vh = bd.prepare(dev["q"], dev["k"], dev["v"], dev["wk_s"], dev["wk_t"], dev["wv_s"], dev["wv_t"],
                            grid=(w.grid_h, w.grid_w))
    torch.cuda.synchronize()
    prepared = {}
    errs = {}
    for b in range(w.B):
        for h in heads:
            sl = lambda a: a[b, :, :, h:h + 1]
            f = G.oracle_view({"q": sl(x["q"]), "k": sl(x["k"]), "v": sl(x["v"])}, w)
            ws_ = lambda n: x[n][h * w.d:(h + 1) * w.d].astype(np.float64)
            rq, rk, rv = oracle.prep(f["q"], f["k"], f["v"], ws_("wk_s"), ws_("wk_t"), ws_("wv_s"), ws_("wv_t"),
                                     w.grid_h, w.grid_w, l2_eps=1e-6)
            for name, ref, got in (("q", rq, qh), ("k", rk, kh), ("v", rv, vh)):
                g = G.to_host_f64(got[b, :, :, h:h + 1])
                errs[name] = max(errs.get(name, 0.0), G.slice_rel_err(g[None], ref[None]))
                if b == 0:
                    prepared.setdefault(name, []).append(ref)
    G.say(f"prep errors {errs}")
    for name, e in errs.items():
        assert e <= (1e-2 if w.dtype == "bf16" else 1e-5), (name, e)
    return x, dev, (qh, kh, vh), {k: np.concatenate(v, axis=2)[None] for k, v in prepared.items()}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prepare_small(dtype):
    w = synth.WORKLOADS["long_prep_bf16"].scaled(name=f"prep_small_{dtype}", dtype=dtype, H=2, T=9,
                                                   grid_h=6, grid_w=10, L=8)
    _prep_case(w, heads=[0, 1])


# The d = 128 bfloat16 prep runs 8 x 12 output tiles that sweep every frame:
# ragged tiles in both directions, clips shorter than the 5 temporal taps, and
# the head-per-XCD block order (H divisible by 8) with two batch elements.
PREP_EDGE = {
    "prep_T1_ragged": dict(H=2, T=1, grid_h=9, grid_w=13, L=4),
    "prep_T2_ragged": dict(H=1, T=2, grid_h=9, grid_w=13, L=4),
    "prep_B2_H8_tiles": dict(B=2, H=8, T=7, grid_h=17, grid_w=25, L=4),
}


@pytest.mark.parametrize("name", list(PREP_EDGE))
def test_prepare_edges(name):
    w = synth.WORKLOADS["long_prep_bf16"].scaled(name=name, **PREP_EDGE[name])
    _prep_case(w, heads=list(range(min(w.H, 3))) + ([w.H - 1] if w.H > 3 else []))


def _fused_query_prepare(dev, w, kh, vh):
    """prepare under VDN_VDA_QUERY_L2: no q_hat, and k_hat, v_hat bit-identical to the unfused call."""
    import torch
    from frame_wise_delta_02_amd import binding as bd
    G.say(f"prepare (query left to the readout) {w.name}")
    qn, kf, vf = bd.prepare(None, dev["k"], dev["v"], dev["wk_s"], dev["wk_t"], dev["wv_s"], dev["wv_t"],
                            grid=(w.grid_h, w.grid_w), query_l2=True)
    torch.cuda.synchronize()
    assert qn is None
    assert torch.equal(kf.view(torch.int16) if kf.dtype == torch.bfloat16 else kf,
                       kh.view(torch.int16) if kh.dtype == torch.bfloat16 else kh)
    assert torch.equal(vf.view(torch.int16) if vf.dtype == torch.bfloat16 else vf,
                       vh.view(torch.int16) if vh.dtype == torch.bfloat16 else vh)
    return kf, vf


_LONG = {}


def _long_clip():
    """The long clip at full size, run once for the tests below: prepare, the
    forward on the prepared features, the prepare that leaves the query to the
    readout (checked bit-identical on K^, V^) and the forward with the fused
    query normalisation.  Both forwards run in the benchmarked configuration."""
    import torch
    from frame_wise_delta_02_amd import binding as bd
    if _LONG:
        return _LONG
    w = synth.WORKLOADS["long_prep_bf16"]
    x = synth.make_inputs(w)
    dev = {k: G.to_device(v, w.dtype) for k, v in x.items()}
    G.say(f"prepare {w.name} T={w.T} grid={w.grid_h}x{w.grid_w} H={w.H}")
    qh, kh, vh = bd.prepare(dev["q"], dev["k"], dev["v"], dev["wk_s"], dev["wk_t"], dev["wv_s"], dev["wv_t"],
                            grid=(w.grid_h, w.grid_w))
    torch.cuda.synchronize()
    out, _, _, _ = G.run_forward(x, w, epilogue=True, dev_inputs=dict(dev, q=qh, k=kh, v=vh))
    kf, vf = _fused_query_prepare(dev, w, kh, vh)
    del kh, vh
    out2, _, _, _ = G.run_forward(x, w, epilogue=True, dev_inputs=dict(dev, k=kf, v=vf), query_l2=True)
    _LONG.update(w=w, x=x, prepared=(qh, kf, vf), out=out, out_fused=out2)
    return _LONG


def _long_clip_heads(heads):
    L = _long_clip()
    w, x = L["w"], L["x"]
    qh, kh, vh = L["prepared"]
    for h in heads:
        f = G.oracle_view({n: x[n][:, :, :, h:h + 1] for n in ("q", "k", "v")}, w)
        wsl = lambda n: x[n][h * w.d:(h + 1) * w.d].astype(np.float64)
        rq, rk, rv = oracle.prep(f["q"][0], f["k"][0], f["v"][0], wsl("wk_s"), wsl("wk_t"), wsl("wv_s"),
                                 wsl("wv_t"), w.grid_h, w.grid_w, l2_eps=1e-6)
        perr = {n: G.slice_rel_err(G.to_host_f64(t[:, :, :, h:h + 1]), r[None])
                for n, r, t in (("q", rq, qh), ("k", rk, kh), ("v", rv, vh))}
        prepared = {"q": rq[None], "k": rk[None], "v": rv[None], "gate": x["gate"][:, :, :, [h]]}
        ref = _oracle_heads(x, w, [h], gate=True, prepared=prepared)
        e1 = G.slice_rel_err(G.to_host_f64(L["out"][:, :, :, [h]]), ref["y"])
        e2 = G.slice_rel_err(G.to_host_f64(L["out_fused"][:, :, :, [h]]), ref["y"])
        G.say(f"long_prep_bf16 head {h}: prep {perr}, err(y)={e1:.3e}, fused query L2 err(y)={e2:.3e}")
        for n, e in perr.items():
            assert e <= 1e-2, (h, n, e)
        assert e1 <= G.TOL["bf16"], (h, e1)
        assert e2 <= G.TOL["bf16"], (h, e2)


# The long clip at full size: one head from each group of eight (the prep's and
# the scan's blocks map heads to XCDs by h mod 8) and from both ends.
def test_long_prep_full_size_heads_a():
    _long_clip_heads([0, 5, 8])


def test_long_prep_full_size_heads_b():
    try:
        _long_clip_heads([15, 16, 23])
    finally:
        _LONG.clear()


# The query's L2 normalisation fused into the readout (VDN_VDA_QUERY_L2): raw q
# into the forward pass, for both readout kernels, every head width, with and
# without the epilogue and the RMSNorm gain.
QL2 = {
    "ql2_bf16_128": dict(H=2, T=9, grid_h=6, grid_w=10, L=8),
    "ql2_bf16_64_ragged": dict(H=3, T=11, grid_h=7, grid_w=9, L=8, d=64),
    "ql2_bf16_32": dict(H=2, T=7, grid_h=5, grid_w=13, L=4, d=32),
    "ql2_bf16_16": dict(H=2, T=6, grid_h=4, grid_w=9, L=4, d=16),
    "ql2_f32_128": dict(H=2, T=8, grid_h=6, grid_w=7, L=8, dtype="f32"),
    "ql2_f32_16": dict(H=2, T=6, grid_h=5, grid_w=5, L=4, d=16, dtype="f32"),
}


@pytest.mark.parametrize("name", list(QL2))
def test_query_l2_fused(name):
    w = synth.WORKLOADS["long_prep_bf16"].scaled(name=name, **QL2[name])
    heads = list(range(w.H))
    x, dev, (qh, kh, vh), prepared = _prep_case(w, heads=heads)
    kf, vf = _fused_query_prepare(dev, w, kh, vh)
    rw = np.random.default_rng(11).uniform(0.5, 1.5, w.d)
    dev2 = dict(dev, k=kf, v=vf)  # q stays raw
    tol = G.TOL[w.dtype]
    for epi, gain in ((False, None), (True, None), (True, rw)):
        out, _, _, _ = G.run_forward(x, w, epilogue=epi, rms_weight=gain, dev_inputs=dev2, query_l2=True)
        ref = _oracle_heads(x, w, heads, gate=True, rms_weight=gain, prepared=prepared)
        err = G.slice_rel_err(G.to_host_f64(out), ref["y" if epi else "o"])
        G.say(f"{name} epilogue={epi} gain={gain is not None}: err={err:.3e} tol={tol}")
        assert err <= tol, (epi, gain is not None, err)


def test_values_beyond_the_half_range():
    """Value entries with |sqrt(beta) v| far above 65504 (the largest IEEE half,
    the statistics kernel's operand type) in two video frames and in the text
    frame: the kernel rescales those units' operands by powers of two and the
    result matches the oracle as for ordinary inputs."""
    w = EDGE["ragged_bf16_128"]
    x = synth.make_inputs(w)
    v = oracle.widen_bf16_bits(x["v"])
    v[:, 3, :30, 1] *= 1.0e5
    v[:, 7, 50:, 0] *= 3.0e4
    x["v"] = synth.f64_to_bf16_bits(v)
    vt = oracle.widen_bf16_bits(x["v_text"])
    vt[:, :5, 2] *= 2.0e5
    x["v_text"] = synth.f64_to_bf16_bits(vt)
    beta = oracle.widen_bf16_bits(x["beta"])
    big = np.abs(np.sqrt(beta)[..., None] * v).max()
    assert big > 1.0e5, big
    out, ws, desc, _ = G.run_forward(x, w, epilogue=True)
    inter = G.intermediates(ws, desc, w)
    ref = _oracle_heads(x, w, list(range(w.H)), gate=True)
    tol = G.TOL[w.dtype]
    err = G.slice_rel_err(G.to_host_f64(out), ref["y"])
    eb = G.mat_rel_err(inter["B"][:, :, 1:w.T - 1], ref["B"][:, :, 1:w.T - 1])
    est = G.mat_rel_err(inter["S_T"], ref["S_T"])
    G.say(f"values beyond half range (max |sqrt(beta) v| = {big:.3g}): err(y)={err:.3e} err(B)={eb:.3e} err(S_T)={est:.3e}")
    assert np.isfinite(G.to_host_f64(out)).all()
    assert err <= tol and eb <= tol and est <= tol, (err, eb, est)
