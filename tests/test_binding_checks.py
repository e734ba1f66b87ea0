"""The binding's own argument checks (frame_wise_delta_02_amd/binding.py), on the
host: the library addresses every tensor from the descriptor alone, so the
binding must pass on tensors of exactly the sizes and element types the
descriptor implies, and refuse any other before a call reaches the library.

A stub stands in for libvdn_vda.so (it records each call and returns VDN_OK),
the device test is relaxed to CPU tensors, and the tensors are built as the GPU
tests, smoke() and bench.py build theirs: from the seeded inputs, bfloat16 bits
viewed as torch.bfloat16, outputs as empty_like of the inputs.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from frame_wise_delta_02_amd import binding as bd  # noqa: E402
from frame_wise_delta_02_amd import synth  # noqa: E402


class _StubLib:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def call(*args):
            self.calls.append(name)
            if name.endswith("_workspace_bytes"):
                return 4096
            if name == "vdn_vda_status_string":
                return b"stub"
            return bd.VDN_OK
        return call


@pytest.fixture
def lib(monkeypatch):
    stub = _StubLib()

    def check(x, name, dev):
        if x is not None and not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    monkeypatch.setattr(bd, "_lib", stub)
    monkeypatch.setattr(bd, "_check", check)
    monkeypatch.setattr(bd, "_stream", lambda: None)
    return stub


def _t(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


BF16 = synth.WORKLOADS["768p_bf16"].scaled(name="bind_bf16", B=2, H=2, T=5, grid_h=3, grid_w=4, d=32, L=6)
F32 = synth.WORKLOADS["stress_f32"].scaled(name="bind_f32", B=1, H=3, T=4, grid_h=2, grid_w=5, d=16, L=3)
NO_TEXT = BF16.scaled(name="bind_no_text", L=0)


def _inputs(w):
    return {k: _t(v) for k, v in synth.make_inputs(w).items()}


def _fwd_args(d):
    return (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["k_text"], d["v_text"], d["beta_text"], d["gate"])


@pytest.mark.parametrize("w", [BF16, F32, NO_TEXT], ids=lambda w: w.name)
def test_forward_accepts_the_tensors_the_callers_pass(lib, w):
    d = _inputs(w)
    grid = (w.grid_h, w.grid_w)
    rw = torch.from_numpy(np.linspace(0.5, 1.5, w.d).astype(np.float32))
    ws = torch.empty(4096, dtype=torch.uint8)
    for epi in (True, False):
        bd.forward(*_fwd_args(d), rw, grid=grid, chunk=w.chunk, epilogue=epi, workspace=ws,
                   out=torch.empty_like(d["q"]))
        bd.forward(*_fwd_args(d), None, grid=grid, chunk=w.chunk, epilogue=epi)
        bd.forward_noalloc(*_fwd_args(d), None, grid=grid, chunk=w.chunk, epilogue=epi)
    # without text tokens the text tensors may be left out
    bd.forward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None, None, None, d["gate"], None, grid=grid,
               chunk=w.chunk)
    assert lib.calls.count("vdn_vda_forward") == 5 and lib.calls.count("vdn_vda_forward_noalloc") == 2


def _bad_forward_cases(w):
    """(label, function that changes the arguments) for the forward pass."""
    def put(name, value):
        def f(a):
            a[name] = value(a)
        return f
    return [
        ("k one token short", put("k", lambda a: a["k"].reshape(-1)[: -w.d].clone())),
        ("v of another dtype", put("v", lambda a: a["v"].float() if a["v"].dtype != torch.float32
                                   else a["v"].to(torch.bfloat16))),
        ("gate one head short", put("gate", lambda a: a["gate"][:, :, :, 1:].contiguous())),
        ("alpha in the input dtype", put("alpha", lambda a: a["alpha"].to(torch.bfloat16)
                                         if a["q"].dtype != torch.bfloat16 else a["alpha"].to(torch.float64))),
        ("alpha per token", put("alpha", lambda a: torch.zeros(a["q"].shape, dtype=torch.float32))),
        ("beta per channel", put("beta", lambda a: torch.zeros(a["q"].shape, dtype=a["q"].dtype))),
        ("beta_text one token short", put("beta_text", lambda a: a["beta_text"][:, 1:].contiguous())),
        ("v_text missing", put("v_text", lambda a: None)),
        ("rms_weight too long", put("rms_weight", lambda a: torch.ones(w.d + 16, dtype=torch.float32))),
        ("rms_weight in bfloat16", put("rms_weight", lambda a: torch.ones(w.d, dtype=torch.bfloat16))),
        ("out one frame short", put("out", lambda a: torch.empty_like(a["q"][:, 1:]))),
        ("out of another dtype", put("out", lambda a: torch.empty(a["q"].shape, dtype=torch.float16))),
        ("grid of other tokens", put("grid", lambda a: (w.grid_h + 1, w.grid_w))),
        ("grid transposed onto fewer tokens", put("grid", lambda a: (w.grid_h, w.grid_w - 1))),
        ("workspace of float32", put("workspace", lambda a: torch.empty(1024, dtype=torch.float32))),
    ]


@pytest.mark.parametrize("label", [c[0] for c in _bad_forward_cases(BF16)])
def test_forward_refuses_before_the_library(lib, label):
    w = BF16
    a = dict(_inputs(w), rms_weight=torch.ones(w.d, dtype=torch.float32), out=None, workspace=None,
             grid=(w.grid_h, w.grid_w))
    dict(_bad_forward_cases(w))[label](a)
    for fn in (bd.forward, bd.forward_noalloc):
        kw = dict(grid=a["grid"], chunk=w.chunk, epilogue=True, out=a["out"])
        if fn is bd.forward:
            kw["workspace"] = a["workspace"]
        elif label.startswith("workspace"):
            continue
        with pytest.raises((ValueError, TypeError)):
            fn(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["k_text"], a["v_text"], a["beta_text"], a["gate"],
               a["rms_weight"], **kw)
    assert lib.calls == []


def test_forward_f32_refuses_bfloat16_alpha(lib):
    d = _inputs(F32)
    with pytest.raises(TypeError):
        bd.forward(d["q"], d["k"], d["v"], d["alpha"].to(torch.bfloat16), d["beta"], d["k_text"], d["v_text"],
                   d["beta_text"], d["gate"], None, grid=(F32.grid_h, F32.grid_w))
    assert lib.calls == []


PREP = synth.WORKLOADS["long_prep_bf16"].scaled(name="bind_prep", B=1, H=2, T=4, grid_h=3, grid_w=5, d=32, L=4)


def test_prepare_accepts_and_refuses(lib):
    d = _inputs(PREP)
    grid = (PREP.grid_h, PREP.grid_w)
    w4 = (d["wk_s"], d["wk_t"], d["wv_s"], d["wv_t"])
    qh, kh, vh = bd.prepare(d["q"], d["k"], d["v"], *w4, grid=grid)
    assert qh.shape == d["q"].shape and kh.dtype == d["k"].dtype
    qn, kf, vf = bd.prepare(None, d["k"], d["v"], *w4, grid=grid, query_l2=True)
    assert qn is None
    assert lib.calls.count("vdn_vda_prepare") == 2
    lib.calls.clear()
    bad = [
        dict(args=(None, d["k"], d["v"], *w4), kw={}),                       # q needed without query_l2
        dict(args=(d["q"], d["k"], d["v"][:, 1:].contiguous(), *w4), kw={}),
        dict(args=(d["q"], d["k"], d["v"], d["wk_s"][:, :, :4].contiguous(), *w4[1:]), kw={}),
        dict(args=(d["q"], d["k"], d["v"], d["wk_s"], d["wk_t"].double(), *w4[2:]), kw={}),
        dict(args=(d["q"], d["k"], d["v"], d["wk_s"], d["wk_t"], d["wv_s"], None), kw={}),
        dict(args=(d["q"], d["k"], d["v"], *w4), kw=dict(grid=(PREP.grid_w, PREP.grid_h + 1))),
    ]
    for b in bad:
        with pytest.raises((ValueError, TypeError)):
            bd.prepare(*b["args"], **dict(dict(grid=grid), **b["kw"]))
    assert lib.calls == []


def test_backward_stages_accept_and_refuse(lib):
    w = BF16
    d = _inputs(w)
    grid = (w.grid_h, w.grid_w)
    dy = torch.randn(d["q"].shape).to(torch.bfloat16)
    fws = torch.empty(4096, dtype=torch.uint8)
    bws = torch.empty(4096, dtype=torch.uint8)
    dq, dg = torch.empty_like(d["q"]), torch.empty_like(d["gate"])
    dalpha = torch.empty((w.B, w.T, w.H, w.d), dtype=torch.float32)
    gout = tuple(torch.empty_like(d[k]) for k in ("k", "v", "beta", "k_text", "v_text", "beta_text"))
    rw = torch.ones(w.d, dtype=torch.float32)
    bd.backward_readout(d["q"], d["gate"], rw, d["alpha"], dy, fws, grid=grid, n_text=w.L, chunk=w.chunk, dq=dq,
                        dgate=dg, workspace=bws, d_rms_weight=torch.empty(w.d, dtype=torch.float32))
    bd.backward_scan(d["alpha"], fws, bws, shape=(w.B, w.T, w.H, w.d), grid=grid, n_text=w.L, chunk=w.chunk,
                     dalpha=dalpha)
    bd.backward_gram(d["k"], d["v"], d["beta"], d["k_text"], d["v_text"], d["beta_text"], bws, grid=grid,
                     chunk=w.chunk, out=gout)
    r = bd.backward(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["k_text"], d["v_text"], d["beta_text"],
                    d["gate"], None, dy, fws, grid=grid, chunk=w.chunk)
    assert r["dk_text"].shape == d["k_text"].shape
    assert lib.calls == ["vdn_vda_backward_readout", "vdn_vda_backward_scan", "vdn_vda_backward_gram",
                         "vdn_vda_backward_workspace_bytes", "vdn_vda_backward_readout", "vdn_vda_backward_scan",
                         "vdn_vda_backward_gram"]
    lib.calls.clear()
    bad = [
        lambda: bd.backward_readout(d["q"], d["gate"], None, d["alpha"], dy.float(), fws, grid=grid, n_text=w.L),
        lambda: bd.backward_readout(d["q"], d["gate"], None, d["alpha"], dy, fws, grid=grid, n_text=w.L,
                                    dq=dq[:, 1:].contiguous()),
        lambda: bd.backward_readout(d["q"], d["gate"], None, d["alpha"], dy, fws.float(), grid=grid, n_text=w.L),
        lambda: bd.backward_readout(d["q"], d["gate"], None, d["alpha"], dy, fws, grid=(1, 1), n_text=w.L),
        lambda: bd.backward_readout(d["q"], d["gate"], None, d["alpha"], dy, fws, grid=grid, n_text=w.L,
                                    d_rms_weight=torch.empty(w.d + 1, dtype=torch.float32)),
        lambda: bd.backward_readout(d["q"], d["gate"], None, d["alpha"], dy, fws, grid=grid, n_text=w.L,
                                    d_rms_weight=torch.empty(w.d, dtype=torch.bfloat16)),
        lambda: bd.backward_readout(d["q"], None, None, d["alpha"], dy, fws, grid=grid, n_text=w.L, epilogue=False,
                                    d_rms_weight=torch.empty(w.d, dtype=torch.float32)),
        lambda: bd.backward_scan(d["alpha"], fws, bws, shape=(w.B, w.T, w.H, w.d), grid=grid,
                                 dalpha=dalpha[:, 1:].contiguous()),
        lambda: bd.backward_scan(d["alpha"].to(torch.bfloat16), fws, bws, shape=(w.B, w.T, w.H, w.d), grid=grid),
        lambda: bd.backward_gram(d["k"], d["v"], d["beta"], d["k_text"], d["v_text"], d["beta_text"], bws, grid=grid,
                                 out=gout[:5]),
        lambda: bd.backward_gram(d["k"], d["v"], d["beta"], d["k_text"], d["v_text"], d["beta_text"], bws, grid=grid,
                                 out=gout[:3] + (gout[3][:, 1:].contiguous(),) + gout[4:]),
        lambda: bd.backward_gram(d["k"], d["v"], d["beta"][..., :1].contiguous(), d["k_text"], d["v_text"],
                                 d["beta_text"], bws, grid=grid),
    ]
    for f in bad:
        with pytest.raises((ValueError, TypeError)):
            f()
    assert lib.calls == []


def test_adjacent_maps_accept_and_refuse(lib):
    w, dm = BF16.scaled(name="bind_adj", L=0), 48
    p = {k: _t(v) for k, v in synth.make_adjacent_inputs(w, dm).items()}
    grid = (w.grid_h, w.grid_w)
    gate, beta, alpha = bd.gates(p["x"], p["w_gb"], p["w_alpha"], heads=w.H, d=w.d, grid=grid)
    assert gate.shape == (w.B, w.T, w.U, w.H, w.d) and beta.shape == (w.B, w.T, w.U, w.H)
    bd.gates(p["x"], p["w_gb"], p["w_alpha"], heads=w.H, d=w.d, grid=grid, out=(gate, beta, alpha),
             workspace=torch.empty(4096, dtype=torch.uint8))
    bd.out_proj(p["o"], p["w_o"], p["y_in"], grid=grid)
    bd.out_proj(p["o"], p["w_o"], p["y_in"], grid=grid, out=p["y_in"])
    bd.out_proj(p["o"], p["w_o"], None, grid=grid)
    assert lib.calls.count("vdn_vda_gates") == 2 and lib.calls.count("vdn_vda_out_proj") == 3
    lib.calls.clear()
    bad = [
        lambda: bd.gates(p["x"], p["w_gb"][1:].contiguous(), p["w_alpha"], heads=w.H, d=w.d, grid=grid),
        lambda: bd.gates(p["x"], p["w_gb"], p["w_alpha"].to(torch.bfloat16), heads=w.H, d=w.d, grid=grid),
        lambda: bd.gates(p["x"], p["w_gb"], p["w_alpha"], heads=w.H, d=w.d, grid=(w.grid_h, w.grid_w + 1)),
        lambda: bd.gates(p["x"], p["w_gb"], p["w_alpha"], heads=w.H, d=w.d, grid=grid,
                         out=(gate, beta[:, 1:].contiguous(), alpha)),
        lambda: bd.out_proj(p["o"], p["w_o"][:, 1:].contiguous(), p["y_in"], grid=grid),
        lambda: bd.out_proj(p["o"], p["w_o"], p["y_in"][:, 1:].contiguous(), grid=grid),
        lambda: bd.out_proj(p["o"].float(), p["w_o"], p["y_in"], grid=grid),
        lambda: bd.out_proj(p["o"], p["w_o"], p["y_in"], grid=grid, out=torch.empty(3, dtype=torch.bfloat16)),
    ]
    for f in bad:
        with pytest.raises((ValueError, TypeError)):
            f()
    assert lib.calls == []
