"""The CPU build of the library (libvdn_vda_sim.so, tests/cpu_build/build.py)
driven from numpy: the same C ABI as the HIP library, with host buffers in
place of device memory.  Mirrors the GPU harness (tests/gpu_harness.py) so that
the CPU-build tests compare with the oracle exactly as the GPU parity tests do.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from frame_wise_delta_02_amd import binding as bd
from frame_wise_delta_02_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(ROOT, "_build", "cpu_build")


def load(path: str) -> ctypes.CDLL:
    return bd.declare(ctypes.CDLL(path))


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _aligned(nbytes: int, align: int = 256) -> np.ndarray:
    """A zeroed uint8 buffer of ``nbytes`` whose data pointer is ``align``-aligned."""
    raw = np.zeros(nbytes + align, np.uint8)
    off = (-raw.ctypes.data) % align
    return raw[off:off + nbytes]


def _c(a):
    return None if a is None else np.ascontiguousarray(a)


def run_forward(L, x: dict, w: synth.Workload, epilogue=True, rms_weight=None, bridge=False, query_l2=False,
                scan=None, inputs=None):
    """vdn_vda_forward on host copies of ``x`` (or on ``inputs``, the prepared
    features); returns (out, workspace, desc) as numpy arrays."""
    src = dict(x) if inputs is None else {**x, **inputs}
    desc = bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, w.L, w.chunk, w.dtype, epilogue,
                        flags=(bd.VDN_VDA_EPILOGUE if epilogue else 0) | (bd.VDN_VDA_DECAY_BRIDGE if bridge else 0)
                        | (bd.VDN_VDA_QUERY_L2 if query_l2 else 0) | bd._SCAN_FLAGS[scan])
    st = L.vdn_vda_validate(ctypes.byref(desc))
    assert st == bd.VDN_OK, st
    a = {k: _c(src[k]) for k in ("q", "k", "v", "alpha", "beta", "gate")}
    for k in ("k_text", "v_text", "beta_text"):
        a[k] = _c(src[k]) if w.L else None
    rw = None if rms_weight is None else np.ascontiguousarray(rms_weight, np.float32)
    out = np.zeros_like(a["q"])
    ws = _aligned(L.vdn_vda_workspace_bytes(ctypes.byref(desc)))
    st = L.vdn_vda_forward(ctypes.byref(desc), _ptr(a["q"]), _ptr(a["k"]), _ptr(a["v"]), _ptr(a["alpha"]),
                           _ptr(a["beta"]), _ptr(a["k_text"]), _ptr(a["v_text"]), _ptr(a["beta_text"]),
                           _ptr(a["gate"]) if epilogue else None, _ptr(rw), _ptr(out), _ptr(ws), ws.size, None)
    assert st == bd.VDN_OK, L.vdn_vda_status_string(st)
    return out, ws, desc


def run_prepare(L, x: dict, w: synth.Workload, query_l2=False):
    """vdn_vda_prepare; returns (q_hat or None, k_hat, v_hat)."""
    desc = bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, w.L, w.chunk, w.dtype, False,
                        flags=bd.VDN_VDA_QUERY_L2 if query_l2 else 0)
    a = {k: _c(x[k]) for k in ("q", "k", "v", "wk_s", "wk_t", "wv_s", "wv_t")}
    q_hat = None if query_l2 else np.zeros_like(a["q"])
    k_hat, v_hat = np.zeros_like(a["k"]), np.zeros_like(a["v"])
    st = L.vdn_vda_prepare(ctypes.byref(desc), None if query_l2 else _ptr(a["q"]), _ptr(a["k"]), _ptr(a["v"]),
                           _ptr(a["wk_s"]), _ptr(a["wk_t"]), _ptr(a["wv_s"]), _ptr(a["wv_t"]),
                           None if query_l2 else _ptr(q_hat), _ptr(k_hat), _ptr(v_hat), None)
    assert st == bd.VDN_OK, L.vdn_vda_status_string(st)
    return q_hat, k_hat, v_hat


def to_f64(a: np.ndarray) -> np.ndarray:
    """Host output in the input dtype (bfloat16 bits or float32) as float64."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def intermediates(L, ws: np.ndarray, desc, w: synth.Workload) -> dict:
    """float64 copies of the workspace intermediates (as tests/gpu_harness.py)."""
    import gpu_harness as G
    lay = bd.Layout()
    assert L.vdn_vda_workspace_layout(ctypes.byref(desc), ctypes.byref(lay)) == bd.VDN_OK
    B, H, T, D = w.B, w.H, w.T, w.d
    nc = -(-T // w.chunk)

    def arr(off, shape):
        n = int(np.prod(shape)) * 4
        return ws[off:off + n].view(np.float32).reshape(shape).astype(np.float64)

    stats = arr(lay.stats, (B, H, T + 1, 2 * D, D))
    if w.dtype == "bf16" and D >= 32:
        n = B * H * (T + 1) * D * D * 4
        raw = ws[lay.pinv:lay.pinv + n].view(np.int16).reshape(B * H * (T + 1), 2, D * D)
        pinv = G.decode_split_pinv(raw, D).reshape(B, H, T + 1, D, D)
    else:
        pinv = arr(lay.pinv, (B, H, T + 1, D, D))
    return dict(A=stats[:, :, :, :D], B=stats[:, :, :, D:], Pinv=pinv,
                S_T=arr(lay.s_text, (B, H, D, D)), F=arr(lay.fwd, (B, H, nc, D, D)),
                R=arr(lay.rev, (B, H, nc, D, D)))


def run_backward(L, x: dict, w: synth.Workload, dy: np.ndarray, fwd_ws: np.ndarray, epilogue=True, rms_weight=None,
                 bridge=False, query_l2=False, l2_eps=1e-6, gain=False):
    """The three backward stages (vdn_vda_backward_readout, _scan, _gram) after a
    forward that left ``fwd_ws``; returns a dict of numpy results (with ``gain``
    the RMSNorm gain's gradient as dgamma), the backward workspace and its
    layout."""
    flags = (bd.VDN_VDA_EPILOGUE if epilogue else 0) | (bd.VDN_VDA_DECAY_BRIDGE if bridge else 0) \
        | (bd.VDN_VDA_QUERY_L2 if query_l2 else 0)
    desc = bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, w.L, w.chunk, w.dtype, epilogue, l2_eps=l2_eps,
                        flags=flags)
    a = {k: _c(x[k]) for k in ("q", "k", "v", "alpha", "beta", "gate")}
    for k in ("k_text", "v_text", "beta_text"):
        a[k] = _c(x[k]) if w.L else None
    rw = None if rms_weight is None else np.ascontiguousarray(rms_weight, np.float32)
    dy = np.ascontiguousarray(dy)
    bws = _aligned(L.vdn_vda_backward_workspace_bytes(ctypes.byref(desc)))
    lay = bd.BackwardLayout()
    assert L.vdn_vda_backward_workspace_layout(ctypes.byref(desc), ctypes.byref(lay)) == bd.VDN_OK
    dq = np.zeros_like(a["q"])
    dgate = np.zeros_like(dy) if epilogue else None
    dgamma = np.full(w.d, np.nan, np.float32) if gain else None
    st = L.vdn_vda_backward_readout(ctypes.byref(desc), _ptr(a["q"]), _ptr(a["gate"]) if epilogue else None,
                                    _ptr(rw), _ptr(a["alpha"]), _ptr(dy), _ptr(fwd_ws), fwd_ws.size, _ptr(dq),
                                    _ptr(dgate), _ptr(dgamma), _ptr(bws), bws.size, None)
    assert st == bd.VDN_OK, L.vdn_vda_status_string(st)
    dalpha = np.zeros((w.B, w.T, w.H, w.d), np.float32)
    st = L.vdn_vda_backward_scan(ctypes.byref(desc), _ptr(a["alpha"]), _ptr(fwd_ws), fwd_ws.size, _ptr(dalpha),
                                 _ptr(bws), bws.size, None)
    assert st == bd.VDN_OK, L.vdn_vda_status_string(st)
    grads = [np.zeros_like(a["k"]), np.zeros_like(a["v"]), np.zeros_like(a["beta"])]
    grads += [None if a[k] is None else np.zeros_like(a[k]) for k in ("k_text", "v_text", "beta_text")]
    st = L.vdn_vda_backward_gram(ctypes.byref(desc), _ptr(a["k"]), _ptr(a["v"]), _ptr(a["beta"]),
                                 _ptr(a["k_text"]), _ptr(a["v_text"]), _ptr(a["beta_text"]), *map(_ptr, grads),
                                 _ptr(bws), bws.size, None)
    assert st == bd.VDN_OK, L.vdn_vda_status_string(st)
    return dict(dq=dq, dgate=dgate, dalpha=dalpha, dk=grads[0], dv=grads[1], dbeta=grads[2], dk_text=grads[3],
                dv_text=grads[4], dbeta_text=grads[5], dgamma=dgamma), bws, lay


def section(ws: np.ndarray, off: int, shape, dtype="f32") -> np.ndarray:
    n = int(np.prod(shape))
    if dtype == "bf16":
        return to_f64(ws[off:off + 2 * n].view(np.uint16).reshape(shape))
    return ws[off:off + 4 * n].view(np.float32).reshape(shape).astype(np.float64)


def run_gates(L, p: dict, w: synth.Workload, dm: int):
    """vdn_vda_gates on synth.make_adjacent_inputs' arrays; returns (gate, beta, alpha)."""
    desc = bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, 0, w.chunk, "bf16", False)
    x, wgb, wal = _c(p["x"]), _c(p["w_gb"]), _c(p["w_alpha"])
    gate = np.zeros((w.B, w.T, w.U, w.H, w.d), np.uint16)
    beta = np.zeros((w.B, w.T, w.U, w.H), np.uint16)
    alpha = np.zeros((w.B, w.T, w.H, w.d), np.float32)
    ws = _aligned(max(1, L.vdn_vda_gates_workspace_bytes(ctypes.byref(desc), dm)))
    st = L.vdn_vda_gates(ctypes.byref(desc), dm, _ptr(x), _ptr(wgb), _ptr(wal), _ptr(gate), _ptr(beta), _ptr(alpha),
                         _ptr(ws), ws.size, None)
    assert st == bd.VDN_OK, L.vdn_vda_status_string(st)
    return gate, beta, alpha


def run_out_proj(L, p: dict, w: synth.Workload, mode: str):
    """vdn_vda_out_proj with y_in ("y_in"), over y_in ("in_place") or without it ("no_y_in")."""
    desc = bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, 0, w.chunk, "bf16", False)
    o, wo = _c(p["o"]), _c(p["w_o"])
    dm = wo.shape[0]
    yin = np.array(p["y_in"], copy=True)
    out = yin if mode == "in_place" else np.zeros((w.B, w.T, w.U, dm), np.uint16)
    st = L.vdn_vda_out_proj(ctypes.byref(desc), dm, _ptr(o), _ptr(wo), None if mode == "no_y_in" else _ptr(yin),
                            _ptr(out), None)
    assert st == bd.VDN_OK, L.vdn_vda_status_string(st)
    return out


def run_forward_noalloc(L, x: dict, w: synth.Workload, epilogue=True):
    """vdn_vda_forward_noalloc (the library's own workspace array); returns out."""
    desc = bd.make_desc(w.B, w.H, w.T, w.grid_h, w.grid_w, w.d, w.L, w.chunk, w.dtype, epilogue)
    a = {k: _c(x[k]) for k in ("q", "k", "v", "alpha", "beta", "gate")}
    for k in ("k_text", "v_text", "beta_text"):
        a[k] = _c(x[k]) if w.L else None
    out = np.zeros_like(a["q"])
    st = L.vdn_vda_forward_noalloc(ctypes.byref(desc), _ptr(a["q"]), _ptr(a["k"]), _ptr(a["v"]), _ptr(a["alpha"]),
                                   _ptr(a["beta"]), _ptr(a["k_text"]), _ptr(a["v_text"]), _ptr(a["beta_text"]),
                                   _ptr(a["gate"]) if epilogue else None, None, _ptr(out), None)
    assert st == bd.VDN_OK, L.vdn_vda_status_string(st)
    return out
