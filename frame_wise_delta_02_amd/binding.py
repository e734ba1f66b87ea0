"""ctypes binding of the VDA C ABI (include/vdn_vda.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the HIP kernels of
libvdn_vda.so.  A missing library is an error: there is no fallback.  Since the
library sizes every buffer from the descriptor, each wrapper first checks that
every tensor holds exactly the elements and element type the descriptor
implies, on the caller's device and contiguous, and that the grid tiles the
frame's tokens.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvdn_vda.so")

VDN_OK, VDN_ERR_INVALID_ARG, VDN_ERR_UNSUPPORTED, VDN_ERR_WORKSPACE, VDN_ERR_ALIGNMENT, VDN_ERR_HIP = range(6)
VDN_F32, VDN_BF16 = 0, 1
VDN_VDA_EPILOGUE = 1 << 0
VDN_VDA_DEBUG_KEEP = 1 << 1
VDN_VDA_DECAY_BRIDGE = 1 << 2
VDN_VDA_QUERY_L2 = 1 << 3
VDN_VDA_SCAN_FRAMES = 1 << 4
VDN_VDA_SCAN_CHUNKS = 1 << 5
_SCAN_FLAGS = {None: 0, "frames": VDN_VDA_SCAN_FRAMES, "chunks": VDN_VDA_SCAN_CHUNKS}

EXPORTS = ("vdn_vda_validate", "vdn_vda_workspace_bytes", "vdn_vda_workspace_layout",
           "vdn_vda_prepare", "vdn_vda_forward", "vdn_vda_forward_timed", "vdn_vda_forward_noalloc",
           "vdn_vda_status_string", "vdn_vda_backward_workspace_bytes",
           "vdn_vda_backward_workspace_layout", "vdn_vda_backward_readout", "vdn_vda_backward_scan",
           "vdn_vda_backward_gram", "vdn_vda_gates_workspace_bytes", "vdn_vda_gates", "vdn_vda_out_proj")
STAGES = ("gram", "solve", "scan", "gather", "readout")


class VdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("n_text", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("dtype", ctypes.c_int), ("flags", ctypes.c_uint32),
                ("l2_eps", ctypes.c_float), ("rms_eps", ctypes.c_float)]


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("stats", "pinv", "s_text", "fwd", "rev", "readout_states", "chunk_m", "chunk_j", "total")]


class BackwardLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("readout_states_t", "d_out", "d_state_q", "d_record_f", "d_record_r",
                                               "d_text_q", "lam_f", "lam_r", "d_a", "d_b", "total")]


_lib = None


def declare(L: ctypes.CDLL) -> ctypes.CDLL:
    """Set the argument and result types of every exported function on a
    loaded library with this C ABI; returns it."""
    p, sz = ctypes.c_void_p, ctypes.c_size_t
    dp = ctypes.POINTER(Desc)
    L.vdn_vda_validate.argtypes = [dp]
    L.vdn_vda_validate.restype = ctypes.c_int
    L.vdn_vda_workspace_bytes.argtypes = [dp]
    L.vdn_vda_workspace_bytes.restype = sz
    L.vdn_vda_workspace_layout.argtypes = [dp, ctypes.POINTER(Layout)]
    L.vdn_vda_workspace_layout.restype = ctypes.c_int
    L.vdn_vda_prepare.argtypes = [dp] + [p] * 11
    L.vdn_vda_prepare.restype = ctypes.c_int
    L.vdn_vda_forward.argtypes = [dp] + [p] * 12 + [sz, p]
    L.vdn_vda_forward.restype = ctypes.c_int
    L.vdn_vda_forward_timed.argtypes = [dp] + [p] * 12 + [sz, p, p, ctypes.c_int32]
    L.vdn_vda_forward_timed.restype = ctypes.c_int
    L.vdn_vda_forward_noalloc.argtypes = [dp] + [p] * 12
    L.vdn_vda_forward_noalloc.restype = ctypes.c_int
    L.vdn_vda_status_string.argtypes = [ctypes.c_int]
    L.vdn_vda_status_string.restype = ctypes.c_char_p
    L.vdn_vda_backward_workspace_bytes.argtypes = [dp]
    L.vdn_vda_backward_workspace_bytes.restype = sz
    L.vdn_vda_backward_workspace_layout.argtypes = [dp, ctypes.POINTER(BackwardLayout)]
    L.vdn_vda_backward_workspace_layout.restype = ctypes.c_int
    L.vdn_vda_backward_readout.argtypes = [dp] + [p] * 6 + [sz] + [p] * 4 + [sz, p]
    L.vdn_vda_backward_readout.restype = ctypes.c_int
    L.vdn_vda_backward_scan.argtypes = [dp, p, p, sz, p, p, sz, p]
    L.vdn_vda_backward_scan.restype = ctypes.c_int
    L.vdn_vda_backward_gram.argtypes = [dp] + [p] * 13 + [sz, p]
    L.vdn_vda_backward_gram.restype = ctypes.c_int
    L.vdn_vda_gates_workspace_bytes.argtypes = [dp, ctypes.c_int32]
    L.vdn_vda_gates_workspace_bytes.restype = sz
    L.vdn_vda_gates.argtypes = [dp, ctypes.c_int32] + [p] * 7 + [sz, p]
    L.vdn_vda_gates.restype = ctypes.c_int
    L.vdn_vda_out_proj.argtypes = [dp, ctypes.c_int32] + [p] * 5
    L.vdn_vda_out_proj.restype = ctypes.c_int
    return L


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m frame_wise_delta_02_amd.build`")
        _lib = declare(ctypes.CDLL(LIB_PATH))
    return _lib


def status_string(status: int) -> str:
    return lib().vdn_vda_status_string(status).decode()


def make_desc(B, H, T, grid_h, grid_w, d, n_text, chunk=5, dtype="bf16", epilogue=True,
              l2_eps=1e-6, rms_eps=1e-6, flags=None) -> Desc:
    f = (VDN_VDA_EPILOGUE if epilogue else 0) if flags is None else flags
    dt = {"bf16": VDN_BF16, "f32": VDN_F32}.get(dtype, dtype)
    return Desc(B, H, T, grid_h, grid_w, d, d, n_text, chunk, dt, f, l2_eps, rms_eps)


def validate(desc: Desc) -> int:
    return lib().vdn_vda_validate(ctypes.byref(desc))


def workspace_bytes(desc: Desc) -> int:
    return lib().vdn_vda_workspace_bytes(ctypes.byref(desc))


def workspace_layout(desc: Desc) -> Layout:
    out = Layout()
    st = lib().vdn_vda_workspace_layout(ctypes.byref(desc), ctypes.byref(out))
    if st != VDN_OK:
        raise VdaError(st, "vdn_vda_workspace_layout")
    return out


# ----------------------------------------------------------------------------
# torch marshalling
# ----------------------------------------------------------------------------


def _ptr(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_of(x) -> str:
    import torch
    if x.dtype == torch.bfloat16:
        return "bf16"
    if x.dtype == torch.float32:
        return "f32"
    raise TypeError(f"unsupported dtype {x.dtype}")


def _check(x, name, dev):
    if x is None:
        return
    if not x.is_cuda or x.device != dev:
        raise ValueError(f"{name} must be on {dev}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# The library addresses every tensor from the descriptor alone, so each one must
# hold exactly the elements and the element type the descriptor implies: a
# smaller tensor would be read or written past its end.
def _expect(x, name, numel, dtype):
    if x is None:
        return
    if x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {x.dtype}")
    if x.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, not {x.numel()} (shape {tuple(x.shape)})")


def _expect_grid(grid, U):
    if len(grid) != 2 or grid[0] < 1 or grid[1] < 1 or grid[0] * grid[1] != U:
        raise ValueError(f"grid {tuple(grid)} does not tile the {U} tokens of a frame")


def _expect_bytes(x, name):
    import torch
    if x is not None and x.dtype != torch.uint8:
        raise TypeError(f"{name} must be a uint8 tensor (its element count is passed as its size in bytes)")


def _expect_forward(q, k, v, alpha, beta, k_text, v_text, beta_text, gate, rms_weight, out, grid, epilogue):
    """Shapes and types of the forward pass's tensors, those of [B, T, U, H, d]
    taken from q; returns the text length."""
    import torch
    B, T, U, H, d = q.shape
    _dtype_of(q)
    _expect_grid(grid, U)
    L = 0 if k_text is None else k_text.shape[1]
    for name, x in (("k", k), ("v", v), ("gate", gate if epilogue else None), ("out", out)):
        _expect(x, name, q.numel(), q.dtype)
    if k is None or v is None or alpha is None or beta is None:
        raise ValueError("k, v, alpha and beta are required")
    _expect(alpha, "alpha", B * T * H * d, torch.float32)
    _expect(beta, "beta", B * T * U * H, q.dtype)
    if L:
        _expect(k_text, "k_text", B * L * H * d, q.dtype)
        _expect(v_text, "v_text", B * L * H * d, q.dtype)
        _expect(beta_text, "beta_text", B * L * H, q.dtype)
        if v_text is None or beta_text is None:
            raise ValueError("v_text and beta_text are required with k_text")
    _expect(rms_weight, "rms_weight", d, torch.float32)
    return L


def forward(q, k, v, alpha, beta, k_text, v_text, beta_text, gate=None, rms_weight=None, *,
            grid, chunk=5, epilogue=True, rms_eps=1e-6, out=None, workspace=None, bridge=False,
            query_l2=False, l2_eps=1e-6, scan=None, events=None):
    """VDA forward on prepared features; returns ``out`` [B, T, U, H, d].

    Shapes as in include/vdn_vda.h.  ``grid`` = (grid_h, grid_w) with
    grid_h * grid_w = U.  ``workspace`` (uint8, on the device) is allocated
    when not given.  ``bridge`` sets VDN_VDA_DECAY_BRIDGE; ``query_l2`` sets
    VDN_VDA_QUERY_L2 (``q`` is then the raw query, normalised with ``l2_eps``);
    ``scan`` = "frames" or "chunks" forces that scan (None: the library picks).
    ``events``: hipEvent_t handles (ints), one before and one after each of the
    ``STAGES``, recorded on the stream by vdn_vda_forward_timed.
    """
    import torch
    B, T, U, H, d = q.shape
    L = _expect_forward(q, k, v, alpha, beta, k_text, v_text, beta_text, gate, rms_weight, out, grid, epilogue)
    _expect_bytes(workspace, "workspace")
    dt = _dtype_of(q)
    dev = q.device
    for name, x in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta),
                    ("k_text", k_text), ("v_text", v_text), ("beta_text", beta_text),
                    ("gate", gate), ("rms_weight", rms_weight), ("out", out), ("workspace", workspace)):
        _check(x, name, dev)
    desc = make_desc(B, H, T, grid[0], grid[1], d, L, chunk, dt, epilogue, l2_eps=l2_eps, rms_eps=rms_eps,
                     flags=(VDN_VDA_EPILOGUE if epilogue else 0) | (VDN_VDA_DECAY_BRIDGE if bridge else 0)
                     | (VDN_VDA_QUERY_L2 if query_l2 else 0) | _SCAN_FLAGS[scan])
    st = validate(desc)
    if st != VDN_OK:
        raise VdaError(st, "vdn_vda_validate")
    if out is None:
        out = torch.empty((B, T, U, H, d), dtype=q.dtype, device=dev)
    need = workspace_bytes(desc)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
            _ptr(k_text), _ptr(v_text), _ptr(beta_text),
            _ptr(gate) if epilogue else None, _ptr(rms_weight), _ptr(out),
            _ptr(workspace), workspace.numel(), _stream())
    if events is None:
        st = lib().vdn_vda_forward(*args)
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        st = lib().vdn_vda_forward_timed(*args, ctypes.cast(arr, ctypes.c_void_p), len(events))
    if st != VDN_OK:
        raise VdaError(st, "vdn_vda_forward")
    return out


def forward_noalloc(q, k, v, alpha, beta, k_text, v_text, beta_text, gate=None, rms_weight=None, *,
                    grid, chunk=5, epilogue=True, rms_eps=1e-6, out=None, bridge=False, query_l2=False,
                    l2_eps=1e-6, scan=None):
    """vdn_vda_forward_noalloc: the forward pass with the library's own device
    array as its workspace (no workspace argument); returns ``out``."""
    import torch
    B, T, U, H, d = q.shape
    L = _expect_forward(q, k, v, alpha, beta, k_text, v_text, beta_text, gate, rms_weight, out, grid, epilogue)
    dev = q.device
    for name, x in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta),
                    ("k_text", k_text), ("v_text", v_text), ("beta_text", beta_text),
                    ("gate", gate), ("rms_weight", rms_weight), ("out", out)):
        _check(x, name, dev)
    desc = make_desc(B, H, T, grid[0], grid[1], d, L, chunk, _dtype_of(q), epilogue, l2_eps=l2_eps,
                     rms_eps=rms_eps,
                     flags=(VDN_VDA_EPILOGUE if epilogue else 0) | (VDN_VDA_DECAY_BRIDGE if bridge else 0)
                     | (VDN_VDA_QUERY_L2 if query_l2 else 0) | _SCAN_FLAGS[scan])
    if out is None:
        out = torch.empty((B, T, U, H, d), dtype=q.dtype, device=dev)
    st = lib().vdn_vda_forward_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                       _ptr(k_text), _ptr(v_text), _ptr(beta_text),
                                       _ptr(gate) if epilogue else None, _ptr(rms_weight), _ptr(out), _stream())
    if st != VDN_OK:
        raise VdaError(st, "vdn_vda_forward_noalloc")
    return out


def prepare(q, k, v, wk_s, wk_t, wv_s, wv_t, *, grid, l2_eps=1e-6, n_text=0, chunk=5, query_l2=False):
    """Feature prep (conv, SiLU, L2); returns (q_hat, k_hat, v_hat).

    With ``query_l2`` (VDN_VDA_QUERY_L2) the query is left to the forward pass:
    ``q`` may be None and q_hat is returned as None.
    """
    import torch
    B, T, U, H, d = k.shape
    _dtype_of(k)
    _expect_grid(grid, U)
    _expect(v, "v", k.numel(), k.dtype)
    if query_l2:
        q = None
    elif q is None:
        raise ValueError("q is required unless query_l2 is set")
    _expect(q, "q", k.numel(), k.dtype)
    for name, x, taps in (("wk_s", wk_s, 25), ("wk_t", wk_t, 5), ("wv_s", wv_s, 25), ("wv_t", wv_t, 5)):
        if x is None:
            raise ValueError(f"{name} is required")
        _expect(x, name, H * d * taps, torch.float32)
    dev = k.device
    for name, x in (("q", q), ("k", k), ("v", v), ("wk_s", wk_s), ("wk_t", wk_t),
                    ("wv_s", wv_s), ("wv_t", wv_t)):
        _check(x, name, dev)
    desc = make_desc(B, H, T, grid[0], grid[1], d, n_text, chunk, _dtype_of(k), False, l2_eps=l2_eps,
                     flags=VDN_VDA_QUERY_L2 if query_l2 else 0)
    q_hat = None if query_l2 else torch.empty_like(q)
    k_hat, v_hat = torch.empty_like(k), torch.empty_like(v)
    st = lib().vdn_vda_prepare(ctypes.byref(desc), None if query_l2 else _ptr(q), _ptr(k), _ptr(v),
                               _ptr(wk_s), _ptr(wk_t), _ptr(wv_s), _ptr(wv_t),
                               None if query_l2 else _ptr(q_hat), _ptr(k_hat), _ptr(v_hat), _stream())
    if st != VDN_OK:
        raise VdaError(st, "vdn_vda_prepare")
    return q_hat, k_hat, v_hat


def backward_workspace_bytes(desc: Desc) -> int:
    return lib().vdn_vda_backward_workspace_bytes(ctypes.byref(desc))


def backward_layout(desc: Desc) -> BackwardLayout:
    out = BackwardLayout()
    st = lib().vdn_vda_backward_workspace_layout(ctypes.byref(desc), ctypes.byref(out))
    if st != VDN_OK:
        raise VdaError(st, "vdn_vda_backward_workspace_layout")
    return out


def backward_readout(q, gate, rms_weight, alpha, dy, fwd_workspace, *, grid, n_text=0, chunk=5, epilogue=True,
                     bridge=False, rms_eps=1e-6, dq=None, dgate=None, workspace=None, query_l2=False, l2_eps=1e-6,
                     d_rms_weight=None):
    """First stage of the backward pass (vdn_vda_backward_readout): returns
    (dq, dgate or None, workspace); the workspace holds do and dS_q at the
    offsets of ``backward_layout``.  ``fwd_workspace`` is the forward's, for the
    same descriptor and inputs.  A float32 tensor of d elements given as
    ``d_rms_weight`` (with the epilogue) receives the RMSNorm gain's gradient."""
    import torch
    B, T, U, H, d = q.shape
    _dtype_of(q)
    _expect_grid(grid, U)
    for name, x in (("gate", gate if epilogue else None), ("dy", dy), ("dq", dq),
                    ("dgate", dgate if epilogue else None)):
        _expect(x, name, q.numel(), q.dtype)
    _expect(alpha, "alpha", B * T * H * d, torch.float32)
    _expect(rms_weight, "rms_weight", d, torch.float32)
    _expect(d_rms_weight, "d_rms_weight", d, torch.float32)
    if d_rms_weight is not None and not epilogue:
        raise ValueError("d_rms_weight needs the epilogue")
    _expect_bytes(fwd_workspace, "fwd_workspace")
    _expect_bytes(workspace, "workspace")
    dev = q.device
    for name, x in (("q", q), ("gate", gate), ("rms_weight", rms_weight), ("alpha", alpha), ("dy", dy),
                    ("fwd_workspace", fwd_workspace), ("dq", dq), ("dgate", dgate), ("workspace", workspace),
                    ("d_rms_weight", d_rms_weight)):
        _check(x, name, dev)
    desc = make_desc(B, H, T, grid[0], grid[1], d, n_text, chunk, _dtype_of(q), epilogue, rms_eps=rms_eps,
                     l2_eps=l2_eps, flags=(VDN_VDA_EPILOGUE if epilogue else 0) | (VDN_VDA_DECAY_BRIDGE if bridge else 0)
                     | (VDN_VDA_QUERY_L2 if query_l2 else 0))
    if dq is None:
        dq = torch.empty_like(q)
    if epilogue and dgate is None:
        dgate = torch.empty_like(dy)
    if workspace is None:
        workspace = torch.empty(backward_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    st = lib().vdn_vda_backward_readout(ctypes.byref(desc), _ptr(q), _ptr(gate) if epilogue else None,
                                        _ptr(rms_weight), _ptr(alpha), _ptr(dy), _ptr(fwd_workspace),
                                        fwd_workspace.numel(), _ptr(dq), _ptr(dgate) if epilogue else None,
                                        _ptr(d_rms_weight), _ptr(workspace), workspace.numel(), _stream())
    if st != VDN_OK:
        raise VdaError(st, "vdn_vda_backward_readout")
    return dq, (dgate if epilogue else None), workspace


def backward_scan(alpha, fwd_workspace, workspace, *, shape, grid, n_text=0, chunk=5, dtype="bf16", epilogue=True,
                  dalpha=None, bridge=False):
    """Second stage of the backward pass (vdn_vda_backward_scan) on the first
    stage's workspace; returns dalpha [B, T, H, d] float32.  ``shape`` = (B, T, H, d)."""
    import torch
    B, T, H, d = shape
    _expect(alpha, "alpha", B * T * H * d, torch.float32)
    _expect(dalpha, "dalpha", B * T * H * d, torch.float32)
    _expect_bytes(fwd_workspace, "fwd_workspace")
    _expect_bytes(workspace, "workspace")
    dev = alpha.device
    for name, x in (("alpha", alpha), ("fwd_workspace", fwd_workspace), ("workspace", workspace), ("dalpha", dalpha)):
        _check(x, name, dev)
    desc = make_desc(B, H, T, grid[0], grid[1], d, n_text, chunk, dtype, epilogue,
                     flags=(VDN_VDA_EPILOGUE if epilogue else 0) | (VDN_VDA_DECAY_BRIDGE if bridge else 0))
    if dalpha is None:
        dalpha = torch.empty((B, T, H, d), dtype=torch.float32, device=dev)
    st = lib().vdn_vda_backward_scan(ctypes.byref(desc), _ptr(alpha), _ptr(fwd_workspace), fwd_workspace.numel(),
                                     _ptr(dalpha), _ptr(workspace), workspace.numel(), _stream())
    if st != VDN_OK:
        raise VdaError(st, "vdn_vda_backward_scan")
    return dalpha


def backward_gram(k, v, beta, k_text, v_text, beta_text, workspace, *, grid, chunk=5, epilogue=True, out=None):
    """Third stage of the backward pass (vdn_vda_backward_gram) on the second
    stage's workspace; returns (dk, dv, dbeta, dk_text, dv_text, dbeta_text),
    the text ones None without text tokens.  ``out`` may give the six output
    tensors."""
    import torch
    B, T, U, H, d = k.shape
    L = 0 if k_text is None else k_text.shape[1]
    _dtype_of(k)
    _expect_grid(grid, U)
    _expect(v, "v", k.numel(), k.dtype)
    _expect(beta, "beta", B * T * U * H, k.dtype)
    if L:
        _expect(k_text, "k_text", B * L * H * d, k.dtype)
        _expect(v_text, "v_text", B * L * H * d, k.dtype)
        _expect(beta_text, "beta_text", B * L * H, k.dtype)
    _expect_bytes(workspace, "workspace")
    if out is not None:
        if len(out) != 6:
            raise ValueError("out must give (dk, dv, dbeta, dk_text, dv_text, dbeta_text)")
        for name, x, n in (("dk", out[0], k.numel()), ("dv", out[1], k.numel()), ("dbeta", out[2], B * T * U * H)):
            if x is None:
                raise ValueError(f"{name} is required")
            _expect(x, name, n, k.dtype)
        if L:
            for name, x, n in (("dk_text", out[3], B * L * H * d), ("dv_text", out[4], B * L * H * d),
                               ("dbeta_text", out[5], B * L * H)):
                if x is None:
                    raise ValueError(f"{name} is required with text tokens")
                _expect(x, name, n, k.dtype)
    dev = k.device
    if out is None:
        out = (torch.empty_like(k), torch.empty_like(v), torch.empty_like(beta),
               None if L == 0 else torch.empty_like(k_text), None if L == 0 else torch.empty_like(v_text),
               None if L == 0 else torch.empty_like(beta_text))
    for name, x in (("k", k), ("v", v), ("beta", beta), ("k_text", k_text), ("v_text", v_text),
                    ("beta_text", beta_text), ("workspace", workspace)) + tuple(zip(
                        ("dk", "dv", "dbeta", "dk_text", "dv_text", "dbeta_text"), out)):
        _check(x, name, dev)
    desc = make_desc(B, H, T, grid[0], grid[1], d, L, chunk, _dtype_of(k), epilogue)
    text = [x if L else None for x in (k_text, v_text, beta_text)]
    st = lib().vdn_vda_backward_gram(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(beta), *map(_ptr, text),
                                     *(_ptr(x if (L or i < 3) else None) for i, x in enumerate(out)),
                                     _ptr(workspace), workspace.numel(), _stream())
    if st != VDN_OK:
        raise VdaError(st, "vdn_vda_backward_gram")
    return tuple(out[:3]) + (tuple(out[3:]) if L else (None, None, None))


def backward(q, k, v, alpha, beta, k_text, v_text, beta_text, gate, rms_weight, dy, fwd_workspace, *, grid,
             chunk=5, epilogue=True, rms_eps=1e-6, workspace=None, query_l2=False, l2_eps=1e-6, bridge=False,
             gain_grad=False):
    """The whole backward pass (the three stages in order) after a forward
    that left ``fwd_workspace`` (with ``query_l2`` the forward took the raw
    query and dq is its gradient); returns a dict of input gradients dq, dk, dv,
    dalpha, dbeta, dk_text, dv_text, dbeta_text, dgate (the last four None
    where absent), with ``gain_grad`` (and the epilogue) drms_weight, the
    RMSNorm gain's gradient [d] float32, and the workspace."""
    import torch
    B, T, U, H, d = q.shape
    L = 0 if k_text is None else k_text.shape[1]
    drms = torch.empty(d, dtype=torch.float32, device=q.device) if gain_grad else None
    dq, dgate, workspace = backward_readout(q, gate, rms_weight, alpha, dy, fwd_workspace, grid=grid, n_text=L,
                                            chunk=chunk, epilogue=epilogue, rms_eps=rms_eps, workspace=workspace,
                                            query_l2=query_l2, l2_eps=l2_eps, bridge=bridge, d_rms_weight=drms)
    dalpha = backward_scan(alpha, fwd_workspace, workspace, shape=(B, T, H, d), grid=grid, n_text=L,
                           chunk=chunk, dtype=_dtype_of(q), epilogue=epilogue, bridge=bridge)
    dk, dv, dbeta, dkt, dvt, dbt = backward_gram(k, v, beta, k_text, v_text, beta_text, workspace, grid=grid,
                                                 chunk=chunk, epilogue=epilogue)
    return dict(dq=dq, dk=dk, dv=dv, dalpha=dalpha, dbeta=dbeta, dk_text=dkt, dv_text=dvt, dbeta_text=dbt,
                dgate=dgate, drms_weight=drms, workspace=workspace)


def gates(x, w_gb, w_alpha, *, heads, d, grid, chunk=5, out=None, workspace=None):
    """Gate logits, write gate and decay gate from the block input x
    [B, T, U, d_model] (vdn_vda_gates): w_gb [heads * d + heads, d_model]
    bfloat16 (the gate rows, then the beta rows), w_alpha [heads * d, d_model]
    float32.  Returns (gate [B, T, U, H, d], beta [B, T, U, H], alpha [B, T, H, d])."""
    import torch
    B, T, U, Dm = x.shape
    _expect(x, "x", x.numel(), torch.bfloat16)
    _expect_grid(grid, U)
    _expect(w_gb, "w_gb", (heads * d + heads) * Dm, torch.bfloat16)
    _expect(w_alpha, "w_alpha", heads * d * Dm, torch.float32)
    if out is not None:
        for name, t, n, dt in (("gate", out[0], B * T * U * heads * d, torch.bfloat16),
                               ("beta", out[1], B * T * U * heads, torch.bfloat16),
                               ("alpha", out[2], B * T * heads * d, torch.float32)):
            _expect(t, name, n, dt)
    _expect_bytes(workspace, "workspace")
    dev = x.device
    desc = make_desc(B, heads, T, grid[0], grid[1], d, 0, chunk, "bf16", False)
    if out is None:
        out = (torch.empty((B, T, U, heads, d), dtype=torch.bfloat16, device=dev),
               torch.empty((B, T, U, heads), dtype=torch.bfloat16, device=dev),
               torch.empty((B, T, heads, d), dtype=torch.float32, device=dev))
    if workspace is None:
        workspace = torch.empty(max(1, lib().vdn_vda_gates_workspace_bytes(ctypes.byref(desc), Dm)), dtype=torch.uint8,
                                device=dev)
    for name, t in (("x", x), ("w_gb", w_gb), ("w_alpha", w_alpha), ("gate", out[0]), ("beta", out[1]),
                    ("alpha", out[2]), ("workspace", workspace)):
        _check(t, name, dev)
    st = lib().vdn_vda_gates(ctypes.byref(desc), Dm, _ptr(x), _ptr(w_gb), _ptr(w_alpha), *map(_ptr, out),
                             _ptr(workspace), workspace.numel(), _stream())
    if st != VDN_OK:
        raise VdaError(st, "vdn_vda_gates")
    return out


def out_proj(o, w_o, y_in=None, *, grid, chunk=5, out=None):
    """Y = y_in + o W_O^T (vdn_vda_out_proj): o [B, T, U, H, d], w_o [d_model, H * d]
    and y_in [B, T, U, d_model] bfloat16; ``out`` may be y_in itself."""
    import torch
    B, T, U, H, d = o.shape
    Dm = w_o.shape[0]
    _expect(o, "o", o.numel(), torch.bfloat16)
    _expect_grid(grid, U)
    _expect(w_o, "w_o", Dm * H * d, torch.bfloat16)
    _expect(y_in, "y_in", B * T * U * Dm, torch.bfloat16)
    _expect(out, "out", B * T * U * Dm, torch.bfloat16)
    dev = o.device
    desc = make_desc(B, H, T, grid[0], grid[1], d, 0, chunk, "bf16", False)
    if out is None:
        out = torch.empty((B, T, U, Dm), dtype=torch.bfloat16, device=dev)
    for name, t in (("o", o), ("w_o", w_o), ("y_in", y_in), ("out", out)):
        _check(t, name, dev)
    st = lib().vdn_vda_out_proj(ctypes.byref(desc), Dm, _ptr(o), _ptr(w_o), _ptr(y_in), _ptr(out), _stream())
    if st != VDN_OK:
        raise VdaError(st, "vdn_vda_out_proj")
    return out

