"""The C ABI without a GPU: exports, descriptor validation, workspace layout and
argument errors that are caught before anything is enqueued."""

import ctypes
import os
import re

import numpy as np
import pytest

from frame_wise_delta_02_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:vdn_status|size_t|const char\*)\s+(vdn_\w+)\s*\(", txt, re.M))
    return names


def test_library_exports_every_declared_symbol():
    lib = bd.lib()
    declared = _declared()
    assert {"vdn_vda_prepare", "vdn_vda_forward", "vdn_vda_validate",
            "vdn_vda_workspace_bytes", "vdn_vda_status_string"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(bd.EXPORTS) <= declared


def good(**kw):
    base = dict(B=1, H=24, T=60, grid_h=48, grid_w=84, d=128, n_text=256, chunk=5, dtype="bf16")
    base.update(kw)
    return bd.make_desc(**base)


def test_valid_descriptors():
    for d in (16, 32, 64, 128):
        assert bd.validate(good(d=d)) == bd.VDN_OK
    assert bd.validate(good(T=1)) == bd.VDN_OK
    assert bd.validate(good(n_text=0)) == bd.VDN_OK
    assert bd.validate(good(dtype="f32", chunk=1)) == bd.VDN_OK


@pytest.mark.parametrize("field,value", [
    ("B", 0), ("H", 0), ("T", 0), ("grid_h", 0), ("grid_w", -1), ("n_text", -1), ("chunk", 0),
    ("d_k", 0), ("d_k", 144), ("d_k", 24), ("dtype", 7), ("flags", 1 << 6),
    ("flags", (1 << 4) | (1 << 5))])
def test_invalid_descriptors(field, value):
    desc = good()
    setattr(desc, field, value)
    if field == "d_k":
        desc.d_v = value
    assert bd.validate(desc) == bd.VDN_ERR_INVALID_ARG
    assert bd.workspace_bytes(desc) == 0


def test_bad_eps_and_unsupported_widths():
    d = good()
    d.rms_eps = 0.0
    assert bd.validate(d) == bd.VDN_ERR_INVALID_ARG
    d = good()
    d.l2_eps = float("nan")
    assert bd.validate(d) == bd.VDN_ERR_INVALID_ARG
    d = good()
    d.d_v = 64
    assert bd.validate(d) == bd.VDN_ERR_UNSUPPORTED
    assert bd.lib().vdn_vda_validate(None) == bd.VDN_ERR_INVALID_ARG


def test_widths_between_the_built_ones():
    """d = 48, 80, 96, 112: the forward and backward passes run them
    (zero-padded to the next built width, the padded copies in their
    workspaces), the prep and the adjacent maps at the width itself."""
    lib = bd.lib()
    for w, D in ((48, 64), (80, 128), (96, 128), (112, 128)):
        d = good(d=w)
        assert bd.validate(d) == bd.VDN_OK
        # the workspace holds the built width's sections plus the padded copies
        L = bd.workspace_layout(d)
        built = bd.workspace_layout(good(d=D))
        assert L.readout_states == built.readout_states and L.chunk_j == built.chunk_j
        x = 60 * 4032 * 24 * D * 2
        assert L.total >= built.total + 5 * x
        # the backward workspace: the built width's sections plus padded dy, dq,
        # dgate, dalpha, k, v, dk, dv and the text's
        bw, bw_built = bd.backward_workspace_bytes(d), bd.backward_workspace_bytes(good(d=D))
        assert bw >= bw_built + 7 * x
        assert bd.backward_layout(d).d_out == bd.backward_layout(good(d=D)).d_out
        # the adjacent maps run at the caller's width (their workspace: the frames' token sums)
        assert lib.vdn_vda_gates_workspace_bytes(ctypes.byref(d), 3072) == \
            lib.vdn_vda_gates_workspace_bytes(ctypes.byref(good()), 3072)
        P = [ctypes.c_void_p(A16 + (1 << 34) * i) for i in range(10)]
        # the prep runs at the width itself (its arguments pass; no GPU here)
        assert lib.vdn_vda_prepare(ctypes.byref(d), *P, None) == bd.VDN_ERR_HIP
        # the backward's argument checks pass (no GPU here: the launch fails)
        fw = bd.workspace_bytes(d)
        assert lib.vdn_vda_backward_readout(ctypes.byref(d), *P[:6], fw, P[6], P[7], None, P[8], bw,
                                            None) == bd.VDN_ERR_HIP
    # d = 144 and widths that are not multiples of 16 stay invalid
    assert bd.validate(good(d=144)) == bd.VDN_ERR_INVALID_ARG
    assert bd.validate(good(d=40)) == bd.VDN_ERR_INVALID_ARG
    # the 32-bit offset limits are those of the built width the kernels run at:
    # 16384 heads of d = 112 run at 128, where a 48 x 84 frame's rows pass 4 GiB
    assert bd.validate(good(H=16384, n_text=0, grid_h=1, grid_w=1, d=112)) == bd.VDN_OK
    assert bd.validate(good(H=2048, n_text=0, d=112)) == bd.VDN_ERR_INVALID_ARG


def test_workspace_layout_is_consistent():
    for kw in (dict(), dict(d=64, T=40, H=8), dict(T=1), dict(T=23, chunk=3), dict(dtype="f32", d=16)):
        desc = good(**kw)
        L = bd.workspace_layout(desc)
        B, H, T, d = desc.B, desc.H, desc.T, desc.d_k
        nc = -(-T // desc.chunk)
        f = 4 * d * d
        offs = [L.stats, L.pinv, L.s_text, L.fwd, L.rev, L.readout_states, L.chunk_m, L.chunk_j, L.total]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
        assert L.pinv - L.stats >= B * H * (T + 1) * 2 * f
        assert L.s_text - L.pinv >= B * H * (T + 1) * f
        assert L.fwd - L.s_text >= B * H * f
        assert L.rev - L.fwd >= B * H * nc * f
        assert L.readout_states - L.rev >= B * H * nc * f
        assert L.chunk_j - L.chunk_m >= B * H * 2 * nc * f
        assert L.total - L.chunk_j >= B * H * 2 * nc * f
        assert L.total == bd.workspace_bytes(desc)


def test_status_strings():
    for s in range(6):
        assert bd.status_string(s).startswith("VDN_")
    assert "unknown" in bd.status_string(99)


def _fwd(desc, ptrs, ws_bytes):
    lib = bd.lib()
    P = [ctypes.c_void_p(p) if p else None for p in ptrs]
    return lib.vdn_vda_forward(ctypes.byref(desc), *P, ws_bytes, None)


# fake, never dereferenced device addresses: every call below must fail its
# argument checks before it reaches the GPU
A16 = 0x7f0000000000


def _ptrs(**over):
    names = ["q", "k", "v", "alpha", "beta", "k_text", "v_text", "beta_text", "gate", "rms_weight",
             "out", "ws"]
    p = {n: A16 + 0x1000000 * i for i, n in enumerate(names)}
    p.update(over)
    return [p[n] for n in names]


def test_forward_argument_errors_before_launch():
    desc = good()
    need = bd.workspace_bytes(desc)
    assert _fwd(desc, _ptrs(q=0), need) == bd.VDN_ERR_INVALID_ARG
    assert _fwd(desc, _ptrs(out=0), need) == bd.VDN_ERR_INVALID_ARG
    assert _fwd(desc, _ptrs(k_text=0), need) == bd.VDN_ERR_INVALID_ARG
    assert _fwd(desc, _ptrs(gate=0), need) == bd.VDN_ERR_INVALID_ARG
    assert _fwd(desc, _ptrs(ws=0), need) == bd.VDN_ERR_WORKSPACE
    assert _fwd(desc, _ptrs(), need - 1) == bd.VDN_ERR_WORKSPACE
    assert _fwd(desc, _ptrs(q=A16 + 8), need) == bd.VDN_ERR_ALIGNMENT
    assert _fwd(desc, _ptrs(ws=A16 + 0x40000000 + 64), need) == bd.VDN_ERR_ALIGNMENT
    assert _fwd(desc, _ptrs(beta=A16 + 1), need) == bd.VDN_ERR_ALIGNMENT
    bad = good()
    bad.d_v = 64
    assert _fwd(bad, _ptrs(), need) == bd.VDN_ERR_UNSUPPORTED


def test_prepare_argument_errors_before_launch():
    lib = bd.lib()
    desc = good(epilogue=False)
    P = [ctypes.c_void_p(A16 + 0x1000000 * i) for i in range(10)]
    args = list(P)
    args[0] = None
    assert lib.vdn_vda_prepare(ctypes.byref(desc), *args, None) == bd.VDN_ERR_INVALID_ARG
    args = list(P)
    args[8] = args[1]  # k_hat aliases k
    assert lib.vdn_vda_prepare(ctypes.byref(desc), *args, None) == bd.VDN_ERR_INVALID_ARG
    args = list(P)
    args[2] = ctypes.c_void_p(A16 + 0x2000000 + 4)
    assert lib.vdn_vda_prepare(ctypes.byref(desc), *args, None) == bd.VDN_ERR_ALIGNMENT


@pytest.mark.parametrize("D", [32, 64, 128])
def test_split_pinv_decoder_round_trip(D):
    """The test-side decoder of the bfloat16 hi/lo inverse planes inverts an
    encoder written from the layout's definition in include/vdn_vda.h."""
    import gpu_harness as G
    rng = np.random.default_rng(D)
    P = rng.standard_normal((2, D, D)).astype(np.float32)

    def bf16_bits(x):  # round to nearest even, as the kernels convert
        u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)

    hi = bf16_bits(P)
    hi_f = (hi.astype(np.uint32) << 16).view(np.float32)
    lo = bf16_bits(P - hi_f)
    raw = np.zeros((2, 2, D * D), np.uint16)
    for n in range(2):
        for w in range(D // 32):
            for e in range(2):
                for s in range(D // 32):
                    for lane in range(64):
                        f = ((2 * w + e) * (D // 32) + s) * 64 + lane
                        for j in range(8):
                            r, c = 32 * s + 8 * (lane // 16) + j, 32 * w + 2 * (lane % 16) + e
                            raw[n, 0, 8 * f + j] = hi[n, r, c]
                            raw[n, 1, 8 * f + j] = lo[n, r, c]
    got = G.decode_split_pinv(raw.view(np.int16), D)
    assert np.abs(got - P).max() <= 2.0 ** -16 * np.abs(P).max()


def test_chunk_record_limit():
    """Each head's chunk records (n_c * d_k * d_v * 4 bytes) must stay below 2^31
    bytes: the scan sends steps that record nothing to offset 2^31 of that buffer."""
    assert bd.validate(good(T=32767, chunk=1, grid_h=1, grid_w=1, H=1)) == bd.VDN_OK
    assert bd.validate(good(T=32768, chunk=1, grid_h=1, grid_w=1, H=1)) == bd.VDN_ERR_INVALID_ARG
    assert bd.validate(good(T=32768, chunk=2, grid_h=1, grid_w=1, H=1)) == bd.VDN_OK
    assert bd.validate(good(T=131072, chunk=4, grid_h=1, grid_w=1, H=1, d=64)) == bd.VDN_OK


def test_query_l2_flag():
    """VDN_VDA_QUERY_L2 is a valid flag; under it vdn_vda_prepare neither requires
    nor checks q and q_hat, and still checks everything else before a launch."""
    flags = bd.VDN_VDA_EPILOGUE | bd.VDN_VDA_QUERY_L2
    assert bd.validate(good(flags=flags)) == bd.VDN_OK
    assert bd.validate(good(flags=bd.VDN_VDA_QUERY_L2 | bd.VDN_VDA_DECAY_BRIDGE)) == bd.VDN_OK
    lib = bd.lib()
    desc = good(flags=bd.VDN_VDA_QUERY_L2)
    P = [ctypes.c_void_p(A16 + 0x1000000 * i) for i in range(10)]
    args = list(P)
    args[0] = args[7] = None   # q, q_hat absent
    args[1] = None             # k absent
    assert lib.vdn_vda_prepare(ctypes.byref(desc), *args, None) == bd.VDN_ERR_INVALID_ARG
    args = list(P)
    args[0] = ctypes.c_void_p(A16 + 4)  # a misaligned q is ignored ...
    args[8] = args[1]                   # ... so the k_hat alias is what fails
    assert lib.vdn_vda_prepare(ctypes.byref(desc), *args, None) == bd.VDN_ERR_INVALID_ARG
    args = list(P)
    args[0] = args[7] = None
    args[9] = ctypes.c_void_p(A16 + 0x9000000 + 2)  # v_hat misaligned
    assert lib.vdn_vda_prepare(ctypes.byref(desc), *args, None) == bd.VDN_ERR_ALIGNMENT
    # without the flag a missing q is an error
    args = list(P)
    args[0] = None
    assert lib.vdn_vda_prepare(ctypes.byref(good(epilogue=False)), *args, None) == bd.VDN_ERR_INVALID_ARG


def test_scan_flags():
    """Either scan may be forced; both at once is an error."""
    assert bd.validate(good(flags=bd.VDN_VDA_EPILOGUE | bd.VDN_VDA_SCAN_FRAMES)) == bd.VDN_OK
    assert bd.validate(good(flags=bd.VDN_VDA_EPILOGUE | bd.VDN_VDA_SCAN_CHUNKS)) == bd.VDN_OK
    assert bd.validate(good(flags=bd.VDN_VDA_SCAN_FRAMES | bd.VDN_VDA_SCAN_CHUNKS)) == bd.VDN_ERR_INVALID_ARG
    # the scan flags change nothing in the workspace
    a, b = good(flags=bd.VDN_VDA_SCAN_CHUNKS), good(flags=bd.VDN_VDA_SCAN_FRAMES)
    assert bd.workspace_bytes(a) == bd.workspace_bytes(b) > 0


def test_backward_readout_argument_errors_before_launch():
    lib = bd.lib()
    desc = good()
    fw = bd.workspace_bytes(desc)
    bw = bd.backward_workspace_bytes(desc)
    assert bw == bd.backward_layout(desc).total > 0
    L = bd.backward_layout(desc)
    offs = [L.readout_states_t, L.d_out, L.d_state_q, L.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert L.d_state_q - L.d_out >= desc.B * desc.T * 48 * 84 * desc.H * desc.d_v * 2
    assert L.total - L.d_state_q >= desc.B * desc.H * desc.T * desc.d_v * desc.d_k * 4
    names = ["q", "gate", "rms", "alpha", "dy", "fws", "dq", "dgate", "drms", "ws"]
    base = {n: A16 + 0x1000000 * i for i, n in enumerate(names)}

    def call(d=desc, fwb=fw, bwb=bw, **over):
        p = dict(base, rms=0, drms=0)
        p.update(over)
        P = [ctypes.c_void_p(p[n]) if p[n] else None for n in names]
        return lib.vdn_vda_backward_readout(ctypes.byref(d), P[0], P[1], P[2], P[3], P[4], P[5], fwb,
                                            P[6], P[7], P[8], P[9], bwb, None)

    assert call(q=0) == bd.VDN_ERR_INVALID_ARG
    assert call(dy=0) == bd.VDN_ERR_INVALID_ARG
    assert call(gate=0) == bd.VDN_ERR_INVALID_ARG           # the epilogue needs the gate ...
    assert call(dgate=0) == bd.VDN_ERR_INVALID_ARG          # ... and its adjoint's buffer
    assert call(dq=base["q"]) == bd.VDN_ERR_INVALID_ARG     # aliasing
    assert call(fwb=fw - 1) == bd.VDN_ERR_WORKSPACE
    assert call(bwb=bw - 1) == bd.VDN_ERR_WORKSPACE
    assert call(ws=0) == bd.VDN_ERR_WORKSPACE
    assert call(dy=base["dy"] + 8) == bd.VDN_ERR_ALIGNMENT
    assert call(ws=base["ws"] + 16) == bd.VDN_ERR_ALIGNMENT
    # float32: do is kept in float32, so the workspace sized for bfloat16 is short
    f32 = good(dtype="f32")
    assert bd.backward_workspace_bytes(f32) > bw
    assert call(d=f32, fwb=bd.workspace_bytes(f32)) == bd.VDN_ERR_WORKSPACE
    assert call(d=f32, q=0) == bd.VDN_ERR_INVALID_ARG
    assert call(d=good(flags=bd.VDN_VDA_QUERY_L2)) == bd.VDN_ERR_UNSUPPORTED   # the raw query needs the epilogue
    # the gain's gradient: 4-byte aligned, and only with the epilogue
    assert call(drms=base["drms"] + 2) == bd.VDN_ERR_ALIGNMENT
    # without the epilogue the gate is not needed
    raw = good(epilogue=False)
    assert call(d=raw, gate=0, dgate=0, q=0) == bd.VDN_ERR_INVALID_ARG  # (q still is)
    assert call(d=raw, gate=0, dgate=0, drms=base["drms"]) == bd.VDN_ERR_INVALID_ARG  # no gain without it


def test_backward_gram_argument_errors_before_launch():
    lib = bd.lib()
    desc = good()
    bw = bd.backward_workspace_bytes(desc)
    names = ["k", "v", "beta", "kt", "vt", "bt", "dk", "dv", "dbeta", "dkt", "dvt", "dbt", "ws"]
    # 8 GiB apart: every tensor of the 768p clip fits between two bases
    base = {n: A16 + (1 << 33) * i for i, n in enumerate(names)}

    def call(d=desc, bwb=bw, **over):
        p = dict(base)
        p.update(over)
        P = [ctypes.c_void_p(p[n]) if p[n] else None for n in names]
        return lib.vdn_vda_backward_gram(ctypes.byref(d), *P, bwb, None)

    assert call(k=0) == bd.VDN_ERR_INVALID_ARG
    assert call(dbeta=0) == bd.VDN_ERR_INVALID_ARG
    assert call(dkt=0) == bd.VDN_ERR_INVALID_ARG                    # text tokens need their outputs
    assert call(dk=base["k"] + 4096) == bd.VDN_ERR_INVALID_ARG     # an output inside an input
    assert call(dv=base["dk"] + 4096) == bd.VDN_ERR_INVALID_ARG    # two outputs overlapping
    assert call(dbt=base["ws"] + 512) == bd.VDN_ERR_INVALID_ARG    # an output inside the workspace
    assert call(bwb=bw - 1) == bd.VDN_ERR_WORKSPACE
    assert call(ws=0) == bd.VDN_ERR_WORKSPACE
    assert call(dk=base["dk"] + 8) == bd.VDN_ERR_ALIGNMENT
    assert call(dbeta=base["dbeta"] + 1) == bd.VDN_ERR_ALIGNMENT
    assert call(ws=base["ws"] + 16) == bd.VDN_ERR_ALIGNMENT
    # float32: 4-byte beta and dbeta, and the arguments pass to the launch
    # (which fails here, with no GPU)
    f32, bw32 = good(dtype="f32"), bd.backward_workspace_bytes(good(dtype="f32"))
    assert call(d=f32, bwb=bw32, dbeta=base["dbeta"] + 2) == bd.VDN_ERR_ALIGNMENT
    assert call(d=f32, bwb=bw32) == bd.VDN_ERR_HIP
    # neither the decay bridge nor the raw query's normalisation reaches this
    # stage: with either flag the arguments are still checked
    assert call(d=good(flags=bd.VDN_VDA_EPILOGUE | bd.VDN_VDA_DECAY_BRIDGE), k=0) == bd.VDN_ERR_INVALID_ARG
    assert call(d=good(flags=bd.VDN_VDA_EPILOGUE | bd.VDN_VDA_QUERY_L2), k=0) == bd.VDN_ERR_INVALID_ARG
    # without text tokens the text pointers are not needed: the call gets as
    # far as the alignment checks
    notext = good(n_text=0)
    assert call(d=notext, kt=0, vt=0, bt=0, dkt=0, dvt=0, dbt=0, bwb=bd.backward_workspace_bytes(notext),
                dk=base["dk"] + 8) == bd.VDN_ERR_ALIGNMENT
    # the third stage's operands are an internal section: the workspace grew by them
    assert bw >= bd.backward_layout(desc).d_b + desc.B * desc.H * (desc.T + 1) * (3 * 128 * 128 * 2 + 128 * 128 * 4)


def test_frame_rows_stay_within_32_bit_offsets():
    """A frame's token rows are addressed with 32-bit byte offsets."""
    # (U + 64) H d 4 bytes must stay below 4 GiB
    assert bd.validate(good(grid_h=1000, grid_w=1000, H=8, d=128)) == bd.VDN_OK
    assert bd.validate(good(grid_h=1000, grid_w=1000, H=16, d=128)) == bd.VDN_ERR_INVALID_ARG
    assert bd.validate(good(n_text=1 << 20, H=16, d=128)) == bd.VDN_ERR_INVALID_ARG
    # the statistics kernel's prefetch reads a few tiles of 64 tokens past the
    # last token: (U + 640) H d 2 bytes must stay below 4 GiB as well, which
    # binds for wide rows of few tokens
    assert bd.validate(good(grid_h=1, grid_w=1, H=16384, n_text=380, d=128)) == bd.VDN_OK
    assert bd.validate(good(grid_h=1, grid_w=1, H=32768, n_text=0, d=128)) == bd.VDN_ERR_INVALID_ARG
    assert bd.validate(good(grid_h=1, grid_w=1, H=16384, n_text=420, d=128)) == bd.VDN_ERR_INVALID_ARG


def test_adjacent_maps_argument_errors_before_launch():
    lib = bd.lib()
    desc = good(n_text=0)
    dm = 3072
    wsb = lib.vdn_vda_gates_workspace_bytes(ctypes.byref(desc), dm)
    assert wsb >= desc.B * desc.T * dm * 4 * 2
    assert lib.vdn_vda_gates_workspace_bytes(ctypes.byref(desc), 100) == 0      # not a multiple of 8
    assert lib.vdn_vda_gates_workspace_bytes(ctypes.byref(good(dtype="f32")), dm) == 0
    names = ["x", "wgb", "wa", "gate", "beta", "alpha", "ws"]
    base = {n: A16 + (1 << 33) * i for i, n in enumerate(names)}

    def gates(d=desc, dmodel=dm, wsbytes=wsb, **over):
        p = dict(base)
        p.update(over)
        P = [ctypes.c_void_p(p[n]) if p[n] else None for n in names]
        return lib.vdn_vda_gates(ctypes.byref(d), dmodel, *P[:6], P[6], wsbytes, None)

    assert gates(x=0) == bd.VDN_ERR_INVALID_ARG
    assert gates(alpha=0) == bd.VDN_ERR_INVALID_ARG
    assert gates(dmodel=100) == bd.VDN_ERR_INVALID_ARG
    assert gates(wsbytes=wsb - 1) == bd.VDN_ERR_WORKSPACE
    assert gates(ws=0) == bd.VDN_ERR_WORKSPACE
    assert gates(gate=base["gate"] + 8) == bd.VDN_ERR_ALIGNMENT
    assert gates(beta=base["beta"] + 1) == bd.VDN_ERR_ALIGNMENT
    assert gates(ws=base["ws"] + 16) == bd.VDN_ERR_ALIGNMENT
    assert gates(beta=base["x"] + 4096) == bd.VDN_ERR_INVALID_ARG           # an output inside x
    assert gates(alpha=base["gate"] + 4096) == bd.VDN_ERR_INVALID_ARG       # outputs overlapping
    assert gates(d=good(n_text=0, dtype="f32")) == bd.VDN_ERR_UNSUPPORTED

    onames = ["o", "wo", "yin", "y"]
    obase = {n: A16 + (1 << 33) * i for i, n in enumerate(onames)}

    def oproj(d=desc, dmodel=dm, **over):
        p = dict(obase)
        p.update(over)
        P = [ctypes.c_void_p(p[n]) if p[n] else None for n in onames]
        return lib.vdn_vda_out_proj(ctypes.byref(d), dmodel, *P, None)

    assert oproj(o=0) == bd.VDN_ERR_INVALID_ARG
    assert oproj(y=0) == bd.VDN_ERR_INVALID_ARG
    assert oproj(dmodel=12) == bd.VDN_ERR_INVALID_ARG
    assert oproj(y=obase["o"] + 4096) == bd.VDN_ERR_INVALID_ARG              # y inside o
    assert oproj(y=obase["yin"] + 4096) == bd.VDN_ERR_INVALID_ARG            # y partly over y_in
    assert oproj(yin=obase["yin"] + 8) == bd.VDN_ERR_ALIGNMENT
    assert oproj(d=good(n_text=0, dtype="f32")) == bd.VDN_ERR_UNSUPPORTED


def test_forward_rejects_overlapping_buffers():
    """The output and the workspace are written while every input is read: any
    shared byte is an error, found before a launch."""
    desc = good()
    need = bd.workspace_bytes(desc)
    gib = 1 << 30
    names = ["q", "k", "v", "alpha", "beta", "k_text", "v_text", "beta_text", "gate", "rms_weight", "out", "ws"]
    # 4 GiB apart: every tensor of the 768p clip fits between two bases
    base = {n: A16 + 4 * gib * i for i, n in enumerate(names)}
    call = lambda **o: _fwd(desc, [dict(base, **o)[n] for n in names], need)
    xbytes = 60 * 4032 * 24 * 128 * 2
    assert call(out=base["q"] + xbytes - 4096) == bd.VDN_ERR_INVALID_ARG       # out's head over q's tail
    assert call(out=base["gate"] - xbytes + 4096) == bd.VDN_ERR_INVALID_ARG    # out's tail over the gate
    assert call(ws=base["k"] + 256 * 1024) == bd.VDN_ERR_INVALID_ARG           # workspace inside k
    assert call(out=base["ws"] + need - 16) == bd.VDN_ERR_INVALID_ARG          # out over the workspace's end
    assert call(ws=base["alpha"] + 256) == bd.VDN_ERR_INVALID_ARG              # workspace over alpha
    assert call(out=base["rms_weight"] - xbytes + 16) == bd.VDN_ERR_INVALID_ARG  # out over the RMSNorm gain
    # ranges that only touch (one ends where the next starts) do not overlap;
    # the call then fails later, on a check that is independent of the ranges
    assert call(out=base["q"] + xbytes, q=base["q"] + 8) == bd.VDN_ERR_ALIGNMENT


def test_forward_timed_checks_its_events():
    lib = bd.lib()
    desc = good()
    need = bd.workspace_bytes(desc)
    P = [ctypes.c_void_p(p) for p in _ptrs()]
    ev = (ctypes.c_void_p * 6)(*([0x1234] * 6))
    few = (ctypes.c_void_p * 5)(*([0x1234] * 5))
    nul = (ctypes.c_void_p * 6)(*([0x1234] * 5 + [0]))
    call = lambda arr, n: lib.vdn_vda_forward_timed(ctypes.byref(desc), *P[:11], P[11], need, None,
                                                    ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None, n)
    assert call(None, 6) == bd.VDN_ERR_INVALID_ARG
    assert call(few, 5) == bd.VDN_ERR_INVALID_ARG
    assert call(nul, 6) == bd.VDN_ERR_INVALID_ARG
    # valid events: the forward's own checks still run before anything is recorded
    P2 = [ctypes.c_void_p(p) for p in _ptrs(q=0)]
    assert lib.vdn_vda_forward_timed(ctypes.byref(desc), *P2[:11], P2[11], need, None,
                                     ctypes.cast(ev, ctypes.c_void_p), 6) == bd.VDN_ERR_INVALID_ARG


def test_prepare_rejects_overlapping_buffers():
    lib = bd.lib()
    desc = good(epilogue=False)
    gib = 1 << 30
    xbytes = 60 * 4032 * 24 * 128 * 2
    base = [A16 + 4 * gib * i for i in range(10)]   # q k v wks wkt wvs wvt q_hat k_hat v_hat

    def call(**o):
        p = list(base)
        for i, v in o.items():
            p[int(i[1:])] = v
        return lib.vdn_vda_prepare(ctypes.byref(desc), *[ctypes.c_void_p(x) for x in p], None)

    assert call(a8=base[1] + 4096) == bd.VDN_ERR_INVALID_ARG          # k_hat inside k
    assert call(a9=base[8] + xbytes - 4096) == bd.VDN_ERR_INVALID_ARG  # v_hat over k_hat's tail
    assert call(a7=base[3] - xbytes + 64) == bd.VDN_ERR_INVALID_ARG    # q_hat over the spatial weights


def test_backward_rejects_overlapping_buffers():
    lib = bd.lib()
    desc = good()
    fw = bd.workspace_bytes(desc)
    bw = bd.backward_workspace_bytes(desc)
    names = ["q", "gate", "rms", "alpha", "dy", "fws", "dq", "dgate", "drms", "ws"]
    base = {n: A16 + (1 << 34) * i for i, n in enumerate(names)}
    xbytes = 60 * 4032 * 24 * 128 * 2

    def call(**over):
        p = dict(base, rms=0, drms=0)
        p.update(over)
        P = [ctypes.c_void_p(p[n]) if p[n] else None for n in names]
        return lib.vdn_vda_backward_readout(ctypes.byref(desc), P[0], P[1], P[2], P[3], P[4], P[5], fw,
                                            P[6], P[7], P[8], P[9], bw, None)

    assert call(dq=base["q"] + 4096) == bd.VDN_ERR_INVALID_ARG              # dq inside q
    assert call(dgate=base["dq"] + xbytes - 4096) == bd.VDN_ERR_INVALID_ARG  # two outputs
    assert call(ws=base["fws"] + 256) == bd.VDN_ERR_INVALID_ARG            # workspace over the forward's
    assert call(dq=base["ws"] + bw - 4096) == bd.VDN_ERR_INVALID_ARG        # dq over the workspace's end
    assert call(drms=base["dy"] + 64) == bd.VDN_ERR_INVALID_ARG              # the gain's gradient inside dy
    assert call(drms=base["ws"] + bw - 256) == bd.VDN_ERR_INVALID_ARG        # ... over the workspace's end
    assert call(drms=base["rms"], rms=base["rms"] + 256) == bd.VDN_ERR_INVALID_ARG  # ... over the gain
    snames = ["alpha", "fws", "dalpha", "ws"]
    sb = {n: A16 + (1 << 34) * i for i, n in enumerate(snames)}

    def scall(**over):
        p = dict(sb, **over)
        return lib.vdn_vda_backward_scan(ctypes.byref(desc), ctypes.c_void_p(p["alpha"]), ctypes.c_void_p(p["fws"]),
                                         fw, ctypes.c_void_p(p["dalpha"]), ctypes.c_void_p(p["ws"]), bw, None)

    assert scall(dalpha=sb["alpha"] + 256) == bd.VDN_ERR_INVALID_ARG
    assert scall(ws=sb["fws"] + fw - 256) == bd.VDN_ERR_INVALID_ARG


def test_adjacent_row_count_is_32_bit():
    """The adjacent maps' GEMMs take B T U rows in 32-bit arithmetic."""
    lib = bd.lib()
    ok = good(n_text=0, T=32767, grid_h=256, grid_w=256, H=1, d=16)     # B T U = 2^31 - 65536
    assert lib.vdn_vda_gates_workspace_bytes(ctypes.byref(ok), 16) > 0
    big = good(n_text=0, T=32768, grid_h=256, grid_w=256, H=1, d=16)    # B T U = 2^31
    assert bd.validate(big) == bd.VDN_OK                      # the forward itself accepts it
    assert lib.vdn_vda_gates_workspace_bytes(ctypes.byref(big), 16) == 0


def test_forward_noalloc_checks_before_touching_the_gpu():
    """vdn_vda_forward_noalloc checks every argument, and its workspace against
    the library's own array, before any HIP call."""
    lib = bd.lib()
    names = ["q", "k", "v", "alpha", "beta", "k_text", "v_text", "beta_text", "gate", "rms_weight", "out"]
    gib = 1 << 30
    base = {n: A16 + 4 * gib * i for i, n in enumerate(names)}

    def call(desc, **over):
        p = dict(base, **over)
        return lib.vdn_vda_forward_noalloc(ctypes.byref(desc), *[ctypes.c_void_p(p[n]) if p[n] else None
                                                                for n in names], None)

    assert call(good(), q=0) == bd.VDN_ERR_INVALID_ARG
    assert call(good(), q=base["q"] + 8) == bd.VDN_ERR_ALIGNMENT
    assert call(good(), out=base["gate"] + 4096) == bd.VDN_ERR_INVALID_ARG
    # the 768p clip needs ~400 MiB of workspace, beyond the 64 MiB array
    assert bd.workspace_bytes(good()) > 64 << 20
    assert call(good()) == bd.VDN_ERR_WORKSPACE
    share = good(H=8, T=60)
    assert bd.workspace_bytes(share) > 64 << 20 and call(share) == bd.VDN_ERR_WORKSPACE
    # a width between the built ones takes its padded copies from the array too
    small = good(H=2, T=6, grid_h=6, grid_w=11, n_text=12, d=48)
    assert bd.workspace_bytes(small) < 64 << 20
    assert call(good(d=48)) == bd.VDN_ERR_WORKSPACE
    bad = good()
    bad.d_v = 64
    assert call(bad) == bd.VDN_ERR_UNSUPPORTED
