"""Address-range model of the HIP kernels' global memory accesses, on the host.

Each ``model_*`` function re-derives, from the kernel's own index arithmetic
(``frame_wise_delta_02_amd/csrc``), every global address a launch can touch:
the work-items are enumerated with numpy (every block, every thread), and loop
indices are taken at the extremes the loop bounds allow (every offset below is
non-decreasing in its loop index, which the model asserts where it matters).
Two kinds of access are checked:

* plain loads and stores through a pointer: the byte range must lie inside the
  buffer the entry point passes;
* loads and stores through a raw buffer descriptor (base, num_records): the
  descriptor's range must lie inside the buffer, and every 32-bit offset the
  kernel computes must not wrap (a wrapped offset could land back inside the
  range); accesses past num_records read zero or are dropped by the hardware.

Covered: the forward pass and the prep (``model_forward``), the three backward
stages (``model_backward``, every part of the backward workspace as a buffer of
its own) and the adjacent maps (``model_gates``, ``model_out_proj``).

The model has no knowledge of the kernels beyond what is written here: a kernel
change that moves an address must be mirrored in its model, and the test then
checks the new arithmetic for every shape the GPU tests and the benchmark run.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

U32 = 1 << 32


@dataclass
class Prob:
    B: int
    H: int
    T: int
    gh: int
    gw: int
    D: int
    L: int
    C: int = 5
    bf16: bool = True
    chunked: bool = False
    epilogue: bool = True
    gamma: bool = False
    bridge: bool = False
    dgain: bool = False   # the backward readout also forms the gain's gradient
    Du: int = 0           # the caller's head width where it lies between the built ones (D is then the built one)

    @property
    def U(self):
        return self.gh * self.gw

    @property
    def nc(self):
        return -(-self.T // self.C)

    @property
    def esz(self):
        return 2 if self.bf16 else 4

    @property
    def split(self):
        return self.bf16 and self.D >= 32


@dataclass
class Report:
    """Every violation found, as readable strings."""
    errors: list = field(default_factory=list)
    checked: int = 0

    def ptr(self, kernel, buf, size, lo, hi):
        """[lo, hi) bytes through a pointer into a buffer of `size` bytes."""
        self.checked += 1
        lo, hi = int(np.min(lo)), int(np.max(hi))
        if lo < 0 or hi > size:
            self.errors.append(f"{kernel}: {buf} [{lo}, {hi}) outside [0, {size})")

    def rsrc(self, kernel, buf, size, base, nrec, max_off, width):
        """A buffer descriptor at byte `base` of `nrec` records; the largest
        32-bit offset used is `max_off` for an access of `width` bytes."""
        self.checked += 1
        base = np.asarray(base, dtype=np.int64)
        nrec = np.asarray(nrec, dtype=np.int64)
        live = nrec > 0
        if np.any(live):
            lo = int(np.min(base[live] if base.ndim else base))
            hi = int(np.max((base + nrec)[live] if (base + nrec).ndim else base + nrec))
            if lo < 0 or hi > size:
                self.errors.append(f"{kernel}: {buf} descriptor [{lo}, {hi}) outside [0, {size})")
        if np.any(nrec >= U32):
            self.errors.append(f"{kernel}: {buf} descriptor of {int(np.max(nrec))} records does not fit 32 bits")
        if int(np.max(max_off)) + width > U32 - 1:
            self.errors.append(f"{kernel}: {buf} offset {int(np.max(max_off))} + {width} wraps 32 bits")


# ---------------------------------------------------------------------------
# buffers of the forward pass (bytes), as the entry points size them
# ---------------------------------------------------------------------------


def sizes(p: Prob) -> dict:
    tok = p.B * p.T * p.U * p.H
    heads = p.B * p.H
    dd = p.D * p.D * 4
    DP = max(p.D, 32)
    MT = DP // 32
    slot = (2 * MT * (p.D // 16) * 64 * 16) if p.bf16 else (MT * (p.D // 8) * 64 * 16)
    return dict(
        q=tok * p.D * p.esz, k=tok * p.D * p.esz, v=tok * p.D * p.esz, gate=tok * p.D * p.esz,
        out=tok * p.D * p.esz, beta=tok * p.esz, alpha=p.B * p.T * p.H * p.D * 4,
        k_text=p.B * p.L * p.H * p.D * p.esz, v_text=p.B * p.L * p.H * p.D * p.esz,
        beta_text=p.B * p.L * p.H * p.esz, rms=p.D * 4,
        stats=heads * (p.T + 1) * 2 * dd, pinv=heads * (p.T + 1) * dd, s_text=heads * dd,
        fwd=heads * p.nc * dd, rev=heads * p.nc * dd, rstates=heads * (p.nc + 1) * slot,
        chunk_m=heads * 2 * p.nc * dd, chunk_j=heads * 2 * p.nc * dd,
        wk_s=p.H * p.D * 25 * 4, wk_t=p.H * p.D * 5 * 4)


def _grid(*dims):
    """All index tuples of a launch, as flat int64 arrays."""
    g = np.meshgrid(*[np.arange(n, dtype=np.int64) for n in dims], indexing="ij")
    return [x.ravel() for x in g]


# ---------------------------------------------------------------------------
# vda_gram.hip
# ---------------------------------------------------------------------------


def model_gram(p: Prob, r: Report, S=None, parts=None, out="stats", t_slots=None):
    """gram_bf16<D> / gram_f32<D>: two parts in one launch -- frames 1..T-2 of
    K, V, beta, then the text frame (slot T).  With ``parts`` (bfloat16 only)
    the backward's PLAIN mode: V^T K of each frame, no beta (``bb`` None), one
    d x d slot per frame of ``out`` with ``t_slots`` slots per head."""
    plain = parts is not None
    S = S or sizes(p)
    D, H = p.D, p.H
    if not plain:
        # with no text tokens the text units' (empty) descriptors sit on the video tensors
        text = ("k_text", "v_text", "beta_text") if p.L > 0 else ("k", "v", "beta")
        parts = [("k", "v", "beta", p.T, p.U, 1, max(p.T - 2, 0), 0),
                 (*text, 1, p.L, 0, 1, p.T)]
        t_slots = p.T + 1
    R = D if plain else 2 * D
    for kb, vb, bb, T_in, U, t_first, n_frames, slot_off in parts:
        nblk = p.B * n_frames * H
        if nblk == 0:
            continue
        (blk,) = _grid(nblk)
        h = blk % H
        fi = (blk // H) % n_frames
        b = blk // (H * n_frames)
        t = t_first + fi
        tok0 = (b * T_in + t) * U
        if p.bf16:
            CGT, NS = D // 8, 2
            TPT = CGT // 2
            nstep = ((U + 63) // 64 + NS - 1) // NS * NS
            rowbytes = H * D * 2
            xbytes = (U - 1) * rowbytes + D * 2 if U > 0 else 0
            blk2, wave, lane = _grid(nblk, 4, 64)
            hh = blk2 % H
            t2 = t_first + (blk2 // H) % n_frames
            b2 = blk2 // (H * n_frames)
            tok02 = (b2 * T_in + t2) * U
            local = (wave & 1) * 64 + lane
            cg, tq = local % CGT, local // CGT
            tokk = TPT * tq
            # loads of tiles 0 .. nstep + NS (the prefetch runs NS tiles ahead)
            it_max = nstep + NS
            max_off = (tokk + TPT - 1 + 64 * it_max) * rowbytes + cg * 16
            base = (tok02 * H + hh) * D * 2
            for buf in (kb, vb):
                r.rsrc("gram_bf16", buf, S[buf], base, np.full_like(base, xbytes), max_off, 16)
            if bb is not None:
                bbase = (tok02 * H + hh) * 2
                bbytes = (U - 1) * H * 2 + 2 if U > 0 else 0
                boff = (32 * (wave & 1) + (lane & 31)) * H * 2 + 64 * it_max * H * 2
                r.rsrc("gram_bf16", bb, S[bb], bbase, np.full_like(bbase, bbytes), boff, 2)
        else:
            TT = 16
            ntile = (U + TT - 1) // TT
            if ntile > 0:
                # rows clamped to token 0 of the frame past U: read range of the frame's rows
                lo = (tok0 * H + h) * D * 4
                hi = ((tok0 + U - 1) * H + h) * D * 4 + D * 4
                r.ptr("gram_f32", kb, S[kb], lo, hi)
                r.ptr("gram_f32", vb, S[vb], lo, hi)
                r.ptr("gram_f32", bb, S[bb], (tok0 * H + h) * 4, ((tok0 + U - 1) * H + h) * 4 + 4)
        # consumer stores: one (2d x d) slot per (b, h, t + slot_off) of [B, H, T+1]
        # (PLAIN: one d x d slot of [B, H, T])
        slot = (b * H + h) * t_slots + (t + slot_off)
        r.ptr("gram", out, S[out], slot * R * D * 4, (slot + 1) * R * D * 4)
        if p.bf16 and not plain:
            # the largest element index a consumer writes inside its slot
            MT, NT = R // 16, D // 16
            WM = 4 if MT >= 4 else MT
            MTW = MT // WM
            wm, mi, nj, lane, rr = _grid(WM, MTW, NT, 64, 4)
            idx = (16 * (wm * MTW + mi) + 4 * (lane >> 4) + rr) * D + 16 * nj + (lane & 15)
            assert idx.max() < R * D and idx.min() >= 0, "gram: a consumer store leaves its slot"


# ---------------------------------------------------------------------------
# vda_solve.hip
# ---------------------------------------------------------------------------


def model_solve(p: Prob, r: Report):
    S = sizes(p)
    D, H = p.D, p.H
    n_video = max(p.T - 2, 0)
    (blk,) = _grid(p.B * H * (n_video + 1))
    si = blk % (n_video + 1)
    h = (blk // (n_video + 1)) % H
    b = blk // ((n_video + 1) * H)
    slot = np.where(si < n_video, 1 + si, p.T)
    mat = (b * H + h) * (p.T + 1) + slot
    # loads of A: D*D floats from the slot's first row; stores: D*D floats
    r.ptr("solve", "stats", S["stats"], mat * 2 * D * D * 4, mat * 2 * D * D * 4 + D * D * 4)
    r.ptr("solve", "pinv", S["pinv"], mat * D * D * 4, (mat + 1) * D * D * 4)
    if p.split:
        # solve_sweep: float4 loads of the lower 16 x 16 tiles of A only, rows
        # 16 R + row, columns 16 C + 4 c4 (C <= R): a subset of the slot's first
        # D x D floats; fragment stores f and NFR + f (16 B each)
        NB = D // 16
        RR, CC, row, c4 = _grid(NB, NB, 16, 4)
        low = CC <= RR
        off = ((16 * RR + row) * D + 16 * CC + 4 * c4)[low] * 4
        assert off.min() >= 0 and off.max() + 16 <= D * D * 4
        NFR = D * D // 8
        f = np.arange(NFR)
        assert (NFR + f).max() * 16 + 16 <= D * D * 4


# ---------------------------------------------------------------------------
# vda_scan.hip
# ---------------------------------------------------------------------------


def _scan_steps(p: Prob, mode: str, dir_, cj=None):
    """(frames or chunk slots visited incl. the prefetch of the last, alpha frames)."""
    T, C, nc = p.T, p.C, p.nc
    nch = max(nc - 2, 0)
    if mode == "compose":
        lo, hi = max(C * cj, 1), min(C * (cj + 1) - 1, T - 2)
        n = max(0, hi - lo + 1)
        s = list(range(lo, hi + 1))
        return (s if n else [T]), (s if n else [0])
    if mode == "chunks":
        first = 0 if dir_ == 0 else nc - 1
        step = 1 if dir_ == 0 else -1
        s = [first + step * i for i in range(nch)]
        return (s if nch else [0]), []
    if dir_ == 0:
        first, last = 1, (min(C * (nc - 2) - 1, T - 2) if nc >= 3 else 0)
        s = list(range(first, last + 1))
    else:
        first, last = T - 2, (max(2 * C, 1) if nc >= 3 else T - 1)
        s = list(range(first, last - 1, -1))
    return (s if s else [T]), (s if s else [0])


def model_scan(p: Prob, r: Report):
    S = sizes(p)
    D, H, T, nc = p.D, p.H, p.T, p.nc
    split = p.split
    NV = 2 if D >= 32 else 1
    RB = 16 * (2 if split else 1)
    NRB = D // RB
    nch = max(nc - 2, 0)
    modes = ["compose", "chunks"] if p.chunked and nch > 0 else (["chunks"] if p.chunked else ["frames"])
    dd = D * D * 4
    for mode in modes:
        groups = p.B * H * 2
        units = groups * nch if mode == "compose" else groups
        rbpu = 2 * NRB if mode == "compose" else NRB
        nblk = (units + 7) // 8 * 8 * rbpu
        (bid,) = _grid(nblk)
        xcd, sl = bid % 8, bid // 8
        rbi = sl % rbpu
        u = (sl // rbpu) * 8 + xcd
        live = u < units
        bid, rbi, u = bid[live], rbi[live], u[live]
        g = u // nch if mode == "compose" else u
        dir_ = g % 2
        h = (g // 2) % H
        b = g // (2 * H)
        head = b * H + h
        mpart = (rbi < NRB) if mode == "compose" else np.zeros_like(rbi, dtype=bool)
        row0 = np.where((mode == "compose") & ~mpart, rbi - NRB, rbi) * RB
        assert row0.max() + RB <= D
        # in-slot offsets of one state block (rows row0..row0+RB-1, every column)
        blk_hi = (row0 + RB) * D * 4
        blk_lo = row0 * D * 4
        for d_ in (0, 1):
            sel = dir_ == d_
            if not np.any(sel):
                continue
            hd = head[sel]
            if mode == "compose":
                cis = (u[sel] % nch)
                cjs = np.where(d_ == 0, cis, nc - 1 - cis)
                frames, alphas = set(), set()
                for cj in np.unique(cjs):
                    f, a = _scan_steps(p, mode, d_, int(cj))
                    frames |= set(f)
                    alphas |= set(a)
            else:
                f, a = _scan_steps(p, mode, d_)
                frames, alphas = set(f), set(a)
                if mode == "frames":
                    frames.add(T)  # the text slot (S_T) first
            fr = np.array(sorted(frames))
            if mode == "chunks":
                # products with M_c, rows of J_c: slots j of [B, H, 2, nc, d, d]
                cs = (hd[:, None] * 2 + d_) * nc + fr[None, :]
                assert fr.max() < nc and fr.min() >= 0
                r.ptr("scan", "chunk_m", S["chunk_m"], cs * dd, (cs + 1) * dd)
                r.ptr("scan", "chunk_j", S["chunk_j"], cs * dd, (cs + 1) * dd)
                # the text frame from stats / pinv slot T
                r.ptr("scan", "pinv", S["pinv"], (hd * (T + 1) + T) * dd, (hd * (T + 1) + T + 1) * dd)
                r.ptr("scan", "stats", S["stats"], (hd * (T + 1) + T) * 2 * dd + dd,
                      (hd * (T + 1) + T) * 2 * dd + 2 * dd)
            else:
                assert fr.min() >= 0 and fr.max() <= T
                ps = hd[:, None] * (T + 1) + fr[None, :]
                r.ptr("scan", "pinv", S["pinv"], ps * dd, (ps + 1) * dd)
                r.ptr("scan", "stats", S["stats"], ps * 2 * dd + dd, ps * 2 * dd + 2 * dd)
                al = np.array(sorted(alphas | {0}))
                assert al.min() >= 0 and al.max() < T
                # alpha [B, T, H, d]: row s of (b, h)
                bb = (hd // H)[:, None]
                hh = (hd % H)[:, None]
                lo = ((bb * T + al[None, :]) * H + hh) * D * 4
                r.ptr("scan", "alpha", S["alpha"], lo, lo + D * 4)
            if mode == "compose":
                cs = (hd * 2 + d_) * nc + cjs
                r.ptr("scan", "chunk_m/j", S["chunk_m"], cs * dd, (cs + 1) * dd)
            else:
                # records through a descriptor over this head's n_c states; steps
                # that record nothing store at offset 2^31
                buf = "fwd" if d_ == 0 else "rev"
                r.rsrc("scan", buf, S[buf], hd * nc * dd, np.full_like(hd, nc * dd),
                       np.array([0x80000000 + D * D * 4 - 4 * NV, (nc - 1) * dd + D * D * 4 - 4 * NV]), 4 * NV)
                if (1 << 31) < nc * dd:
                    r.errors.append("scan: the no-record sentinel 2^31 lies inside a head's records")
                if d_ == 0:
                    r.ptr("scan", "s_text", S["s_text"], hd * dd, (hd + 1) * dd)


def model_gather(p: Prob, r: Report):
    S = sizes(p)
    D, nc, T, H = p.D, p.nc, p.T, p.H
    dd = D * D * 4
    (blk,) = _grid(p.B * H * (nc + 1))
    slot = blk % (nc + 1)
    head = blk // (nc + 1)
    r.ptr("gather", "s_text", S["s_text"], head * dd, (head + 1) * dd)
    fsel = (slot < nc) & (slot >= 2)
    if np.any(fsel):
        j = head[fsel] * nc + slot[fsel] - 2
        r.ptr("gather", "fwd", S["fwd"], j * dd, (j + 1) * dd)
    rsel = (slot < nc) & (slot + 2 <= nc - 1)
    if np.any(rsel):
        j = head[rsel] * nc + slot[rsel] + 2
        r.ptr("gather", "rev", S["rev"], j * dd, (j + 1) * dd)
    if p.bridge:
        frames = [s for c in range(nc) for s in list(range(p.C * (c - 1), p.C * c)) * (c >= 1)
                  + list(range(p.C * (c + 1), min(p.C * (c + 2), T))) * (c + 1 <= nc - 1)]
        if frames:
            assert min(frames) >= 0 and max(frames) < T
    slot_bytes = S["rstates"] // (p.B * H * (nc + 1))
    r.ptr("gather", "rstates", S["rstates"], blk * slot_bytes, (blk + 1) * slot_bytes)


def model_readout(p: Prob, r: Report, S=None, q="q", out="out", rstates="rstates"):
    """readout_bf16 / readout_f32; the backward pass runs it on dy with the
    transposed states (``q``, ``out``, ``rstates`` name those buffers)."""
    S = S or sizes(p)
    D, H, T, U = p.D, p.H, p.T, p.U
    (blk,) = _grid(p.B * T * H)
    h = blk % H
    t = (blk // H) % T
    b = blk // (H * T)
    nc = p.nc
    slot = np.where((t == 0) | (t == T - 1), nc, t // p.C)
    slot_bytes = S[rstates] // (p.B * H * (nc + 1))
    rs = (b * H + h) * (nc + 1) + slot
    r.ptr("readout", rstates, S[rstates], rs * slot_bytes, (rs + 1) * slot_bytes)
    if p.gamma:
        r.ptr("readout", "rms", S["rms"], 0, D * 4)
    if p.bf16:
        NW, CH = 8, D // 8
        RPI = 64 // CH
        NL = 32 // RPI
        rowbytes = H * D * 2
        nbytes = (U - 1) * rowbytes + D * 2 if U > 0 else 0
        fbase = (((b * T + t) * U * H + h) * D) * 2
        ntiles = (U + 31) // 32
        per_wave = (ntiles + NW - 1) // NW
        steps = (per_wave + 1) & ~1
        # fetch(tile + 2 NW) at the last loop pass reaches tile wave + NW * steps;
        # process(tile + NW) stores up to tile wave + NW * (steps - 1)
        wave, lane = _grid(NW, 64)
        loff = (lane // CH) * rowbytes + 16 * (lane % CH)
        tile_max = wave + NW * max(steps, 0)
        max_off = tile_max * 32 * rowbytes + loff + (RPI * (NL - 1)) * rowbytes
        for buf in [q, out] + (["gate"] if p.epilogue else []):
            r.rsrc("readout_bf16", buf, S[buf], fbase, np.full_like(fbase, nbytes), max_off, 16)
    else:
        lo = (((b * T + t) * U) * H + h) * D * 4
        hi = (((b * T + t) * U + U - 1) * H + h) * D * 4 + D * 4
        for buf in [q, out] + (["gate"] if p.epilogue else []):
            r.ptr("readout_f32", buf, S[buf], lo, hi)


# ---------------------------------------------------------------------------
# vda_prep.hip
# ---------------------------------------------------------------------------


def model_prep(p: Prob, r: Report):
    """The prep runs on the caller's tensors at the caller's width (Du where it
    lies between the built ones: the generic kernel, its last lanes idle)."""
    D = p.Du or p.D
    H, T, gh, gw = p.H, p.T, p.gh, p.gw
    U = gh * gw
    tok = p.B * T * U * H
    S = dict(q=tok * D * p.esz, k=tok * D * p.esz, v=tok * D * p.esz, wk_s=H * D * 25 * 4, wk_t=H * D * 5 * 4)
    tokstride = H * D
    if p.bf16 and D == 128:
        PTY, PTX = 8, 12
        ntx, nty = -(-gw // PTX), -(-gh // PTY)
        ntile = ntx * nty
        (bid,) = _grid(p.B * H * ntile)
        if H % 8 == 0:
            xcd, j = bid % 8, bid // 8
            tile = j % ntile
            hq = j // ntile
            h = (hq % (H // 8)) * 8 + xcd
            b = hq // (H // 8)
        else:
            tile = bid % ntile
            h = (bid // ntile) % H
            b = bid // (ntile * H)
        assert h.max() < H and b.max() < p.B and np.unique(b * H * ntile + h * ntile + tile).size == bid.size
        # slab loads: positions clamped to the frame by the `ok` test; frames < T
        y0, x0 = (tile // ntx) * PTY, (tile % ntx) * PTX
        yy_lo, yy_hi = np.maximum(y0 - 2, 0), np.minimum(y0 + PTY + 1, gh - 1)
        xx_lo, xx_hi = np.maximum(x0 - 2, 0), np.minimum(x0 + PTX + 1, gw - 1)
        lo = ((b * T + 0) * U + yy_lo * gw + xx_lo) * tokstride + h * D
        hi = ((b * T + T - 1) * U + yy_hi * gw + xx_hi) * tokstride + h * D + D
        for buf in ("k", "v"):
            r.ptr("prep_conv_tile", buf, S[buf], lo * 2, hi * 2)
        # stores: positions inside the grid of frames 0..T-1
        yo = np.minimum(y0 + PTY - 1, gh - 1)
        xo = np.minimum(x0 + PTX - 1, gw - 1)
        lo = ((b * T) * U + y0 * gw + x0) * tokstride + h * D
        hi = ((b * T + T - 1) * U + yo * gw + xo) * tokstride + h * D + D
        for buf in ("k", "v"):
            r.ptr("prep_conv_tile", buf + "_hat", S[buf], lo * 2, hi * 2)
        c = h * D
        r.ptr("prep_conv_tile", "wk_s", S["wk_s"], c * 25 * 4, (c + D) * 25 * 4)
        r.ptr("prep_conv_tile", "wk_t", S["wk_t"], c * 5 * 4, (c + D) * 5 * 4)
    else:
        (blk,) = _grid(p.B * T * H * gh)
        y = blk % gh
        h = (blk // gh) % H
        t = (blk // (gh * H)) % T
        b = blk // (gh * H * T)
        lo = ((b * T + np.maximum(t - 2, 0)) * U + np.maximum(y - 2, 0) * gw) * H + h
        hi = ((b * T + np.minimum(t + 2, T - 1)) * U + np.minimum(y + 2, gh - 1) * gw + gw - 1) * H + h
        for buf in ("k", "v"):
            r.ptr("prep_conv", buf, S[buf], lo * D * p.esz, (hi * D + D) * p.esz)
        r.ptr("prep_conv", "wk_s", S["wk_s"], h * D * 25 * 4, (h * D + D) * 25 * 4)
    # prep_l2: rows = B T U H, one thread per 8 channels, guarded by row < rows
    rows = p.B * T * U * H
    r.ptr("prep_l2", "q", S["q"], 0, rows * D * p.esz)


def model_copy_rows(r: Report, src, src_size, dst, dst_size, src_row, dst_row, copy, rows):
    """copy_rows (vda_pad.hip): thread i of rows * dst_row / 16 writes 16 bytes
    at 16 i and, for chunk c = i % (dst_row / 16) < copy / 16 of row
    r = i / (dst_row / 16), reads 16 bytes at src_row r + 16 c."""
    ss, ds, nc = src_row // 16, dst_row // 16, copy // 16
    assert src_row % 16 == 0 and dst_row % 16 == 0 and copy % 16 == 0 and nc <= ds and nc <= ss
    n = rows * ds
    if n == 0:
        return
    r.ptr("copy_rows", dst, dst_size, np.array([0]), np.array([n * 16]))
    if nc:
        r.ptr("copy_rows", src, src_size, np.array([0]), np.array([((rows - 1) * ss + nc - 1) * 16 + 16]))


def model_forward(p: Prob, prep: bool = False) -> Report:
    """Every kernel of vdn_vda_forward (and vdn_vda_prepare) for one problem.
    With Du set (a width between the built ones) the pipeline's kernels run at
    p.D on zero-padded copies in the workspace: the caller's q, k, v, gate,
    alpha and text tensors (width Du) are copied in and the output copied back."""
    r = Report()
    if prep:
        model_prep(p, r)
    if p.Du and p.Du != p.D:
        S = sizes(p)  # the padded copies
        tok, trows = p.B * p.T * p.U * p.H, p.B * p.L * p.H
        ub, pb = p.Du * p.esz, p.D * p.esz
        for x in ("q", "k", "v") + (("gate",) if p.epilogue else ()):
            model_copy_rows(r, "caller " + x, tok * ub, "padded " + x, S[x], ub, pb, ub, tok)
        model_copy_rows(r, "caller alpha", p.B * p.T * p.H * p.Du * 4, "padded alpha", S["alpha"], p.Du * 4,
                        p.D * 4, p.Du * 4, p.B * p.T * p.H)
        if p.L:
            for x in ("k_text", "v_text"):
                model_copy_rows(r, "caller " + x, trows * ub, "padded " + x, S[x], ub, pb, ub, trows)
        if p.epilogue:  # pad_gain: one workgroup, thread j < D writes dst[j], reads w[j] for j < Du
            r.ptr("pad_gain", "padded rms", S["rms"], np.arange(p.D) * 4, np.arange(p.D) * 4 + 4)
            if p.gamma:
                r.ptr("pad_gain", "caller rms", p.Du * 4, np.arange(p.Du) * 4, np.arange(p.Du) * 4 + 4)
        model_copy_rows(r, "padded out", S["out"], "caller out", tok * ub, pb, ub, ub, tok)
    model_gram(p, r)
    model_solve(p, r)
    model_scan(p, r)
    model_gather(p, r)
    model_readout(p, r)
    return r


# ---------------------------------------------------------------------------
# the backward pass: vda_backward.hip, the scan's STATES and ADJOINT modes and
# the statistics kernel's PLAIN mode, on the buffers vdn_vda_backward_readout,
# _scan and _gram are given (every part of the backward workspace is checked
# as a buffer of its own, so an access that runs from one part into the next
# is caught, which a sanitizer watching the whole allocation would miss)
# ---------------------------------------------------------------------------


def bwd_sizes(p: Prob) -> dict:
    """Bytes of every buffer the three backward stages touch."""
    S = dict(sizes(p))
    tok, ttok, heads = p.B * p.T * p.U * p.H, p.B * p.L * p.H, p.B * p.H
    dd = p.D * p.D * 4
    x, xt = tok * p.D * p.esz, ttok * p.D * p.esz
    S.update(dy=x, dq=x, dgate=x, dout=x, dk=x, dv=x, dbeta=tok * p.esz, dk_text=xt, dv_text=xt,
             dbeta_text=ttok * p.esz,
             dalpha=p.B * p.T * p.H * p.D * 4, rstates_t=S["rstates"], dsq=heads * p.T * dd,
             dF=heads * p.nc * dd, dR=heads * p.nc * dd, dST=heads * dd, lam_final=heads * 2 * dd,
             states_f=heads * (p.T + 2) * dd, states_r=heads * (p.T + 2) * dd,
             gmats=heads * (p.T + 1) * 5 * max(p.D, 32) * p.D * 2,
             gain=p.B * p.T * p.H * p.D * 4, dgamma=(p.Du or p.D) * 4)
    for n in ("lam_f", "lam_r", "dA", "dB", "p32", "M", "dPinv", "tmp"):
        S[n] = heads * (p.T + 1) * dd
    return S


def _readout_frags(D):
    """16-byte fragments of one plane of a readout state slot."""
    DP = max(D, 32)
    return (DP // 32) * (D // 16) * 64


def model_pack_states_t(p: Prob, r: Report, S):
    D, H, T, C, nc = p.D, p.H, p.T, p.C, p.nc
    NF = _readout_frags(D)
    dd = D * D * 4
    (blk,) = _grid(p.B * H * (nc + 1))
    slot = blk % (nc + 1)
    bh = blk // (nc + 1)
    h, b = bh % H, bh // H
    r.ptr("pack_states_t", "rstates_t", S["rstates_t"], blk * 2 * NF * 16, (blk + 1) * 2 * NF * 16)
    r.ptr("pack_states_t", "s_text", S["s_text"], bh * dd, (bh + 1) * dd)
    has_f = (slot < nc) & (slot >= 2)
    has_r = (slot < nc) & (slot + 2 <= nc - 1)
    if np.any(has_f):
        j = bh[has_f] * nc + slot[has_f] - 2
        r.ptr("pack_states_t", "fwd", S["fwd"], j * dd, (j + 1) * dd)
    if np.any(has_r):
        j = bh[has_r] * nc + slot[has_r] + 2
        r.ptr("pack_states_t", "rev", S["rev"], j * dd, (j + 1) * dd)
    if p.bridge:
        frames = []
        for sl in range(nc):
            if sl >= 1:
                frames += list(range(C * (sl - 1), C * sl))
            if sl + 1 <= nc - 1:
                frames += list(range(C * (sl + 1), min(C * (sl + 2), T)))
        if frames:
            s_ = np.array(frames)
            lo = ((b[:, None] * T + s_[None, :]) * H + h[:, None]) * D * 4
            r.ptr("pack_states_t", "alpha", S["alpha"], lo, lo + D * 4)


def model_readout_bwd(p: Prob, r: Report, S):
    """readout_bwd_bf16 (with the epilogue), else the forward readout on dy."""
    D, H, T, U, C, nc = p.D, p.H, p.T, p.U, p.C, p.nc
    if not p.epilogue:
        model_readout(p, r, S, q="dy", out="dq", rstates="rstates_t")
        return
    NF = _readout_frags(D)
    (blk,) = _grid(p.B * T * H)
    h = blk % H
    t = (blk // H) % T
    b = blk // (H * T)
    slot = np.where((t == 0) | (t == T - 1), nc, t // C)
    sl = (b * H + h) * (nc + 1) + slot
    sb = 2 * NF * 16
    r.ptr("readout_bwd", "rstates", S["rstates"], sl * sb, sl * sb + 2 * NF * 16)
    r.ptr("readout_bwd", "rstates_t", S["rstates_t"], sl * sb, sl * sb + NF * 16)
    if p.gamma:
        r.ptr("readout_bwd", "rms", S["rms"], 0, D * 4)
    NW, CH = 4, D // 8
    RPI = 64 // CH
    NL = 32 // RPI
    HALF = max(D, 32) // 2
    NG = HALF // 8
    rowbytes = H * D * 2
    nbytes = (U - 1) * rowbytes + D * 2 if U > 0 else 0
    fbase = (((b * T + t) * U * H + h) * D) * 2
    ntiles = (U + 31) // 32
    per_wave = (ntiles + NW - 1) // NW
    loff = (RPI - 1) * rowbytes + 16 * (CH - 1)
    # fetch_q(tile + NW) inside the last process: tile (NW - 1) + NW per_wave
    fetch_max = ((NW - 1) + NW * per_wave) * 32 * rowbytes + loff + RPI * (NL - 1) * rowbytes
    tile_max = (NW - 1) + NW * max(per_wave - 1, 0)
    row_max = tile_max * 32 * rowbytes + loff + RPI * (NL - 1) * rowbytes
    # this tile's q again, by token: the lanes owning outputs (dv0 < D)
    qc_max = (tile_max * 32 + 31) * rowbytes + max(dv0 for dv0 in (0, HALF) if dv0 < D) * 2 + 16 * (NG - 1)
    n = np.full_like(fbase, nbytes)
    r.rsrc("readout_bwd", "q", S["q"], fbase, n, max(fetch_max, qc_max), 16)
    for buf in ("gate", "dy", "dout", "dgate", "dq"):
        r.rsrc("readout_bwd", buf, S[buf], fbase, n, row_max, 16)
    if p.dgain:
        # readout_bwd_gain_bf16: threads tid < D store row blockIdx.x of the
        # per-(frame, head) sums; gain_grad_sum: one workgroup of 1024 threads,
        # thread (s, j) reading rows s, s + 1024 / D, ... < B T H, and dgamma[j]
        r.ptr("readout_bwd", "gain", S["gain"], blk * D * 4, blk * D * 4 + D * 4)
        rows = p.B * T * H
        sl = np.arange(1024) // D
        j = np.arange(1024) % D
        last = sl + ((rows - 1 - sl) // (1024 // D)) * (1024 // D)
        live = sl < rows
        r.ptr("gain_grad_sum", "gain", S["gain"], (sl[live] * D + j[live]) * 4, (last[live] * D + j[live]) * 4 + 4)
        n_out = p.Du or D  # the caller's channels only
        r.ptr("gain_grad_sum", "dgamma", S["dgamma"], j[:n_out] * 4, j[:n_out] * 4 + 4)


def model_gram_plain(p: Prob, r: Report, S):
    """dS_q(t) = do_t^T q_t for every frame: the statistics kernel's PLAIN mode."""
    do = "dout" if p.epilogue else "dy"
    model_gram(p, r, S, parts=[("q", do, None, p.T, p.U, 0, p.T, 0)], out="dsq", t_slots=p.T)


def _ptr_heads(r, kern, S, buf, heads, per_head, lo_slot, hi_slot, dd):
    """Slots lo_slot .. hi_slot - 1 of per_head-slot blocks of every head."""
    lo = (heads * per_head + lo_slot) * dd
    hi = (heads * per_head + hi_slot) * dd
    r.ptr(kern, buf, S[buf], lo, hi)


def _token_rows(r, kern, buf, size, b, t, h, T_in, U, H, D, esz, per_token=None):
    """Every token row [u < U] of frame t of batch b, head h, in a [B, T_in, U,
    H, D] tensor (or, with per_token, one element per token: [B, T_in, U, H])."""
    tok0 = (b * T_in + t) * U
    first = (tok0 * H + h)
    last = ((tok0 + U - 1) * H + h)
    if per_token:
        r.ptr(kern, buf, size, first * esz, last * esz + esz)
    else:
        r.ptr(kern, buf, size, first * D * esz, last * D * esz + D * esz)


def model_backward_f32(p: Prob, r: Report, S):
    """The float32 first and third stages (vda_backward_f32.hip)."""
    D, H, T, U, C, nc = p.D, p.H, p.T, p.U, p.C, p.nc
    dd = D * D * 4
    # slot_states_f32: one workgroup per (batch, head, slot), the slot's D x D
    # floats written, the records and S_T read as pack_states_t reads them
    (blk,) = _grid(p.B * H * (nc + 1))
    r.ptr("slot_states_f32", "rstates_t", S["rstates_t"], blk * dd, blk * dd + dd)
    rr = Report()
    model_pack_states_t(p, rr, dict(S, rstates_t=1 << 62))
    r.errors += [e.replace("pack_states_t", "slot_states_f32") for e in rr.errors]
    r.checked += rr.checked
    # readout_bwd_f32 and state_adjoint_f32: one workgroup per (frame, head)
    (blk,) = _grid(p.B * T * H)
    h, t, b = blk % H, (blk // H) % T, blk // (H * T)
    slot = np.where((t == 0) | (t == T - 1), nc, t // C)
    sl = (b * H + h) * (nc + 1) + slot
    r.ptr("readout_bwd_f32", "rstates_t", S["rstates_t"], sl * dd, sl * dd + dd)
    ins = ("q", "gate", "dy") if p.epilogue else ("q", "dy")
    outs = ("dq", "dgate", "dout") if p.epilogue else ("dq",)
    for buf in ins + outs:
        _token_rows(r, "readout_bwd_f32", buf, S[buf], b, t, h, T, U, H, D, 4)
    if p.gamma:
        r.ptr("readout_bwd_f32", "rms", S["rms"], np.array([0]), np.array([D * 4]))
    if p.dgain and p.epilogue:
        r.ptr("readout_bwd_f32", "gain", S["gain"], blk * D * 4, blk * D * 4 + D * 4)
    for buf in ("q", "dout" if p.epilogue else "dy"):
        _token_rows(r, "state_adjoint_f32", buf, S[buf], b, t, h, T, U, H, D, 4)
    m = ((b * H + h) * T + t) * dd
    r.ptr("state_adjoint_f32", "dsq", S["dsq"], m, m + dd)


def model_gram_bwd_f32(p: Prob, r: Report, S):
    """gram_bwd_f32: every frame (slots 0 .. T-1), then the text frame (slot T)."""
    D, H, T, U, L = p.D, p.H, p.T, p.U, p.L
    dd = D * D * 4
    parts = [("k", "v", "beta", "dk", "dv", "dbeta", T, U, T, 0)]
    if L:
        parts.append(("k_text", "v_text", "beta_text", "dk_text", "dv_text", "dbeta_text", 1, L, 1, T))
    for k, v, be, dk, dv, dbe, T_in, n_tok, n_frames, off in parts:
        (blk,) = _grid(p.B * n_frames * H)
        h, f, b = blk % H, (blk // H) % n_frames, blk // (H * n_frames)
        m = ((b * H + h) * (T + 1) + f + off) * dd
        for buf in ("dA", "dB"):
            r.ptr("gram_bwd_f32", buf, S[buf], m, m + dd)
        for buf in (k, v, dk, dv):
            _token_rows(r, "gram_bwd_f32", buf, S[buf], b, f, h, T_in, n_tok, H, D, 4)
        for buf in (be, dbe):
            _token_rows(r, "gram_bwd_f32", buf, S[buf], b, f, h, T_in, n_tok, H, D, 4, per_token=True)


def model_backward_scan(p: Prob, r: Report, S):
    D, H, T, C, nc = p.D, p.H, p.T, p.C, p.nc
    heads = np.arange(p.B * H, dtype=np.int64)
    dd = D * D * 4
    # fill_zero over whole buffers (n16 = bytes / 16 entries of 16 bytes)
    for buf in ("states_f", "states_r", "lam_f", "lam_r", "dA", "dB", "dalpha"):
        assert S[buf] % 16 == 0
        r.ptr("fill_zero", buf, S[buf], 0, S[buf] // 16 * 16)
    # backward_gather: dsq of all T frames of a head; dF, dR of all n_c slots; dST
    _ptr_heads(r, "backward_gather", S, "dsq", heads, T, 0, T, dd)
    _ptr_heads(r, "backward_gather", S, "dF", heads, nc, 0, nc, dd)
    _ptr_heads(r, "backward_gather", S, "dR", heads, nc, 0, nc, dd)
    _ptr_heads(r, "backward_gather", S, "dST", heads, 1, 0, 1, dd)
    if p.bridge:
        frames = []
        for j in range(nc):
            if j >= 1:
                frames += list(range(C * (j - 1), C * j))
            if j + 1 <= nc - 1:
                frames += list(range(C * (j + 1), min(C * (j + 2), T)))
        if frames:
            s_ = np.array(frames)
            b, h = heads // H, heads % H
            lo = ((b[:, None] * T + s_[None, :]) * H + h[:, None]) * D * 4
            r.ptr("backward_gather", "alpha", S["alpha"], lo, lo + D * 4)
    # the scan's STATES and ADJOINT modes: frame by frame, every frame's state
    # (T + 2 slots) and every frame's adjoint (T + 1 slots) through a
    # descriptor per (head, direction)
    NV = 2 if D >= 32 else 1
    for d_ in (0, 1):
        frames, alphas = _scan_steps(p, "frames", d_)
        fr = np.array(sorted(set(frames) | {T}))
        assert fr.min() >= 0 and fr.max() <= T
        ps = heads[:, None] * (T + 1) + fr[None, :]
        for kern in ("scan_states", "scan_adjoint"):
            r.ptr(kern, "pinv", S["pinv"], ps * dd, (ps + 1) * dd)
            al = np.array(sorted(set(alphas) | {0}))
            assert al.max() < T
            b, h = (heads // H)[:, None], (heads % H)[:, None]
            lo = ((b * T + al[None, :]) * H + h) * D * 4
            r.ptr(kern, "alpha", S["alpha"], lo, lo + D * 4)
        r.ptr("scan_states", "stats", S["stats"], ps * 2 * dd + dd, ps * 2 * dd + 2 * dd)
        # STATES: the start state in slot 0 / T - 1, then slot s after frame s
        rec = "states_f" if d_ == 0 else "states_r"
        slots = [0 if d_ == 0 else T - 1] + [s for s in frames if s != T]
        assert max(slots) <= T + 1
        r.rsrc("scan_states", rec, S[rec], heads * (T + 2) * dd, np.full_like(heads, (T + 2) * dd),
               np.array([max(slots) * dd + dd - 4 * NV]), 4 * NV)
        # ADJOINT: the record adjoints of chunk min(s / C, n_c - 1) (or 0),
        # lambda at frame s into slot s, the start state's adjoint into lam_final
        real = [s for s in frames if s != T]
        js = sorted({min(s // C, nc - 1) for s in real} | {0})
        assert max(js) < nc
        src = "dF" if d_ == 0 else "dR"
        jj = heads[:, None] * nc + np.array(js)[None, :]
        r.ptr("scan_adjoint", src, S[src], jj * dd, (jj + 1) * dd)
        lam = "lam_f" if d_ == 0 else "lam_r"
        top = max(real) if real else 0
        r.rsrc("scan_adjoint", lam, S[lam], heads * (T + 1) * dd, np.full_like(heads, (T + 1) * dd),
               np.array([top * dd + dd - 4 * NV]), 4 * NV)
        _ptr_heads(r, "scan_adjoint", S, "lam_final", heads, 2, d_, d_ + 1, dd)
    # text_adjoint: slot T of lam_f, dST, both final adjoints
    _ptr_heads(r, "text_adjoint", S, "lam_f", heads, T + 1, T, T + 1, dd)
    _ptr_heads(r, "text_adjoint", S, "dST", heads, 1, 0, 1, dd)
    _ptr_heads(r, "text_adjoint", S, "lam_final", heads, 2, 0, 2, dd)
    # decode_pinv: every slot's two planes into a float32 matrix
    P = "pinv"
    if p.split:
        _ptr_heads(r, "decode_pinv", S, "pinv", heads, T + 1, 0, T + 1, dd)
        _ptr_heads(r, "decode_pinv", S, "p32", heads, T + 1, 0, T + 1, dd)
        P = "p32"
    # gemm_dd: (head, slot) for slots 1 .. T-2 and T; matrix slot + shift of
    # each operand, head strides of T + 2 (states), 2 (T + 1) (stats) or T + 1
    slots = np.array(list(range(1, T - 1)) + [T])
    hs = heads[:, None]
    sl = slots[None, :]

    def mat(kern, buf, per_head, shift, stride=1, off=0):
        i = (hs * per_head + (sl + shift) * stride) * dd + off
        r.ptr(kern, buf, S[buf], i, i + dd)

    for buf, per, sh in (("states_f", T + 2, -1), ("lam_f", T + 1, 0), ("states_r", T + 2, 1), ("lam_r", T + 1, 0),
                         (P, T + 1, 0), ("M", T + 1, 0)):
        mat("gemm_dd rowdot", buf, per, sh)
    mat("gemm_dd diag", "stats", 2 * (T + 1), 0, stride=2, off=dd)
    for buf in ("lam_f", "lam_r", "M", "dPinv"):
        mat("gemm_dd diag", buf, T + 1, 0)
    for buf in ("lam_f", "lam_r", P, "dB", "dPinv", "tmp", "dA"):
        mat("gemm_dd", buf, T + 1, 0)
    frames_ = slots[slots < T]
    if frames_.size:
        b, h = (heads // H)[:, None], (heads % H)[:, None]
        lo = ((b * T + frames_[None, :]) * H + h) * D * 4
        r.ptr("gemm_dd diag", "alpha", S["alpha"], lo, lo + D * 4)
        r.ptr("gemm_dd rowdot", "dalpha", S["dalpha"], lo, lo + D * 4)
    # bridge_dalpha: (head, chunk j); query chunks j + 1 (forward) and j - 1 (reverse)
    if p.bridge:
        for j in range(nc):
            if j + 1 <= nc - 1 and j + 1 >= 2:
                _ptr_heads(r, "bridge_dalpha", S, "fwd", heads, nc, j - 1, j, dd)
            if j >= 1 and j + 1 <= nc - 1:
                _ptr_heads(r, "bridge_dalpha", S, "rev", heads, nc, j + 1, j + 2, dd)
            cs = [c for c in (j + 1, j - 1) if 0 <= c <= nc - 1]
            ts = [t for c in cs for t in range(C * c, min(C * (c + 1), T))]
            if ts:
                _ptr_heads(r, "bridge_dalpha", S, "dsq", heads, T, min(ts), max(ts) + 1, dd)
            s_ = np.arange(C * j, min(C * (j + 1), T))
            b, h = (heads // H)[:, None], (heads % H)[:, None]
            lo = ((b * T + s_[None, :]) * H + h) * D * 4
            r.ptr("bridge_dalpha", "alpha", S["alpha"], lo, lo + D * 4)
            r.ptr("bridge_dalpha", "dalpha", S["dalpha"], lo, lo + D * 4)
        _ptr_heads(r, "bridge_dalpha", S, "s_text", heads, 1, 0, 1, dd)


def model_backward_gram(p: Prob, r: Report, S):
    D, H, T, U, L = p.D, p.H, p.T, p.U, p.L
    heads = np.arange(p.B * H, dtype=np.int64)
    dd = D * D * 4
    # pack_grad_mats(16): slot i of dA, dB into five bfloat16 planes of slot i
    DP = max(D, 32)
    NF = (DP // 16) * (D // 32) * 64 if D >= 32 else (DP // 32) * (D // 16) * 64
    slot_b = 5 * NF * 16  # the layout gives each slot 5 max(d, 32) d bfloat16 values
    for buf in ("dA", "dB"):
        _ptr_heads(r, "pack_grad_mats", S, buf, heads, T + 1, 0, T + 1, dd)
    _ptr_heads(r, "pack_grad_mats", S, "gmats", heads, T + 1, 0, T + 1, slot_b)
    # gram_bwd16 (d >= 32) / gram_bwd_bf16 (d = 16): every frame, then the text
    # frame (launched only with text tokens)
    parts = [("k", "v", "beta", "dk", "dv", "dbeta", T, U, 0, T, 0)]
    if L > 0:
        parts.append(("k_text", "v_text", "beta_text", "dk_text", "dv_text", "dbeta_text", 1, L, 0, 1, T))
    rowbytes = H * D * 2
    for kb, vb, bb, dkb, dvb, dbb, T_in, Up, t_first, n_frames, slot_off in parts:
        (blk,) = _grid(p.B * n_frames * H)
        h = blk % H
        fi = (blk // H) % n_frames
        b = blk // (H * n_frames)
        t = t_first + fi
        src = (b * H + h) * (T + 1) + (t + slot_off)
        r.ptr("gram_bwd", "gmats", S["gmats"], src * slot_b, (src + 1) * slot_b)
        tok0 = (b * T_in + t) * Up
        fbase = (tok0 * H + h) * D * 2
        nbytes = (Up - 1) * rowbytes + D * 2 if Up > 0 else 0
        ntiles = (Up + 31) // 32
        row = max(ntiles * 32 - 1, 0)  # every load and store is guarded by tile < ntiles
        max_off = row * rowbytes + (D * 2 - 16)
        for buf in (kb, vb, dkb, dvb):
            r.rsrc("gram_bwd", buf, S[buf], fbase, np.full_like(fbase, nbytes), max_off, 16)
        bbase = (tok0 * H + h) * 2
        bbytes = (Up - 1) * H * 2 + 2 if Up > 0 else 0
        for buf in (bb, dbb):
            r.rsrc("gram_bwd", buf, S[buf], bbase, np.full_like(bbase, bbytes), row * H * 2, 2)


def model_backward(p: Prob) -> Report:
    """Every kernel of vdn_vda_backward_readout, _scan and _gram for one
    problem (bfloat16 inputs)."""
    S = bwd_sizes(p)
    r = Report()
    pad = bool(p.Du) and p.Du != p.D
    tok, trows, frames = p.B * p.T * p.U * p.H, p.B * p.L * p.H, p.B * p.T * p.H
    ub, pb = p.Du * 2, p.D * 2
    if pad:  # stage 1: dy in (q, gate, alpha and the gain are the forward's padded copies)
        model_copy_rows(r, "caller dy", tok * ub, "padded dy", S["dy"], ub, pb, ub, tok)
    if p.bf16:
        model_pack_states_t(p, r, S)
        model_readout_bwd(p, r, S)
        model_gram_plain(p, r, S)
    else:
        model_backward_f32(p, r, S)
    if pad:  # dq, dgate out
        for x in ("dq",) + (("dgate",) if p.epilogue else ()):
            model_copy_rows(r, "padded " + x, S[x], "caller " + x, tok * ub, pb, ub, ub, tok)
    model_backward_scan(p, r, S)
    if pad:  # dalpha out
        model_copy_rows(r, "padded dalpha", S["dalpha"], "caller dalpha", frames * p.Du * 4, p.D * 4, p.Du * 4,
                        p.Du * 4, frames)
        # stage 3: k, v (and the text's) in
        for x in ("k", "v"):
            model_copy_rows(r, "caller " + x, tok * ub, "padded " + x, S[x], ub, pb, ub, tok)
        if p.L:
            for x in ("k_text", "v_text"):
                model_copy_rows(r, "caller " + x, trows * ub, "padded " + x, S[x], ub, pb, ub, trows)
    if p.bf16:
        model_backward_gram(p, r, S)
    else:
        model_gram_bwd_f32(p, r, S)
    if pad:  # dk, dv (and the text's) out
        for x in ("dk", "dv"):
            model_copy_rows(r, "padded " + x, S[x], "caller " + x, tok * ub, pb, ub, ub, tok)
        if p.L:
            for x in ("dk_text", "dv_text"):
                model_copy_rows(r, "padded " + x, S[x], "caller " + x, trows * ub, pb, ub, ub, trows)
    return r


# ---------------------------------------------------------------------------
# vda_proj.hip: the gates before the path and the output projection after it
# ---------------------------------------------------------------------------

GBM = GBN = 256
GROUP_M = 4


def proj_sizes(p: Prob, dm: int) -> dict:
    """Bytes of the adjacent maps' buffers (bfloat16, float32 where noted)."""
    M, F, HD = p.B * p.T * p.U, p.B * p.T, p.H * p.D
    S = min(8, max(1, p.U // 64))
    return dict(x=M * dm * 2, w_gb=(HD + p.H) * dm * 2, w_alpha=HD * dm * 4, gate=M * HD * 2, beta=M * p.H * 2,
                alpha=F * HD * 4, partial=F * S * dm * 4, xbar=F * dm * 4, o=M * HD * 2, w_o=dm * HD * 2,
                y_in=M * dm * 2, y=M * dm * 2, splits=S)


def model_gemm(r: Report, S, kern, M, N, K, a, w, epi, outs):
    """gemm_nt_bf16: C [M, N] = A [M, K] W [N, K]^T, one 256 x 256 tile per live
    block in the XCD-banded order; ``outs`` names (gate, beta) for PROJ_GATE
    with the gate's column count first, else (y, y_in or None)."""
    mtiles, ntiles = -(-M // GBM), -(-N // GBN)
    ntot = mtiles * ntiles
    grid = (ntot + 7) // 8 * 8
    (bid,) = _grid(grid)
    xcd, slot = bid & 7, bid >> 3
    per_xcd = (ntot + 7) // 8
    tau = xcd * per_xcd + slot
    live = (slot < per_xcd) & (tau < ntot)
    tau = tau[live]
    band, rem = tau // (GROUP_M * ntiles), tau % (GROUP_M * ntiles)
    gm = np.minimum(GROUP_M, mtiles - band * GROUP_M)
    nt, mt = rem // gm, band * GROUP_M + rem % gm
    tiles = mt * ntiles + nt
    if not (mt.max() < mtiles and nt.max() < ntiles and np.unique(tiles).size == ntot == tiles.size):
        r.errors.append(f"{kern}: the tile order does not visit every tile once")
    m0, n0 = mt * GBM, nt * GBN
    mrows, nrows = np.minimum(GBM, M - m0), np.minimum(GBN, N - n0)
    # panel loads: row < 256, k <= K - 8 (16 bytes); past K the offset 2^31
    kmax = (GBM * K - 8) * 2
    r.rsrc(kern, a, S[a], m0 * K * 2, mrows * K * 2, np.array([kmax, 0x80000000]), 16)
    r.rsrc(kern, w, S[w], n0 * K * 2, nrows * K * 2, np.array([kmax, 0x80000000]), 16)
    if 0x80000000 < GBM * K * 2:
        r.errors.append(f"{kern}: the past-K sentinel 2^31 lies inside a panel")
    # epilogue: 128 rows per wave row, 16-byte stores inside a row
    for wm in (0, 1):
        rb = m0 + 128 * wm
        rows = np.where(rb < M, np.minimum(128, M - rb), 0)
        if epi == "gate":
            (g, ng), (b_, nb) = outs
            r.rsrc(kern, g, S[g], rb * ng * 2, rows * ng * 2, np.array([128 * ng * 2 - 16]), 16)
            r.rsrc(kern, b_, S[b_], rb * nb * 2, rows * nb * 2, np.array([128 * nb * 2 - 2]), 2)
        else:
            y, yin = outs
            for buf in [y] + ([yin] if yin else []):
                r.rsrc(kern, buf, S[buf], rb * N * 2, rows * N * 2, np.array([128 * N * 2 - 16]), 16)


def model_gates(p: Prob, dm: int) -> Report:
    """vdn_vda_gates: the gate/beta GEMM, the frame means, the decay gate."""
    S = proj_sizes(p, dm)
    r = Report()
    M, F, HD, U = p.B * p.T * p.U, p.B * p.T, p.H * p.D, p.U
    model_gemm(r, S, "gemm_nt_bf16 gates", M, HD + p.H, dm, "x", "w_gb", "gate", (("gate", HD), ("beta", p.H)))
    SP = S["splits"]
    per = -(-U // SP)
    f, s = _grid(F, SP)
    u0 = s * per
    u1 = np.minimum(U, u0 + per)
    has = u1 > u0
    # frame_col_sums: rows u0 .. u1 - 1 of frame f, columns 0 .. dm - 1
    lo = (f[has] * U + u0[has]) * dm * 2
    hi = (f[has] * U + u1[has] - 1) * dm * 2 + dm * 2
    r.ptr("frame_col_sums", "x", S["x"], lo, hi)
    r.ptr("frame_col_sums", "partial", S["partial"], (f * SP + s) * dm * 4, (f * SP + s + 1) * dm * 4)
    r.ptr("frame_mean", "partial", S["partial"], 0, F * SP * dm * 4)
    r.ptr("frame_mean", "xbar", S["xbar"], 0, F * dm * 4)
    # alpha_proj: guarded reads of xbar [F, K] and W_alpha [HD, K], alpha [F, HD]
    r.ptr("alpha_proj", "xbar", S["xbar"], 0, F * dm * 4)
    r.ptr("alpha_proj", "w_alpha", S["w_alpha"], 0, HD * dm * 4)
    r.ptr("alpha_proj", "alpha", S["alpha"], 0, F * HD * 4)
    return r


def model_out_proj(p: Prob, dm: int, y_in: bool = True) -> Report:
    """vdn_vda_out_proj: Y = Y_in + O W_O^T."""
    S = proj_sizes(p, dm)
    r = Report()
    model_gemm(r, S, "gemm_nt_bf16 out_proj", p.B * p.T * p.U, dm, p.H * p.D, "o", "w_o", "add",
               ("y", "y_in" if y_in else None))
    return r
