"""Lane-level host model of solve_sweep<D> (frame_wise_delta_02_amd/csrc/vda_solve.hip).

The kernel inverts P = I + A_t by a symmetric block sweep over the lower
triangle of 16 x 16 tiles held in LDS and writes P^{-1} as bfloat16 hi + lo
fragments in the scan's operand order.  This model repeats, with numpy
float32 arithmetic, the kernel's own index arithmetic: the float4 load of the
lower tiles (identity added on the diagonal), the one-wave scalar leaf sweep
(lane = row, the pivot row broadcast by readlane, reciprocal plus one Newton
step), the products on v_mfma_f32_16x16x4f32 with the kernel's operand and
accumulator lane layouts (lane l supplies A[l%16][l/16] and B[l/16][l%16];
accumulator register r of lane l is D[4(l/16)+r][l%16]), the permuted k order
that lets C_i = P_ik X serve as the update's left operand, and the output
fragment order.  The arithmetic order of a real matrix core differs, so the
model gives the algorithm's float32 error, not the kernel's bits.

Like tests/kernel_bounds.py, the model knows only what is written here: a
change to the kernel's layouts must be mirrored in it.
"""

from __future__ import annotations

import numpy as np

LANE = np.arange(64)
LM, LG = LANE & 15, LANE >> 4
LDT = 17
TS = 16 * LDT


def mfma_16x16x4(a: np.ndarray, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    """c + A B for per-lane operands a, b (64,) and accumulators c (64, 4)."""
    A = np.zeros((16, 4), np.float32)
    Bm = np.zeros((4, 16), np.float32)
    A[LM, LG] = a
    Bm[LG, LM] = b
    prod = (A @ Bm).astype(np.float32)
    out = c.copy()
    for r in range(4):
        out[:, r] = (out[:, r] + prod[4 * LG + r, LM]).astype(np.float32)
    return out


def sweep_inverse(a_t: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Run the modelled kernel on A_t (d x d).  Returns (P^{-1} as float32
    from the hi + lo fragments' exact sum, fragment write counts per element)."""
    D = a_t.shape[0]
    assert a_t.shape == (D, D) and D in (32, 64, 128)
    NB = D // 16
    NT = NB * (NB + 1) // 2
    RPW = 2 if NB == 8 else 1
    A = np.asarray(a_t, np.float32)
    tl = np.full((NT + 1) * TS, np.nan, np.float32)
    XS = NT * TS

    def tile(R, C):
        return (R * (R + 1) // 2 + C) * TS

    # ---- the lower tiles of P = I + A into LDS: float4 piece e of 64 per tile
    for e in range(NT * 64):
        t, w = e >> 6, e & 63
        R = 0
        while (R + 1) * (R + 2) // 2 <= t:
            R += 1
        C = t - R * (R + 1) // 2
        row, c4 = w >> 2, w & 3
        x = A[16 * R + row, 16 * C + 4 * c4:16 * C + 4 * c4 + 4].copy()
        if R == C:
            for q in range(4):
                x[q] += np.float32(1.0) if row == 4 * c4 + q else np.float32(0.0)
        dst = (t * 16 + row) * LDT + 4 * c4
        tl[dst:dst + 4] = x

    def leaf(k):
        Tk = tile(k, k)
        a = [tl[Tk + LM * LDT + j].copy() for j in range(16)]  # a[j][lane]: row lm, column j
        for p in range(16):
            rowp = [np.float32(a[j][p]) for j in range(16)]  # readlane(a[j], p): row p
            d = rowp[p]
            r = np.float32(1.0) / d
            r = np.float32(r + r * (np.float32(1.0) - d * r))  # one Newton step
            me = LM == p
            t = np.where(me, np.float32(1.0) - r, a[p] * r).astype(np.float32)
            for j in range(16):
                if j != p:
                    a[j] = (a[j] - t * rowp[j]).astype(np.float32)
            a[p] = np.where(me, -r, t).astype(np.float32)
        lanes = LANE < 16
        for j in range(16):
            tl[Tk + LM[lanes] * LDT + j] = a[j][lanes]
            tl[XS + LM[lanes] * LDT + j] = -a[j][lanes]

    def row_of(wave, u):
        return wave if u == 0 else NB - 1 - wave

    leaf(0)
    for k in range(NB):
        creg = {}
        writes = []
        for wave in range(4):
            for u in range(RPW):
                i = row_of(wave, u)
                if i >= NB or i == k:
                    continue
                acc = np.zeros((64, 4), np.float32)
                Pik = tile(i, k) if i > k else tile(k, i)
                for s in range(4):
                    xa = tl[XS + LM * LDT + 4 * s + LG]
                    pb = tl[Pik + LM * LDT + 4 * s + LG] if i > k else tl[Pik + (4 * s + LG) * LDT + LM]
                    acc = mfma_16x16x4(xa, pb, acc)
                creg[(wave, u)] = acc
                for j in range(i + 1):
                    if j == k:
                        continue
                    Tij = tile(i, j)
                    c = np.stack([tl[Tij + (4 * LG + r) * LDT + LM] for r in range(4)], 1)
                    Pkj = tile(k, j) if j < k else tile(j, k)
                    for s in range(4):
                        pb = tl[Pkj + (4 * LG + s) * LDT + LM] if j < k else tl[Pkj + LM * LDT + 4 * LG + s]
                        c = mfma_16x16x4(-acc[:, s], pb, c)
                    # the updated tiles are row i's own: no other wave reads them this step
                    writes.append((Tij, c))
        for Tij, c in writes:
            for r in range(4):
                tl[Tij + (4 * LG + r) * LDT + LM] = c[:, r]
        # after the barrier: P_ik <- C_i
        for (wave, u), acc in creg.items():
            i = row_of(wave, u)
            for r in range(4):
                if i > k:
                    tl[tile(i, k) + LM * LDT + 4 * LG + r] = acc[:, r]
                else:
                    tl[tile(k, i) + (4 * LG + r) * LDT + LM] = acc[:, r]
        if k + 1 < NB:
            leaf(k + 1)

    # ---- output: fragment f holds P^{-1}[32 s + 8 (l/16) + j][32 w + 2 (l%16) + e]
    NFR = D * D // 8
    KS2 = D // 32
    out = np.zeros((D, D), np.float32)
    count = np.zeros((D, D), np.int64)
    for f in range(NFR):
        fl, ks, we = f & 63, (f >> 6) % KS2, (f >> 6) // KS2
        c = 32 * (we >> 1) + 2 * (fl & 15) + (we & 1)
        r0 = 32 * ks + 8 * (fl >> 4)
        R, rr, Cb, cc = r0 >> 4, r0 & 15, c >> 4, c & 15
        for j in range(8):
            v = -tl[tile(R, Cb) + (rr + j) * LDT + cc] if R >= Cb else -tl[tile(Cb, R) + cc * LDT + rr + j]
            out[r0 + j, c] = v
            count[r0 + j, c] += 1
    return out, count


def split_bf16(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """hi = bf16(x), lo = bf16(x - hi), both round to nearest even, as float32."""
    def to_bf16(v):
        b = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
        b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
        return b.astype(np.uint32).view(np.float32)
    hi = to_bf16(x)
    lo = to_bf16(np.asarray(x, np.float32) - hi)
    return hi, lo
