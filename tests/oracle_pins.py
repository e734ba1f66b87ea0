"""Checks that pin the oracle to facts other than itself.

Each ``check_*`` raises AssertionError on failure.  They look every oracle
function up through the module at call time, so a test can plant a mistake in
the oracle (monkeypatch) and confirm that some check catches it.

Pins (the oracle function each one constrains in brackets):
  P1  normal-equation residual of every frame update      [transition, scan_states]
  P2  brute-force least squares on the frame objective     [frame_stats, transition, frame_update, text_state]
  P3  one token, unit key == the token delta rule with beta/(1+beta)   [frame_update]
  P4  ||Diag(alpha)(I+A)^-1||_2 <= 1, A PSD                 [frame_stats, transition]
  P5  text counted once; pure-decay closed form             [text_state, scan_states, query_states, readout]
  P5b decay bridge: pure-decay closed form with the bridged chunks   [query_states, bridge_decay]
  P6  coverage partitions the clip; closed-form ranges      [coverage]
  P7  time reversal                                          [scan_states, query_states]
  P8  linearity in (V, V_text)                               [whole raw readout]
  P9  chunk / time-shard composition of the affine updates  [scan_states]
  P10 library routines (trace, symmetry, Cholesky, scipy correlate, torch ops)  [frame_stats, prep, epilogue]
  P11 small-beta agreement with the batch form, O(beta^2)    [frame_update]
  P12 zero writes give zero output                           [all]
  P13 brute-force states straight from the coverage sets     [scan_states, query_states, readout]
  G   hand-worked fixtures under tests/golden               [frame_update, epilogue, coverage, text]
"""

from __future__ import annotations

import os

import numpy as np

import oracle.vda as V

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_head(rng, T=12, U=6, dk=5, dv=4, L=3, unit_keys=True, alpha_lo=0.3):
    """Random inputs of one head, float64, the oracle's per-head layout."""
    k = rng.standard_normal((T, U, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((T, U, dk))
    v = rng.standard_normal((T, U, dv))
    beta = rng.uniform(0.0, 2.0, (T, U))
    alpha = rng.uniform(alpha_lo, 1.0, (T, dk))
    kt = rng.standard_normal((L, dk))
    kt /= np.linalg.norm(kt, axis=-1, keepdims=True)
    vt = rng.standard_normal((L, dv))
    bt = rng.uniform(0.0, 2.0, L)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, k_txt=kt, v_txt=vt, beta_txt=bt)


def run_head(x, C=5):
    return V.forward_head(x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                          x["k_txt"], x["v_txt"], x["beta_txt"], chunk=C)


def _objective(S, Sbar, k, v, beta):
    r = S @ k.T - v.T
    return 0.5 * np.sum((S - Sbar) ** 2) + 0.5 * np.sum(beta * np.sum(r * r, axis=0))


# ----------------------------------------------------------------------------


def check_p1_residual(x, C=5, tol=1e-12):
    """S_t (I + A_t) = S_prev Diag(alpha_t) + B_t for every absorbed frame, both directions."""
    r = run_head(x, C)
    T = x["k"].shape[0]
    dk = x["k"].shape[-1]
    for direction in ("fwd", "rev"):
        S = r["S_T"] / 2
        frames = range(1, T - 1) if direction == "fwd" else range(T - 2, 0, -1)
        for s in frames:
            Sn = S @ r["M"][s] + r["J"][s]
            rhs = S * x["alpha"][s][None, :] + r["B"][s]
            A, _ = V.frame_stats(x["k"][s], x["v"][s], x["beta"][s])
            res = np.linalg.norm(Sn @ (np.eye(dk) + A) - rhs) / max(np.linalg.norm(rhs), 1e-300)
            assert res <= tol, (direction, s, res)
            S = Sn


def check_p2_lstsq(rng, trials=20, tol=1e-12):
    """The frame update equals the least-squares minimiser of the frame objective, row by row."""
    for _ in range(trials):
        dk, dv, U = rng.integers(1, 9), rng.integers(1, 9), rng.integers(1, 17)
        k = rng.standard_normal((U, dk))
        v = rng.standard_normal((U, dv))
        beta = rng.uniform(0.0, 3.0, U)
        alpha = rng.uniform(0.0, 1.0, dk)
        S_prev = rng.standard_normal((dv, dk))
        Sbar = S_prev * alpha[None, :]
        want = np.zeros((dv, dk))
        sq = np.sqrt(beta)[:, None]
        Amat = np.vstack([np.eye(dk), sq * k])
        for i in range(dv):
            rhs = np.concatenate([Sbar[i], sq[:, 0] * v[:, i]])
            want[i] = np.linalg.lstsq(Amat, rhs, rcond=None)[0]
        A, B = V.frame_stats(k, v, beta)
        got = V.frame_update(S_prev, A, B, alpha)
        M, J, _ = V.transition(A, B, alpha)
        got2 = S_prev @ M + J
        scale = max(1.0, np.abs(want).max())
        assert np.abs(got - want).max() <= tol * scale * 10, np.abs(got - want).max()
        assert np.abs(got2 - want).max() <= tol * scale * 10, np.abs(got2 - want).max()
        f0 = _objective(want, Sbar, k, v, beta)
        for _ in range(5):
            P = want + 1e-3 * rng.standard_normal(want.shape)
            assert _objective(P, Sbar, k, v, beta) >= f0
        # the text state is the same objective from a zero state with alpha irrelevant
        ST = V.text_state(k, v, beta)
        want0 = np.zeros((dv, dk))
        for i in range(dv):
            rhs = np.concatenate([np.zeros(dk), sq[:, 0] * v[:, i]])
            want0[i] = np.linalg.lstsq(Amat, rhs, rcond=None)[0]
        assert np.abs(ST - want0).max() <= tol * max(1.0, np.abs(want0).max()) * 10


def check_p3_one_token(rng, trials=20, tol=1e-13):
    """U = 1: the frame update is the token delta rule with beta' = beta / (1 + beta ||k||^2)."""
    for _ in range(trials):
        dk, dv = rng.integers(1, 9), rng.integers(1, 9)
        k = rng.standard_normal(dk)
        unit = rng.random() < 0.5
        if unit:
            k /= np.linalg.norm(k)
        v = rng.standard_normal(dv)
        beta = rng.uniform(0.0, 3.0)
        alpha = rng.uniform(0.0, 1.0, dk)
        S_prev = rng.standard_normal((dv, dk))
        A, B = V.frame_stats(k[None, :], v[None, :], np.array([beta]))
        got = V.frame_update(S_prev, A, B, alpha)
        bprime = beta / (1.0 + beta * (k @ k))
        if unit:
            assert abs(bprime - beta / (1.0 + beta)) < 1e-15
        want = V.token_delta_step(S_prev, k, v, alpha, bprime)
        assert np.abs(got - want).max() <= tol * max(1.0, np.abs(want).max()) * 10


def check_p4_nonexpansion(k_frames, beta_frames, alpha_frames, tol=1e-12):
    """Every frame's transition is a non-expansion and its key Gram is PSD."""
    worst = 0.0
    for k, beta, alpha in zip(k_frames, beta_frames, alpha_frames):
        A, B = V.frame_stats(k, np.zeros((k.shape[0], 1)), beta)
        M, _, Pinv = V.transition(A, B, alpha)
        s = np.linalg.svd(M, compute_uv=False)[0]
        worst = max(worst, s)
        assert s <= 1.0 + tol, s
        assert np.linalg.eigvalsh(A).min() >= -1e-12 * max(1.0, np.abs(A).max())
        assert np.linalg.svd(Pinv, compute_uv=False)[0] <= 1.0 + tol
    return worst


def check_p5_text_once(rng, C=5, tol=1e-13):
    """Text counted exactly once; anchors read S_T q; pure decay gives S_T (D_fwd + D_rev) q / 2."""
    for T in (2, 7, 10, 12, 20, 23):
        x = rand_head(rng, T=T)
        x["beta"][:] = 0.0
        # alpha = 1: every frame reads exactly S_T q
        x1 = dict(x, alpha=np.ones_like(x["alpha"]))
        r = run_head(x1, C)
        for t in range(T):
            want = x["q"][t] @ r["S_T"].T
            assert np.abs(r["o"][t] - want).max() <= tol * 10, (T, t)
        # alpha != 1: the decays of the covered frames multiply S_T/2 on each side
        r = run_head(x, C)
        for t in range(T):
            fwd, rev = V.coverage(t, T, C)
            Df = np.ones(x["alpha"].shape[1])
            for s in fwd:
                Df = Df * x["alpha"][s]
            Dr = np.ones_like(Df)
            for s in rev:
                Dr = Dr * x["alpha"][s]
            S = 0.5 * r["S_T"] * (Df + Dr)[None, :]
            want = x["q"][t] @ S.T
            assert np.abs(r["o"][t] - want).max() <= tol * 10, (T, t)
    # with video writes: anchors still read S_T q, and T <= 2C reads S_T q everywhere
    for T in (8, 10, 15, 30):
        x = rand_head(rng, T=T)
        r = run_head(x, C)
        for t in range(T):
            if t in (0, T - 1) or T <= 2 * C:
                want = x["q"][t] @ r["S_T"].T
                assert np.abs(r["o"][t] - want).max() <= tol * 10, (T, t)


def check_p5b_bridge_closed_form(rng, C=5, tol=1e-13):
    """Decay bridge: with zero video writes every frame absorbed on either side
    only decays, so a non-anchor query in chunk c reads S_T (D_f + D_r) q / 2 with
    D_f = prod alpha over frames 1 .. Cc-1 (c >= 2), 0 .. C-1 (c = 1), none (c = 0),
    D_r = prod alpha over C(c+1) .. T-2 (c <= nc-3), C(nc-1) .. T-1 (c = nc-2),
    none (c = nc-1): the summarised frames plus the bridged chunk next to the
    query's.  Anchor queries read S_T q, with or without writes."""
    def run(x, bridge):
        return V.forward_head(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["k_txt"],
                              x["v_txt"], x["beta_txt"], chunk=C, bridge=bridge)
    for T in (2, 5, 7, 10, 12, 20, 23, 31):
        nc = -(-T // C)
        x = rand_head(rng, T=T)
        x["beta"][:] = 0.0
        r = run(x, True)
        a = x["alpha"]
        for t in range(T):
            if t in (0, T - 1):
                want = x["q"][t] @ r["S_T"].T
                assert np.abs(r["o"][t] - want).max() <= tol * 10, (T, t)
                continue
            c = t // C
            fwd = range(1, C * c) if c >= 2 else (range(0, C) if c == 1 else range(0))
            if c <= nc - 3:
                rev = range(C * (c + 1), T - 1)
            elif c == nc - 2:
                rev = range(C * (nc - 1), T)
            else:
                rev = range(0)
            Df = np.prod(a[list(fwd)], axis=0) if len(fwd) else np.ones(a.shape[1])
            Dr = np.prod(a[list(rev)], axis=0) if len(rev) else np.ones(a.shape[1])
            want = x["q"][t] @ (0.5 * r["S_T"] * (Df + Dr)[None, :]).T
            assert np.abs(r["o"][t] - want).max() <= tol * 10, (T, t, c)
        # with writes the bridge leaves anchors and the states themselves alone
        y = rand_head(rng, T=T)
        rb, r0 = run(y, True), run(y, False)
        for name in ("S_T", "F", "R", "Pinv"):
            assert np.array_equal(rb[name], r0[name]), name
        for t in (0, T - 1):
            assert np.abs(rb["o"][t] - y["q"][t] @ rb["S_T"].T).max() <= tol * 10


def check_p6_coverage(C=5, Ts=(1, 2, 3, 7, 10, 15, 20, 23, 30, 40, 60, 120)):
    """F(t), R(t), W(t) and the anchors partition the clip; F and R have their closed forms."""
    for T in Ts:
        nc = V.num_chunks(T, C)
        assert nc == len(range(0, T, C))
        for t in range(T):
            fwd, rev = V.coverage(t, T, C)
            Fs, Rs = set(fwd), set(rev)
            assert len(Fs) == len(fwd) and len(Rs) == len(rev)
            assert not (Fs & Rs)
            assert fwd == sorted(fwd) and rev == sorted(rev, reverse=True)
            A = V.anchors(T)
            if t in A:
                assert not Fs and not Rs
                continue
            W = V.window_frames(t, T, C)
            assert t in W
            parts = [Fs, Rs, W | A]
            assert sum(len(p) for p in parts) == T
            assert Fs | Rs | W | A == set(range(T))
            assert not (Fs & (W | A)) and not (Rs & (W | A))
            c = t // C
            assert Fs == set(range(1, C * (c - 1))) - A
            assert Rs == set(range(C * (c + 2), T - 1))
            # the window is the query chunk and its neighbours, clipped
            chunks = {s // C for s in W}
            assert chunks == set(range(max(0, c - 1), min(nc - 1, c + 1) + 1))


def _ranges(tok):
    if tok.strip() == "-":
        return []
    out = []
    for part in tok.split(","):
        a, _, b = part.strip().partition("-")
        out.extend(range(int(a), int(b or a) + 1))
    return out


def check_golden_coverage():
    path = os.path.join(GOLDEN, "coverage_T20_C5.txt")
    seen = set()
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        qs, fs, rs = [p.strip() for p in line.split(":")]
        for t in _ranges(qs):
            fwd, rev = V.coverage(t, 20, 5)
            assert sorted(fwd) == _ranges(fs), (t, fwd)
            assert sorted(rev) == _ranges(rs), (t, rev)
            seen.add(t)
    assert seen == set(range(20))


def check_golden_hand_cases(tol=1e-7):
    path = os.path.join(GOLDEN, "hand_cases.txt")
    n = 0
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        f = [p.strip() for p in line.split("|")]
        kind = f[0]
        if kind == "frame":
            dk, dv = map(int, f[2].split())
            alpha = np.array(f[3].split(), float)
            S_prev = np.array(f[4].split(), float).reshape(dv, dk)
            ks, vs, bs = [], [], []
            for tok in f[5].split(","):
                b, kk, vv = tok.split(";")
                bs.append(float(b))
                ks.append(np.array(kk.split(), float))
                vs.append(np.array(vv.split(), float))
            k, v, beta = np.array(ks), np.array(vs), np.array(bs)
            want = np.array(f[6].split(), float).reshape(dv, dk)
            A, B = V.frame_stats(k, v, beta)
            got = V.frame_update(S_prev, A, B, alpha)
            M, J, _ = V.transition(A, B, alpha)
            assert np.abs(got - want).max() <= tol, (f[1], got, want)
            assert np.abs(S_prev @ M + J - want).max() <= tol, f[1]
        elif kind == "epilogue":
            o = np.array(f[2].split(), float)
            g = np.array(f[3].split(), float)
            want = np.array(f[4].split(), float)
            got = V.epilogue(o, g, None, 1e-6)
            assert np.abs(got - want).max() <= tol, (f[1], got, want)
        elif kind == "text":
            q = float(f[2])
            want = float(f[3])
            T, U = 2, 3
            x = dict(q=np.full((T, U, 1), q), k=np.ones((T, U, 1)), v=np.ones((T, U, 1)),
                     alpha=np.ones((T, 1)), beta=np.ones((T, U)),
                     k_txt=np.ones((1, 1)), v_txt=np.full((1, 1), 2.0), beta_txt=np.ones(1))
            r = run_head(x)
            assert np.abs(r["o"] - want).max() <= tol, (f[1], r["o"])
        n += 1
    assert n >= 7


def check_p7_time_reversal(rng, C=5, tol=1e-12):
    for T in (10, 20, 30):
        x = rand_head(rng, T=T)
        r = run_head(x, C)
        xf = dict(x)
        for name in ("q", "k", "v", "alpha", "beta"):
            xf[name] = x[name][::-1].copy()
        rf = run_head(xf, C)
        assert np.abs(rf["o"][::-1] - r["o"]).max() <= tol * 10, T


def check_p8_linearity(rng, C=5, tol=1e-12):
    x1 = rand_head(rng, T=20)
    x2 = dict(x1, v=rng.standard_normal(x1["v"].shape), v_txt=rng.standard_normal(x1["v_txt"].shape))
    a, b = 0.7, -1.3
    x3 = dict(x1, v=a * x1["v"] + b * x2["v"], v_txt=a * x1["v_txt"] + b * x2["v_txt"])
    o1, o2, o3 = run_head(x1, C)["o"], run_head(x2, C)["o"], run_head(x3, C)["o"]
    assert np.abs(o3 - (a * o1 + b * o2)).max() <= tol * 10


def check_p9_composition(rng, C=5, tol=1e-12):
    """Composing each chunk's frames into one affine map, then scanning chunks, equals F and R."""
    for T in (20, 23, 40):
        x = rand_head(rng, T=T)
        r = run_head(x, C)
        M, J = r["M"], r["J"]
        d = M.shape[1]
        nc = V.num_chunks(T, C)

        def compose(frames):
            Mc, Jc = np.eye(d), np.zeros_like(J[0])
            for s in frames:
                Mc, Jc = Mc @ M[s], Jc @ M[s] + J[s]
            return Mc, Jc

        S = r["S_T"] / 2
        for j in range(nc):
            frames = [s for s in range(C * j, min(C * (j + 1), T)) if 1 <= s <= T - 2]
            Mc, Jc = compose(frames)
            S = S @ Mc + Jc
            assert np.abs(S - r["F"][j]).max() <= tol * 10, ("F", T, j)
        S = r["S_T"] / 2
        for j in range(nc - 1, -1, -1):
            frames = [s for s in range(min(C * (j + 1), T) - 1, C * j - 1, -1) if 1 <= s <= T - 2]
            Mc, Jc = compose(frames)
            S = S @ Mc + Jc
            if j >= 1:
                assert np.abs(S - r["R"][j]).max() <= tol * 10, ("R", T, j)
        # three emulated time shards on chunk boundaries: local summaries, then an exclusive prefix
        bounds = [0, (nc // 3) * C, (2 * nc // 3) * C, T]
        summaries = [compose([s for s in range(a, b) if 1 <= s <= T - 2])
                     for a, b in zip(bounds[:-1], bounds[1:])]
        S = r["S_T"] / 2
        for (a, b), (Mc, Jc) in zip(zip(bounds[:-1], bounds[1:]), summaries):
            S = S @ Mc + Jc
            j = (b - 1) // C
            if b < T and b % C == 0:
                assert np.abs(S - r["F"][j]).max() <= tol * 10, ("shard", T, b)


def check_p10_library(rng, tol=1e-13):
    import scipy.ndimage
    import torch
    # key Gram: symmetric, trace, Cholesky of I + A reconstructs it
    k = rng.standard_normal((30, 7))
    beta = rng.uniform(0, 2, 30)
    A, B = V.frame_stats(k, rng.standard_normal((30, 3)), beta)
    assert np.abs(A - A.T).max() <= tol
    assert abs(np.trace(A) - np.sum(beta * np.sum(k * k, axis=1))) <= tol * np.trace(A) * 10
    P = np.eye(7) + A
    Lc = np.linalg.cholesky(P)
    assert np.abs(Lc @ Lc.T - P).max() <= tol * np.abs(P).max() * 10
    # prep vs scipy.ndimage.correlate with the outer-product kernel w_t x w_s
    T, gh, gw, H, d = 6, 4, 5, 2, 3
    x = rng.standard_normal((T, gh * gw, H, d))
    ws = rng.standard_normal((H * d, 5, 5))
    wt = rng.standard_normal((H * d, 5))
    q = rng.standard_normal((T, gh * gw, H, d))
    _, k_hat, v_hat = V.prep(q, x, x, ws, wt, ws, wt, gh, gw, l2_eps=1e-6)
    flat = x.reshape(T, gh, gw, H * d)
    for ch in range(H * d):
        kern = wt[ch][:, None, None] * ws[ch][None, :, :]
        conv = scipy.ndimage.correlate(flat[..., ch], kern, mode="constant", cval=0.0)
        want = conv / (1 + np.exp(-conv))
        h, j = divmod(ch, d)
        got = v_hat[:, :, h, j].reshape(T, gh, gw)
        assert np.abs(got - want).max() <= 1e-12 * max(1, np.abs(want).max())
    silu = torch.nn.functional.silu(torch.from_numpy(x.reshape(T, gh, gw, H * d)))
    # delta weights: the conv is the identity, so V^ = SiLU(V) and K^ = L2(SiLU(K))
    wd_s = np.zeros_like(ws)
    wd_s[:, 2, 2] = 1
    wd_t = np.zeros_like(wt)
    wd_t[:, 2] = 1
    q_hat, k_hat, v_hat = V.prep(q, x, x, wd_s, wd_t, wd_s, wd_t, gh, gw, l2_eps=0.0)
    assert np.abs(v_hat.reshape(silu.shape) - silu.numpy()).max() <= tol * 10
    kn = torch.nn.functional.normalize(silu.reshape(T, gh * gw, H, d), dim=-1).numpy()
    assert np.abs(k_hat - kn).max() <= tol * 10
    qn = torch.nn.functional.normalize(torch.from_numpy(q), dim=-1).numpy()
    assert np.abs(q_hat - qn).max() <= tol * 10
    # epilogue vs torch rms_norm and sigmoid
    o = rng.standard_normal((9, 16))
    g = rng.standard_normal((9, 16))
    gamma = rng.uniform(0.5, 1.5, 16)
    to = torch.from_numpy(o)
    want = torch.nn.functional.rms_norm(to, (16,), torch.from_numpy(gamma), eps=1e-6) * torch.sigmoid(torch.from_numpy(g))
    got = V.epilogue(o, g, gamma, 1e-6)
    assert np.abs(got - want.numpy()).max() <= tol * 10


def check_p11_small_beta(rng):
    """The frame update and the batch form differ by O(beta^2) as beta -> 0."""
    U, dk, dv = 6, 5, 4
    k = rng.standard_normal((U, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((U, dv))
    alpha = rng.uniform(0.5, 1.0, dk)
    S_prev = rng.standard_normal((dv, dk))
    b0 = rng.uniform(0.5, 1.5, U)
    scales = np.logspace(-4, -1, 7)
    errs = []
    for s in scales:
        A, B = V.frame_stats(k, v, s * b0)
        errs.append(np.linalg.norm(V.frame_update(S_prev, A, B, alpha) - V.batch_form_step(S_prev, A, B, alpha)))
    slope = np.polyfit(np.log(scales), np.log(errs), 1)[0]
    assert abs(slope - 2.0) <= 0.1, slope


def check_p12_zero(rng, C=5):
    x = rand_head(rng, T=20)
    x["beta"][:] = 0
    x["beta_txt"][:] = 0
    r = run_head(x, C)
    assert np.all(r["o"] == 0)
    y = V.epilogue(r["o"], rng.standard_normal(r["o"].shape), None, 1e-6)
    assert np.all(y == 0)


def check_p13_brute_force(rng, C=5, tol=1e-13):
    """Each query's two states rebuilt from scratch from its coverage sets with the frame update."""
    for T in (2, 3, 9, 12, 20, 23, 31):
        x = rand_head(rng, T=T)
        r = run_head(x, C)
        S_T = V.text_state(x["k_txt"], x["v_txt"], x["beta_txt"])
        for t in range(T):
            fwd, rev = V.coverage(t, T, C)
            states = []
            for frames in (fwd, rev):
                S = S_T / 2
                for s in frames:
                    A, B = V.frame_stats(x["k"][s], x["v"][s], x["beta"][s])
                    S = V.frame_update(S, A, B, x["alpha"][s])
                states.append(S)
            o = x["q"][t] @ (states[0] + states[1]).T
            assert np.abs(r["o"][t] - o).max() <= tol * 100 * max(1, np.abs(o).max()), (T, t)
            sf, sr = V.query_states(r["F"], r["R"], r["S_T"], t, T, C)
            assert np.abs(sf - states[0]).max() <= tol * 100
            assert np.abs(sr - states[1]).max() <= tol * 100
