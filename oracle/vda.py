"""VDA forward, written out as the pages define it, in float64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow on purpose: no
blocking, fusion or reordering beyond what the definitions state.

Notation follows [VDN-summary] "어떻게 쓰나": per frame t of one head, K_t is
U x d_k (rows are token keys k_{t,u}), V_t is U x d_v, beta_t holds one write
strength per token, alpha_t one decay per key channel.  The state S is
d_v x d_k, and a query q (length d_k) reads out S q (length d_v).

Readings of points the pages leave open:

R1  Anchor query frames (0 and T-1) attend to everything in the softmax
    branch, so their linear coverage is empty in both directions and their
    readout is S_T q.
R2  No "decay bridge": the state a query reads is exactly the state after
    its covered frames.
R3  The reverse scan applies the same frame update (each frame with its own
    alpha_t) to the time-reversed frame order.
R4  S_T is the frame update from a zero state over the text tokens (a
    leading virtual frame): S_T = B_T (I + A_T)^{-1}.
R5  Windows are clipped at the clip edges, not shifted.
R6  When T is not a multiple of the chunk size the last chunk is short.
R7  Prep conv: per-channel (depthwise) weights, separate for K and V, no bias,
    cross-correlation orientation, zero padding 2, temporal taps centred
    (t-2 .. t+2).  Q is not convolved; text tokens are not convolved.
R8  L2 normalisation is x / sqrt(sum x^2 + eps_l2).
R9  RMSNorm over d_v per (token, head): o / sqrt(mean(o^2) + eps_rms),
    times an optional per-channel weight gamma; then the elementwise sigmoid
    of the gate logits.
R10 alpha has shape [B, T, H, d_k]; beta has shape [B, T, U, H].
"""

from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# input decoding (not part of the method)
# ----------------------------------------------------------------------------


def widen_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16/int16) to float64.

    A bfloat16 value is the upper half of an IEEE binary32 value, so shifting
    the 16 bits into the top of a 32-bit word gives the float32 exactly.
    """
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# coverage: which frames each direction of the linear branch summarises
# [VDN-summary] "어떻게 동작하나"; [VDN-H3-writeup] hybrid attention structure
# ----------------------------------------------------------------------------


def num_chunks(T: int, C: int) -> int:
    """Number of VAE temporal chunks of C latent frames (last one may be short, R6)."""
    return -(-T // C)


def anchors(T: int) -> set:
    """The two boundary anchor frames: the first and the last latent frame."""
    return {0, T - 1}


def window_frames(t: int, T: int, C: int) -> set:
    """Frames inside the sliding softmax window of query frame t.

    The query's chunk attends to itself and the chunks immediately before and
    after it ([VDN-summary] "어떻게 동작하나"), clipped at the clip edges (R5).
    """
    nc = num_chunks(T, C)
    c = t // C
    lo = max(0, c - 1) * C
    hi = min(nc - 1, c + 1) * C + C - 1
    return set(range(lo, min(hi, T - 1) + 1))


def coverage(t: int, T: int, C: int):
    """(forward frames, reverse frames) summarised by the linear states of query t.

    The forward state covers the frames before the softmax window, the
    reverse state the frames after it; neither covers the anchors, which the
    softmax branch already sees in full ([VDN-summary] "전제와 한계": anchors
    are excluded from the linear state).  Anchor queries get empty coverage
    (R1).  Returned as sorted lists in absorption order: forward ascending,
    reverse descending.
    """
    A = anchors(T)
    if t in A:
        return [], []
    W = window_frames(t, T, C)
    lo, hi = min(W), max(W)
    fwd = [s for s in range(0, lo) if s not in A]
    rev = [s for s in range(T - 1, hi, -1) if s not in A]
    return fwd, rev


# ----------------------------------------------------------------------------
# O0: prep ([VDN-summary] "무엇과 다른가": separable short conv on K and V, then
# SiLU; L2 normalisation on Q and K; readings R7, R8)
# ----------------------------------------------------------------------------


def _silu(x):
    return x / (1.0 + np.exp(-x))


def _l2_normalise(x, eps):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _depthwise_conv(x, w_s, w_t, grid_h, grid_w):
    """Zero-padded 5x5 spatial then 5-tap temporal cross-correlation, per channel.

    x: [T, U, C] with U = grid_h * grid_w in row-major (y, x) order.
    w_s: [C, 5, 5], w_t: [C, 5].
    """
    T, U, Cc = x.shape
    g = x.reshape(T, grid_h, grid_w, Cc)
    pad = np.zeros((T + 4, grid_h + 4, grid_w + 4, Cc))
    pad[2:-2, 2:-2, 2:-2, :] = g
    x1 = np.zeros((T + 4, grid_h, grid_w, Cc))
    for a in range(5):          # spatial row offset a-2
        for c in range(5):      # spatial column offset c-2
            x1 += w_s[:, a, c] * pad[:, a:a + grid_h, c:c + grid_w, :]
    # rows 0,1 and T+2,T+3 of x1 are the zero temporal padding
    x2 = np.zeros((T, grid_h, grid_w, Cc))
    for tau in range(5):        # temporal offset tau-2
        x2 += w_t[:, tau] * x1[tau:tau + T]
    return x2.reshape(T, U, Cc)


def prep(q, k, v, wk_s, wk_t, wv_s, wv_t, grid_h, grid_w, l2_eps=1e-6):
    """Prepared features (Q^, K^, V^) of one batch element.

    q, k, v: [T, U, H, d] float64.  Conv weights are indexed by channel
    h*d + j: wk_s [H*d_k, 5, 5], wk_t [H*d_k, 5], likewise for V.
    K^ = L2(SiLU(conv(K))), V^ = SiLU(conv(V)), Q^ = L2(Q).
    """
    T, U, H, dk = k.shape
    dv = v.shape[-1]
    kc = _depthwise_conv(k.reshape(T, U, H * dk), wk_s, wk_t, grid_h, grid_w)
    vc = _depthwise_conv(v.reshape(T, U, H * dv), wv_s, wv_t, grid_h, grid_w)
    k_hat = _l2_normalise(_silu(kc).reshape(T, U, H, dk), l2_eps)
    v_hat = _silu(vc).reshape(T, U, H, dv)
    q_hat = _l2_normalise(q, l2_eps)
    return q_hat, k_hat, v_hat


# ----------------------------------------------------------------------------
# O1-O3: frame statistics, transition, the frame update
# [VDN-summary] "어떻게 쓰나"
# ----------------------------------------------------------------------------


def frame_stats(k_t, v_t, beta_t):
    """A_t = K_t^T Diag(beta_t) K_t (key correlation), B_t = V_t^T Diag(beta_t) K_t.

    k_t: [U, d_k], v_t: [U, d_v], beta_t: [U].
    """
    A = k_t.T @ (beta_t[:, None] * k_t)
    B = v_t.T @ (beta_t[:, None] * k_t)
    return A, B


def transition(A, B, alpha):
    """M_t = Diag(alpha_t) (I + A_t)^{-1}, J_t = B_t (I + A_t)^{-1}, and (I + A_t)^{-1}.

    These are the per-frame transition and injection terms that make the frame
    update affine in the previous state: S_t = S_{t-1} M_t + J_t.  Solved by
    LU (numpy.linalg.solve); P = I + A_t is symmetric, so X P^{-1} = solve(P, X^T)^T.
    """
    d = A.shape[0]
    P = np.eye(d) + A
    Pinv = np.linalg.solve(P, np.eye(d))
    M = np.linalg.solve(P, np.diag(alpha)).T
    J = np.linalg.solve(P, B.T).T
    return M, J, Pinv


def frame_update(S_prev, A, B, alpha):
    """The frame objective's minimiser, S_t = (S_prev Diag(alpha_t) + B_t)(I + A_t)^{-1}.

    argmin_S 1/2||S - Sbar||_F^2 + 1/2 sum_u beta_u ||S k_u - v_u||^2 with
    Sbar = S_prev Diag(alpha_t); its normal equation is S (I + A_t) = Sbar + B_t.
    """
    d = A.shape[0]
    Sbar = S_prev * alpha[None, :]
    return np.linalg.solve(np.eye(d) + A, (Sbar + B).T).T


def text_state(k_txt, v_txt, beta_txt):
    """S_T: all text tokens summarised into one state before the video scan (R4).

    k_txt: [L, d_k], v_txt: [L, d_v], beta_txt: [L].  The text is a leading
    virtual frame updated from a zero state.  L = 0 gives S_T = 0.
    """
    dk = k_txt.shape[-1]
    dv = v_txt.shape[-1]
    if k_txt.shape[0] == 0:
        return np.zeros((dv, dk))
    A, B = frame_stats(k_txt, v_txt, beta_txt)
    return frame_update(np.zeros((dv, dk)), A, B, np.ones(dk))


# ----------------------------------------------------------------------------
# O5: the bidirectional scan
# ----------------------------------------------------------------------------


def scan_states(M, J, S_T, T, C):
    """Chunk-boundary states of the two directions.

    Each direction starts from S_T / 2 so that the two readouts together count
    the prompt once ([VDN-summary] "어떻게 동작하나").  Forward absorbs frames
    1, 2, ..., T-2 (frame 0 is an anchor) with S <- S M_s + J_s; F[j] is the
    state after the last absorbed frame of chunk j.  Reverse absorbs T-2, T-3,
    ..., 1 (R3); R[j] is the state after the first absorbed frame of chunk j.
    A chunk with no absorbed frame leaves the state where the scan has got to.

    M, J: [T, d, d] (entries for the anchors are unused).
    Returns F, R: [n_c, d_v, d_k].
    """
    nc = num_chunks(T, C)
    half = S_T / 2.0
    # prefix states: fwd[s] = state after absorbing frames 1..s (fwd[0] = S_T/2)
    fwd = [half]
    for s in range(1, T - 1):
        fwd.append(fwd[-1] @ M[s] + J[s])
    # suffix states: rev[s] = state after absorbing frames T-2..s (rev[T-1] = S_T/2)
    rev = {T - 1: half}
    for s in range(T - 2, 0, -1):
        rev[s] = rev[s + 1] @ M[s] + J[s]
    F = np.zeros((nc,) + S_T.shape)
    R = np.zeros((nc,) + S_T.shape)
    for j in range(nc):
        last = min(C * (j + 1) - 1, T - 2)
        F[j] = fwd[max(last, 0)] if T >= 2 else half
        first = max(C * j, 1)
        R[j] = rev[first] if first <= T - 1 else half
    return F, R


def bridge_decay(alpha, frames):
    """Per key channel, the product of alpha over ``frames``: absorbing those
    frames with zero writes (beta = 0, so A = 0 and B = 0) turns the frame
    update S <- (S Diag(alpha_s) + B_s)(I + A_s)^{-1} into S <- S Diag(alpha_s)."""
    d = np.ones(alpha.shape[-1])
    for s in frames:
        d = d * alpha[s]
    return d


def query_states(F, R, S_T, t, T, C, bridge_alpha=None):
    """(S_fwd, S_rev) read by query frame t.

    Forward: the state that has absorbed every non-anchor frame before the
    query's window, F[c-2]; reverse: every non-anchor frame after it, R[c+2];
    S_T / 2 where the range is empty.  Anchors read S_T / 2 twice (R1).

    With ``bridge_alpha`` (alpha [T, d_k]) the VDA-Gather decay bridge
    ([VDN-summary] "전제와 한계": VDA-Gather applies a decay bridge, not defined
    further) is applied, read as: the frames between the summarised range and
    the query chunk -- all of chunk c-1 forward, all of chunk c+1 in reverse,
    anchor frames included -- are absorbed with zero writes, S <- S Diag(alpha_s).
    Anchor queries are unchanged.
    """
    nc = num_chunks(T, C)
    half = S_T / 2.0
    if t in anchors(T):
        return half, half
    c = t // C
    sf = F[c - 2] if c >= 2 else half
    sr = R[c + 2] if c + 2 <= nc - 1 else half
    if bridge_alpha is not None:
        if c >= 1:
            sf = sf * bridge_decay(bridge_alpha, range(C * (c - 1), C * c))[None, :]
        if c + 1 <= nc - 1:
            sr = sr * bridge_decay(bridge_alpha, range(C * (c + 1), min(C * (c + 2), T)))[None, :]
    return sf, sr


def readout(q_t, S_fwd, S_rev):
    """o_t = S_fwd q_t + S_rev q_t for every token of the frame; q_t: [U, d_k] -> [U, d_v]."""
    return q_t @ S_fwd.T + q_t @ S_rev.T


def epilogue(o, g, gamma=None, eps=1e-6):
    """RMSNorm over d_v, then the elementwise sigmoid output gate (R9).

    [VDN-summary] "무엇과 다른가": the linear readout passes RMS normalisation
    and its own sigmoid output gate.  o, g: [..., d_v].
    """
    y = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    if gamma is not None:
        y = y * gamma
    return y / (1.0 + np.exp(-g))


# ----------------------------------------------------------------------------
# the whole forward pass
# ----------------------------------------------------------------------------


def forward_head(q, k, v, alpha, beta, k_txt, v_txt, beta_txt, chunk=5,
                 frames=None, bridge=False):
    """States and raw readout of one (batch element, head).

    q, k: [T, U, d_k]; v: [T, U, d_v]; alpha: [T, d_k]; beta: [T, U];
    k_txt: [L, d_k]; v_txt: [L, d_v]; beta_txt: [L].
    ``frames`` limits which query frames get a readout (all by default);
    the states always use every frame.  ``bridge`` applies the decay bridge
    (query_states).
    Returns a dict with S_T, A, B, Pinv, M, J, F, R and o ([T, U, d_v],
    zero rows for frames not read out).
    """
    T, U, dk = k.shape
    dv = v.shape[-1]
    S_T = text_state(k_txt, v_txt, beta_txt)
    A = np.zeros((T, dk, dk))
    Bw = np.zeros((T, dv, dk))
    M = np.zeros((T, dk, dk))
    J = np.zeros((T, dv, dk))
    Pinv = np.zeros((T, dk, dk))
    for t in range(T):
        A[t], Bw[t] = frame_stats(k[t], v[t], beta[t])
        M[t], J[t], Pinv[t] = transition(A[t], Bw[t], alpha[t])
    F, R = scan_states(M, J, S_T, T, chunk)
    o = np.zeros((T, U, dv))
    for t in (range(T) if frames is None else frames):
        sf, sr = query_states(F, R, S_T, t, T, chunk, alpha if bridge else None)
        o[t] = readout(q[t], sf, sr)
    return dict(S_T=S_T, A=A, B=Bw, Pinv=Pinv, M=M, J=J, F=F, R=R, o=o)


def forward(q, k, v, alpha, beta, k_txt, v_txt, beta_txt, gate=None,
            rms_weight=None, chunk=5, rms_eps=1e-6, heads=None, bridge=False):
    """VDA forward over all batch elements and heads (or the listed heads).

    Layouts as the boundary takes them: q, k, v, gate [B, T, U, H, d];
    alpha [B, T, H, d_k]; beta [B, T, U, H]; k_txt, v_txt [B, L, H, d];
    beta_txt [B, L, H].  All float64.  Returns a dict with the per-head
    intermediates stacked as [B, H, ...], the raw readout ``o`` and, when a
    gate is given, the epilogue output ``y`` (both [B, T, U, H, d_v]; heads
    not computed are zero).  ``bridge`` applies the decay bridge.
    """
    Bn, T, U, H, dk = k.shape
    dv = v.shape[-1]
    hs = list(range(H)) if heads is None else list(heads)
    o = np.zeros((Bn, T, U, H, dv))
    inter = {}
    for b in range(Bn):
        for h in hs:
            r = forward_head(q[b, :, :, h], k[b, :, :, h], v[b, :, :, h],
                             alpha[b, :, h], beta[b, :, :, h],
                             k_txt[b, :, h], v_txt[b, :, h], beta_txt[b, :, h],
                             chunk=chunk, bridge=bridge)
            o[b, :, :, h] = r.pop("o")
            for name, val in r.items():
                inter.setdefault(name, np.zeros((Bn, H) + val.shape))[b, h] = val
    out = dict(inter)
    out["o"] = o
    if gate is not None:
        out["y"] = epilogue(o, gate, rms_weight, rms_eps)
    return out


# ----------------------------------------------------------------------------
# comparators printed on the pages (used by the pins, not by forward)
# ----------------------------------------------------------------------------


def token_delta_step(S_prev, k, v, alpha, beta):
    """The token-level gated delta rule: Sbar = S Diag(alpha); S = Sbar + beta (v - Sbar k) k^T."""
    Sbar = S_prev * alpha[None, :]
    return Sbar + beta * np.outer(v - Sbar @ k, k)


def batch_form_step(S_prev, A, B, alpha):
    """The batch form with every residual at the same Sbar: S = Sbar (I - A) + B."""
    Sbar = S_prev * alpha[None, :]
    return Sbar @ (np.eye(A.shape[0]) - A) + B
