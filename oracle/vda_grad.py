"""Gradients of the VDA forward (its backward pass), float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages define the forward only; training through it ([VDN-summary]
"전제와 한계" and the staged adaptation in "어떻게 쓰나" train the linear
branch) needs its derivative.  The plain definition of that derivative is the
chain rule applied to the forward's own steps, so this module transcribes the
forward of ``vda.py`` literally into torch CPU float64 operations (same steps,
same order, same readings R1-R10: frame statistics, the transition by a
linear solve, the two scans from S_T / 2, the query states with or without the
decay bridge, the readout and the epilogue) and lets reverse-mode automatic
differentiation apply the chain rule.  Nothing here is blocked, fused or
reordered.  The transcription is pinned to ``vda.py`` value for value and its
gradients to central finite differences of ``vda.py`` (tests/test_oracle_grad.py).

Besides the input gradients it returns the adjoints of the intermediates a
staged backward produces: do (readout), dS_q (per frame, the gradient of the
state its queries read: forward and reverse state summed), dF, dR, dS_T, dA,
dB and dPinv per frame.
"""

from __future__ import annotations

import numpy as np
import torch

from . import vda


def _t(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def _keep(x):
    """x as a graph node whose adjoint is kept after backward: x + 0, with the
    zero a leaf that requires grad, so the adjoint exists even where x itself
    depends on no input (S_T = 0 without text, and the states read from it)."""
    if not torch.is_grad_enabled():
        return x
    y = x + torch.zeros_like(x, requires_grad=True)
    y.retain_grad()
    return y


def forward_head_t(q, k, v, alpha, beta, k_txt, v_txt, beta_txt, gate=None, gamma=None,
                   chunk=5, rms_eps=1e-6, bridge=False, keep=None, query_l2=None):
    """``vda.forward_head`` followed by ``vda.epilogue``, in torch ops.

    Same shapes as ``vda.forward_head``; gate [T, U, d_v] (None: return o only),
    gamma [d_v] or None.  ``keep`` (a dict) receives the intermediate tensors
    with ``retain_grad`` set, for reading their adjoints after ``backward``.
    ``query_l2`` (an epsilon, or None) takes q raw and normalises each token
    first, q / sqrt(sum q^2 + eps) (reading R8, the forward's fused query
    normalisation).
    """
    if query_l2 is not None:
        q = q / torch.sqrt(torch.sum(q * q, dim=-1, keepdim=True) + query_l2)
    T, U, dk = k.shape
    dv = v.shape[-1]
    C = chunk
    nc = vda.num_chunks(T, C)
    keep = {} if keep is None else keep
    eye = torch.eye(dk, dtype=torch.float64)

    # text state (R4): the frame update from a zero state over the text tokens
    if k_txt.shape[0] == 0:
        S_T = torch.zeros((dv, dk), dtype=torch.float64)
        A_T = B_T = None
    else:
        A_T = _keep(k_txt.T @ (beta_txt[:, None] * k_txt))
        B_T = _keep(v_txt.T @ (beta_txt[:, None] * k_txt))
        S_T = torch.linalg.solve(eye + A_T, B_T.T).T
    keep["A_T"], keep["B_T"] = A_T, B_T
    S_T = _keep(S_T)
    keep["S_T"] = S_T

    # frame statistics and transitions ("어떻게 쓰나")
    A, Bw, Pinv, M, J = [], [], [], [], []
    for t in range(T):
        A_t = k[t].T @ (beta[t][:, None] * k[t])
        B_t = v[t].T @ (beta[t][:, None] * k[t])
        A_t = _keep(A_t)
        B_t = _keep(B_t)
        P = eye + A_t
        Pi = torch.linalg.solve(P, eye)
        Pi = _keep(Pi)
        A.append(A_t)
        Bw.append(B_t)
        Pinv.append(Pi)
        M.append(alpha[t][:, None] * Pi)       # Diag(alpha_t) (I + A_t)^{-1}
        J.append(B_t @ Pi)                      # B_t (I + A_t)^{-1}
    keep["A"], keep["B"], keep["Pinv"] = A, Bw, Pinv

    # the two scans from S_T / 2 (O5; R3)
    half = S_T / 2.0
    fwd = [half]
    for s in range(1, T - 1):
        fwd.append(_keep(fwd[-1] @ M[s] + J[s]))
    rev = {T - 1: half}
    for s in range(T - 2, 0, -1):
        rev[s] = _keep(rev[s + 1] @ M[s] + J[s])
    keep["fwd"], keep["rev"] = fwd, rev
    F, R = [], []
    for j in range(nc):
        last = min(C * (j + 1) - 1, T - 2)
        Fj = fwd[max(last, 0)] if T >= 2 else half
        first = max(C * j, 1)
        Rj = rev[first] if first <= T - 1 else half
        # a fresh node per record, so each record's adjoint is its own
        Fj = _keep(Fj)
        Rj = _keep(Rj)
        F.append(Fj)
        R.append(Rj)
    keep["F"], keep["R"] = F, R

    # query states (O4; R1, R2 and the bridge option) and the readout (E7)
    anchors = vda.anchors(T)
    o_frames, Sq = [], []
    for t in range(T):
        if t in anchors:
            sf, sr = half, half
        else:
            c = t // C
            sf = F[c - 2] if c >= 2 else half
            sr = R[c + 2] if c + 2 <= nc - 1 else half
            if bridge:
                if c >= 1:
                    df = torch.ones(dk, dtype=torch.float64)
                    for s in range(C * (c - 1), C * c):
                        df = df * alpha[s]
                    sf = sf * df[None, :]
                if c + 1 <= nc - 1:
                    dr = torch.ones(dk, dtype=torch.float64)
                    for s in range(C * (c + 1), min(C * (c + 2), T)):
                        dr = dr * alpha[s]
                    sr = sr * dr[None, :]
        S_q = sf + sr
        S_q = _keep(S_q)
        Sq.append(S_q)
        o_frames.append(q[t] @ S_q.T)
    keep["S_q"] = Sq
    o = torch.stack(o_frames)
    o = _keep(o)
    keep["o"] = o
    if gate is None:
        return o
    # epilogue (R9): RMSNorm over d_v, optional gain, elementwise sigmoid gate
    y = o / torch.sqrt(torch.mean(o * o, dim=-1, keepdim=True) + rms_eps)
    if gamma is not None:
        y = y * gamma
    return y / (1.0 + torch.exp(-gate))


def backward_head(q, k, v, alpha, beta, k_txt, v_txt, beta_txt, dy, gate=None, gamma=None,
                  chunk=5, rms_eps=1e-6, bridge=False, query_l2=None):
    """Gradients of sum(dy * y) (or sum(dy * o) without a gate) for one head.

    Inputs as ``forward_head_t`` (numpy float64); dy has the output's shape.
    Returns numpy float64 arrays: dq, dk, dv, dalpha, dbeta, dk_txt, dv_txt,
    dbeta_txt, dgate (None without a gate), dgamma (None without gamma), and
    the intermediate adjoints do [T, U, d_v], dS_q [T, d_v, d_k], dF, dR
    [n_c, d_v, d_k], dS_T, dA, dB, dPinv [T, ...].
    """
    names = ["q", "k", "v", "alpha", "beta", "k_txt", "v_txt", "beta_txt"]
    xs = {n: _t(a).requires_grad_(True) for n, a in zip(names, (q, k, v, alpha, beta, k_txt, v_txt, beta_txt))}
    g = None if gate is None else _t(gate).requires_grad_(True)
    gm = None if gamma is None else _t(gamma).requires_grad_(True)
    keep = {}
    out = forward_head_t(xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], xs["k_txt"], xs["v_txt"],
                         xs["beta_txt"], g, gm, chunk=chunk, rms_eps=rms_eps, bridge=bridge, keep=keep,
                         query_l2=query_l2)
    (out * _t(dy)).sum().backward()

    def grad_of(x, shape):
        return np.zeros(shape) if x.grad is None else x.grad.detach().numpy().copy()

    res = {"d" + n: grad_of(x, x.shape) for n, x in xs.items()}
    res["dgate"] = None if g is None else grad_of(g, g.shape)
    res["dgamma"] = None if gm is None else grad_of(gm, gm.shape)
    res["do"] = grad_of(keep["o"], keep["o"].shape)
    res["dS_T"] = grad_of(keep["S_T"], keep["S_T"].shape)
    for name in ("S_q", "F", "R", "A", "B", "Pinv"):
        res["d" + name] = np.stack([grad_of(x, x.shape) for x in keep[name]])
    # adjoints of the scan states after each absorbed frame (zero elsewhere)
    # and of the text statistics
    T, dv, dk = len(keep["A"]), keep["S_T"].shape[0], keep["S_T"].shape[1]
    res["dfwd"] = np.zeros((T, dv, dk))
    res["drev"] = np.zeros((T, dv, dk))
    for s in range(1, T - 1):
        res["dfwd"][s] = grad_of(keep["fwd"][s], (dv, dk))
        res["drev"][s] = grad_of(keep["rev"][s], (dv, dk))
    res["dA_T"] = np.zeros((dk, dk)) if keep["A_T"] is None else grad_of(keep["A_T"], (dk, dk))
    res["dB_T"] = np.zeros((dv, dk)) if keep["B_T"] is None else grad_of(keep["B_T"], (dv, dk))
    return res


def backward(q, k, v, alpha, beta, k_txt, v_txt, beta_txt, dy, gate=None, rms_weight=None,
             chunk=5, rms_eps=1e-6, heads=None, bridge=False, query_l2=None):
    """``backward_head`` over every batch element and head (or the listed heads).

    Layouts as ``vda.forward``.  Returns the input gradients in the input
    layouts (heads not computed are zero) and the intermediate adjoints stacked
    as [B, H, ...].  dgamma, shared by all heads, is summed over the heads
    computed.
    """
    Bn, T, U, H, dk = k.shape
    hs = list(range(H)) if heads is None else list(heads)
    out = {n: np.zeros_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha),
                                           ("dbeta", beta), ("dk_txt", k_txt), ("dv_txt", v_txt),
                                           ("dbeta_txt", beta_txt))}
    out["dgate"] = None if gate is None else np.zeros_like(gate)
    out["dgamma"] = None if rms_weight is None else np.zeros_like(rms_weight)
    inter = {}
    for b in range(Bn):
        for h in hs:
            r = backward_head(q[b, :, :, h], k[b, :, :, h], v[b, :, :, h], alpha[b, :, h], beta[b, :, :, h],
                              k_txt[b, :, h], v_txt[b, :, h], beta_txt[b, :, h], dy[b, :, :, h],
                              None if gate is None else gate[b, :, :, h], rms_weight, chunk=chunk,
                              rms_eps=rms_eps, bridge=bridge, query_l2=query_l2)
            out["dq"][b, :, :, h] = r["dq"]
            out["dk"][b, :, :, h] = r["dk"]
            out["dv"][b, :, :, h] = r["dv"]
            out["dalpha"][b, :, h] = r["dalpha"]
            out["dbeta"][b, :, :, h] = r["dbeta"]
            out["dk_txt"][b, :, h] = r["dk_txt"]
            out["dv_txt"][b, :, h] = r["dv_txt"]
            out["dbeta_txt"][b, :, h] = r["dbeta_txt"]
            if gate is not None:
                out["dgate"][b, :, :, h] = r["dgate"]
            if rms_weight is not None:
                out["dgamma"] += r["dgamma"]
            for name in ("do", "dS_q", "dF", "dR", "dS_T", "dA", "dB", "dPinv", "dfwd", "drev", "dA_T", "dB_T"):
                inter.setdefault(name, np.zeros((Bn, H) + r[name].shape))[b, h] = r[name]
    out.update(inter)
    return out
