"""Pins of the oracle's gradients (oracle/vda_grad.py) to something other than itself.

* G1: its torch transcription of the forward equals vda.py value for value.
* G2: every input gradient matches a central finite difference of the numpy
  forward (vda.py, not the transcription) along a random direction.
* G3: the raw readout is linear in (V, V_text) jointly, so the gradient with
  respect to them does not depend on their values.
* G4: the exposed intermediate adjoints obey the relations a staged backward
  uses (dq = do S_q, dS_q = do^T q, dA = -P^{-1} dP^{-1} P^{-1}, and the text
  state and records split the query adjoints as the coverage rules say).
"""

import numpy as np
import pytest

from oracle import vda
from oracle import vda_grad as vg


def _inputs(seed, T=12, U=3, d=4, L=2, C=3):
    rng = np.random.default_rng(seed)

    def unit(*shape):
        x = rng.standard_normal(shape)
        return x / np.linalg.norm(x, axis=-1, keepdims=True)

    return dict(
        q=unit(T, U, d), k=unit(T, U, d), v=rng.standard_normal((T, U, d)),
        alpha=1.0 / (1.0 + np.exp(-(2.0 + rng.standard_normal((T, d))))),
        beta=1.0 / (1.0 + np.exp(-rng.standard_normal((T, U)))),
        k_txt=unit(L, d), v_txt=rng.standard_normal((L, d)),
        beta_txt=1.0 / (1.0 + np.exp(-rng.standard_normal(L))),
        gate=rng.standard_normal((T, U, d)), gamma=rng.uniform(0.5, 1.5, d),
        dy=rng.standard_normal((T, U, d)), chunk=C)


CASES = {
    "T12_C3": dict(seed=1),
    "T12_C3_query_l2": dict(seed=7, query_l2=True),
    "T12_C3_bridge": dict(seed=2, bridge=True),
    "T7_C2_no_text": dict(seed=3, T=7, C=2, L=0),
    "T11_C5_ragged": dict(seed=4, T=11, C=5, U=2),
    "T3_C1": dict(seed=5, T=3, C=1),
    "T16_C5_bridge": dict(seed=6, T=16, C=5, bridge=True),
}


QL2_EPS = 1e-6


def _case(name):
    kw = dict(CASES[name])
    bridge = kw.pop("bridge", False)
    ql2 = kw.pop("query_l2", False)
    x = _inputs(**kw)
    if ql2:  # raw queries of uneven length, normalised inside the forward
        x["q"] = x["q"] * np.random.default_rng(kw["seed"] + 100).uniform(0.3, 3.0, x["q"].shape[:-1] + (1,))
    x["query_l2"] = QL2_EPS if ql2 else None
    return x, bridge


def _numpy_out(x, bridge, gate=True, gamma=True):
    q = x["q"]
    if x.get("query_l2") is not None:  # the forward's fused query normalisation (R8), in numpy
        q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + x["query_l2"])
    r = vda.forward_head(q, x["k"], x["v"], x["alpha"], x["beta"], x["k_txt"], x["v_txt"],
                         x["beta_txt"], chunk=x["chunk"], bridge=bridge)
    if not gate:
        return r["o"]
    return vda.epilogue(r["o"], x["gate"], x["gamma"] if gamma else None)


@pytest.mark.parametrize("name", list(CASES))
def test_g1_transcription_matches_numpy(name):
    import torch
    x, bridge = _case(name)
    t = {k: torch.as_tensor(v) for k, v in x.items() if isinstance(v, np.ndarray)}
    with torch.no_grad():
        o = vg.forward_head_t(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["k_txt"], t["v_txt"],
                              t["beta_txt"], chunk=x["chunk"], bridge=bridge, query_l2=x["query_l2"]).numpy()
        y = vg.forward_head_t(t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["k_txt"], t["v_txt"],
                              t["beta_txt"], t["gate"], t["gamma"], chunk=x["chunk"], bridge=bridge,
                              query_l2=x["query_l2"]).numpy()
    o_ref = _numpy_out(x, bridge, gate=False)
    y_ref = _numpy_out(x, bridge)
    assert np.abs(o - o_ref).max() <= 1e-12 * max(1.0, np.abs(o_ref).max())
    assert np.abs(y - y_ref).max() <= 1e-12 * max(1.0, np.abs(y_ref).max())


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "beta": "dbeta", "k_txt": "dk_txt",
           "v_txt": "dv_txt", "beta_txt": "dbeta_txt", "gate": "dgate", "gamma": "dgamma"}


@pytest.mark.parametrize("gate", [True, False])
@pytest.mark.parametrize("name", list(CASES))
def test_g2_gradients_match_finite_differences(name, gate):
    x, bridge = _case(name)
    g = vg.backward_head(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["k_txt"], x["v_txt"], x["beta_txt"],
                         x["dy"], x["gate"] if gate else None, x["gamma"] if gate else None,
                         chunk=x["chunk"], bridge=bridge, query_l2=x["query_l2"])
    rng = np.random.default_rng(99)
    h = 1e-5
    for inp, gname in GRAD_OF.items():
        if not gate and inp in ("gate", "gamma"):
            continue
        if x[inp].size == 0:
            continue
        delta = rng.standard_normal(x[inp].shape)

        def J(sign):
            xp = dict(x)
            xp[inp] = x[inp] + sign * h * delta
            return float(np.sum(x["dy"] * _numpy_out(xp, bridge, gate=gate)))

        fd = (J(1) - J(-1)) / (2 * h)
        an = float(np.sum(g[gname] * delta))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (inp, fd, an)


@pytest.mark.parametrize("name", ["T12_C3", "T12_C3_bridge", "T7_C2_no_text"])
def test_g3_value_gradient_does_not_depend_on_values(name):
    x, bridge = _case(name)
    rng = np.random.default_rng(7)
    res = []
    for trial in range(2):
        v = x["v"] if trial == 0 else rng.standard_normal(x["v"].shape)
        vt = x["v_txt"] if trial == 0 else rng.standard_normal(x["v_txt"].shape)
        g = vg.backward_head(x["q"], x["k"], v, x["alpha"], x["beta"], x["k_txt"], vt, x["beta_txt"],
                             x["dy"], chunk=x["chunk"], bridge=bridge)
        res.append((g["dv"], g["dv_txt"]))
    for a, b in zip(res[0], res[1]):
        if a.size:
            assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(a).max())


@pytest.mark.parametrize("name", list(CASES))
def test_g4_intermediate_adjoints(name):
    x, bridge = _case(name)
    T, C = x["q"].shape[0], x["chunk"]
    nc = vda.num_chunks(T, C)
    g = vg.backward_head(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["k_txt"], x["v_txt"], x["beta_txt"],
                         x["dy"], x["gate"], x["gamma"], chunk=C, bridge=bridge)
    f = vda.forward_head(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["k_txt"], x["v_txt"], x["beta_txt"],
                         chunk=C, bridge=bridge)
    tol = 1e-11
    for t in range(T):
        sf, sr = vda.query_states(f["F"], f["R"], f["S_T"], t, T, C, x["alpha"] if bridge else None)
        # readout: o_t = q_t S_q^T  =>  dq_t = do_t S_q, dS_q = do_t^T q_t
        assert np.abs(g["dq"][t] - g["do"][t] @ (sf + sr)).max() <= tol
        assert np.abs(g["dS_q"][t] - g["do"][t].T @ x["q"][t]).max() <= tol
    # (I + A)^{-1}: dA = -P^{-1} dPinv P^{-1} (A enters only through P)
    for t in range(T):
        P = f["Pinv"][t]
        assert np.abs(g["dA"][t] - (-P @ g["dPinv"][t] @ P)).max() <= tol * max(1.0, np.abs(g["dA"][t]).max())
    if not bridge:
        # records: a query in chunk c reads F_{c-2} and R_{c+2} (R1, O4)
        anchors = vda.anchors(T)
        for j in range(nc):
            zero = np.zeros_like(g["dF"][j])
            want_f = sum((g["dS_q"][t] for t in range(T) if t not in anchors and t // C - 2 == j), zero)
            want_r = sum((g["dS_q"][t] for t in range(T) if t not in anchors and t // C + 2 == j), zero)
            assert np.abs(g["dF"][j] - want_f).max() <= tol
            assert np.abs(g["dR"][j] - want_r).max() <= tol


@pytest.mark.parametrize("name", ["T12_C3", "T11_C5_ragged", "T16_C5_bridge", "T7_C2_no_text"])
def test_g5_scan_adjoint_recurrence(name):
    """The adjoint of the forward scan state after frame s-1 is that after
    frame s times P_s Diag(alpha_s), plus the record adjoint where frame s-1
    ends a chunk (the recurrence the staged backward runs); the reverse scan
    likewise with the frame order reversed."""
    x, bridge = _case(name)
    T, C = x["q"].shape[0], x["chunk"]
    nc = vda.num_chunks(T, C)
    g = vg.backward_head(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["k_txt"], x["v_txt"], x["beta_txt"],
                         x["dy"], x["gate"], x["gamma"], chunk=C, bridge=bridge)
    f = vda.forward_head(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["k_txt"], x["v_txt"], x["beta_txt"],
                         chunk=C, bridge=bridge)
    tol = 1e-10 * max(1.0, np.abs(g["dfwd"]).max(), np.abs(g["drev"]).max())
    for s in range(2, T - 1):
        want = (g["dfwd"][s] @ f["Pinv"][s]) * x["alpha"][s][None, :]
        for j in range(nc):  # F_j is the state after frame min(C(j+1)-1, T-2)
            if min(C * (j + 1) - 1, T - 2) == s - 1:
                want = want + g["dF"][j]
        assert np.abs(g["dfwd"][s - 1] - want).max() <= tol, s
    for s in range(1, T - 2):
        want = (g["drev"][s] @ f["Pinv"][s]) * x["alpha"][s][None, :]
        for j in range(nc):  # R_j is the state after frame max(C j, 1)
            if max(C * j, 1) == s + 1:
                want = want + g["dR"][j]
        assert np.abs(g["drev"][s + 1] - want).max() <= tol, s


def test_one_text_token_leaves_dq_to_rmsnorms_epsilon():
    """With one text token and every frame reading S_T (three frames in one
    chunk: the anchors read S_T, the middle frame S_T / 2 from each side),
    S_T q = v_T (beta / (1 + beta)) (k_T . q) points along one direction for
    every query and RMSNorm removes its length: y depends on q only through
    RMSNorm's epsilon, so dq is proportional to epsilon (and largest for the
    tokens whose k_T . q is tiny).  This is why, in such clips, a bfloat16 dq
    fails a bound relative to its own size.  With three text tokens dq does
    not depend on epsilon."""
    def dq_max(L, eps):
        x = _inputs(seed=11, T=3, U=4, d=8, L=L, C=5)
        r = vg.backward_head(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["k_txt"], x["v_txt"], x["beta_txt"],
                             x["dy"], gate=x["gate"], gamma=x["gamma"], chunk=5, rms_eps=eps)
        return np.abs(r["dq"]).max()

    assert dq_max(1, 1e-9) / dq_max(1, 1e-6) == pytest.approx(1e-3, rel=0.05)
    assert dq_max(1, 1e-12) / dq_max(1, 1e-9) == pytest.approx(1e-3, rel=0.05)
    assert dq_max(3, 1e-9) / dq_max(3, 1e-6) == pytest.approx(1.0, rel=1e-3)
