"""Pins of the adjacent linear maps' oracle (oracle/vda_adjacent.py).

* A1 pure-Python loops (no array library) on a tiny case give the same gate
  logits, write gate, decay gate and branch merge: catches a transposed weight,
  a head/channel order swapped in the reshape, a sum for the frame mean, a
  missing sigmoid, the decay gate read per token.
* A2 one-hot weights select input channels exactly; zero weights give 1/2.
* A3 permuting the tokens of a frame permutes g and beta and leaves alpha
  unchanged (the frame mean is order-free).
* A4 the merge is linear in O and passes Y_in through when W_O = 0.
"""

import math

import numpy as np
import pytest

from oracle import vda_adjacent as adj

B, T, U, H, D, DM = 2, 3, 4, 2, 3, 5   # D != DM and H * D != DM: a transposition cannot hide


def _inputs(seed=0):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((B, T, U, DM)), w_g=rng.standard_normal((H * D, DM)),
                w_beta=rng.standard_normal((H, DM)), w_alpha=rng.standard_normal((H * D, DM)),
                o=rng.standard_normal((B, T, U, H, D)), w_o=rng.standard_normal((DM, H * D)),
                y_in=rng.standard_normal((B, T, U, DM)))


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def test_a1_loops():
    p = _inputs()
    x = p["x"].tolist()
    g, beta, alpha = adj.gate_proj(p["x"], p["w_g"], p["w_beta"], p["w_alpha"], H, D)
    y = adj.out_proj(p["o"], p["w_o"], p["y_in"])
    for b in range(B):
        for t in range(T):
            xbar = [sum(x[b][t][u][k] for u in range(U)) / U for k in range(DM)]
            for h in range(H):
                for e in range(D):
                    want = _sig(sum(p["w_alpha"][h * D + e][k] * xbar[k] for k in range(DM)))
                    assert abs(alpha[b, t, h, e] - want) <= 1e-12
            for u in range(U):
                for h in range(H):
                    want = _sig(sum(p["w_beta"][h][k] * x[b][t][u][k] for k in range(DM)))
                    assert abs(beta[b, t, u, h] - want) <= 1e-12
                    for e in range(D):
                        want = sum(p["w_g"][h * D + e][k] * x[b][t][u][k] for k in range(DM))
                        assert abs(g[b, t, u, h, e] - want) <= 1e-12
                for n in range(DM):
                    want = p["y_in"][b, t, u, n] + sum(
                        p["o"][b, t, u, h, e] * p["w_o"][n][h * D + e] for h in range(H) for e in range(D))
                    assert abs(y[b, t, u, n] - want) <= 1e-12


def test_a2_one_hot_and_zero_weights():
    p = _inputs(1)
    pick = [(3 * i + 1) % DM for i in range(H * D)]
    w = np.zeros((H * D, DM))
    w[np.arange(H * D), pick] = 1.0
    g, beta, alpha = adj.gate_proj(p["x"], w, np.zeros((H, DM)), w, H, D)
    assert np.array_equal(g.reshape(B, T, U, H * D), p["x"][..., pick])
    assert np.all(beta == 0.5)
    np.testing.assert_allclose(alpha.reshape(B, T, H * D),
                               adj.sigmoid(p["x"].mean(axis=2)[..., pick]), rtol=0, atol=1e-15)


def test_a3_token_order_within_a_frame():
    p = _inputs(2)
    perm = np.array([2, 0, 3, 1])
    g, beta, alpha = adj.gate_proj(p["x"], p["w_g"], p["w_beta"], p["w_alpha"], H, D)
    g2, beta2, alpha2 = adj.gate_proj(p["x"][:, :, perm], p["w_g"], p["w_beta"], p["w_alpha"], H, D)
    np.testing.assert_allclose(g2, g[:, :, perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(beta2, beta[:, :, perm], rtol=0, atol=1e-15)
    np.testing.assert_allclose(alpha2, alpha, rtol=0, atol=1e-15)
    # alpha is one value per frame: changing one frame's tokens leaves the others'
    x3 = p["x"].copy()
    x3[:, 1] += 1.0
    _, _, alpha3 = adj.gate_proj(x3, p["w_g"], p["w_beta"], p["w_alpha"], H, D)
    assert np.array_equal(alpha3[:, [0, 2]], alpha[:, [0, 2]]) and not np.allclose(alpha3[:, 1], alpha[:, 1])


@pytest.mark.parametrize("scale", [0.0, 2.5])
def test_a4_merge_linear_and_pass_through(scale):
    p = _inputs(3)
    y0 = adj.out_proj(p["o"], p["w_o"] * 0.0, p["y_in"])
    assert np.array_equal(y0, p["y_in"])
    a = adj.out_proj(p["o"] * scale, p["w_o"], None)
    b = scale * adj.out_proj(p["o"], p["w_o"], np.zeros_like(p["y_in"]))
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-14)
