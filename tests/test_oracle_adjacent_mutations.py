"""Plant plausible mistakes in the adjacent maps' oracle (oracle/vda_adjacent.py,
on the CPU) and check that one of its pins (tests/test_oracle_adjacent.py)
fails for each.  A pin set that passes a wrong oracle pins nothing."""

import numpy as np
import pytest

import oracle.vda_adjacent as A
import test_oracle_adjacent as PINS

_gate_proj, _out_proj = A.gate_proj, A.out_proj


def _pins():
    checks = [PINS.test_a1_loops, PINS.test_a2_one_hot_and_zero_weights, PINS.test_a3_token_order_within_a_frame,
              lambda: PINS.test_a4_merge_linear_and_pass_through(0.0),
              lambda: PINS.test_a4_merge_linear_and_pass_through(2.5)]
    failed = 0
    for c in checks:
        try:
            c()
        except AssertionError:  # a pin fails; any other exception is a broken mutant
            failed += 1
    return failed


def _sum_not_mean(x, w_g, w_beta, w_alpha, H, d):
    g, beta, _ = _gate_proj(x, w_g, w_beta, w_alpha, H, d)
    alpha = A.sigmoid(x.sum(axis=2) @ w_alpha.T).reshape(x.shape[0], x.shape[1], H, d)
    return g, beta, alpha


def _beta_no_sigmoid(x, w_g, w_beta, w_alpha, H, d):
    g, _, alpha = _gate_proj(x, w_g, w_beta, w_alpha, H, d)
    return g, x @ w_beta.T, alpha


def _gate_sigmoid(x, w_g, w_beta, w_alpha, H, d):
    g, beta, alpha = _gate_proj(x, w_g, w_beta, w_alpha, H, d)
    return A.sigmoid(g), beta, alpha


def _head_channel_swapped(x, w_g, w_beta, w_alpha, H, d):
    g, beta, alpha = _gate_proj(x, w_g, w_beta, w_alpha, H, d)
    B, T, U = x.shape[:3]
    g2 = (x @ w_g.T).reshape(B, T, U, d, H).swapaxes(-1, -2)
    return g2, beta, alpha


def _alpha_first_token(x, w_g, w_beta, w_alpha, H, d):
    g, beta, _ = _gate_proj(x, w_g, w_beta, w_alpha, H, d)
    alpha = A.sigmoid(x[:, :, 0] @ w_alpha.T).reshape(x.shape[0], x.shape[1], H, d)
    return g, beta, alpha


def _alpha_whole_clip_mean(x, w_g, w_beta, w_alpha, H, d):
    g, beta, _ = _gate_proj(x, w_g, w_beta, w_alpha, H, d)
    xbar = np.broadcast_to(x.mean(axis=(1, 2))[:, None], x.shape[:2] + x.shape[3:])
    alpha = A.sigmoid(xbar @ w_alpha.T).reshape(x.shape[0], x.shape[1], H, d)
    return g, beta, alpha


def _merge_drops_y_in(o, w_o, y_in=None):
    return _out_proj(o, w_o, None)


def _merge_transposed_o(o, w_o, y_in=None):
    B, T, U, H, d = o.shape
    y = o.swapaxes(-1, -2).reshape(B, T, U, H * d) @ w_o.T
    return y if y_in is None else y_in + y


MUTANTS = {
    "alpha from the frame's token sum": ("gate_proj", _sum_not_mean),
    "beta without its sigmoid": ("gate_proj", _beta_no_sigmoid),
    "sigmoid applied to the gate logits": ("gate_proj", _gate_sigmoid),
    "heads and channels swapped in the gate layout": ("gate_proj", _head_channel_swapped),
    "alpha from the frame's first token": ("gate_proj", _alpha_first_token),
    "alpha from the whole clip's mean": ("gate_proj", _alpha_whole_clip_mean),
    "merge drops Y_in": ("out_proj", _merge_drops_y_in),
    "merge reads O with heads and channels swapped": ("out_proj", _merge_transposed_o),
}


def test_pins_pass_on_the_oracle():
    assert _pins() == 0


@pytest.mark.parametrize("name", list(MUTANTS))
def test_each_mutant_fails_a_pin(name, monkeypatch):
    fn, mutant = MUTANTS[name]
    monkeypatch.setattr(A, fn, mutant)
    assert _pins() >= 1, name
