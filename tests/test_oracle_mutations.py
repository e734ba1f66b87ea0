"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

A pin set that passes a wrong oracle pins nothing; each case here swaps one
oracle function for a subtly wrong version and expects some check to fail.
"""

import numpy as np
import pytest

import oracle.vda as V
import oracle_pins as P

_orig = {name: getattr(V, name) for name in (
    "frame_stats", "transition", "frame_update", "text_state", "scan_states",
    "query_states", "bridge_decay", "coverage", "window_frames", "epilogue", "prep", "readout")}


def _all_checks():
    rng = np.random.default_rng(123)
    checks = [
        lambda: P.check_p1_residual(P.rand_head(rng, T=20)),
        lambda: P.check_p2_lstsq(rng, trials=5),
        lambda: P.check_p3_one_token(rng, trials=5),
        lambda: P.check_p5_text_once(rng),
        lambda: P.check_p5b_bridge_closed_form(rng),
        lambda: P.check_p6_coverage(),
        P.check_golden_coverage,
        P.check_golden_hand_cases,
        lambda: P.check_p7_time_reversal(rng),
        lambda: P.check_p9_composition(rng),
        lambda: P.check_p10_library(rng),
        lambda: P.check_p12_zero(rng),
        lambda: P.check_p13_brute_force(rng),
    ]
    failed = 0
    for c in checks:
        try:
            c()
        except AssertionError:  # a pin fails; any other exception is a broken mutant
            failed += 1
    return failed


def _stats_no_beta(k, v, beta):
    return k.T @ k, v.T @ k


def _stats_sign(k, v, beta):
    A, B = _orig["frame_stats"](k, v, beta)
    return A, -B


def _transition_col_scaled(A, B, alpha):
    M, J, Pinv = _orig["transition"](A, B, alpha)
    return Pinv @ np.diag(alpha), J, Pinv


def _update_no_decay(S_prev, A, B, alpha):
    return _orig["frame_update"](S_prev, A, B, np.ones_like(alpha))


def _text_no_inverse(k, v, beta):
    if k.shape[0] == 0:
        return np.zeros((v.shape[-1], k.shape[-1]))
    return _orig["frame_stats"](k, v, beta)[1]


def _scan_full_text(M, J, S_T, T, C):
    return _orig["scan_states"](M, J, 2 * S_T, T, C)


def _scan_rev_off_by_one(M, J, S_T, T, C):
    F, R = _orig["scan_states"](M, J, S_T, T, C)
    R2 = R.copy()
    R2[:-1] = R[1:]
    return F, R2


def _query_fwd_one_chunk_late(F, R, S_T, t, T, C, bridge_alpha=None):
    sf, sr = _orig["query_states"](F, R, S_T, t, T, C, bridge_alpha)
    c = t // C
    if t not in V.anchors(T) and c >= 1:
        sf = F[c - 1]
    return sf, sr


def _query_bridge_own_chunk(F, R, S_T, t, T, C, bridge_alpha=None):
    sf, sr = _orig["query_states"](F, R, S_T, t, T, C, None)
    if bridge_alpha is not None and t not in V.anchors(T):
        c = t // C
        sf = sf * V.bridge_decay(bridge_alpha, range(C * c, min(C * (c + 1), T)))[None, :]
    return sf, sr


def _bridge_drops_last_frame(alpha, frames):
    return _orig["bridge_decay"](alpha, list(frames)[:-1])


def _window_shifted(t, T, C):
    nc = V.num_chunks(T, C)
    c = min(max(t // C, 1), nc - 2) if nc >= 3 else t // C
    lo, hi = max(0, c - 1) * C, min(T - 1, (c + 1) * C + C - 1)
    return set(range(lo, hi + 1))


def _epilogue_no_sqrt(o, g, gamma=None, eps=1e-6):
    y = o / (np.mean(o * o, axis=-1, keepdims=True) + eps)
    return y / (1 + np.exp(-g))


def _epilogue_gate_sign(o, g, gamma=None, eps=1e-6):
    return _orig["epilogue"](o, -g, gamma, eps)


def _prep_causal(q, k, v, wk_s, wk_t, wv_s, wv_t, gh, gw, l2_eps=1e-6):
    T = k.shape[0]
    sh = lambda x: np.concatenate([np.zeros_like(x[:2]), x[:-2]])  # taps t-4..t
    return _orig["prep"](q, sh(k), sh(v), wk_s, wk_t, wv_s, wv_t, gh, gw, l2_eps)


def _readout_fwd_only(q_t, S_fwd, S_rev):
    return 2 * q_t @ S_fwd.T


MUTANTS = {
    "frame_stats drops beta": ("frame_stats", _stats_no_beta),
    "frame_stats sign of the write": ("frame_stats", _stats_sign),
    "transition scales columns by alpha": ("transition", _transition_col_scaled),
    "frame_update forgets the decay": ("frame_update", _update_no_decay),
    "text_state without the inverse": ("text_state", _text_no_inverse),
    "scan starts from S_T, not S_T/2": ("scan_states", _scan_full_text),
    "reverse boundary state one chunk off": ("scan_states", _scan_rev_off_by_one),
    "forward state one chunk late": ("query_states", _query_fwd_one_chunk_late),
    "bridge decays the query's own chunk": ("query_states", _query_bridge_own_chunk),
    "bridge misses a frame": ("bridge_decay", _bridge_drops_last_frame),
    "window shifted at the clip edges": ("window_frames", _window_shifted),
    "RMSNorm without the square root": ("epilogue", _epilogue_no_sqrt),
    "gate sign flipped": ("epilogue", _epilogue_gate_sign),
    "causal temporal taps": ("prep", _prep_causal),
    "readout reads one direction twice": ("readout", _readout_fwd_only),
}


@pytest.mark.parametrize("label", list(MUTANTS))
def test_pins_catch_planted_mistake(label, monkeypatch):
    name, fn = MUTANTS[label]
    monkeypatch.setattr(V, name, fn)
    assert _all_checks() >= 1, f"no pin caught: {label}"


def test_unmutated_oracle_passes_every_check():
    assert _all_checks() == 0
