"""Plant plausible mistakes in the gradient oracle's transcription
(oracle/vda_grad.py, on the CPU) and check that a pin of
tests/test_oracle_grad.py fails for each: an input detached somewhere in the
transcription (the forward unchanged, one gradient path lost) must fail the
finite-difference pin G2, a changed forward the transcription pin G1."""

import pytest

import oracle.vda_grad as VG
import test_oracle_grad as PINS

_fwd = VG.forward_head_t


def _detached(name):
    pos = ["q", "k", "v", "alpha", "beta", "k_txt", "v_txt", "beta_txt"].index(name)

    def f(*args, **kw):
        args = list(args)
        args[pos] = args[pos].detach()
        return _fwd(*args, **kw)
    return f


def _gate_detached(*args, **kw):
    args = list(args)
    if len(args) > 8 and args[8] is not None:
        args[8] = args[8].detach()
    elif kw.get("gate") is not None:
        kw["gate"] = kw["gate"].detach()
    return _fwd(*args, **kw)


def _scaled_output(*args, **kw):
    return _fwd(*args, **kw) * (1.0 + 1e-6)


MUTANTS = {f"{n} detached": _detached(n) for n in ("q", "k", "v", "alpha", "beta", "k_txt", "v_txt", "beta_txt")}
MUTANTS["gate detached"] = _gate_detached
MUTANTS["output off by 1e-6"] = _scaled_output


def _pins(case):
    failed = 0
    for check in (lambda: PINS.test_g1_transcription_matches_numpy(case),
                  lambda: PINS.test_g2_gradients_match_finite_differences(case, True),
                  lambda: PINS.test_g2_gradients_match_finite_differences(case, False)):
        try:
            check()
        except AssertionError:
            failed += 1
    return failed


def test_pins_pass_on_the_oracle():
    assert _pins("T12_C3") == 0


@pytest.mark.parametrize("name", list(MUTANTS))
def test_each_mutant_fails_a_pin(name, monkeypatch):
    monkeypatch.setattr(VG, "forward_head_t", MUTANTS[name])
    assert _pins("T12_C3") >= 1, name
