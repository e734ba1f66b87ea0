"""Host checks of the block-sweep inverse (solve_sweep<D>, bfloat16 inputs,
d >= 32) through its lane-level model (tests/sweep_model.py):

* the output fragments cover every element of P^{-1} exactly once, in the
  order include/vdn_vda.h states for the split pinv format;
* on frames of the workloads' own synthetic inputs the model's float32 result
  is within 2^-16 of the float64 inverse (the resolution of the hi + lo
  bfloat16 planes the kernel stores);
* on matrices with a geometric spectrum the error grows with the condition
  number, which is why float32 inputs keep the Cholesky kernel (the bounds
  below are the model's measured values with headroom)."""

import numpy as np
import pytest

import sweep_model as SM
from frame_wise_delta_02_amd import synth
from oracle import vda


def _rel(a, b):
    return float(np.abs(a - b).max() / np.abs(b).max())


@pytest.mark.parametrize("d", [32, 64, 128])
def test_fragments_cover_every_element_once(d):
    rng = np.random.default_rng(d)
    K = rng.standard_normal((3 * d, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    A = (K.T * rng.uniform(0, 1, 3 * d)) @ K
    got, count = SM.sweep_inverse(A.astype(np.float32))
    assert (count == 1).all()
    assert np.isfinite(got).all()
    assert _rel(got, np.linalg.inv(np.eye(d) + A)) < 2.0 ** -16


def _frames(name, **kw):
    """A_t of frames 1 and 3 of every head of a small draw of workload `name`
    (the prepared keys for the long clip), as float64."""
    w = synth.WORKLOADS[name].scaled(name="sweep", **kw)
    x = synth.make_inputs(w)
    f = lambda a: synth.to_f64(a, w.dtype)
    k = f(x["k"])[0]
    if w.prep:
        _, kh, _ = vda.prep(f(x["q"])[0], k, f(x["v"])[0], x["wk_s"].astype(np.float64),
                            x["wk_t"].astype(np.float64), x["wv_s"].astype(np.float64),
                            x["wv_t"].astype(np.float64), w.grid_h, w.grid_w)
        k = synth.to_f64(synth._round(kh, w.dtype), w.dtype)
    beta = f(x["beta"])[0]
    for t in (1, 3):
        for h in range(w.H):
            yield (k[t, :, h, :].T * beta[t, :, h]) @ k[t, :, h, :]


@pytest.mark.parametrize("name", ["768p_bf16", "small_bf16", "long_prep_bf16"])
def test_workload_frames_within_split_resolution(name):
    worst = 0.0
    for A in _frames(name, H=2, T=6):
        d = A.shape[0]
        got, _ = SM.sweep_inverse(A.astype(np.float32))
        ref = np.linalg.inv(np.eye(d) + A)
        worst = max(worst, _rel(got, ref))
        # the stored planes: hi + lo of the float32 result
        hi, lo = SM.split_bf16(got)
        assert _rel(hi.astype(np.float64) + lo, ref) < 2.0 ** -16
    assert worst < 2.0 ** -16, worst


@pytest.mark.parametrize("d", [32, 128])
def test_error_grows_with_condition(d):
    """Geometric spectra of I + A: condition 10 and 100 stay within 2^-16;
    700 and 3000 do not stay there (measured 1.3-4.2e-5 and 2.5e-4-1.2e-3)."""
    rng = np.random.default_rng(7 + d)
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    errs = {}
    for cond in (10, 100, 700, 3000):
        A = (Q * (np.geomspace(1, cond, d) - 1)) @ Q.T
        A = (A + A.T) / 2
        got, _ = SM.sweep_inverse(A.astype(np.float32))
        errs[cond] = _rel(got, np.linalg.inv(np.eye(d) + A.astype(np.float32).astype(np.float64)))
    assert errs[10] < 2.0 ** -16 and errs[100] < 2.0 ** -16, errs
    assert errs[700] < 2e-4 and errs[3000] < 1e-2, errs
    assert errs[10] < errs[700] < errs[3000], errs
