"""The oracle against what the pages and the mathematics fix (CPU only)."""

import numpy as np
import pytest

import oracle_pins as P
from frame_wise_delta_02_amd import synth
import oracle


def test_p1_normal_equation_residual():
    rng = np.random.default_rng(1)
    for T in (12, 20, 23):
        P.check_p1_residual(P.rand_head(rng, T=T))
    # the stress workload's key geometry at one head
    w = synth.WORKLOADS["stress_tight_f32"].scaled(H=1, T=12, grid_h=8, grid_w=8, d=32, L=8)
    x = synth.make_inputs(w)
    f = {k: synth.to_f64(v, w.dtype) for k, v in x.items()}
    P.check_p1_residual(dict(q=f["q"][0, :, :, 0], k=f["k"][0, :, :, 0], v=f["v"][0, :, :, 0],
                             alpha=f["alpha"][0, :, 0], beta=f["beta"][0, :, :, 0],
                             k_txt=f["k_text"][0, :, 0], v_txt=f["v_text"][0, :, 0],
                             beta_txt=f["beta_text"][0, :, 0]), tol=1e-11)


def test_p2_bruteforce_least_squares():
    P.check_p2_lstsq(np.random.default_rng(2))


def test_p3_one_token_is_token_delta_rule():
    P.check_p3_one_token(np.random.default_rng(3))


@pytest.mark.parametrize("name", ["stress_f32", "stress_tight_f32", "tiny_f32"])
def test_p4_nonexpansion_on_workloads(name):
    w = synth.WORKLOADS[name]
    x = synth.make_inputs(w)
    k = synth.to_f64(x["k"], w.dtype)
    beta = synth.to_f64(x["beta"], w.dtype)
    alpha = x["alpha"].astype(np.float64)
    for h in range(w.H):
        worst = P.check_p4_nonexpansion(k[0, :, :, h], beta[0, :, :, h], alpha[0, :, h])
        assert worst <= 1.0


def test_p4_nonexpansion_768p_shape():
    w = synth.WORKLOADS["768p_bf16"].scaled(H=1, T=6)
    x = synth.make_inputs(w)
    k = synth.to_f64(x["k"], w.dtype)
    beta = synth.to_f64(x["beta"], w.dtype)
    P.check_p4_nonexpansion(k[0, :, :, 0], beta[0, :, :, 0], x["alpha"][0, :, 0].astype(np.float64))


def test_p5_text_counted_once():
    P.check_p5_text_once(np.random.default_rng(5))


def test_p5b_bridge_closed_form():
    P.check_p5b_bridge_closed_form(np.random.default_rng(15))
    P.check_p5b_bridge_closed_form(np.random.default_rng(16), C=3)


def test_p6_coverage_partition():
    P.check_p6_coverage()
    P.check_p6_coverage(C=3, Ts=(1, 2, 4, 9, 11, 30))


def test_golden_coverage_fixture():
    P.check_golden_coverage()


def test_golden_hand_cases():
    P.check_golden_hand_cases()


def test_p7_time_reversal():
    P.check_p7_time_reversal(np.random.default_rng(7))


def test_p8_linearity():
    P.check_p8_linearity(np.random.default_rng(8))


def test_p9_chunk_and_shard_composition():
    P.check_p9_composition(np.random.default_rng(9))


def test_p10_library_routines():
    P.check_p10_library(np.random.default_rng(10))


def test_p11_small_beta_matches_batch_form():
    P.check_p11_small_beta(np.random.default_rng(11))


def test_p12_zero_writes():
    P.check_p12_zero(np.random.default_rng(12))


def test_p13_bruteforce_states():
    P.check_p13_brute_force(np.random.default_rng(13))


def test_forward_layout_matches_forward_head():
    """The [B, T, U, H, d] driver slices heads and batch elements correctly."""
    rng = np.random.default_rng(14)
    Bn, T, U, H, dk, dv, L = 2, 12, 5, 3, 4, 3, 2
    q = rng.standard_normal((Bn, T, U, H, dk))
    k = rng.standard_normal((Bn, T, U, H, dk))
    v = rng.standard_normal((Bn, T, U, H, dv))
    alpha = rng.uniform(0.3, 1, (Bn, T, H, dk))
    beta = rng.uniform(0, 2, (Bn, T, U, H))
    kt = rng.standard_normal((Bn, L, H, dk))
    vt = rng.standard_normal((Bn, L, H, dv))
    bt = rng.uniform(0, 2, (Bn, L, H))
    g = rng.standard_normal((Bn, T, U, H, dv))
    r = oracle.forward(q, k, v, alpha, beta, kt, vt, bt, gate=g)
    for b in range(Bn):
        for h in range(H):
            x = dict(q=q[b, :, :, h], k=k[b, :, :, h], v=v[b, :, :, h], alpha=alpha[b, :, h],
                     beta=beta[b, :, :, h], k_txt=kt[b, :, h], v_txt=vt[b, :, h], beta_txt=bt[b, :, h])
            rh = P.run_head(x)
            assert np.array_equal(r["o"][b, :, :, h], rh["o"])
            assert np.array_equal(r["F"][b, h], rh["F"])
    assert np.array_equal(r["y"], oracle.epilogue(r["o"], g, None, 1e-6))


def test_bf16_rounding_of_inputs():
    """The input rounding agrees with torch's float64 -> bfloat16 cast (nearest-even)."""
    import torch
    rng = np.random.default_rng(15)
    x = np.concatenate([rng.standard_normal(100000), 1 + np.arange(1, 2000) * 2.0 ** -9,
                        -(1 + np.arange(1, 2000) * 2.0 ** -9), [0.0]])
    ours = synth.f64_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(oracle.widen_bf16_bits(ours), torch.from_numpy(x).to(torch.bfloat16).double().numpy())
