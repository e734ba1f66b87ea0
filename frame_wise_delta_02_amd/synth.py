"""Seeded synthetic inputs for the VDA forward pass.

This module draws inputs only; it holds none of the method's arithmetic and is
shared by the GPU tests, the benchmark and the oracle checks so that both
sides read the very same arrays.

The five workloads stand in for the pages' 768p latent clips (48 x 84 tokens
per latent frame, 5-frame VAE chunks, 128-wide heads); no dataset, prompt set
or trained weight is used.  Big tensors are drawn per (batch, frame) block from
``numpy.random.Generator(PCG64(SeedSequence(seed, spawn_key=(tensor, b, t))))``
as float32 standard normals, transformed in float64 (L2 normalisation,
sigmoid) and rounded once to the workload's dtype with round-to-nearest-even.
Blocks are independent, so the draw is the same for any thread count.

bfloat16 tensors are returned as uint16 bit patterns; float32 tensors as
float32.  alpha is always float32.  Layouts are the boundary's:
q, k, v, gate [B, T, U, H, d]; alpha [B, T, H, d_k]; beta [B, T, U, H];
k_text, v_text [B, L, H, d]; beta_text [B, L, H]; conv weights
[H*d, 5, 5] and [H*d, 5] (float32).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

# tensor ids in the spawn key (fixed: changing them changes every draw)
_ID = dict(q=0, k=1, v=2, beta=3, alpha=4, k_text=5, v_text=6, beta_text=7,
           gate=8, wk_s=9, wk_t=10, wv_s=11, wv_t=12, centres=13,
           x=14, x_frame=15, w_gb=16, w_alpha=17, w_o=18, o=19, y_in=20)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    grid_h: int
    grid_w: int
    d: int
    L: int
    dtype: str                      # "f32" or "bf16"
    alpha_mu: float = 2.0           # alpha = sigmoid(N(alpha_mu, 1)) unless alpha_uniform
    alpha_uniform: tuple = None     # (lo, hi): alpha ~ U(lo, hi)
    beta_scale: float = 1.0         # beta = beta_scale * sigmoid(N(0, 1))
    clusters: int = 0               # > 0: keys drawn around this many unit centres
    cluster_noise_std: float = 0.1
    prep: bool = False              # raw q, k, v + conv weights; prepare() runs first
    conv_std: float = 0.2           # conv weights ~ N(0, conv_std^2)
    chunk: int = 5
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def U(self) -> int:
        return self.grid_h * self.grid_w

    def scaled(self, **kw) -> "Workload":
        """The same distributions at other sizes (for parity cases)."""
        return replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", B=1, H=2, T=20, grid_h=4, grid_w=4, d=16,
                         L=8, dtype="f32", alpha_mu=2.0),
    "small_bf16": Workload("small_bf16", B=1, H=8, T=40, grid_h=30, grid_w=52,
                           d=64, L=64, dtype="bf16", alpha_mu=2.0),
    "768p_bf16": Workload("768p_bf16", B=1, H=24, T=60, grid_h=48, grid_w=84,
                          d=128, L=256, dtype="bf16", alpha_mu=3.0),
    "stress_f32": Workload("stress_f32", B=1, H=4, T=30, grid_h=32, grid_w=32,
                           d=128, L=64, dtype="f32", alpha_uniform=(0.9, 1.0),
                           beta_scale=10.0, clusters=8, cluster_noise_std=0.1),
    "stress_tight_f32": Workload("stress_tight_f32", B=1, H=4, T=30, grid_h=32,
                                 grid_w=32, d=128, L=64, dtype="f32",
                                 alpha_uniform=(0.9, 1.0), beta_scale=10.0,
                                 clusters=8, cluster_noise_std=0.01),
    "long_prep_bf16": Workload("long_prep_bf16", B=1, H=24, T=120, grid_h=48,
                               grid_w=84, d=128, L=512, dtype="bf16",
                               alpha_mu=3.0, prep=True, conv_std=0.2),
    # one GPU's share of the 768p clip when its 24 heads are split over 8 GPUs:
    # the few-heads regime where the serial frame scan dominates
    "768p_share8_bf16": Workload("768p_share8_bf16", B=1, H=3, T=60, grid_h=48,
                                 grid_w=84, d=128, L=256, dtype="bf16", alpha_mu=3.0),
}
# the five workloads in their published order (the stress case twice: two noise readings)
ORDER = ["tiny_f32", "small_bf16", "768p_bf16", "stress_f32", "long_prep_bf16"]


# ----------------------------------------------------------------------------
# rounding
# ----------------------------------------------------------------------------


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 to bfloat16 (nearest, ties to even) in one step; returns uint16 bits.

    Works on the binary64 encoding: keep the top 7 mantissa bits with RNE on
    the dropped 45, then re-bias the exponent.  Inputs here are zero or normal
    numbers well inside bfloat16's range.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    u = x.view(np.uint64)
    sign = ((u >> np.uint64(48)) & np.uint64(0x8000)).astype(np.uint16)
    mag = u & np.uint64(0x7FFFFFFFFFFFFFFF)
    lsb = (mag >> np.uint64(45)) & np.uint64(1)
    r = (mag + lsb + np.uint64((1 << 44) - 1)) >> np.uint64(45)
    exp = (r >> np.uint64(7)).astype(np.int64) - 1023 + 127
    man = (r & np.uint64(0x7F)).astype(np.int64)
    zero = mag == 0
    if np.any(~zero & ((exp < 1) | (exp > 254))):
        raise ValueError("value outside the normal bfloat16 range")
    bits = np.where(zero, 0, (exp << 7) | man).astype(np.uint16)
    return bits | sign


def _round(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f64_to_bf16_bits(x64)
    return x64.astype(np.float32)


def _rng(seed, tensor, b=0, t=0):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(seed, spawn_key=(_ID[tensor], b, t))))


def _normal(g, shape):
    return g.standard_normal(shape, dtype=np.float32).astype(np.float64)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _l2(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _threads(n):
    if n:
        return n
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------
# the draw
# ----------------------------------------------------------------------------


def _centres(w: Workload, b):
    """Per head: `clusters` unit key directions (the stress workload)."""
    g = _rng(w.seed, "centres", b)
    return _l2(_normal(g, (w.H, w.clusters, w.d)))


def _keys(w: Workload, g, n, centres):
    """n x H unit keys: isotropic, or around cluster centres plus Gaussian noise."""
    if w.clusters:
        m = g.integers(0, w.clusters, size=(n, w.H))
        noise = _normal(g, (n, w.H, w.d)) * w.cluster_noise_std
        x = centres[np.arange(w.H)[None, :], m] + noise
    else:
        x = _normal(g, (n, w.H, w.d))
    return _l2(x)


def _beta(w: Workload, g, shape):
    return w.beta_scale * _sigmoid(_normal(g, shape))


def make_inputs(w: Workload, threads: int = 0) -> dict:
    """Draw every input of workload ``w``; see the module docstring for layouts."""
    B, T, U, H, d, L = w.B, w.T, w.U, w.H, w.d, w.L
    big = np.uint16 if w.dtype == "bf16" else np.float32
    out = {
        "q": np.empty((B, T, U, H, d), big),
        "k": np.empty((B, T, U, H, d), big),
        "v": np.empty((B, T, U, H, d), big),
        "gate": np.empty((B, T, U, H, d), big),
        "beta": np.empty((B, T, U, H), big),
        "alpha": np.empty((B, T, H, d), np.float32),
    }
    centres = [_centres(w, b) if w.clusters else None for b in range(B)]

    def frame(bt):
        b, t = bt
        if w.prep:
            q = _normal(_rng(w.seed, "q", b, t), (U, H, d))
            k = _normal(_rng(w.seed, "k", b, t), (U, H, d))
        else:
            q = _l2(_normal(_rng(w.seed, "q", b, t), (U, H, d)))
            k = _keys(w, _rng(w.seed, "k", b, t), U, centres[b])
        out["q"][b, t] = _round(q, w.dtype)
        out["k"][b, t] = _round(k, w.dtype)
        out["v"][b, t] = _round(_normal(_rng(w.seed, "v", b, t), (U, H, d)), w.dtype)
        out["gate"][b, t] = _round(_normal(_rng(w.seed, "gate", b, t), (U, H, d)), w.dtype)
        out["beta"][b, t] = _round(_beta(w, _rng(w.seed, "beta", b, t), (U, H)), w.dtype)
        ga = _rng(w.seed, "alpha", b, t)
        if w.alpha_uniform is not None:
            lo, hi = w.alpha_uniform
            a = lo + (hi - lo) * ga.random((H, d))
        else:
            a = _sigmoid(w.alpha_mu + _normal(ga, (H, d)))
        out["alpha"][b, t] = a.astype(np.float32)

    jobs = [(b, t) for b in range(B) for t in range(T)]
    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(frame, jobs))

    kt = np.empty((B, L, H, d), big)
    vt = np.empty((B, L, H, d), big)
    bt = np.empty((B, L, H), big)
    for b in range(B):
        kt[b] = _round(_keys(w, _rng(w.seed, "k_text", b), L, centres[b]), w.dtype)
        vt[b] = _round(_normal(_rng(w.seed, "v_text", b), (L, H, d)), w.dtype)
        bt[b] = _round(_beta(w, _rng(w.seed, "beta_text", b), (L, H)), w.dtype)
    out.update(k_text=kt, v_text=vt, beta_text=bt)

    if w.prep:
        for name, shape in (("wk_s", (H * d, 5, 5)), ("wk_t", (H * d, 5)),
                            ("wv_s", (H * d, 5, 5)), ("wv_t", (H * d, 5))):
            out[name] = (w.conv_std * _normal(_rng(w.seed, name), shape)).astype(np.float32)
    return out


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a drawn tensor (bfloat16 bits or float32)."""
    if dtype == "bf16" and x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def make_adjacent_inputs(w: Workload, d_model: int, threads: int = 0) -> dict:
    """Inputs of the linear maps either side of the path, bfloat16 bits except
    w_alpha (float32):

    * x [B, T, U, d_model]: a per-frame offset ~ N(0, 1) plus per-token N(0, 1)
      (so the frame means carry a signal for the decay gate);
    * w_gb [H d + H, d_model] ~ N(0, 1 / d_model) (gate rows, then beta rows);
    * w_alpha [H d, d_model] ~ N(0, 1 / d_model), float32;
    * o [B, T, U, H, d] ~ N(0, 1) (a stand-in for the forward's output);
    * w_o [d_model, H d] ~ N(0, 1 / (H d)); y_in [B, T, U, d_model] ~ N(0, 1).
    """
    B, T, U, H, d = w.B, w.T, w.U, w.H, w.d
    out = {"x": np.empty((B, T, U, d_model), np.uint16), "o": np.empty((B, T, U, H, d), np.uint16),
           "y_in": np.empty((B, T, U, d_model), np.uint16)}

    def frame(bt):
        b, t = bt
        off = _normal(_rng(w.seed, "x_frame", b, t), (1, d_model))
        out["x"][b, t] = f64_to_bf16_bits(off + _normal(_rng(w.seed, "x", b, t), (U, d_model)))
        out["o"][b, t] = f64_to_bf16_bits(_normal(_rng(w.seed, "o", b, t), (U, H, d)))
        out["y_in"][b, t] = f64_to_bf16_bits(_normal(_rng(w.seed, "y_in", b, t), (U, d_model)))

    jobs = [(b, t) for b in range(B) for t in range(T)]
    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(frame, jobs))
    out["w_gb"] = f64_to_bf16_bits(_normal(_rng(w.seed, "w_gb"), (H * d + H, d_model)) / np.sqrt(d_model))
    out["w_alpha"] = (_normal(_rng(w.seed, "w_alpha"), (H * d, d_model)) / np.sqrt(d_model)).astype(np.float32)
    out["w_o"] = f64_to_bf16_bits(_normal(_rng(w.seed, "w_o"), (d_model, H * d)) / np.sqrt(H * d))
    return out

