"""The linear maps either side of the VDA path, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:

* [VDN-summary] "무엇과 다른가": the linear branch ends in RMSNorm and its own
  sigmoid output gate; separate decay and write gates steer how much memory a
  frame keeps and how strongly it writes; each branch has its own output
  projection and the two are summed, Y = O^S W_O^S + O^L W_O^L, into the
  pretrained residual stream.
* [VDN-summary] "어떻게 쓰나": alpha_t per key channel per frame in [0, 1],
  beta_{t,u} per token, beta >= 0.
* [VDN-summary] "전제와 한계": the decay module runs in FP32.
* [VDN-H3-writeup] "VDN-H3의 하이브리드 어텐션 구조": a content-dependent
  sigmoid gate on each branch, a separate output projection per branch, then
  the residual stream.

The pages name these maps but not their form.  Readings (the plainest that
the pages support):

* every gate reads the attention block's input x (the tokens the shared QKV
  projection reads) through a linear map without bias, weights stored
  [out, in];
* gate logits  g[t, u] = W_g x[t, u]                 (H * d_v per token; the
  VDA epilogue applies the sigmoid);
* write gate   beta[t, u, h] = sigmoid(w_beta[h] . x[t, u]);
* decay gate   alpha[t, h, :] = sigmoid(W_alpha[h] xbar_t), xbar_t the mean of
  frame t's tokens (alpha is per frame, so it reads a per-frame summary);
* branch merge Y = Y_in + O W_O^T, O the linear branch's output after its
  epilogue, Y_in whatever the caller adds (the softmax branch's O^S W_O^S and
  the residual stream).
"""

from __future__ import annotations

import numpy as np


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def gate_proj(x, w_g, w_beta, w_alpha, H, d):
    """Gate logits, write gate and decay gate from the block input.

    x [B, T, U, Dm]; w_g [H * d, Dm]; w_beta [H, Dm]; w_alpha [H * d, Dm].
    Returns g [B, T, U, H, d], beta [B, T, U, H], alpha [B, T, H, d] (float64).
    """
    B, T, U, Dm = x.shape
    g = (x @ w_g.T).reshape(B, T, U, H, d)
    beta = sigmoid(x @ w_beta.T)
    xbar = x.mean(axis=2)                                     # [B, T, Dm]
    alpha = sigmoid(xbar @ w_alpha.T).reshape(B, T, H, d)
    return g, beta, alpha


def out_proj(o, w_o, y_in=None):
    """The linear branch's output projection merged into what the caller adds.

    o [B, T, U, H, d]; w_o [Dm, H * d]; y_in [B, T, U, Dm] or None (zero).
    Returns Y [B, T, U, Dm] = y_in + o W_O^T.
    """
    B, T, U, H, d = o.shape
    y = o.reshape(B, T, U, H * d) @ w_o.T
    return y if y_in is None else y_in + y
