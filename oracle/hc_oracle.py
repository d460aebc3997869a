"""Plain fp64 CPU oracle of the Hyper-Connection mixer around the attention block.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path, and sharing no code with it.

Source: P1 = "【#3】ds4.c を読み解く", section 10 (Hyper-Connection: four
streams mixed with Sinkhorn).  The page fixes: the hidden state is carried as
n_hc = 4 residual streams; a per-token mixer row is split into pre weights,
post gates and an n_hc x n_hc coupling matrix between the streams; the
coupling matrix is normalised by Sinkhorn iterations (20 at the Flash shape)
that alternate a row normalisation and a column normalisation, each dividing
by (sum + eps); the loop the page shows runs from the second iteration on, so
the first one is done when the matrix is built.

Readings taken where the page is silent (each also listed in the design
notes; "parity unpinned" for the parts no invariant fixes):

* mixer row layout: [pre (n) | post (n) | coupling (n * n, row-major)];
* pre weights and post gates are the logistic sigmoid of their entries;
* building the matrix = a softmax along each row (the first iteration's row
  normalisation), then the first column normalisation; iterations 2..iters
  are (row, column) normalisations; eps = 1e-6;
* the streams h_0..h_{n-1} (each a hidden-size vector) feed the block with
  x = sum_i pre_i h_i, and after the block (output y) become
  h'_j = sum_i C[j][i] h_i + post_j y  (row j of C gathers into stream j).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64

HC_N = 4
HC_SINKHORN_ITERS = 20
HC_EPS = 1e-6


def sigmoid(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, F64)
    return 1.0 / (1.0 + np.exp(-x))


def sinkhorn(m: np.ndarray, iters: int = HC_SINKHORN_ITERS, eps: float = HC_EPS) -> np.ndarray:
    """Coupling matrix [..., n, n] from its mixer entries, by the alternating
    normalisation of P1 s10: the first iteration is the row softmax and a
    column normalisation, each later one a row then a column normalisation."""
    m = np.asarray(m, F64)
    e = np.exp(m - m.max(axis=-1, keepdims=True))
    c = e / e.sum(axis=-1, keepdims=True)                 # iteration 1: rows
    c = c / (c.sum(axis=-2, keepdims=True) + eps)         #              columns
    for _ in range(1, iters):
        c = c / (c.sum(axis=-1, keepdims=True) + eps)     # rows
        c = c / (c.sum(axis=-2, keepdims=True) + eps)     # columns
    return c


def hc_split(mix: np.ndarray, n: int = HC_N, iters: int = HC_SINKHORN_ITERS, eps: float = HC_EPS):
    """Mixer rows [..., n (n + 2)] -> (pre [..., n], post [..., n], C [..., n, n])."""
    mix = np.asarray(mix, F64)
    pre = sigmoid(mix[..., :n])
    post = sigmoid(mix[..., n:2 * n])
    comb = sinkhorn(mix[..., 2 * n:].reshape(mix.shape[:-1] + (n, n)), iters, eps)
    return pre, post, comb


def hc_pre(pre: np.ndarray, h: np.ndarray) -> np.ndarray:
    """Block input x [..., D] = sum_i pre_i h_i for streams h [..., n, D]."""
    h = np.asarray(h, F64)
    pre = np.asarray(pre, F64)
    x = np.zeros(h.shape[:-2] + h.shape[-1:])
    for i in range(h.shape[-2]):
        x += pre[..., i:i + 1] * h[..., i, :]
    return x


def hc_post(post: np.ndarray, comb: np.ndarray, h: np.ndarray, y: np.ndarray) -> np.ndarray:
    """Streams after the block: h'_j = sum_i C[j][i] h_i + post_j y."""
    h = np.asarray(h, F64)
    y = np.asarray(y, F64)
    n = h.shape[-2]
    out = np.zeros_like(h)
    for j in range(n):
        acc = post[..., j:j + 1] * y
        for i in range(n):
            acc = acc + comb[..., j, i:i + 1] * h[..., i, :]
        out[..., j, :] = acc
    return out
