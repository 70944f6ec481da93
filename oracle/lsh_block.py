"""CPU oracle for one reversible Reformer block around the LSH attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP path
and never imports it; the product path must not call it.

Sources (the pages): the Reformer abstract names reversible residual layers in
place of standard residuals; the Reformer explainer names reversible residual
layers and a chunked feed-forward as the memory savings that, with LSH
attention, fit about 64K tokens on one accelerator; the Korean Reformer page
lists the reversible layers and the chunked feed-forward among Reformer's
ideas and gives the "Reformer-mlm-small" shape (dim 512, 8 heads).

Readings where the pages are silent (listed in the design notes):
  * reversible block (RevNet form): y1 = x1 + F(x2), y2 = x2 + G(y1), so the
    inputs follow from the outputs: x2 = y2 - G(y1), x1 = y1 - F(x2);
  * F = the attention sublayer: LayerNorm, a shared query/key projection and
    a value projection (no biases), the LSH attention per head (dim = heads x
    64, head h takes features 64h .. 64h+63), an output projection (no bias);
  * G = the feed-forward sublayer: LayerNorm, Linear(dim, 4 dim) + bias, GELU
    (the erf form), Linear(4 dim, dim) + bias;
  * "chunked feed-forward": G is applied to consecutive chunks of rows, one
    chunk at a time; every row is computed exactly as without chunking;
  * LayerNorm(x) = (x - mean) / sqrt(var + 1e-5) * gamma + beta over the
    feature dimension (biased variance).
Float64 numpy throughout; matrix products, erf and the attention oracle are
the library primitives.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from . import lsh_oracle as O

LN_EPS = 1e-5


def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + LN_EPS) * gamma + beta


def gelu(x: np.ndarray) -> np.ndarray:
    """x * Phi(x), Phi the standard normal CDF."""
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def feed_forward(x: np.ndarray, p: dict, chunk_rows: int | None = None) -> np.ndarray:
    """G(x) for rows x [N, dim]; with chunk_rows, row chunks one at a time."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    step = n if chunk_rows is None else chunk_rows
    out = np.empty((n, p["w2"].shape[1]))
    for r0 in range(0, n, step):
        h = layer_norm(x[r0:r0 + step], p["ln2_g"], p["ln2_b"])
        h = gelu(h @ p["w1"] + p["b1"])
        out[r0:r0 + step] = h @ p["w2"] + p["b2"]
    return out


def attention_sublayer(x: np.ndarray, p: dict, rot, n_buckets: int, n_hashes: int, causal: bool,
                       chunk_len: int = 64) -> np.ndarray:
    """F(x) for one sequence x [L, dim]: LayerNorm, projections, LSH attention per
    head with the shared rotations `rot` [n_h, 64, n_b/2], output projection."""
    x = np.asarray(x, dtype=np.float64)
    L, dim = x.shape
    heads = dim // 64
    h = layer_norm(x, p["ln1_g"], p["ln1_b"])
    qk = h @ p["w_qk"]
    v = h @ p["w_v"]
    att = np.empty((L, dim))
    for hd in range(heads):
        sl = slice(64 * hd, 64 * hd + 64)
        r = O.forward_problem(qk[:, sl], v[:, sl], rot, n_buckets, n_hashes, chunk_len, causal)
        att[:, sl] = r["out"]
    return att @ p["w_o"]


def block_forward(x1, x2, p: dict, rot, n_buckets: int, n_hashes: int, causal: bool,
                  chunk_rows: int | None = None):
    """One reversible block on a batch: x1, x2 [B, L, dim] -> (y1, y2)."""
    x1 = np.asarray(x1, dtype=np.float64)
    x2 = np.asarray(x2, dtype=np.float64)
    y1 = np.empty_like(x1)
    y2 = np.empty_like(x2)
    for b in range(x1.shape[0]):
        y1[b] = x1[b] + attention_sublayer(x2[b], p, rot, n_buckets, n_hashes, causal)
        y2[b] = x2[b] + feed_forward(y1[b], p, chunk_rows)
    return y1, y2


def block_inverse(y1, y2, p: dict, rot, n_buckets: int, n_hashes: int, causal: bool,
                  chunk_rows: int | None = None):
    """The inputs recovered from the outputs: x2 = y2 - G(y1), x1 = y1 - F(x2)."""
    y1 = np.asarray(y1, dtype=np.float64)
    y2 = np.asarray(y2, dtype=np.float64)
    x1 = np.empty_like(y1)
    x2 = np.empty_like(y2)
    for b in range(y1.shape[0]):
        x2[b] = y2[b] - feed_forward(y1[b], p, chunk_rows)
        x1[b] = y1[b] - attention_sublayer(x2[b], p, rot, n_buckets, n_hashes, causal)
    return x1, x2


def attention_rows(x, p: dict, rot, n_buckets: int, n_hashes: int, causal: bool, rows,
                   chunk_len: int = 64) -> np.ndarray:
    """F(x)[rows] for one sequence, each head's rows from their own windows (for
    sampled checks of long sequences): the permutation of every head is computed
    in full, the attention only for the requested tokens."""
    x = np.asarray(x, dtype=np.float64)
    L, dim = x.shape
    heads = dim // 64
    h = layer_norm(x, p["ln1_g"], p["ln1_b"])
    qk = h @ p["w_qk"]
    v = h @ p["w_v"]
    att = np.empty((len(rows), dim))
    for hd in range(heads):
        sl = slice(64 * hd, 64 * hd + 64)
        if n_buckets == 1:
            buckets = np.zeros((n_hashes, L), dtype=np.int64)
        else:
            buckets, _ = O.hash_buckets(qk[:, sl], rot, n_buckets)
        sidx, undo = O.sort_by_bucket(buckets)
        for k, i in enumerate(rows):
            att[k, sl], _ = O.token_output(qk[:, sl], v[:, sl], sidx, undo, chunk_len, causal, int(i))
    return att @ p["w_o"]
