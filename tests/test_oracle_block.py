"""Pins of the reversible-block oracle (CPU only): textbook values of GELU and
LayerNorm, the chunked feed-forward against the unchunked one, the inverse of
the block against its inputs, head handling of the attention sublayer against
a permutation of the heads, and the sampled-row form against the full one."""
import math

import numpy as np
import pytest

import oracle as O
from oracle import lsh_block as OBk
from lsh_attention_amd import inputs as I


def test_gelu_is_x_times_the_normal_cdf():
    # Phi(1) and Phi(-1) from the normal table; gelu(x) - gelu(-x) = x since erf is odd
    assert OBk.gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(OBk.gelu(np.array([1.0]))[0], 0.8413447460685429, rtol=1e-15)
    np.testing.assert_allclose(OBk.gelu(np.array([-1.0]))[0], -0.15865525393145707, rtol=1e-14)
    x = np.linspace(-6, 6, 97)
    np.testing.assert_allclose(OBk.gelu(x) - OBk.gelu(-x), x, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(OBk.gelu(np.array([30.0])), [30.0], rtol=1e-15)


def test_layer_norm_hand_example_and_moments():
    g, b = np.ones(4), np.zeros(4)
    y = OBk.layer_norm(np.array([[1.0, 2.0, 3.0, 4.0]]), g, b)
    np.testing.assert_allclose(y[0], (np.array([1, 2, 3, 4]) - 2.5) / math.sqrt(1.25 + 1e-5), rtol=1e-15)
    rng = np.random.default_rng(1)
    x = 3.0 + 2.0 * rng.standard_normal((5, 512))
    y = OBk.layer_norm(x, np.ones(512), np.zeros(512))
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose(y.var(axis=1), 1.0, rtol=1e-5)
    gam, bet = rng.standard_normal(512), rng.standard_normal(512)
    np.testing.assert_allclose(OBk.layer_norm(x, gam, bet), y * gam + bet, rtol=1e-13, atol=1e-13)


def _block(L=256, heads=2, n_h=2, name="mlm_small_512"):
    bi = I.make_block_inputs(name, n_hashes=n_h, B=1, L=L, heads=heads)
    p = bi.params_math()
    rot = None if bi.rot is None else bi.rot.values.astype(np.float64)
    return bi, p, rot


@pytest.mark.parametrize("chunk", [1, 7, 64, 100])
def test_chunked_feed_forward_equals_unchunked(chunk):
    bi, p, _ = _block(L=256)
    x = bi.x1.values[0].astype(np.float64)
    full = OBk.feed_forward(x, p)
    np.testing.assert_allclose(OBk.feed_forward(x, p, chunk_rows=chunk), full, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_block_inverse_recovers_the_inputs(causal):
    bi, p, rot = _block(L=192)
    w = bi.workload
    x1, x2 = bi.x1.values.astype(np.float64), bi.x2.values.astype(np.float64)
    y1, y2 = OBk.block_forward(x1, x2, p, rot, w.n_buckets, 2, causal, chunk_rows=64)
    assert np.max(np.abs(y1 - x1)) > 0.1 and np.max(np.abs(y2 - x2)) > 0.1
    r1, r2 = OBk.block_inverse(y1, y2, p, rot, w.n_buckets, 2, causal, chunk_rows=64)
    np.testing.assert_allclose(r1, x1, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(r2, x2, rtol=1e-10, atol=1e-10)


def test_attention_sublayer_is_equivariant_under_a_permutation_of_the_heads():
    """Swapping head 0 and head 1 (columns of W_qk and W_v, rows of W_o) gives the
    same F: each head attends with its own 64 features only."""
    bi, p, rot = _block(L=128, heads=3)
    w = bi.workload
    x = bi.x2.values[0].astype(np.float64)
    ref = OBk.attention_sublayer(x, p, rot, w.n_buckets, 2, False)
    perm = np.r_[64:128, 0:64, 128:192]
    q = dict(p)
    q["w_qk"] = p["w_qk"][:, perm]
    q["w_v"] = p["w_v"][:, perm]
    q["w_o"] = p["w_o"][perm, :]
    np.testing.assert_allclose(OBk.attention_sublayer(x, q, rot, w.n_buckets, 2, False), ref, rtol=1e-12,
                               atol=1e-12)


def test_one_head_with_identity_output_is_the_attention_oracle():
    """dim = 64 (one head) and W_o = I: F is the attention oracle's output on the
    LayerNorm-ed projections."""
    bi, p, rot = _block(L=128, heads=1)
    w = bi.workload
    x = bi.x2.values[0].astype(np.float64)
    q = dict(p)
    q["w_o"] = np.eye(64)
    h = OBk.layer_norm(x, p["ln1_g"], p["ln1_b"])
    r = O.forward_problem(h @ p["w_qk"], h @ p["w_v"], rot, w.n_buckets, 2, 64, True)
    np.testing.assert_allclose(OBk.attention_sublayer(x, q, rot, w.n_buckets, 2, True), r["out"], rtol=1e-13,
                               atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_attention_rows_equal_the_full_sublayer(causal):
    bi, p, rot = _block(L=256)
    w = bi.workload
    x = bi.x2.values[0].astype(np.float64)
    full = OBk.attention_sublayer(x, p, rot, w.n_buckets, 2, causal)
    rows = [0, 13, 128, 255]
    np.testing.assert_allclose(OBk.attention_rows(x, p, rot, w.n_buckets, 2, causal, rows), full[rows],
                               rtol=1e-11, atol=1e-12)
