"""Pins of the backward oracle (CPU only): its differentiable forward against
the numpy oracle, its gradients against central finite differences of the
numpy oracle with the permutation held fixed, exact invariants, and the
sampled single-token form against the whole-problem gradient."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import lsh_backward as OB


def _problem(seed, L, n_b, n_h, D=64):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    rot = None if n_b == 1 else rng.standard_normal((n_h, D, n_b // 2))
    if rot is None:
        buckets = np.zeros((n_h, L), dtype=np.int64)
    else:
        buckets, _ = O.hash_buckets(x, rot, n_b)
    sidx, undo = O.sort_by_bucket(buckets)
    dout = rng.standard_normal((L, D))
    dlse = rng.standard_normal(L)
    return x, v, sidx, undo, dout, dlse


def _loss_np(x, v, sidx, undo, causal, dout, dlse, lse0):
    """sum dout . out + sum dlse (LSE - LSE0): the constant LSE0 (the unperturbed
    LSE) is taken off element by element, so that self-only tokens (LSE near
    -1e5, independent of x) do not swamp the central differences in rounding."""
    o, l = O.chunk_attention(x, v, sidx, 64, causal)
    out, lse = O.unsort_combine(o, l, undo)
    f = float(np.sum(out * dout))
    return f + (float(np.sum((lse - lse0) * dlse)) if dlse is not None else 0.0)


CASES = [(11, 128, 4, 2, False), (12, 128, 4, 2, True), (13, 192, 2, 3, True), (14, 64, 1, 1, False),
         (15, 64, 1, 1, True), (16, 128, 8, 1, False), (17, 256, 16, 2, True)]


@pytest.mark.parametrize("seed,L,n_b,n_h,causal", CASES)
def test_differentiable_forward_equals_numpy_oracle(seed, L, n_b, n_h, causal):
    x, v, sidx, undo, _, _ = _problem(seed, L, n_b, n_h)
    o, l = O.chunk_attention(x, v, sidx, 64, causal)
    out, lse = O.unsort_combine(o, l, undo)
    t_out, t_lse = OB.token_forward_torch(torch.tensor(x), torch.tensor(v), sidx, undo, 64, causal, np.arange(L))
    np.testing.assert_allclose(t_out.detach().numpy(), out, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(t_lse.detach().numpy(), lse, rtol=1e-10, atol=1e-9)


@pytest.mark.parametrize("with_dlse", [True, False])
@pytest.mark.parametrize("seed,L,n_b,n_h,causal", CASES)
def test_gradient_matches_finite_differences(seed, L, n_b, n_h, causal, with_dlse):
    """Directional derivatives along random directions, and single coordinates,
    by central differences of the numpy oracle (the permutation held fixed)."""
    x, v, sidx, undo, dout, dlse = _problem(seed, L, n_b, n_h)
    dlse = dlse if with_dlse else None
    dx, dv = OB.backward_problem(x, v, sidx, undo, 64, causal, dout, dlse)
    rng = np.random.default_rng(seed + 100)
    h = 1e-5
    lse0 = O.unsort_combine(*O.chunk_attention(x, v, sidx, 64, causal), undo)[1]
    f = lambda xx, vv: _loss_np(xx, vv, sidx, undo, causal, dout, dlse, lse0)  # noqa: E731
    for _ in range(2):
        u = rng.standard_normal(x.shape)
        w = rng.standard_normal(v.shape)
        fd_x = (f(x + h * u, v) - f(x - h * u, v)) / (2 * h)
        fd_v = (f(x, v + h * w) - f(x, v - h * w)) / (2 * h)
        assert abs(fd_x - np.sum(dx * u)) <= 1e-6 * (abs(fd_x) + np.sqrt(np.sum(dx * dx))), (fd_x, np.sum(dx * u))
        assert abs(fd_v - np.sum(dv * w)) <= 1e-6 * (abs(fd_v) + np.sqrt(np.sum(dv * dv))), (fd_v, np.sum(dv * w))
    for _ in range(4):
        i, d = int(rng.integers(0, L)), int(rng.integers(0, 64))
        e = np.zeros_like(x)
        e[i, d] = 1.0
        fd_x = (f(x + h * e, v) - f(x - h * e, v)) / (2 * h)
        fd_v = (f(x, v + h * e) - f(x, v - h * e)) / (2 * h)
        assert abs(fd_x - dx[i, d]) <= 1e-6 * (1.0 + abs(fd_x)), (i, d, fd_x, dx[i, d])
        assert abs(fd_v - dv[i, d]) <= 1e-6 * (1.0 + abs(fd_v)), (i, d, fd_v, dv[i, d])


@pytest.mark.parametrize("seed,L,n_b,n_h,causal", CASES)
def test_value_gradients_sum_to_the_output_gradients(seed, L, n_b, n_h, causal):
    """Each token's combined weights over its key occurrences sum to 1, so the
    value gradients sum to sum_i dout_i; and the LSE term never reaches v."""
    x, v, sidx, undo, dout, dlse = _problem(seed, L, n_b, n_h)
    _, dv = OB.backward_problem(x, v, sidx, undo, 64, causal, dout, dlse)
    np.testing.assert_allclose(dv.sum(axis=0), dout.sum(axis=0), rtol=1e-10, atol=1e-10)
    _, dv0 = OB.backward_problem(x, v, sidx, undo, 64, causal, np.zeros_like(dout), dlse)
    assert np.all(dv0 == 0.0)


def test_self_only_token_passes_its_output_gradient_to_its_own_value():
    """Causal position 0 attends only to itself in every round: out_0 = v_0, so
    dv gets dout_0 at row 0 from that token, and x_0 gets nothing from it."""
    x, v, sidx, undo, dout, _ = _problem(21, 128, 4, 2)
    d1 = np.zeros_like(dout)
    d1[0] = dout[0]
    dx, dv = OB.backward_problem(x, v, sidx, undo, 64, True, d1, None)
    np.testing.assert_allclose(dv[0], dout[0], rtol=1e-12, atol=1e-12)
    assert np.all(dv[1:] == 0.0) and np.all(dx == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_token_gradient_equals_the_whole_problem(causal):
    x, v, sidx, undo, dout, dlse = _problem(22, 256, 8, 3)
    dx, dv = OB.backward_problem(x, v, sidx, undo, 64, causal, dout, dlse)
    for j in (0, 7, 100, 255):
        gx, gv = OB.token_grads(x, v, sidx, undo, 64, causal, dout, dlse, j)
        np.testing.assert_allclose(gx, dx[j], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(gv, dv[j], rtol=1e-10, atol=1e-12)
