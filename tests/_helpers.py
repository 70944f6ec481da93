"""Shared helpers for the GPU tests: device upload of the seeded inputs and
the elementwise tolerance check."""
import numpy as np
import torch

from lsh_attention_amd import inputs as I

# Output tolerance (relative, in the sense of rel_check below): fp32 1e-4, bf16 2e-2.
TOL = {"f32": 1e-4, "bf16": 2e-2}
# lse is computed from fp32 logits of exact inputs in both dtypes.
LSE_TOL = 1e-4


def to_device(t):
    if t is None:
        return None
    if t.bits is not None:
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(t.values)).cuda()


def f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def rel_check(got, ref, tol, what):
    """|got - ref| <= tol * (|ref| + rms(ref row)) elementwise, the rms taken over
    each output row (one token's head vector).  A pure relative error is
    ill-posed for entries near zero, and a row's rounding errors scale with the
    row's magnitude (a causal token early in the sequence averages few values)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True)) if ref.size else 0.0
    err = np.abs(got - ref)
    bound = tol * (np.abs(ref) + rms)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / np.maximum(bound, 1e-300)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())}/{err.size} elements outside tol {tol}; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} (ratio {float(err[i] / bound[i]):.3g})")
    return float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0


def lse_check(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bound = LSE_TOL * (np.abs(ref) + 1.0)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())}/{err.size} lse values outside tol; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r}")


def upload(inp: I.Inputs):
    return to_device(inp.qk), to_device(inp.v), to_device(inp.rot)
