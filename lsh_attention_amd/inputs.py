"""Seeded synthetic inputs for the shared-QK LSH-attention forward pass.

This module only draws random numbers and rounds them to the storage type.
It holds none of the attention method's arithmetic, so both the CPU oracle
(via the tests) and the HIP path consume the exact same arrays.

Workloads (shapes follow the Reformer-mlm-small table of the Korean Reformer
language-model page and the ~64K-token single-accelerator claim of the
Reformer explainer page):

=================  ====  ==  =====  ====  ===  ===  ======  ======================
workload           B     H   L      dt    n_b  n_h  causal  shared-QK distribution
=================  ====  ==  =====  ====  ===  ===  ======  ======================
single_head_fp32   1     1   1024   f32   16   1    no      iid N(0,1)
mlm_small_512      128   8   512    bf16  8    4    no      iid N(0,1)
causal_lm_4k       8     8   4096   bf16  64   4    yes     iid N(0,1)
long_seq_64k       1     8   65536  bf16  1024 8    yes     iid N(0,1)
peaked_vmf_16k     4     8   16384  bf16  256  2,8  no      256 vMF clusters, kappa 50
=================  ====  ==  =====  ====  ===  ===  ======  ======================

d_head = 64 and chunk_len = 64 everywhere.  V is iid N(0,1).  Rotations are
iid N(0,1) of shape [n_h, 64, n_b/2], rounded to the QK storage type.

Seeds: workload k (1-based, table order) uses seed 1000*k + stream, with
stream 0 = QK, 1 = V, 2 = rotations, 3 = vMF means, 4 = cluster assignment,
5 = vMF draws.  Every array is drawn in float32 by numpy's PCG64 and, for bf16
workloads, rounded to nearest-even bf16; the float32 view of the bf16 bits is
the exact value both sides see.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

D_HEAD = 64
CHUNK_LEN = 64


@dataclass(frozen=True)
class Workload:
    name: str
    index: int  # 1-based position in the table above (seed base)
    B: int
    H: int
    L: int
    dtype: str  # "f32" or "bf16"
    n_buckets: int
    n_hashes: tuple
    causal: bool
    qk_dist: str = "gauss"  # "gauss" or "vmf"
    D: int = D_HEAD
    chunk_len: int = CHUNK_LEN
    n_clusters: int = 0
    kappa: float = 0.0


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_head_fp32", 1, 1, 1, 1024, "f32", 16, (1,), False),
        Workload("mlm_small_512", 2, 128, 8, 512, "bf16", 8, (4,), False),
        Workload("causal_lm_4k", 3, 8, 8, 4096, "bf16", 64, (4,), True),
        Workload("long_seq_64k", 4, 1, 8, 65536, "bf16", 1024, (8,), True),
        Workload("peaked_vmf_16k", 5, 4, 8, 16384, "bf16", 256, (2, 8), False,
                 qk_dist="vmf", n_clusters=256, kappa=50.0),
    ]
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Tensor:
    """One input array: `values` is float32 holding the exact stored values;
    `bits` is the uint16 bf16 storage (None for float32 storage)."""
    values: np.ndarray
    bits: np.ndarray | None = None

    @property
    def dtype(self) -> str:
        return "f32" if self.bits is None else "bf16"

    def storage(self) -> np.ndarray:
        return self.values if self.bits is None else self.bits

    def sha256(self) -> str:
        return hashlib.sha256(np.ascontiguousarray(self.storage()).tobytes()).hexdigest()


def _store(a32: np.ndarray, dtype: str) -> Tensor:
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "f32":
        return Tensor(a32)
    if dtype == "bf16":
        bits = bf16_bits_from_f32(a32)
        return Tensor(f32_from_bf16_bits(bits), bits)
    raise ValueError(f"unknown dtype {dtype}")


def gaussian(seed: int, shape, dtype: str) -> Tensor:
    rng = np.random.Generator(np.random.PCG64(seed))
    return _store(rng.standard_normal(shape, dtype=np.float32), dtype)


def rotations(seed: int, n_hashes: int, D: int, n_buckets: int, dtype: str) -> Tensor | None:
    """Random rotations [n_hashes, D, n_buckets/2]; None when n_buckets == 1."""
    if n_buckets == 1:
        return None
    return gaussian(seed, (n_hashes, D, n_buckets // 2), dtype)


def vmf_wood(rng: np.random.Generator, mu: np.ndarray, kappa: float) -> np.ndarray:
    """Draw one von Mises-Fisher sample per row of the unit vectors `mu` [N, d]
    with Wood's (1994) rejection sampler for the cosine w = mu.x, then a
    uniform direction orthogonal to mu.  float64."""
    N, d = mu.shape
    b = (-2.0 * kappa + np.sqrt(4.0 * kappa * kappa + (d - 1.0) ** 2)) / (d - 1.0)
    x0 = (1.0 - b) / (1.0 + b)
    c = kappa * x0 + (d - 1.0) * np.log(1.0 - x0 * x0)
    w = np.empty(N)
    todo = np.arange(N)
    while todo.size:
        n = todo.size
        z = rng.beta((d - 1.0) / 2.0, (d - 1.0) / 2.0, size=n)
        wc = (1.0 - (1.0 + b) * z) / (1.0 - (1.0 - b) * z)
        u = rng.uniform(size=n)
        ok = kappa * wc + (d - 1.0) * np.log(1.0 - x0 * wc) - c >= np.log(u)
        w[todo[ok]] = wc[ok]
        todo = todo[~ok]
    v = rng.standard_normal((N, d))
    v -= np.sum(v * mu, axis=1, keepdims=True) * mu
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    return w[:, None] * mu + np.sqrt(np.maximum(0.0, 1.0 - w * w))[:, None] * v


def vmf_clustered(seed_means: int, seed_assign: int, seed_draw: int, B: int, H: int, L: int,
                  D: int, n_clusters: int, kappa: float, dtype: str) -> Tensor:
    """Shared QK on the unit sphere: per (b, h), `n_clusters` normalised-Gaussian
    means; each token picks a cluster uniformly and is a vMF(mean, kappa) draw."""
    rm = np.random.Generator(np.random.PCG64(seed_means))
    ra = np.random.Generator(np.random.PCG64(seed_assign))
    rd = np.random.Generator(np.random.PCG64(seed_draw))
    means = rm.standard_normal((B * H, n_clusters, D))
    means /= np.linalg.norm(means, axis=2, keepdims=True)
    assign = ra.integers(0, n_clusters, size=(B * H, L))
    mu = np.take_along_axis(means, assign[:, :, None], axis=1).reshape(B * H * L, D)
    x = vmf_wood(rd, mu, kappa).reshape(B, H, L, D)
    return _store(x.astype(np.float32), dtype)


@dataclass
class Inputs:
    workload: Workload
    n_hashes: int
    qk: Tensor
    v: Tensor
    rot: Tensor | None
    meta: dict = field(default_factory=dict)


def make_inputs(name: str, n_hashes: int | None = None, B: int | None = None,
                H: int | None = None, L: int | None = None) -> Inputs:
    """Inputs of a named workload.  B, H, L may be shrunk for fast tests; the
    draw is then of the smaller shape with the same seeds (not a slice)."""
    w = WORKLOADS[name]
    n_h = w.n_hashes[-1] if n_hashes is None else n_hashes
    B = w.B if B is None else B
    H = w.H if H is None else H
    L = w.L if L is None else L
    s = 1000 * w.index
    shape = (B, H, L, w.D)
    if w.qk_dist == "vmf":
        qk = vmf_clustered(s + 3, s + 4, s + 5, B, H, L, w.D, w.n_clusters, w.kappa, w.dtype)
    else:
        qk = gaussian(s + 0, shape, w.dtype)
    v = gaussian(s + 1, shape, w.dtype)
    # The largest round count is drawn and sliced, so runs with fewer rounds
    # share their leading rotations with the larger ones.
    rot_all = rotations(s + 2, max(w.n_hashes), w.D, w.n_buckets, w.dtype)
    rot = None
    if rot_all is not None:
        if n_h <= rot_all.values.shape[0]:
            rot = Tensor(rot_all.values[:n_h].copy(),
                         None if rot_all.bits is None else rot_all.bits[:n_h].copy())
        else:
            rot = rotations(s + 2, n_h, w.D, w.n_buckets, w.dtype)
    meta = {"seed_base": s, "qk_sha256": qk.sha256(), "v_sha256": v.sha256(),
            "rot_sha256": None if rot is None else rot.sha256()}
    return Inputs(w, n_h, qk, v, rot, meta)


# ---- one reversible block (attention sublayer + feed-forward sublayer) ----
@dataclass
class BlockInputs:
    """Seeded synthetic inputs of one reversible block: the two input streams
    x1, x2 [B, L, dim], the rotations of the attention, and the parameters.
    Weights are stored [out, in] (a Linear layer's layout); `params_math`
    gives them [in, out] for x @ W.  Random weights scaled by 1/sqrt(in) keep
    the activations of order one; there are no trained weights."""
    workload: Workload
    n_hashes: int
    x1: Tensor
    x2: Tensor
    rot: Tensor | None
    params: dict  # name -> Tensor

    def params_math(self) -> dict:
        out = {}
        for k, t in self.params.items():
            a = t.values.astype(np.float64)
            out[k] = a.T if a.ndim == 2 else a
        return out


def make_block_inputs(name: str, n_hashes: int | None = None, B: int | None = None, L: int | None = None,
                      heads: int | None = None) -> BlockInputs:
    w = WORKLOADS[name]
    n_h = w.n_hashes[-1] if n_hashes is None else n_hashes
    B = w.B if B is None else B
    L = w.L if L is None else L
    H = w.H if heads is None else heads
    dim = H * w.D
    s = 1000 * w.index + 500
    x1 = gaussian(s + 0, (B, L, dim), w.dtype)
    x2 = gaussian(s + 1, (B, L, dim), w.dtype)
    rot = rotations(1000 * w.index + 2, n_h, w.D, w.n_buckets, w.dtype)

    def lin(seed, n_out, n_in):
        g = gaussian(seed, (n_out, n_in), "f32").values / np.sqrt(n_in)
        return _store(g, w.dtype)

    def vec(seed, n, mean, scale):
        return _store(mean + scale * gaussian(seed, (n,), "f32").values, w.dtype)

    p = {
        "ln1_g": vec(s + 10, dim, 1.0, 0.1), "ln1_b": vec(s + 11, dim, 0.0, 0.1),
        "w_qk": lin(s + 12, dim, dim), "w_v": lin(s + 13, dim, dim), "w_o": lin(s + 14, dim, dim),
        "ln2_g": vec(s + 15, dim, 1.0, 0.1), "ln2_b": vec(s + 16, dim, 0.0, 0.1),
        "w1": lin(s + 17, 4 * dim, dim), "b1": vec(s + 18, 4 * dim, 0.0, 0.1),
        "w2": lin(s + 19, dim, 4 * dim), "b2": vec(s + 20, dim, 0.0, 0.1),
    }
    return BlockInputs(w, n_h, x1, x2, rot, p)
