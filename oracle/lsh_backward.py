"""CPU oracle for the backward pass of the shared-QK LSH-attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP path
and never imports it; the product path must not call it.

What it computes: the gradient of L = sum_i dout_i . out_i + sum_i dlse_i LSE_i
with respect to the shared query/key vectors x and the values v, for the
forward pass defined in lsh_oracle (chunked windows of the sorted order,
rounds combined with softmax_r(lse_r)).  Hashing and sorting are piecewise
constant in x, so the permutation of the forward pass is an input here, as
the Reformer explainer's pipeline reuses it (the bucket of a token does not
move under an infinitesimal change of x); the gradient flows through the
logits, the key normalisation, the softmax weights, the values and the
combine.

How: float64 PyTorch autograd (a library primitive, used as the definition of
the gradient) through a differentiable transcription of the forward pass,
written per token: token i's output is computed from its own window in every
round (the previous chunk and its own chunk of the sorted order), then the
rounds are combined.  This is a different arrangement of the same steps than
the numpy oracle's chunk-by-chunk pass, and the tests pin the two to each
other, and the gradient to central finite differences of the numpy oracle.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from .lsh_oracle import KEY_NORM_FLOOR, SELF_LOGIT


def _windows(sorted_idx: np.ndarray, undo_idx: np.ndarray, chunk_len: int, tokens: np.ndarray):
    """Key positions of every (token, round) window: [len(tokens), n_h, 2 * chunk_len]
    (previous chunk, cyclic over the round-major slots, then the token's chunk)."""
    n_slots = sorted_idx.shape[0]
    n_chunks = n_slots // chunk_len
    chunk = undo_idx[:, tokens].T // chunk_len               # [nq, n_h]
    prev = (chunk - 1) % n_chunks
    ar = np.arange(chunk_len)
    slots = np.concatenate([prev[..., None] * chunk_len + ar, chunk[..., None] * chunk_len + ar], axis=-1)
    return sorted_idx[slots]


def token_forward_torch(X: torch.Tensor, V: torch.Tensor, sorted_idx: np.ndarray, undo_idx: np.ndarray,
                        chunk_len: int, causal: bool, tokens: np.ndarray):
    """Differentiable float64 forward for the given tokens: (out [nq, D], LSE [nq]).
    Logit (x_i . x_j / max(|x_j|, 1e-12)) / sqrt(D), the self key at -1e5, causal
    drops keys after the query; per round a softmax over the window (keys
    counted as often as they occur); rounds combined with weights softmax_r(lse_r)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    D = X.shape[1]
    kpos = torch.as_tensor(_windows(sorted_idx, undo_idx, chunk_len, tokens))     # [nq, n_h, 2C]
    qpos = torch.as_tensor(tokens)[:, None, None]
    K = X[kpos]                                                                   # [nq, n_h, 2C, D]
    k_hat = K / torch.clamp(torch.linalg.vector_norm(K, dim=-1, keepdim=True), min=KEY_NORM_FLOOR)
    s = torch.einsum("qd,qrkd->qrk", X[torch.as_tensor(tokens)], k_hat) / math.sqrt(D)
    s = torch.where(kpos == qpos, torch.full_like(s, SELF_LOGIT), s)
    if causal:
        s = torch.where(kpos > qpos, torch.full_like(s, -math.inf), s)
    lse_r = torch.logsumexp(s, dim=-1)                                            # [nq, n_h]
    o_r = torch.einsum("qrk,qrkd->qrd", torch.exp(s - lse_r[..., None]), V[kpos])  # [nq, n_h, D]
    LSE = torch.logsumexp(lse_r, dim=-1)
    out = torch.einsum("qr,qrd->qd", torch.exp(lse_r - LSE[:, None]), o_r)
    return out, LSE


def backward_problem(x, v, sorted_idx, undo_idx, chunk_len: int, causal: bool, dout, dlse=None):
    """One (batch, head) problem: (dx [L, D], dv [L, D]) for the loss
    sum_i dout_i . out_i + sum_i dlse_i LSE_i (dlse None: no LSE term)."""
    L = x.shape[0]
    X = torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)
    V = torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True)
    out, LSE = token_forward_torch(X, V, np.asarray(sorted_idx), np.asarray(undo_idx), chunk_len, causal,
                                   np.arange(L))
    loss = (out * torch.as_tensor(np.asarray(dout, dtype=np.float64))).sum()
    if dlse is not None:
        loss = loss + (LSE * torch.as_tensor(np.asarray(dlse, dtype=np.float64))).sum()
    loss.backward()
    return X.grad.numpy(), V.grad.numpy()


def attending_tokens(sorted_idx: np.ndarray, undo_idx: np.ndarray, chunk_len: int, j: int) -> np.ndarray:
    """Tokens whose output depends on x_j or v_j: j itself, and every token with
    a query slot in a chunk whose window holds one of j's slots (j's own chunk
    and the next chunk, cyclically, in every round)."""
    n_slots = sorted_idx.shape[0]
    n_chunks = n_slots // chunk_len
    qs = {int(j)}
    for g in undo_idx[:, j]:
        c = int(g) // chunk_len
        for cq in (c, (c + 1) % n_chunks):
            qs.update(int(t) for t in sorted_idx[cq * chunk_len:(cq + 1) * chunk_len])
    return np.array(sorted(qs), dtype=np.int64)


def token_grads(x, v, sorted_idx, undo_idx, chunk_len: int, causal: bool, dout, dlse, j: int):
    """(dx_j, dv_j) of one token, from the loss restricted to the tokens whose
    output depends on row j (for sampled checks of long sequences)."""
    X = torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)
    V = torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=True)
    qs = attending_tokens(np.asarray(sorted_idx), np.asarray(undo_idx), chunk_len, j)
    out, LSE = token_forward_torch(X, V, np.asarray(sorted_idx), np.asarray(undo_idx), chunk_len, causal, qs)
    loss = (out * torch.as_tensor(np.asarray(dout, dtype=np.float64)[qs])).sum()
    if dlse is not None:
        loss = loss + (LSE * torch.as_tensor(np.asarray(dlse, dtype=np.float64)[qs])).sum()
    loss.backward()
    return X.grad[j].numpy().copy(), V.grad[j].numpy().copy()
