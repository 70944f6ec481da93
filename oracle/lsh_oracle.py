"""CPU oracle for Reformer's shared-QK angular-LSH attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP path
and never imports it; the product path must not call it.

Plain, slow and meant to be checked by eye: float64 numpy, one (batch, head)
problem at a time, one chunk at a time, exactly in the order of the method's
steps.  Library primitives used as steps: a matrix product, argmax, a stable
argsort, exp/log.

Sources (the pages):
  * Reformer explainer (akshathtiwari.co.in/blog/reformer), the one-paragraph
    description: a bucket is the angular sector a vector lands in after a
    random rotation, with collision probability 1 - theta/pi; queries and keys
    are tied (shared-QK); tokens are sorted by bucket and processed in equal
    chunks; several hash rounds with independent rotations are unioned.
  * Reformer abstract (codewithpapers.app, "Reformer: The Efficient
    Transformer"): LSH attention replaces dot-product attention, O(L log L).

Readings where the pages are silent (each listed in the design notes):
  * hash: argmax over the concatenation [x R_r ; -x R_r] (R_r has n_b/2
    columns), lowest index on exact ties, computed on the raw vector (positive
    scaling does not move an argmax); n_b = 1 puts every token in bucket 0.
  * sort key (round, bucket, position), i.e. a stable sort per round.
  * chunks tile the round-major concatenation of all rounds' sorted slots; a
    chunk attends to itself and to the previous chunk, cyclically over that
    concatenation (round r's first chunk looks back at round r-1's last one).
  * logits (x_i . x_j / max(|x_j|, 1e-12)) / sqrt(D): keys normalised,
    queries not; the self logit is replaced by -1e5, so a token attends to
    itself only when nothing else is in its window; causal drops keys whose
    original position is after the query's.
  * rounds are combined with weights softmax_r(lse_r), i.e. duplicates across
    rounds are counted with multiplicity.
  * attended-set variants (the explainer's "attends to its bucket-mates" and
    "unions the buckets", taken literally): with `same_bucket` a key slot
    counts only if it holds the query's (round, bucket); with `dedup` every
    distinct key token counts once over the union of the query's windows,
    by subtracting log N from each occurrence's logit, N = the number of
    kept (query occurrence, key occurrence) pairs of that token pair.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

SELF_LOGIT = -1.0e5
KEY_NORM_FLOOR = 1e-12


# --------------------------------------------------------------------------
# Step 1: angular LSH (explainer page: random rotation, angular sector)
# --------------------------------------------------------------------------

def _exact_value(x_row: np.ndarray, col: np.ndarray) -> Fraction:
    """x . col in exact rational arithmetic (binary floating-point inputs are
    dyadic rationals n / 2^k; the sum is formed over a common power of two)."""
    terms = []
    for a, r in zip(x_row.tolist(), col.tolist()):
        if a == 0.0 or r == 0.0:
            continue
        na, da = float(a).as_integer_ratio()
        nr, dr = float(r).as_integer_ratio()
        terms.append((na * nr, (da.bit_length() - 1) + (dr.bit_length() - 1)))
    if not terms:
        return Fraction(0)
    K = max(k for _, k in terms)
    return Fraction(sum(n << (K - k) for n, k in terms), 1 << K)


def _exact_bucket(x_row: np.ndarray, rot_r: np.ndarray, candidates=None) -> int:
    """Argmax of [x R ; -x R] in exact arithmetic, lowest index on ties, over the
    given entry indices (all 2 * n_b/2 entries when None)."""
    half = rot_r.shape[1]
    idxs = range(2 * half) if candidates is None else sorted(int(c) for c in candidates)
    cols = {}
    best_val, best_idx = None, 0
    for idx in idxs:
        j = idx % half
        if j not in cols:
            cols[j] = _exact_value(x_row, rot_r[:, j])
        val = cols[j] if idx < half else -cols[j]
        if best_val is None or val > best_val:
            best_val, best_idx = val, idx
    return best_idx


def hash_buckets(x: np.ndarray, rot: np.ndarray | None, n_buckets: int):
    """Bucket of every token in every round.

    x: [L, D] exact input values; rot: [n_h, D, n_b/2] (None when n_b == 1).
    Returns (buckets int64 [n_h, L], margin float64 [n_h, L]) where margin is
    the gap between the two largest entries of [p ; -p] divided by |x|, i.e.
    on the unit-normalised vector (inf when n_b == 1).
    """
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[0]
    if n_buckets == 1:
        n_h = 1 if rot is None else rot.shape[0]
        return np.zeros((n_h, L), dtype=np.int64), np.full((n_h, L), np.inf)
    if n_buckets < 2 or n_buckets % 2:
        raise ValueError("n_buckets must be 1 or even")
    rot = np.asarray(rot, dtype=np.float64)
    n_h, D, half = rot.shape
    assert half == n_buckets // 2 and D == x.shape[1]
    xnorm = np.linalg.norm(x, axis=1)
    buckets = np.empty((n_h, L), dtype=np.int64)
    margin = np.empty((n_h, L))
    for r in range(n_h):
        p = x @ rot[r]                                   # projection, [L, n_b/2]
        c = np.concatenate([p, -p], axis=1)              # [x R ; -x R], [L, n_b]
        b = np.argmax(c, axis=1)                         # first maximum = lowest index
        top2 = np.partition(c, -2, axis=1)[:, -2:]       # [second largest, largest]
        gap = top2[:, 1] - top2[:, 0]
        with np.errstate(divide="ignore", invalid="ignore"):
            margin[r] = np.where(xnorm > 0, gap / xnorm, 0.0)
        # float64 rounding of a D-term dot product is below D * 2^-53 * |x||r_j|;
        # any gap under a far larger band is re-decided in exact arithmetic,
        # among the entries within twice the band of the float64 maximum (a
        # superset of the exact maximisers).
        band = 1e-9 * xnorm * np.max(np.linalg.norm(rot[r], axis=0))
        for i in np.nonzero(gap <= band)[0]:
            cand = np.nonzero(c[i] >= c[i, b[i]] - 2.0 * band[i])[0]
            b[i] = _exact_bucket(x[i], rot[r], cand)
        buckets[r] = b
    return buckets, margin


# --------------------------------------------------------------------------
# Step 2: sort by (round, bucket, position)  (explainer page: sort by bucket)
# --------------------------------------------------------------------------

def sort_by_bucket(buckets: np.ndarray):
    """Stable sort of positions by bucket, independently per round.

    Returns sorted_idx [n_h*L] (slot g = r*L + k holds the original position of
    the k-th token of round r's order) and undo_idx [n_h, L] (the slot of
    position i in round r)."""
    n_h, L = buckets.shape
    sorted_idx = np.empty(n_h * L, dtype=np.int64)
    undo_idx = np.empty((n_h, L), dtype=np.int64)
    for r in range(n_h):
        order = np.argsort(buckets[r], kind="stable")
        sorted_idx[r * L:(r + 1) * L] = order
        undo_idx[r, order] = r * L + np.arange(L)
    return sorted_idx, undo_idx


# --------------------------------------------------------------------------
# Step 3: attention inside equal chunks (explainer page: equal chunks)
# --------------------------------------------------------------------------

def window_slots(n_slots: int, chunk_len: int, c: int) -> np.ndarray:
    """Slots attended by chunk c: the previous chunk (cyclic), then chunk c."""
    n_chunks = n_slots // chunk_len
    p = (c - 1) % n_chunks
    return np.concatenate([np.arange(p * chunk_len, (p + 1) * chunk_len),
                           np.arange(c * chunk_len, (c + 1) * chunk_len)])


def slot_codes(buckets: np.ndarray, sorted_idx: np.ndarray) -> np.ndarray:
    """(round, bucket) of every sorted slot, as one integer per slot: slot g of
    round r = g // L holds token sorted_idx[g], whose bucket in that round is
    buckets[r, token]."""
    n_h, L = buckets.shape
    g = np.arange(sorted_idx.shape[0])
    r = g // L
    return r * (int(buckets.max()) + 1) + buckets[r, sorted_idx]


def pair_multiplicity(sorted_idx: np.ndarray, undo_idx: np.ndarray, chunk_len: int, causal: bool,
                      codes=None, tokens=None) -> list:
    """For every token i, a dict {token j: N_ij}: how many times j is a kept key
    of i over all of i's windows (one query occurrence of i per round, each
    window counted with multiplicity, the masks of the variant applied).
    With `tokens` given, only those query tokens are counted (the others get
    empty dicts), for sampled checks of long sequences."""
    n_h, L = undo_idx.shape
    n_slots = sorted_idx.shape[0]
    wanted = None if tokens is None else set(int(t) for t in tokens)
    counts = []
    for i in range(L):
        cnt = {}
        if wanted is not None and i not in wanted:
            counts.append(cnt)
            continue
        for r in range(n_h):
            g = int(undo_idx[r, i])
            for gk in window_slots(n_slots, chunk_len, g // chunk_len):
                j = int(sorted_idx[gk])
                if causal and j > i:
                    continue
                if codes is not None and codes[gk] != codes[g]:
                    continue
                cnt[j] = cnt.get(j, 0) + 1
        counts.append(cnt)
    return counts


def chunk_attention(x: np.ndarray, v: np.ndarray, sorted_idx: np.ndarray, chunk_len: int,
                    causal: bool, chunks=None, codes=None, mult=None):
    """Per-round attention of every sorted slot over its window.

    Returns (o_sorted [n_slots, D], lse_sorted [n_slots]); with `chunks`
    given, only those chunks' rows are filled (the rest are NaN).
    Variants: `codes` (from slot_codes) drops key slots whose (round, bucket)
    differs from the query slot's; `mult` (from pair_multiplicity) subtracts
    log N_ij from each kept logit."""
    x = np.asarray(x, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_slots = sorted_idx.shape[0]
    if n_slots % chunk_len:
        raise ValueError("chunk_len must divide n_hashes * L")
    n_chunks = n_slots // chunk_len
    D = x.shape[1]
    o = np.full((n_slots, v.shape[1]), np.nan)
    lse = np.full(n_slots, np.nan)
    for c in (range(n_chunks) if chunks is None else chunks):
        q_slots = np.arange(c * chunk_len, (c + 1) * chunk_len)
        k_slots = window_slots(n_slots, chunk_len, c)
        q_pos = sorted_idx[q_slots]
        k_pos = sorted_idx[k_slots]
        q = x[q_pos]
        k = x[k_pos]
        k_hat = k / np.maximum(np.linalg.norm(k, axis=1), KEY_NORM_FLOOR)[:, None]
        s = (q @ k_hat.T) / math.sqrt(D)
        s = np.where(q_pos[:, None] == k_pos[None, :], SELF_LOGIT, s)
        if mult is not None:  # every kept pair, the self pair included
            n = np.array([[mult[qi].get(kj, 1) for kj in k_pos] for qi in q_pos], dtype=np.float64)
            s = s - np.log(n)
        if causal:
            s = np.where(k_pos[None, :] > q_pos[:, None], -np.inf, s)
        if codes is not None:
            s = np.where(codes[k_slots][None, :] != codes[q_slots][:, None], -np.inf, s)
        m = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - m)
        den = np.sum(e, axis=1)
        o[c * chunk_len:(c + 1) * chunk_len] = (e @ v[k_pos]) / den[:, None]
        lse[c * chunk_len:(c + 1) * chunk_len] = m[:, 0] + np.log(den)
    return o, lse


# --------------------------------------------------------------------------
# Steps 4-5: unsort and combine the rounds (explainer page: union of rounds)
# --------------------------------------------------------------------------

def unsort_combine(o_sorted: np.ndarray, lse_sorted: np.ndarray, undo_idx: np.ndarray):
    """out_i = sum_r exp(lse_r(i) - LSE_i) o_r(i), LSE_i = logsumexp_r lse_r(i)."""
    o_r = o_sorted[undo_idx]          # [n_h, L, D]
    l_r = lse_sorted[undo_idx]        # [n_h, L]
    m = np.max(l_r, axis=0)
    lse = m + np.log(np.sum(np.exp(l_r - m), axis=0))
    w = np.exp(l_r - lse)
    out = np.sum(w[:, :, None] * o_r, axis=0)
    return out, lse


# --------------------------------------------------------------------------
# Whole forward pass
# --------------------------------------------------------------------------

def forward_problem(x, v, rot, n_buckets: int, n_hashes: int, chunk_len: int, causal: bool,
                    same_bucket: bool = False, dedup: bool = False):
    """One (batch, head) problem.  Returns a dict with every intermediate."""
    if n_buckets == 1:
        L = x.shape[0]
        buckets, margin = np.zeros((n_hashes, L), dtype=np.int64), np.full((n_hashes, L), np.inf)
    else:
        assert rot.shape[0] == n_hashes
        buckets, margin = hash_buckets(x, rot, n_buckets)
    sorted_idx, undo_idx = sort_by_bucket(buckets)
    codes = slot_codes(buckets, sorted_idx) if same_bucket else None
    mult = pair_multiplicity(sorted_idx, undo_idx, chunk_len, causal, codes) if dedup else None
    o_sorted, lse_sorted = chunk_attention(x, v, sorted_idx, chunk_len, causal, codes=codes, mult=mult)
    out, lse = unsort_combine(o_sorted, lse_sorted, undo_idx)
    return dict(buckets=buckets, margin=margin, sorted_idx=sorted_idx, undo_idx=undo_idx,
                o_sorted=o_sorted, lse_sorted=lse_sorted, out=out, lse=lse)


def forward(x, v, rot, n_buckets: int, n_hashes: int, chunk_len: int, causal: bool,
            same_bucket: bool = False, dedup: bool = False):
    """x, v: [B, H, L, D]; rot: [n_h, D, n_b/2] shared by every (b, h).
    Returns (out [B, H, L, D], lse [B, H, L]) in float64."""
    B, H, L, D = x.shape
    out = np.empty((B, H, L, v.shape[-1]))
    lse = np.empty((B, H, L))
    for b in range(B):
        for h in range(H):
            r = forward_problem(x[b, h], v[b, h], rot, n_buckets, n_hashes, chunk_len, causal, same_bucket, dedup)
            out[b, h], lse[b, h] = r["out"], r["lse"]
    return out, lse


def token_output(x, v, sorted_idx, undo_idx, chunk_len: int, causal: bool, i: int, codes=None, mult=None):
    """Output and LSE of the single token i of one problem, computed from its
    own window in every round (for sampled checks at sizes where the full
    oracle would be slow).  `codes` / `mult` as in chunk_attention."""
    n_h, L = undo_idx.shape
    o_r, l_r = [], []
    for r in range(n_h):
        g = int(undo_idx[r, i])
        c = g // chunk_len
        o, l = chunk_attention(x, v, sorted_idx, chunk_len, causal, chunks=[c], codes=codes, mult=mult)
        o_r.append(o[g])
        l_r.append(l[g])
    l_r = np.array(l_r)
    m = np.max(l_r)
    lse = m + np.log(np.sum(np.exp(l_r - m)))
    out = np.sum(np.exp(l_r - lse)[:, None] * np.array(o_r), axis=0)
    return out, lse


# --------------------------------------------------------------------------
# Exact attention and recall (explainer page: attention as nearest-neighbour
# search; it measures how much the hashed windows recover)
# --------------------------------------------------------------------------

def full_attention(x, v, causal: bool):
    """Dense shared-QK attention with the same key normalisation, scale,
    self rule and causal rule, one query at a time.  [L, D] -> ([L, D], [L])."""
    x = np.asarray(x, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L, D = x.shape
    k_hat = x / np.maximum(np.linalg.norm(x, axis=1), KEY_NORM_FLOOR)[:, None]
    out = np.empty((L, v.shape[1]))
    lse = np.empty(L)
    for i in range(L):
        s = (k_hat @ x[i]) / math.sqrt(D)
        s[i] = SELF_LOGIT
        if causal:
            s[i + 1:] = -np.inf
        m = np.max(s)
        e = np.exp(s - m)
        out[i] = (e @ v) / np.sum(e)
        lse[i] = m + np.log(np.sum(e))
    return out, lse


def union_attention(x, v, sorted_idx, undo_idx, chunk_len: int, causal: bool, codes=None):
    """Attention of every token over the SET of distinct tokens that are kept
    keys in any of its windows (each counted once), computed directly from
    that set: the definition the set-union variant must reproduce."""
    x = np.asarray(x, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_h, L = undo_idx.shape
    n_slots = sorted_idx.shape[0]
    D = x.shape[1]
    out = np.empty((L, v.shape[1]))
    lse = np.empty(L)
    for i in range(L):
        keys = set()
        for r in range(n_h):
            g = int(undo_idx[r, i])
            for gk in window_slots(n_slots, chunk_len, g // chunk_len):
                j = int(sorted_idx[gk])
                if causal and j > i:
                    continue
                if codes is not None and codes[gk] != codes[g]:
                    continue
                keys.add(j)
        ks = np.array(sorted(keys))
        k = x[ks]
        s = (x[i] @ (k / np.maximum(np.linalg.norm(k, axis=1), KEY_NORM_FLOOR)[:, None]).T) / math.sqrt(D)
        s = np.where(ks == i, SELF_LOGIT, s)
        m = np.max(s)
        e = np.exp(s - m)
        out[i] = e @ v[ks] / np.sum(e)
        lse[i] = m + np.log(np.sum(e))
    return out, lse


def attended_positions(sorted_idx, undo_idx, chunk_len: int, i: int) -> set:
    """Set of original positions inside token i's windows over all rounds."""
    n_h, L = undo_idx.shape
    n_slots = n_h * L
    seen = set()
    for r in range(n_h):
        c = int(undo_idx[r, i]) // chunk_len
        seen.update(int(p) for p in sorted_idx[window_slots(n_slots, chunk_len, c)])
    return seen


def recall_at_k(x, sorted_idx, undo_idx, chunk_len: int, queries, k: int) -> float:
    """Mean over `queries` of the fraction of the query's k nearest keys
    (largest logits, j != i) that fall inside its union of windows."""
    x = np.asarray(x, dtype=np.float64)
    k_hat = x / np.maximum(np.linalg.norm(x, axis=1), KEY_NORM_FLOOR)[:, None]
    hits = 0
    for i in queries:
        s = k_hat @ x[i]
        s[i] = -np.inf
        top = np.argpartition(-s, k)[:k]
        seen = attended_positions(sorted_idx, undo_idx, chunk_len, int(i))
        hits += sum(1 for j in top if int(j) in seen)
    return hits / (k * len(queries))


def attention_mass_recall(x, sorted_idx, undo_idx, chunk_len: int, queries) -> float:
    """Mean over `queries` of the exact (non-causal) attention weight that
    falls on keys inside the query's union of windows."""
    x = np.asarray(x, dtype=np.float64)
    L, D = x.shape
    k_hat = x / np.maximum(np.linalg.norm(x, axis=1), KEY_NORM_FLOOR)[:, None]
    tot = 0.0
    for i in queries:
        s = (k_hat @ x[i]) / math.sqrt(D)
        s[i] = SELF_LOGIT
        w = np.exp(s - np.max(s))
        w /= np.sum(w)
        seen = attended_positions(sorted_idx, undo_idx, chunk_len, int(i))
        tot += float(np.sum(w[sorted(seen)]))
    return tot / len(queries)
