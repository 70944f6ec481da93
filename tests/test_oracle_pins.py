"""Pins for the CPU oracle, against facts that do not come from the oracle.

Each test states what it pins and where the fact comes from: the collision law
and the angular-sector picture of the Reformer explainer page
(akshathtiwari.co.in/blog/reformer), closed forms worked by hand, exact
invariants, and brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O

_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    """A hand-worked fixture of tests/golden (each states its source and derivation)."""
    with open(os.path.join(_GOLDEN, name)) as f:
        return json.load(f)


def _unit(v):
    return v / np.linalg.norm(v)


# ---------------------------------------------------------------- hashing --

@pytest.mark.parametrize("theta", [math.pi / 12, math.pi / 6, math.pi / 3, math.pi / 2, 2 * math.pi / 3])
def test_collision_law_two_buckets(theta):
    """Explainer page, angular-LSH passage: P[h(x) = h(y)] = 1 - theta/pi.
    With two buckets the hash is one random hyperplane, where the law is exact."""
    rng = np.random.default_rng(11)
    D, N = 64, 20000
    q, _ = np.linalg.qr(rng.standard_normal((D, 2)))
    x = q[:, 0]
    y = math.cos(theta) * q[:, 0] + math.sin(theta) * q[:, 1]
    rot = rng.standard_normal((N, D, 1))
    b, _ = O.hash_buckets(np.stack([x, y]), rot, 2)
    freq = np.mean(b[:, 0] == b[:, 1])
    p = 1 - theta / math.pi
    assert abs(freq - p) < 5 * math.sqrt(p * (1 - p) / N) + 1e-12


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_two_dimensional_sectors_closed_form(k):
    """Explainer page, angular sectors after a rotation.  In two dimensions,
    with the n_b/2 = k projection directions at angles phi + j*pi/k, the entry
    m of [p ; -p] is |x| cos(alpha - phi - m*pi/k), so the bucket is the
    sector round((alpha - phi) * k / pi) mod 2k.  Pins the [+p ; -p] index
    layout and the argmax."""
    rng = np.random.default_rng(100 + k)
    D = 64
    phi = rng.uniform(0, 2 * math.pi)
    rot = np.zeros((1, D, k))
    for j in range(k):
        rot[0, 0, j] = math.cos(phi + j * math.pi / k)
        rot[0, 1, j] = math.sin(phi + j * math.pi / k)
    x = rng.standard_normal((3000, D))
    alpha = np.arctan2(x[:, 1], x[:, 0])
    t = (alpha - phi) * k / math.pi
    keep = np.abs((t - np.floor(t)) - 0.5) > 1e-6
    expect = np.mod(np.round(t[keep]).astype(np.int64), 2 * k)
    b, _ = O.hash_buckets(x[keep], rot, 2 * k)
    np.testing.assert_array_equal(b[0], expect)


def test_two_dimensional_sector_collision_rate():
    """Same construction with phi uniform: P_coll = max(0, 1 - k theta / pi)."""
    rng = np.random.default_rng(7)
    k, theta, N, D = 2, math.pi / 6, 20000, 64
    x = np.zeros((2, D))
    x[0, 0] = 1.0
    x[1, 0], x[1, 1] = math.cos(theta), math.sin(theta)
    phis = rng.uniform(0, 2 * math.pi, size=N)
    rot = np.zeros((N, D, k))
    for j in range(k):
        rot[:, 0, j] = np.cos(phis + j * math.pi / k)
        rot[:, 1, j] = np.sin(phis + j * math.pi / k)
    b, _ = O.hash_buckets(x, rot, 2 * k)
    p = max(0.0, 1 - k * theta / math.pi)
    assert abs(np.mean(b[:, 0] == b[:, 1]) - p) < 5 * math.sqrt(p * (1 - p) / N)


def test_hash_negation_and_scaling_invariants():
    """Negating x swaps every entry of [p ; -p] with its partner n_b/2 away, so
    h(-x) = (h(x) + n_b/2) mod n_b; scaling by a power of two is exact and
    leaves the argmax alone."""
    rng = np.random.default_rng(3)
    for n_b in (2, 8, 64, 1024):
        x = rng.standard_normal((200, 64)).astype(np.float32).astype(np.float64)
        rot = rng.standard_normal((3, 64, n_b // 2)).astype(np.float32).astype(np.float64)
        b, _ = O.hash_buckets(x, rot, n_b)
        bn, _ = O.hash_buckets(-x, rot, n_b)
        np.testing.assert_array_equal(bn, (b + n_b // 2) % n_b)
        for s in (0.125, 4.0):
            bs, _ = O.hash_buckets(s * x, rot, n_b)
            np.testing.assert_array_equal(bs, b)


def test_hash_exact_ties_take_lowest_index():
    """Ties in [p ; -p] go to the lowest index (duplicate or negated rotation
    columns make exact ties); x = 0 and n_b = 1 give bucket 0."""
    rng = np.random.default_rng(5)
    D, half = 64, 16
    rot = rng.standard_normal((1, D, half))
    dup = rot.copy()
    dup[0, :, 9] = dup[0, :, 2]
    b, _ = O.hash_buckets(dup[0, :, 2][None, :], dup, 2 * half)
    assert b[0, 0] == 2
    neg = rot.copy()
    neg[0, :, 9] = -neg[0, :, 2]
    b, _ = O.hash_buckets(neg[0, :, 2][None, :], neg, 2 * half)       # +p_2 ties -p_9
    assert b[0, 0] == 2
    b, _ = O.hash_buckets(-neg[0, :, 2][None, :], neg, 2 * half)      # +p_9 ties -p_2
    assert b[0, 0] == 9
    b, _ = O.hash_buckets(np.zeros((1, D)), rot, 2 * half)
    assert b[0, 0] == 0
    b, _ = O.hash_buckets(rng.standard_normal((5, D)), None, 1)
    assert not b.any()


def test_hash_decides_below_float64_resolution():
    """Exact p_9 = 1 + 2^-70 beats p_2 = 1, a difference float64 sums cannot
    see (they return a tie, which the lowest-index rule would give to 2).
    Pins that near-ties are decided in exact arithmetic."""
    D, half = 64, 16
    rot = np.zeros((1, D, half))
    rot[0, 0, 2] = 1.0
    rot[0, 0, 9], rot[0, 1, 9] = 1.0, 2.0 ** -70
    x = np.zeros((1, D))
    x[0, 0], x[0, 1] = 1.0, 1.0
    b, _ = O.hash_buckets(x, rot, 2 * half)
    assert b[0, 0] == 9
    b, _ = O.hash_buckets(-x, rot, 2 * half)
    assert b[0, 0] == half + 9


def test_hash_matches_exact_arithmetic_on_tiny_inputs():
    """Brute force in exact rational arithmetic on every token of a tiny case."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 8)).astype(np.float32).astype(np.float64)
    rot = rng.standard_normal((2, 8, 4)).astype(np.float32).astype(np.float64)
    b, _ = O.hash_buckets(x, rot, 8)
    for r in range(2):
        for i in range(6):
            assert b[r, i] == O.lsh_oracle._exact_bucket(x[i], rot[r])


# ------------------------------------------------------------------- sort --

def test_sort_counting_rank_closed_form():
    """Stable sort by (round, bucket, position): position i of round r lands in
    slot r*L + #{j : b_j < b_i} + #{j < i : b_j = b_i}; also a permutation per
    round with non-decreasing buckets, and undo . sorted = identity."""
    rng = np.random.default_rng(1)
    n_h, L, n_b = 3, 200, 7
    bk = rng.integers(0, n_b, size=(n_h, L))
    s, u = O.sort_by_bucket(bk)
    for r in range(n_h):
        seg = s[r * L:(r + 1) * L]
        assert sorted(seg.tolist()) == list(range(L))
        assert np.all(np.diff(bk[r, seg]) >= 0)
        for i in range(L):
            rank = sum(1 for j in range(L) if bk[r, j] < bk[r, i]) + \
                   sum(1 for j in range(i) if bk[r, j] == bk[r, i])
            assert s[r * L + rank] == i
            assert u[r, i] == r * L + rank
    assert np.array_equal(s[u.reshape(-1)], np.tile(np.arange(L), n_h))


# -------------------------------------------------------------- attention --

def _problem(seed, L, n_b, n_h, D=64):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    rot = None if n_b == 1 else rng.standard_normal((n_h, D, n_b // 2))
    return x, v, rot


@pytest.mark.parametrize("causal", [False, True])
def test_weights_sum_to_one(causal):
    """Every round's attention weights sum to 1: V = 1 gives o_r = 1 and out = 1.
    (A self-only round has lse near -1e5, where float64 differences of lse
    values carry about 1e5 * 2^-53 of absolute error, hence the combined bound.)"""
    x, _, rot = _problem(2, 48, 4, 3)
    r = O.forward_problem(x, np.ones((48, 64)), rot, 4, 3, 8, causal)
    np.testing.assert_allclose(r["o_sorted"], 1.0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["out"], 1.0, rtol=0, atol=1e-10)


def test_causal_first_position_is_self_only():
    """Causal: position 0 has no earlier key, so it attends only to itself
    (every round exactly; the combine of rounds whose lse is -1e5 carries
    float64 rounding of order 1e5 * 2^-53)."""
    x, v, rot = _problem(4, 64, 8, 3)
    r = O.forward_problem(x, v, rot, 8, 3, 8, True)
    np.testing.assert_allclose(r["out"][0], v[0], rtol=0, atol=1e-10)
    for rr in range(3):
        np.testing.assert_array_equal(r["o_sorted"][r["undo_idx"][rr, 0]], v[0])


def _brute_force(x, v, causal):
    """Textbook dense attention written as loops: logit x_i . x_j / |x_j| / sqrt(D),
    self at -1e5, causal excludes j > i."""
    L, D = x.shape
    out = np.zeros_like(v)
    lse = np.zeros(L)
    for i in range(L):
        logits = []
        for j in range(L):
            if causal and j > i:
                continue
            s = -1e5 if j == i else float(x[i] @ x[j]) / math.sqrt(float(x[j] @ x[j])) / math.sqrt(D)
            logits.append((j, s))
        m = max(s for _, s in logits)
        z = sum(math.exp(s - m) for _, s in logits)
        for j, s in logits:
            out[i] += math.exp(s - m) / z * v[j]
        lse[i] = m + math.log(z)
    return out, lse


@pytest.mark.parametrize("n_h", [1, 2, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_one_bucket_one_chunk_is_full_attention(n_h, causal):
    """n_b = 1 and chunk_len = L: every window holds all tokens (twice), so the
    result is dense attention; duplicates scale every weight alike."""
    L = 12
    x, v, _ = _problem(20 + n_h, L, 1, n_h)
    r = O.forward_problem(x, v, None, 1, n_h, L, causal)
    out, lse = _brute_force(x, v, causal)
    np.testing.assert_allclose(r["out"], out, rtol=0, atol=1e-10)
    # each token appears twice per round and once per round in n_h rounds
    np.testing.assert_allclose(r["lse"], lse + math.log(2 * n_h), rtol=1e-14, atol=1e-12)
    fo, fl = O.full_attention(x, v, causal)
    np.testing.assert_allclose(fo, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(fl, lse, rtol=0, atol=1e-12)


def test_hand_worked_logits_scale_and_key_normalisation():
    """Four tokens, one bucket, one chunk (the window is the chunk twice), logits
    worked by hand in tests/golden/hand_logits.json: keys normalised, queries
    not, scale 1/sqrt(64) = 1/8, self excluded.  With one-hot values, out_i is
    the weight vector."""
    g = _golden("hand_logits.json")
    D = 64
    x = np.zeros((4, D))
    for i, d, val in g["x_nonzero"]:
        x[i, d] = val
    v = np.eye(4, D)
    w = [[0.0 if lg is None else math.exp(lg) for lg in row] for row in g["logits"]]
    expect = np.zeros((4, D))
    for i in range(4):
        expect[i, :4] = np.array(w[i]) / sum(w[i])
    r = O.forward_problem(x, v, None, 1, 1, 4, False)
    np.testing.assert_allclose(r["out"], expect, rtol=0, atol=1e-14)
    np.testing.assert_allclose(r["lse"], [math.log(g["window_multiplicity"] * sum(wi)) for wi in w], rtol=0,
                               atol=1e-14)


# Two buckets, two rounds, x_i = +e0 for even i and -e0 for odd i; round 0's
# single rotation column is +e0 and round 1's is -e0.  The chunks of the sorted
# slots and each chunk's window (previous chunk, cyclic over all rounds, plus
# itself) are worked by hand in tests/golden/windows_two_rounds.json.
_WIN = _golden("windows_two_rounds.json")
HAND_WINDOWS = {int(c): set(w) for c, w in _WIN["windows"].items()}
_CPR = _WIN["L"] // _WIN["chunk_len"]  # chunks per round
HAND_CHUNK_OF = {(int(c) // _CPR, p): int(c) for c, ps in _WIN["chunks"].items() for p in ps}


@pytest.mark.parametrize("causal", [False, True])
def test_hand_enumerated_windows(causal):
    """Pins the look-back to the previous chunk, its wrap across rounds, the
    hash sign layout and the stable sort: with one-hot values each round's
    output is its weight vector, whose support must be the hand-enumerated
    window minus the token itself (keys after it dropped when causal; the
    token alone when nothing else is left)."""
    L, D, n_h = _WIN["L"], 64, _WIN["n_hashes"]
    x = np.zeros((L, D))
    x[:, 0] = _WIN["x_dim0"]
    rot = np.zeros((n_h, D, _WIN["n_buckets"] // 2))
    rot[:, 0, 0] = _WIN["rotation_dim0"]
    v = np.eye(L, D)
    r = O.forward_problem(x, v, rot, _WIN["n_buckets"], n_h, _WIN["chunk_len"], causal)
    for rr in range(n_h):
        for i in range(L):
            win = HAND_WINDOWS[HAND_CHUNK_OF[(rr, i)]] - {i}
            if causal:
                win = {j for j in win if j < i}
            expect = win if win else {i}
            o = r["o_sorted"][r["undo_idx"][rr, i]]
            assert set(np.nonzero(o > 0)[0].tolist()) == expect, (rr, i)


def test_uniform_logits_window_means():
    """All keys in one direction: every non-self logit is 1/8, so each round's
    output is the plain mean of the window's values without the token itself.
    One bucket, L = 16, chunks of 4, two rounds with the identity order, so the
    windows are {12..15, 0..3}, {0..7}, {4..11}, {8..15} for tokens in 0..3,
    4..7, 8..11, 12..15.  With v_j = j the outputs are (60 - i)/7,
    (28 - i)/7, (60 - i)/7, (92 - i)/7 and every LSE is 1/8 + log 14."""
    L, D = 16, 64
    x = np.zeros((L, D))
    x[:, 0] = 1.0
    v = np.repeat(np.arange(L, dtype=np.float64)[:, None], D, axis=1)
    r = O.forward_problem(x, v, None, 1, 2, 4, False)
    sums = [60, 28, 60, 92]
    expect = np.array([(sums[i // 4] - i) / 7 for i in range(L)])
    np.testing.assert_allclose(r["out"][:, 0], expect, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["lse"], 0.125 + math.log(14), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- combine --

def test_single_round_combine_is_identity():
    x, v, rot = _problem(6, 64, 8, 1)
    r = O.forward_problem(x, v, rot, 8, 1, 16, False)
    np.testing.assert_array_equal(r["out"], r["o_sorted"][r["undo_idx"][0]])
    np.testing.assert_allclose(r["lse"], r["lse_sorted"][r["undo_idx"][0]], rtol=0, atol=1e-14)


def test_identical_rounds_equal_one_round():
    """Repeating the same rotation gives identical windows in every round
    (the wrap joins identical chunks), so the combined output equals one round."""
    x, v, rot = _problem(8, 64, 8, 1)
    one = O.forward_problem(x, v, rot, 8, 1, 16, True)
    three = O.forward_problem(x, v, np.repeat(rot, 3, axis=0), 8, 3, 16, True)
    np.testing.assert_allclose(three["out"], one["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(three["lse"], one["lse"] + math.log(3), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_combine_equals_softmax_over_the_multiset_union(causal):
    """The log-sum-exp combine equals one softmax over the concatenation of all
    rounds' windows (duplicates kept), computed here with plain loops."""
    L, C, n_h, n_b = 32, 8, 3, 4
    x, v, rot = _problem(12, L, n_b, n_h)
    r = O.forward_problem(x, v, rot, n_b, n_h, C, causal)
    s_idx, u = r["sorted_idx"], r["undo_idx"]
    n_slots = n_h * L
    for i in range(L):
        pairs = []
        for rr in range(n_h):
            c = u[rr, i] // C
            for g in list(range(((c - 1) % (n_slots // C)) * C, ((c - 1) % (n_slots // C)) * C + C)) + \
                    list(range(c * C, c * C + C)):
                j = int(s_idx[g])
                if causal and j > i:
                    continue
                s = -1e5 if j == i else float(x[i] @ x[j]) / float(np.linalg.norm(x[j])) / 8.0
                pairs.append((j, s))
        m = max(s for _, s in pairs)
        z = sum(math.exp(s - m) for _, s in pairs)
        out = sum(math.exp(s - m) / z * v[j] for j, s in pairs)
        np.testing.assert_allclose(r["out"][i], out, rtol=0, atol=1e-12)
        assert abs(r["lse"][i] - (m + math.log(z))) < 1e-12


# ----------------------------------------------------------------- recall --
# Recall is what the explainer's nearest-neighbour reading of attention and its
# multi-round sentence are about: the share of a query's true nearest keys that
# its hashed windows (union over rounds) contain.  The pins below fix the
# neighbour order, the windows and the expected fractions by hand.

_REC = _golden("recall_circle.json")


def _circle_tokens():
    """Eight tokens in the plane of the first two dims (D = 64, the rest zero) at
    the angles and norms of tests/golden/recall_circle.json (token i at 2^i - 1
    degrees, norm 2^i): the neighbours of query i by cosine are i-1, ..., 0, then
    i+1, ..., 7.  The norms grow with i, so a key left unnormalised would reorder
    them."""
    deg = np.array(_REC["angles_deg"], dtype=np.float64)
    rho = np.array(_REC["norms"], dtype=np.float64)
    x = np.zeros((8, 64))
    x[:, 0] = rho * np.cos(np.radians(deg))
    x[:, 1] = rho * np.sin(np.radians(deg))
    return x


# One round, chunk_len 2, sorted order 0 1 | 4 5 | 2 3 | 6 7; a second round in
# position order, whose first chunk looks back at round 0's last chunk {6, 7}
# (and round 0's first chunk at round 1's last, again {6, 7}).  Windows and
# expected fractions: tests/golden/recall_circle.json.
_C = _REC["chunk_len"]
_S1 = np.array(_REC["one_round"]["sorted_idx"])
_U1 = np.array(_REC["one_round"]["undo_idx"])
_S2 = np.array(_REC["two_rounds"]["sorted_idx"])
_U2 = np.array(_REC["two_rounds"]["undo_idx"])


def _frac(nd):
    return nd[0] / nd[1]


def test_hand_windows_of_the_recall_pins():
    for key, s, u in (("one_round", _S1, _U1), ("two_rounds", _S2, _U2)):
        for i, w in _REC[key]["windows"].items():
            assert O.attended_positions(s, u, _C, int(i)) == set(w), (key, i)


def test_recall_at_k_hand_counts_one_round():
    """Hand counts of the first three neighbours inside the one-round windows:
    R@1 = 5/8, R@2 = 5/16, R@3 = 8/24.  A query counted as its own neighbour
    gives R@1 = 1; the smallest logits, or keys left unnormalised, give other
    counts."""
    x = _circle_tokens()
    g = _REC["one_round"]
    for k, nd in g["recall_at_k"].items():
        assert O.recall_at_k(x, _S1, _U1, _C, range(8), int(k)) == _frac(nd), k
    # the mean is over the queries given
    for sub in g["recall_subsets"]:
        assert O.recall_at_k(x, _S1, _U1, _C, sub["queries"], sub["k"]) == _frac(sub["value"])


def test_recall_at_k_hand_counts_two_rounds():
    """Over the union of both rounds' windows every nearest neighbour is in
    (R@1 = 1); second neighbours miss for q0 and q1 only (R@2 = 14/16), third
    ones too (R@3 = 20/24).  The union contains the first round's windows, so
    recall cannot drop."""
    x = _circle_tokens()
    for k, nd in _REC["two_rounds"]["recall_at_k"].items():
        assert O.recall_at_k(x, _S2, _U2, _C, range(8), int(k)) == _frac(nd), k


def test_recall_at_k_equals_a_full_sort_on_random_problems():
    """Second definition: the k best keys by a full stable sort of the cosine
    (ties impossible on Gaussian data), the window membership by enumerating
    every round's window slots, per query."""
    rng = np.random.default_rng(31)
    for L, n_h, C, k in ((64, 2, 8, 1), (96, 3, 16, 5), (128, 1, 32, 16)):
        x = rng.standard_normal((L, 64))
        s, u = O.sort_by_bucket(rng.integers(0, 4, (n_h, L)))
        q = rng.choice(L, 20, replace=False)
        hits = 0
        for i in q:
            cos = [float(x[j] @ x[i]) / float(np.linalg.norm(x[j])) if j != i else -math.inf for j in range(L)]
            best = sorted(range(L), key=lambda j: -cos[j])[:k]
            win = set()
            for r in range(n_h):
                c = int(u[r, i]) // C
                prev = (c - 1) % (n_h * L // C)
                win |= {int(s[g]) for g in range(prev * C, prev * C + C)} | {int(s[g]) for g in range(c * C, c * C + C)}
            hits += sum(1 for j in best if j in win)
        assert O.recall_at_k(x, s, u, C, q, k) == hits / (k * len(q))


def test_attention_mass_recall_uniform_logits():
    """All tokens along one direction with distinct norms: with keys normalised
    every logit j != i equals |x_i| / 8, so the exact weights are uniform over
    the L - 1 other tokens and the mass inside a window set W (which holds the
    query itself, at weight 0) is (|W| - 1) / (L - 1).  One round: |W| = 4 for
    every query -> 3/7.  Two rounds: |W| = 4 for q0, q1 and 6 for the others ->
    (2 * 3/7 + 6 * 5/7) / 8 = 9/14."""
    x = np.zeros((8, 64))
    x[:, 5] = np.arange(1, 9, dtype=np.float64)
    assert abs(O.attention_mass_recall(x, _S1, _U1, _C, range(8)) - _frac(_REC["one_round"]["mass_uniform"])) < 1e-14
    assert abs(O.attention_mass_recall(x, _S2, _U2, _C, range(8)) - _frac(_REC["two_rounds"]["mass_uniform"])) < 1e-14


def test_attention_mass_recall_two_directions():
    """Tokens 0-3 at +e1 (norm 1), tokens 4-7 at -2 e1 (norm 2); scale 1/8, keys
    normalised.  A query in the first group sees logit +1/8 on the three others
    of its group and -1/8 on the second group; a query in the second group sees
    +1/4 on its group and -1/4 on the first.  One-round windows:
      q0..q3 (W holds 1 other of its group, 2 of the other):
          (e^{1/8} + 2 e^{-1/8}) / (3 e^{1/8} + 4 e^{-1/8})
      q4..q7 (W holds 1 other of its group, 2 of the other):
          (e^{1/4} + 2 e^{-1/4}) / (3 e^{1/4} + 4 e^{-1/4})
    The mean is the average of the two.  Negated logits, another scale or a
    query weighting its own key give other values."""
    x = np.zeros((8, 64))
    x[:4, 0] = 1.0
    x[4:, 0] = -2.0
    a = math.exp(1 / 8)
    b = math.exp(1 / 4)
    first = (a + 2 / a) / (3 * a + 4 / a)
    second = (b + 2 / b) / (3 * b + 4 / b)
    assert abs(O.attention_mass_recall(x, _S1, _U1, 2, range(4)) - first) < 1e-14
    assert abs(O.attention_mass_recall(x, _S1, _U1, 2, range(4, 8)) - second) < 1e-14
    assert abs(O.attention_mass_recall(x, _S1, _U1, 2, range(8)) - (first + second) / 2) < 1e-14


def test_recall_is_one_when_every_key_is_in_the_window():
    x, _, _ = _problem(14, 32, 1, 1)
    s, u = O.sort_by_bucket(np.zeros((1, 32), dtype=np.int64))
    assert O.recall_at_k(x, s, u, 32, range(32), 5) == 1.0
    assert abs(O.attention_mass_recall(x, s, u, 32, range(32)) - 1.0) < 1e-12


def test_more_rounds_raise_recall_on_clustered_keys():
    """Explainer page, multi-round passage: more independent rounds raise
    recall.  The 8-round run shares its first two rotations with the 2-round
    run, so its windows include the 2-round ones except at the wrap of the
    first chunk."""
    from lsh_attention_amd import inputs as I
    inp = I.make_inputs("peaked_vmf_16k", n_hashes=8, B=1, H=1, L=2048)
    x = inp.qk.values[0, 0].astype(np.float64)
    rot = inp.rot.values.astype(np.float64)[:, :, :16]     # 32 buckets: mean occupancy 64
    q = range(0, 2048, 16)
    rec = {}
    for n_h in (2, 8):
        b, _ = O.hash_buckets(x, rot[:n_h], 32)
        s, u = O.sort_by_bucket(b)
        rec[n_h] = O.recall_at_k(x, s, u, 64, q, 16)
    assert rec[8] > rec[2]


# ----------------------------------------------- attended-set variants --
# Explainer page: a token "attends to its bucket-mates" (same_bucket) and the
# rounds' buckets are "unioned" (dedup: every distinct key once).

def _attend(x, v, i, keys, causal):
    """Loop softmax of query i over an explicit key multiset (self at -1e5,
    causal drops j > i); returns (out, lse)."""
    D = x.shape[1]
    logits = []
    for j in keys:
        if causal and j > i:
            continue
        s = -1e5 if j == i else float(x[i] @ x[j]) / math.sqrt(float(x[j] @ x[j])) / math.sqrt(D)
        logits.append((j, s))
    m = max(s for _, s in logits)
    z = sum(math.exp(s - m) for _, s in logits)
    out = sum(math.exp(s - m) / z * v[j] for j, s in logits)
    return out, m + math.log(z)


def _aligned_rotation(x, seed, L):
    """A one-column rotation (n_b = 2) and sign flips of x such that exactly
    L/2 tokens fall in bucket 0 (x . r > 0) and L/2 in bucket 1."""
    rng = np.random.default_rng(seed)
    r = rng.standard_normal(x.shape[1])
    pos = rng.permutation(L)[: L // 2]
    x = x.copy()
    p = x @ r
    for i in range(L):
        want = i in set(pos.tolist())
        if (p[i] > 0) != want:
            x[i] = -x[i]
    return x, r


def test_same_bucket_with_one_bucket_and_round_is_the_base_method():
    """n_b = 1, one round: every key slot holds the query's (round, bucket), so
    the mask removes nothing."""
    x, v, _ = _problem(31, 192, 1, 1)
    for causal in (False, True):
        a = O.forward_problem(x, v, None, 1, 1, 64, causal)
        b = O.forward_problem(x, v, None, 1, 1, 64, causal, same_bucket=True)
        np.testing.assert_array_equal(a["out"], b["out"])
        np.testing.assert_array_equal(a["lse"], b["lse"])


@pytest.mark.parametrize("causal", [False, True])
def test_same_bucket_aligned_buckets_is_attention_among_bucket_mates(causal):
    """Two buckets of exactly 64 tokens, one round: each bucket is one chunk, the
    look-back chunk is the other bucket and masked, so every token attends to
    exactly its bucket-mates (computed here straight from the bucket sets)."""
    x, v, _ = _problem(32, 128, 2, 1)
    x, r = _aligned_rotation(x, 5, 128)
    rot = r[None, :, None]
    res = O.forward_problem(x, v, rot, 2, 1, 64, causal, same_bucket=True)
    bk = (x @ r <= 0).astype(int)  # argmax of [p, -p]: bucket 0 iff p > 0
    assert np.array_equal(res["buckets"][0], bk)
    for i in range(128):
        mates = [j for j in range(128) if bk[j] == bk[i]]
        out, lse = _attend(x, v, i, mates, causal)
        np.testing.assert_allclose(res["out"][i], out, rtol=0, atol=1e-10)
        assert abs(res["lse"][i] - lse) < 1e-9


def test_same_bucket_two_aligned_rounds_is_the_multiset_union_of_bucket_mates():
    """Two rounds, each with exactly-aligned buckets: the combine is softmax over
    the multiset union of the two rounds' bucket-mate sets."""
    x, v, _ = _problem(33, 128, 2, 2)
    x, r0 = _aligned_rotation(x, 6, 128)
    # second round: another column that splits the (flipped) tokens 64/64
    rng = np.random.default_rng(7)
    while True:
        r1 = rng.standard_normal(64)
        if int(np.sum(x @ r1 > 0)) == 64:
            break
    rot = np.stack([r0, r1])[:, :, None]
    res = O.forward_problem(x, v, rot, 2, 2, 64, False, same_bucket=True)
    b0, b1 = (x @ r0 <= 0).astype(int), (x @ r1 <= 0).astype(int)
    for i in range(0, 128, 5):
        keys = [j for j in range(128) if b0[j] == b0[i]] + [j for j in range(128) if b1[j] == b1[i]]
        out, lse = _attend(x, v, i, keys, False)
        np.testing.assert_allclose(res["out"][i], out, rtol=0, atol=1e-10)
        assert abs(res["lse"][i] - lse) < 1e-9


@pytest.mark.parametrize("causal", [False, True])
def test_dedup_with_identical_rounds_is_one_round(causal):
    """All rounds use the same rotation, so every round's windows hold the same
    tokens: the union of n_h rounds is one round's window set, and the
    set-union variant must equal the one-round result (lse included)."""
    x, v, rot = _problem(34, 256, 8, 1)
    one = O.forward_problem(x, v, rot, 8, 1, 64, causal)
    rot3 = np.repeat(rot, 3, axis=0)
    three = O.forward_problem(x, v, rot3, 8, 3, 64, causal, dedup=True)
    np.testing.assert_allclose(three["out"], one["out"], rtol=0, atol=1e-10)
    np.testing.assert_allclose(three["lse"], one["lse"], rtol=0, atol=1e-9)
    plain = O.forward_problem(x, v, rot3, 8, 3, 64, causal)  # with multiplicity: lse + log 3
    np.testing.assert_allclose(plain["lse"], one["lse"] + math.log(3), rtol=0, atol=1e-9)


def test_dedup_in_one_round_changes_nothing():
    """One round, at least two chunks: a window never holds a token twice."""
    x, v, rot = _problem(35, 192, 8, 1)
    for causal in (False, True):
        a = O.forward_problem(x, v, rot, 8, 1, 64, causal)
        b = O.forward_problem(x, v, rot, 8, 1, 64, causal, dedup=True)
        np.testing.assert_allclose(a["out"], b["out"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(a["lse"], b["lse"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("same_bucket", [False, True])
def test_dedup_equals_attention_over_the_union_set(causal, same_bucket):
    """The per-occurrence -log N route (round softmaxes + combine) equals plain
    softmax over the set of distinct kept keys, built directly per token."""
    x, v, rot = _problem(36, 192, 4, 3)
    res = O.forward_problem(x, v, rot, 4, 3, 64, causal, same_bucket=same_bucket, dedup=True)
    codes = O.slot_codes(res["buckets"], res["sorted_idx"]) if same_bucket else None
    uo, ul = O.union_attention(x, v, res["sorted_idx"], res["undo_idx"], 64, causal, codes)
    np.testing.assert_allclose(res["out"], uo, rtol=0, atol=1e-10)
    np.testing.assert_allclose(res["lse"], ul, rtol=0, atol=1e-9)


def test_dedup_causal_first_position_lse_is_the_self_logit():
    """Causal position 0 keeps only itself in every window; counted once over the
    union, its lse is exactly the self logit."""
    x, v, rot = _problem(37, 128, 4, 3)
    res = O.forward_problem(x, v, rot, 4, 3, 64, True, dedup=True)
    np.testing.assert_allclose(res["out"][0], v[0], rtol=0, atol=1e-10)
    assert abs(res["lse"][0] - (-1e5)) < 1e-9


def test_same_bucket_masks_equal_bucket_ids_of_another_round():
    """Round 0 puts every token in bucket 0 (a zero rotation column: [0, -0]
    ties, lowest index); round 1 splits them 64/64.  Round 1's first chunk
    (bucket 0) looks back at round 0's last chunk, also bucket 0 but another
    round, which must stay masked.  Round 0's chunks hold positions 0-63 and
    64-127 (one bucket, position order); its first chunk looks back at round
    1's last chunk (masked), its second at its first."""
    x, v, _ = _problem(38, 128, 2, 2)
    x, r1 = _aligned_rotation(x, 8, 128)
    rot = np.stack([np.zeros(64), r1])[:, :, None]
    res = O.forward_problem(x, v, rot, 2, 2, 64, False, same_bucket=True)
    assert np.all(res["buckets"][0] == 0)
    b1 = (x @ r1 <= 0).astype(int)
    for i in range(0, 128, 3):
        keys = list(range(64)) if i < 64 else list(range(128))
        keys += [j for j in range(128) if b1[j] == b1[i]]
        out, lse = _attend(x, v, i, keys, False)
        np.testing.assert_allclose(res["out"][i], out, rtol=0, atol=1e-10)
        assert abs(res["lse"][i] - lse) < 1e-9


def test_sampled_multiplicity_and_token_output_agree_with_the_full_variant():
    """The sampled forms used at long sequence lengths (multiplicity for a
    subset of query tokens, one token's output from its own windows) give the
    full variant computation's values for those tokens."""
    x, v, rot = _problem(35, 256, 4, 3)
    for causal in (False, True):
        full = O.forward_problem(x, v, rot, 4, 3, 64, causal, same_bucket=True, dedup=True)
        si, ui = full["sorted_idx"], full["undo_idx"]
        codes = O.slot_codes(full["buckets"], si)
        every = O.pair_multiplicity(si, ui, 64, causal, codes)
        toks = [0, 5, 131, 255]
        some = O.pair_multiplicity(si, ui, 64, causal, codes, tokens=toks)
        for i in range(256):
            assert some[i] == (every[i] if i in toks else {})
        for i in toks:
            o, l = O.token_output(x, v, si, ui, 64, causal, i, codes=codes, mult=some)
            np.testing.assert_allclose(o, full["out"][i], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(l, full["lse"][i], rtol=1e-12, atol=1e-12)
