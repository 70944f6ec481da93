"""HIP path vs the CPU oracle, element by element, through the C ABI.

Integer results (buckets, permutations) must match bit for bit; the hash is
decided exactly on both sides, and oracle near-ties (margin < 1e-6 on the unit
vector) are counted and printed.  Each floating-point stage is fed the GPU's
own upstream results, so a stage is checked on its own; the fused call is also
checked end to end against the oracle's own forward pass.
"""
import numpy as np
import pytest
import torch

import oracle as O
from _helpers import TOL, f64, lse_check, rel_check, to_device, upload
from lsh_attention_amd import binding as bd
from lsh_attention_amd import inputs as I

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-parity]", *a, flush=True)


def run_stages(qk, v, rot, n_b, n_h, causal):
    buckets = bd.lsh_hash(qk, rot, n_b, n_h)
    sorted_idx, undo_idx = bd.lsh_sort(buckets, n_b)
    o_sorted, lse_sorted = bd.lsh_chunk_attn(qk, v, sorted_idx, n_h, 64, causal)
    out, lse = bd.lsh_unsort_combine(o_sorted, lse_sorted, undo_idx)
    torch.cuda.synchronize()
    return buckets, sorted_idx, undo_idx, o_sorted, lse_sorted, out, lse


REDUCED = [
    ("single_head_fp32", dict(), 1),
    ("mlm_small_512", dict(B=4, H=2), 4),
    ("causal_lm_4k", dict(B=1, H=2), 4),
    ("long_seq_64k", dict(B=1, H=2, L=4160), 8),   # 3 sort tiles, ragged hash block
    ("peaked_vmf_16k", dict(B=1, H=2), 2),
    ("peaked_vmf_16k", dict(B=1, H=2), 8),
]


@pytest.mark.parametrize("name,shape,n_h", REDUCED, ids=[f"{n}-h{h}" for n, _, h in REDUCED])
def test_all_stages_match_oracle(gpu_lib, name, shape, n_h):
    inp = I.make_inputs(name, n_hashes=n_h, **shape)
    w = inp.workload
    B, H, L, _ = inp.qk.values.shape
    say(f"case {name} B{B} H{H} L{L} n_b{w.n_buckets} n_h{n_h} causal={w.causal} {w.dtype}")
    qk, v, rot = upload(inp)
    buckets, sidx, undo, o_s, l_s, out, lse = run_stages(qk, v, rot, w.n_buckets, n_h, w.causal)
    out_f, lse_f = bd.reformer_lsh_attn_fwd(qk, v, rot, w.n_buckets, n_h, 64, w.causal)
    torch.cuda.synchronize()
    tol = TOL[w.dtype]
    # The fused call takes its per-token scales from the hash pass and keeps the
    # per-round results in token order; it agrees with the staged calls to rounding.
    rel_check(f64(out_f), f64(out), tol, "fused vs staged")
    gfo, gfl = f64(out_f), f64(lse_f)
    gb, gs, gu = buckets.cpu().numpy(), sidx.cpu().numpy(), undo.cpu().numpy()
    go, gl, gout, glse = f64(o_s), f64(l_s), f64(out), f64(lse)
    rot64 = None if inp.rot is None else inp.rot.values.astype(np.float64)
    near = 0
    for b in range(B):
        for h in range(H):
            x = inp.qk.values[b, h].astype(np.float64)
            vv = inp.v.values[b, h].astype(np.float64)
            ob, margin = O.hash_buckets(x, rot64, w.n_buckets)
            near += int(np.sum(margin < 1e-6))
            np.testing.assert_array_equal(gb[b, h], ob, err_msg=f"buckets b{b} h{h}")
            os_, ou = O.sort_by_bucket(gb[b, h].astype(np.int64))
            np.testing.assert_array_equal(gs[b, h], os_, err_msg=f"sorted_idx b{b} h{h}")
            np.testing.assert_array_equal(gu[b, h], ou, err_msg=f"undo_idx b{b} h{h}")
            oo, ol = O.chunk_attention(x, vv, gs[b, h].astype(np.int64), 64, w.causal)
            rel_check(go[b, h], oo, tol, f"o_sorted b{b} h{h}")
            lse_check(gl[b, h], ol, f"lse_sorted b{b} h{h}")
            co, cl = O.unsort_combine(go[b, h], gl[b, h], gu[b, h].astype(np.int64))
            rel_check(gout[b, h], co, tol, f"combine b{b} h{h}")
            lse_check(glse[b, h], cl, f"combine lse b{b} h{h}")
            ref = O.forward_problem(x, vv, rot64, w.n_buckets, n_h, 64, w.causal)
            rel_check(gout[b, h], ref["out"], tol, f"staged end-to-end b{b} h{h}")
            lse_check(glse[b, h], ref["lse"], f"staged end-to-end lse b{b} h{h}")
            rel_check(gfo[b, h], ref["out"], tol, f"fused end-to-end b{b} h{h}")
            lse_check(gfl[b, h], ref["lse"], f"fused end-to-end lse b{b} h{h}")
    say(f"  ok; oracle near-ties (margin < 1e-6): {near} of {B * H * n_h * L} token-rounds")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n_h", [1, 3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_bucket_one_chunk_equals_full_attention(gpu_lib, dtype, n_h, causal):
    """n_b = 1 and L = chunk_len = 64: the fused pass is dense attention."""
    say(f"case brute-force {dtype} n_h{n_h} causal={causal}")
    qk_t = I.gaussian(77, (1, 2, 64, 64), dtype)
    v_t = I.gaussian(78, (1, 2, 64, 64), dtype)
    out, lse = bd.reformer_lsh_attn_fwd(to_device(qk_t), to_device(v_t), None, 1, n_h, 64, causal)
    torch.cuda.synchronize()
    for h in range(2):
        fo, fl = O.full_attention(qk_t.values[0, h].astype(np.float64), v_t.values[0, h].astype(np.float64), causal)
        rel_check(f64(out)[0, h], fo, TOL[dtype], f"brute force h{h}")
        lse_check(f64(lse)[0, h], fl + np.log(2 * n_h), f"brute force lse h{h}")


def _tie_inputs(dtype, L=320):
    """Rotations with duplicated and negated columns and tokens placed on them,
    plus zero rows: every kind of exact tie of [p ; -p]."""
    rng = np.random.default_rng(5)
    n_h, half = 2, 16
    rot = rng.standard_normal((n_h, 64, half)).astype(np.float32)
    rot[:, :, 9] = rot[:, :, 2]
    rot[:, :, 11] = -rot[:, :, 4]
    rot[:, :, 15] = rot[:, :, 15] * 0
    x = rng.standard_normal((1, 1, L, 64)).astype(np.float32)
    x[0, 0, 0::5] = rot[0, :, 2]
    x[0, 0, 1::5] = -rot[0, :, 4]
    x[0, 0, 2::5] = 0.0
    x[0, 0, 3::5] = rot[1, :, 11]
    if dtype == "bf16":
        rt = I.Tensor(I.f32_from_bf16_bits(I.bf16_bits_from_f32(rot)), I.bf16_bits_from_f32(rot))
        xt = I.Tensor(I.f32_from_bf16_bits(I.bf16_bits_from_f32(x)), I.bf16_bits_from_f32(x))
    else:
        rt, xt = I.Tensor(rot), I.Tensor(x)
    return xt, rt, 2 * half, n_h


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_exact_ties_take_lowest_index(gpu_lib, dtype):
    xt, rt, n_b, n_h = _tie_inputs(dtype)
    say(f"case exact ties {dtype}")
    got = bd.lsh_hash(to_device(xt), to_device(rt), n_b, n_h).cpu().numpy()
    ref, _ = O.hash_buckets(xt.values[0, 0].astype(np.float64), rt.values.astype(np.float64), n_b)
    np.testing.assert_array_equal(got[0, 0], ref)
    assert np.all(got[0, 0, 0, 0::5] == 2)           # +p_2 ties +p_9
    assert np.all(got[0, 0, :, 2::5] == 0)           # zero vector


def test_every_token_needs_the_exact_path(gpu_lib):
    """All rotation columns come in identical pairs, so every token's top two
    scores tie and every token-round goes through the float64 re-decision."""
    say("case all-tied fixup queue")
    rng = np.random.default_rng(8)
    half, n_h = 64, 2
    base = rng.standard_normal((n_h, 64, half // 2)).astype(np.float32)
    rot = np.repeat(base, 2, axis=2)
    rt = I.Tensor(I.f32_from_bf16_bits(I.bf16_bits_from_f32(rot)), I.bf16_bits_from_f32(rot))
    xt = I.gaussian(9, (2, 2, 576, 64), "bf16")
    got = bd.lsh_hash(to_device(xt), to_device(rt), 2 * half, n_h).cpu().numpy()
    for b in range(2):
        for h in range(2):
            ref, _ = O.hash_buckets(xt.values[b, h].astype(np.float64), rt.values.astype(np.float64), 2 * half)
            np.testing.assert_array_equal(got[b, h], ref)
    assert np.all(got % 2 == 0)  # the lower index of each identical pair


def test_near_ties_only_float64_separates(gpu_lib):
    """fp32 rotation columns in pairs that differ by one ulp in coordinate 0: the
    pair's two scores differ by |x_0| ulp(r_0), far inside the fp32 error bound,
    so which of the two wins is decided by the float64 re-scoring of the
    candidates, and depends on the sign of x_0 (both members must occur).
    |x_0| >= 0.5 and |r_0| >= 0.25 keep each pair's gap at or above 2^-26; the
    smallest top-two gap in these inputs is 7.6e-10, both far outside the float64
    sums' rounding (about 1e-13 here), so the exact order is the oracle's."""
    say("case one-ulp column pairs, fp32")
    rng = np.random.default_rng(12)
    half, n_h = 64, 2

    def away_from_zero(a, m):
        return (np.where(a >= 0, 1, -1) * np.maximum(np.abs(a), m)).astype(np.float32)

    base = rng.standard_normal((n_h, 64, half // 2)).astype(np.float32)
    base[:, 0, :] = away_from_zero(base[:, 0, :], 0.25)
    rot = np.repeat(base, 2, axis=2)
    rot[:, 0, 1::2] = np.nextafter(rot[:, 0, 1::2], np.float32(np.inf))
    rt = I.Tensor(rot)
    xv = I.gaussian(13, (2, 2, 576, 64), "f32").values.copy()
    xv[..., 0] = away_from_zero(xv[..., 0], 0.5)
    xt = I.Tensor(xv)
    got = bd.lsh_hash(to_device(xt), to_device(rt), 2 * half, n_h).cpu().numpy()
    for b in range(2):
        for h in range(2):
            ref, _ = O.hash_buckets(xt.values[b, h].astype(np.float64), rot.astype(np.float64), 2 * half)
            np.testing.assert_array_equal(got[b, h], ref)
    col = got % half
    assert np.any(col % 2 == 0) and np.any(col % 2 == 1)


@pytest.mark.parametrize("copies", [8, 9])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_candidate_limit_boundary(gpu_lib, dtype, copies):
    """A rotation whose column 3 appears `copies` times (at 3, 5, 7, ...): a token
    whose best column is one of them has that many exactly tied candidates.  8
    fit the float64 candidate path (unless another column also comes within the
    bound), 9 exceed it and take the all-column float64 loop; either way the
    lowest index wins, as in the oracle."""
    say(f"case {copies} tied copies, {dtype}")
    rng = np.random.default_rng(40 + copies)
    half, n_h = 32, 2
    rot = rng.standard_normal((n_h, 64, half)).astype(np.float32)
    dup = [3 + 2 * k for k in range(copies)]
    rot[:, :, dup] = rot[:, :, 3:4]
    if dtype == "bf16":
        rt = I.Tensor(I.f32_from_bf16_bits(I.bf16_bits_from_f32(rot)), I.bf16_bits_from_f32(rot))
    else:
        rt = I.Tensor(rot)
    xt = I.gaussian(41 + copies, (2, 2, 576, 64), dtype)
    got = bd.lsh_hash(to_device(xt), to_device(rt), 2 * half, n_h).cpu().numpy()
    hits = 0
    for b in range(2):
        for h in range(2):
            ref, _ = O.hash_buckets(xt.values[b, h].astype(np.float64), rt.values.astype(np.float64), 2 * half)
            np.testing.assert_array_equal(got[b, h], ref)
            hits += int(np.sum(np.isin(ref % half, dup)))
    # the tied column wins often, and always as its lowest copy
    assert hits > 0 and not np.any(np.isin(got % half, dup[1:]))


def _dtype_tensor(a, dtype):
    """Values rounded to the dtype (round to nearest even for bf16)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        bits = I.bf16_bits_from_f32(a)
        return I.Tensor(I.f32_from_bf16_bits(bits), bits)
    return I.Tensor(a)


# Crafted tokens (coordinates 0, 1, 2, 6, 34; every other coordinate 0), and
# their buckets for the two rotations of test_gaps_below_float64_resolution.
_T = 2.0**-70
_SUBDOUBLE_TOKENS = [  # (name, {coordinate: value}, bucket with 4 columns, bucket with 16 columns)
    ("+1,+t", {0: 1.0, 1: _T}, 1, 9),
    ("+1,-t", {0: 1.0, 1: -_T}, 0, 0),
    ("-1,+t", {0: -1.0, 1: _T}, 4, 16),
    ("-1,-t", {0: -1.0, 1: -_T}, 5, 25),
    ("+1,0 tie", {0: 1.0}, 0, 0),
    ("-1,0 tie", {0: -1.0}, 4, 16),
    ("sign +", {2: 1.0, 34: _T, 6: -1.0}, 2, 10),
    ("sign -", {2: 1.0, 34: -_T, 6: -1.0}, 6, 26),
    ("sign 0", {2: 1.0, 6: -1.0}, 0, 0),
    ("zero", {}, 0, 0),
]


@pytest.mark.parametrize("half", [4, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gaps_below_float64_resolution(gpu_lib, dtype, half):
    """Top-two gaps far below float64's resolution of the scores, so float64 sums
    tie or even get the sign wrong and only exact summation decides.

    Columns: c0 = e0 and c1 = e0 + e1 (half 4), or c_j = e0 + j 2^-60 e1 for
    j < 10 (half 16); then c = e2 + e6 + e34 (column 2, resp. 10); the rest are
    small random columns on coordinates 8..31.  A token (+-1, +-2^-70) scores
    1 + 2^-70 (or 1 + j 2^-130) against 1 on its rivals: in float64 they are
    equal.  A token (e2 - e6 +- 2^-70 e34) scores +-2^-70 on the sum column,
    which a float64 pairwise sum (1 + 2^-70 first, then - 1) gives as 0.  The
    4-column rotation takes the fixup's candidate short list, the 16-column one
    (10 or more tied candidates) its all-column loop.  Expected buckets are
    worked by hand and also the oracle's (exact rationals)."""
    say(f"case sub-double gaps {dtype} half {half}")
    rng = np.random.default_rng(70 + half)
    rot = np.zeros((1, 64, half), dtype=np.float64)
    n_near = 2 if half == 4 else 10
    for j in range(n_near):
        rot[0, 0, j] = 1.0
        rot[0, 1, j] = 1.0 if half == 4 and j == 1 else j * 2.0**-60
    rot[0, [2, 6, 34], n_near] = 1.0
    rot[0, 8:32, n_near + 1:] = rng.standard_normal((24, half - n_near - 1)) * 2.0**-12
    L = 256
    x = np.zeros((1, 2, L, 64))
    x[0, 1] = rng.standard_normal((L, 64))       # head 1: random tokens, mostly near-tied on c_j
    pos = rng.permutation(L)
    expect = {}
    for k, (name, coords, b4, b16) in enumerate(_SUBDOUBLE_TOKENS):
        for i in pos[k::len(_SUBDOUBLE_TOKENS)]:
            for c, val in coords.items():
                x[0, 0, i, c] = val
            expect[int(i)] = (name, b4 if half == 4 else b16)
    xt = _dtype_tensor(x, dtype)
    rt = _dtype_tensor(rot, dtype)
    assert np.array_equal(xt.values[0, 0], x[0, 0]) and np.array_equal(rt.values[0, :8], rot[0, :8])  # exact
    n_b = 2 * half
    ws = torch.empty(bd.hash_workspace_bytes(1, 2, L, 64, n_b, 1, bd.LSH_BF16 if dtype == "bf16" else bd.LSH_F32),
                     dtype=torch.uint8, device="cuda")
    got = bd.lsh_hash(to_device(xt), to_device(rt), n_b, 1, workspace=ws).cpu().numpy()
    for i, (name, b) in sorted(expect.items()):
        assert got[0, 0, 0, i] == b, f"token {i} ({name}): bucket {got[0, 0, 0, i]}, expected {b}"
    for h in range(2):
        ref, _ = O.hash_buckets(xt.values[0, h].astype(np.float64), rt.values.astype(np.float64), n_b)
        np.testing.assert_array_equal(got[0, h], ref, err_msg=f"head {h}")
    unc = bd.hash_uncertified(ws, 1, 2, L, n_b, 1, torch.bfloat16 if dtype == "bf16" else torch.float32)
    say(f"  hand-worked buckets and the oracle agree; {unc} of {2 * L} token-rounds uncertified in fp32")
    assert unc >= L  # every crafted token is a near-tie


def _uncertified_bracket(x64, rot64):
    """Bounds on the number of token-rounds the GPU cannot certify, from exact
    (float64) scores of one problem.  The kernel certifies a decision when its
    fp32 top-two gap of truncated keys exceeds 2 eps + delta, eps = 65 2^-23 |x|
    max_j |r_j| bounding a 64-term fp32 sum's error and delta = 2^(e - 23 +
    ibits) the key's truncation step (e = exponent of the top score, 2^ibits >=
    columns per lane).  The computed gap lies within 2 eps + delta of the exact
    one, so an exact tie is never certified and an exact gap above 4 eps +
    2 delta always is."""
    n_h, _, half = rot64.shape
    halfp = -(-half // 64) * 64
    ibits = 0
    while (1 << ibits) < halfp // 2:
        ibits += 1
    xn = np.linalg.norm(x64, axis=1)
    lo = hi = 0
    for r in range(n_h):
        a = np.zeros((x64.shape[0], max(halfp, 2)))
        a[:, :half] = np.abs(x64 @ rot64[r])        # padded columns score 0
        top = np.sort(a, axis=1)[:, -2:]
        t1, gap = top[:, 1], top[:, 1] - top[:, 0]
        eps = 65 * 2.0**-23 * xn * np.max(np.linalg.norm(rot64[r], axis=0)) * 1.0001
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(t1 + eps))
        delta = np.where(t1 + eps > 0, 2.0 ** (e - 23 + ibits), 2.0**-126)
        lo += int(np.sum(gap == 0))
        hi += int(np.sum(gap <= 4 * eps + 2 * delta))
    return lo, hi


@pytest.mark.parametrize("name,shape,n_h", REDUCED, ids=[f"{n}-h{h}" for n, _, h in REDUCED])
def test_uncertified_count_is_bracketed(gpu_lib, name, shape, n_h):
    """The GPU's count of float64 re-decisions (lsh_hash_uncertified) lies between
    the exact ties and the exact gaps within the certification band, and the
    fused forward counts the same decisions as the staged hash."""
    inp = I.make_inputs(name, n_hashes=n_h, **shape)
    w = inp.workload
    B, H, L, D = inp.qk.values.shape
    qk, v, rot = upload(inp)
    say(f"case {name} B{B} H{H} L{L} n_b{w.n_buckets} n_h{n_h}")
    dt = bd.LSH_BF16 if qk.dtype == torch.bfloat16 else bd.LSH_F32
    ws = torch.empty(bd.hash_workspace_bytes(B, H, L, D, w.n_buckets, n_h, dt), dtype=torch.uint8, device="cuda")
    bd.lsh_hash(qk, rot, w.n_buckets, n_h, workspace=ws)
    got = bd.hash_uncertified(ws, B, H, L, w.n_buckets, n_h, qk.dtype)
    lo = hi = 0
    rot64 = inp.rot.values.astype(np.float64)
    for b in range(B):
        for h in range(H):
            l, u = _uncertified_bracket(inp.qk.values[b, h].astype(np.float64), rot64)
            lo, hi = lo + l, hi + u
    say(f"  uncertified {got} of {B * H * n_h * L} token-rounds; exact bracket [{lo}, {hi}]")
    assert lo <= got <= hi
    fws = torch.empty(bd.fwd_workspace_bytes(B, H, L, D, w.n_buckets, n_h, 64, dt), dtype=torch.uint8,
                      device="cuda")
    bd.reformer_lsh_attn_fwd(qk, v, rot, w.n_buckets, n_h, 64, w.causal, workspace=fws)
    assert bd.hash_uncertified(fws, B, H, L, w.n_buckets, n_h, qk.dtype) == got


def test_all_tied_rounds_are_all_counted(gpu_lib):
    """With every rotation column duplicated, no decision can be certified: the
    count is every token-round."""
    rng = np.random.default_rng(8)
    half, n_h, B, H, L = 64, 2, 2, 2, 576
    rot = np.repeat(rng.standard_normal((n_h, 64, half // 2)).astype(np.float32), 2, axis=2)
    rt = I.Tensor(I.f32_from_bf16_bits(I.bf16_bits_from_f32(rot)), I.bf16_bits_from_f32(rot))
    xt = I.gaussian(9, (B, H, L, 64), "bf16")
    ws = torch.empty(bd.hash_workspace_bytes(B, H, L, 64, 2 * half, n_h, bd.LSH_BF16), dtype=torch.uint8,
                     device="cuda")
    bd.lsh_hash(to_device(xt), to_device(rt), 2 * half, n_h, workspace=ws)
    assert bd.hash_uncertified(ws, B, H, L, 2 * half, n_h, torch.bfloat16) == B * H * n_h * L


@pytest.mark.parametrize("n_b,n_h,L", [(2, 1, 64), (4096, 2, 4096), (8, 16, 128), (64, 1, 64)])
def test_extreme_bucket_and_round_counts(gpu_lib, n_b, n_h, L):
    say(f"case extremes n_b{n_b} n_h{n_h} L{L}")
    qk_t = I.gaussian(31, (1, 2, L, 64), "bf16")
    v_t = I.gaussian(32, (1, 2, L, 64), "bf16")
    rot_t = I.rotations(33, n_h, 64, n_b, "bf16")
    qk, v, rot = to_device(qk_t), to_device(v_t), to_device(rot_t)
    for causal in (False, True):
        out, lse = bd.reformer_lsh_attn_fwd(qk, v, rot, n_b, n_h, 64, causal)
        torch.cuda.synchronize()
        for h in range(2):
            ref = O.forward_problem(qk_t.values[0, h].astype(np.float64), v_t.values[0, h].astype(np.float64),
                                    rot_t.values.astype(np.float64), n_b, n_h, 64, causal)
            rel_check(f64(out)[0, h], ref["out"], TOL["bf16"], f"out h{h} causal={causal}")
            lse_check(f64(lse)[0, h], ref["lse"], f"lse h{h}")


# The hash stages the rotation in blocks of 128 columns when the padded width
# n_b/2 (rounded up to 64) is a multiple of 128, else 64, two blocks per loop
# trip.  These bucket counts give one block per round with padding (130, 256),
# an odd number of blocks in all (256 with one round, 384 with three rounds: 3
# blocks per round), 64-column blocks beyond one per round (640: 5) and
# 128-column ones (1536: 6), in both dtypes.
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_b,n_h", [(130, 2), (256, 1), (384, 3), (640, 2), (1536, 3)])
def test_hash_staging_block_counts(gpu_lib, n_b, n_h, dtype):
    L = 320  # two hash blocks, the second one ragged
    say(f"case staging n_b{n_b} n_h{n_h} L{L} {dtype}")
    qk_t = I.gaussian(41, (1, 2, L, 64), dtype)
    rot_t = I.rotations(42, n_h, 64, n_b, dtype)
    got = bd.lsh_hash(to_device(qk_t), to_device(rot_t), n_b, n_h).cpu().numpy()
    for h in range(2):
        ref, _ = O.hash_buckets(qk_t.values[0, h].astype(np.float64), rot_t.values.astype(np.float64), n_b)
        np.testing.assert_array_equal(got[0, h], ref, err_msg=f"head {h}")


def test_repeatable_bits(gpu_lib):
    inp = I.make_inputs("causal_lm_4k", B=2, H=2, L=1024)
    say("case determinism")
    qk, v, rot = upload(inp)
    a = bd.reformer_lsh_attn_fwd(qk, v, rot, 64, 4, 64, True)
    b = bd.reformer_lsh_attn_fwd(qk, v, rot, 64, 4, 64, True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_caller_stream_and_workspace_reuse(gpu_lib):
    """Work runs on the caller's stream; one workspace serves repeated calls."""
    inp = I.make_inputs("mlm_small_512", B=2, H=2)
    say("case side stream")
    qk, v, rot = upload(inp)
    ws = torch.empty(bd.fwd_workspace_bytes(2, 2, 512, 64, 8, 4, 64, bd.LSH_BF16), dtype=torch.uint8, device="cuda")
    ref = bd.reformer_lsh_attn_fwd(qk, v, rot, 8, 4, workspace=ws)[0].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got = bd.reformer_lsh_attn_fwd(qk, v, rot, 8, 4, workspace=ws)[0]
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


@pytest.mark.parametrize("shape", [(0, 2, 64), (2, 0, 64), (1, 2, 0)])
def test_empty_problems(gpu_lib, shape):
    """Zero-sized batch, heads or length: every call succeeds and returns empty
    outputs of the right shapes (the library enqueues nothing)."""
    B, H, L = shape
    say(f"case empty B{B} H{H} L{L}")
    qk = torch.zeros((B, H, L, 64), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(qk)
    rot = torch.zeros((2, 64, 8), dtype=torch.bfloat16, device="cuda")
    out, lse = bd.reformer_lsh_attn_fwd(qk, v, rot, 16, 2, 64, True)
    buckets, sidx, undo, o_s, l_s, out_s, lse_s = run_stages(qk, v, rot, 16, 2, True)
    assert out.shape == (B, H, L, 64) and lse.shape == (B, H, L)
    assert buckets.shape == (B, H, 2, L) and sidx.shape == (B, H, 2 * L) and o_s.shape == (B, H, 2 * L, 64)
    assert out_s.shape == (B, H, L, 64) and lse_s.shape == (B, H, L)
