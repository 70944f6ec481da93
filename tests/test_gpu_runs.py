"""Chunk attention walks runs of consecutive chunks of one (batch, head): at most
8 chunks (4 for the attended-set variants), halved while a launch would give
the 256 CUs fewer than 1024 blocks.  The shapes here make the runs 8, 4 and 2
chunks long, each with a one- or five-chunk last run, and the first and last
(batch, head) problems -- every run of them, the ragged one included -- are
checked element by element against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from _helpers import TOL, f64, lse_check, rel_check, to_device
from lsh_attention_amd import binding as bd
from lsh_attention_amd import inputs as I
import oracle as O

pytestmark = pytest.mark.gpu

FILL_BLOCKS = 1024


def run_length(bh, n_chunks, longest):
    """The launch's run length for (batch * heads, chunks per problem)."""
    cpb = longest
    while cpb > 1 and bh * -(-n_chunks // cpb) < FILL_BLOCKS:
        cpb //= 2
    return cpb


def say(*a):
    print("[gpu-runs]", *a, flush=True)


# (B, H, L, n_h): L = 6464 gives 101 chunks per problem with one round
CASES = [(10, 8, 6464, 1), (8, 8, 6464, 1), (4, 8, 6464, 1)]


def _inputs(B, H, L, n_h, n_b, seed):
    x = I.gaussian(seed, (B, H, L, 64), "bf16")
    v = I.gaussian(seed + 1, (B, H, L, 64), "bf16")
    r = I.rotations(seed + 2, n_h, 64, n_b, "bf16")
    return x, v, r


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,L,n_h", CASES, ids=[f"B{b}-H{h}" for b, h, _, _ in CASES])
def test_base_runs_match_oracle(gpu_lib, B, H, L, n_h, causal):
    n_b, n_chunks = 16, n_h * L // 64
    cpb = run_length(B * H, n_chunks, 8)
    say(f"base B{B} H{H} L{L} n_h{n_h} causal={causal}: runs of {cpb}, last run {n_chunks - cpb * (n_chunks // cpb) or cpb}")
    assert (B, cpb) in ((10, 8), (8, 4), (4, 2))
    x, v, r = _inputs(B, H, L, n_h, n_b, 9900 + B)
    qk, vd, rd = to_device(x), to_device(v), to_device(r)
    buckets = bd.lsh_hash(qk, rd, n_b, n_h)
    sidx, undo = bd.lsh_sort(buckets, n_b)
    o_s, l_s = bd.lsh_chunk_attn(qk, vd, sidx, n_h, 64, causal)
    out, lse = bd.lsh_unsort_combine(o_s, l_s, undo)
    torch.cuda.synchronize()
    gs, go, gl = sidx.cpu().numpy().astype(np.int64), f64(o_s), f64(l_s)
    gout, glse = f64(out), f64(lse)
    for b, h in ((0, 0), (B - 1, H - 1)):
        xx, vv = x.values[b, h].astype(np.float64), v.values[b, h].astype(np.float64)
        oo, ol = O.chunk_attention(xx, vv, gs[b, h], 64, causal)
        rel_check(go[b, h], oo, TOL["bf16"], f"o_sorted b{b} h{h}")
        lse_check(gl[b, h], ol, f"lse_sorted b{b} h{h}")
        ref = O.forward_problem(xx, vv, r.values.astype(np.float64), n_b, n_h, 64, causal)
        rel_check(gout[b, h], ref["out"], TOL["bf16"], f"end-to-end b{b} h{h}")
        lse_check(glse[b, h], ref["lse"], f"end-to-end lse b{b} h{h}")


@pytest.mark.parametrize("B,H,L,n_h", CASES, ids=[f"B{b}-H{h}" for b, h, _, _ in CASES])
def test_variant_runs_match_oracle(gpu_lib, B, H, L, n_h):
    """Same-bucket mask and set union together (runs of at most 4)."""
    n_b, n_chunks = 16, n_h * L // 64
    cpb = run_length(B * H, n_chunks, 4)
    say(f"variants B{B} H{H} L{L} n_h{n_h}: runs of {cpb}")
    assert (B, cpb) in ((10, 4), (8, 4), (4, 2))
    x, v, r = _inputs(B, H, L, n_h, n_b, 9950 + B)
    qk, vd, rd = to_device(x), to_device(v), to_device(r)
    buckets = bd.lsh_hash(qk, rd, n_b, n_h)
    sidx, undo = bd.lsh_sort(buckets, n_b)
    o_s, l_s = bd.lsh_chunk_attn(qk, vd, sidx, n_h, 64, True, buckets=buckets, undo_idx=undo, same_bucket=True,
                                 dedup=True)
    torch.cuda.synchronize()
    gb, gs, gu = (t.cpu().numpy().astype(np.int64) for t in (buckets, sidx, undo))
    go, gl = f64(o_s), f64(l_s)
    for b, h in ((0, 0), (B - 1, H - 1)):
        xx, vv = x.values[b, h].astype(np.float64), v.values[b, h].astype(np.float64)
        codes = O.slot_codes(gb[b, h], gs[b, h])
        mult = O.pair_multiplicity(gs[b, h], gu[b, h], 64, True, codes)
        oo, ol = O.chunk_attention(xx, vv, gs[b, h], 64, True, codes=codes, mult=mult)
        rel_check(go[b, h], oo, TOL["bf16"], f"variant o_sorted b{b} h{h}")
        lse_check(gl[b, h], ol, f"variant lse_sorted b{b} h{h}")
