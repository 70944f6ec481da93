"""Attended-set variants (same-bucket mask, set-union correction) of the
HIP path vs the CPU oracle, through the C ABI.

The attention stage is fed the GPU's own hash and sort results, so it is
checked on its own against the oracle's chunk attention with the variant's
slot codes and pair multiplicities; the fused call is checked against the
staged calls and end to end against the oracle's forward pass with the same
variant flags.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from _helpers import TOL, f64, lse_check, rel_check, to_device, upload
from lsh_attention_amd import binding as bd
from lsh_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

VARIANTS = [(True, False), (False, True), (True, True)]
VIDS = ["same_bucket", "dedup", "same_bucket+dedup"]


def say(*a):
    print("[gpu-variants]", *a, flush=True)


def oracle_tables(gb, gs, gu, causal, sb, dd, tokens=None):
    codes = O.slot_codes(gb.astype(np.int64), gs.astype(np.int64)) if sb else None
    mult = (O.pair_multiplicity(gs.astype(np.int64), gu.astype(np.int64), 64, causal, codes, tokens=tokens)
            if dd else None)
    return codes, mult


def check_problem_set(inp_x, inp_v, rot64, n_b, n_h, causal, dtype, qk, v, rot, sb, dd, e2e=((0, 0),)):
    """Staged variant calls on the GPU vs the oracle on every (b, h); fused vs
    staged; fused end to end vs the oracle's forward pass on the `e2e` problems."""
    B, H, L, _ = inp_x.shape
    tol = TOL[dtype]
    buckets = bd.lsh_hash(qk, rot, n_b, n_h)
    sidx, undo = bd.lsh_sort(buckets, n_b)
    o_s, l_s = bd.lsh_chunk_attn(qk, v, sidx, n_h, 64, causal, buckets=buckets, undo_idx=undo, same_bucket=sb,
                                 dedup=dd)
    out, lse = bd.lsh_unsort_combine(o_s, l_s, undo)
    out_f, lse_f = bd.reformer_lsh_attn_fwd(qk, v, rot, n_b, n_h, 64, causal, same_bucket=sb, dedup=dd)
    torch.cuda.synchronize()
    rel_check(f64(out_f), f64(out), tol, "fused vs staged")
    gb, gs, gu = buckets.cpu().numpy(), sidx.cpu().numpy(), undo.cpu().numpy()
    go, gl = f64(o_s), f64(l_s)
    for b in range(B):
        for h in range(H):
            x = inp_x[b, h].astype(np.float64)
            vv = inp_v[b, h].astype(np.float64)
            codes, mult = oracle_tables(gb[b, h], gs[b, h], gu[b, h], causal, sb, dd)
            oo, ol = O.chunk_attention(x, vv, gs[b, h].astype(np.int64), 64, causal, codes=codes, mult=mult)
            rel_check(go[b, h], oo, tol, f"o_sorted b{b} h{h}")
            lse_check(gl[b, h], ol, f"lse_sorted b{b} h{h}")
    gfo, gfl = f64(out_f), f64(lse_f)
    for b, h in e2e:
        x = inp_x[b, h].astype(np.float64)
        vv = inp_v[b, h].astype(np.float64)
        ref = O.forward_problem(x, vv, rot64, n_b, n_h, 64, causal, same_bucket=sb, dedup=dd)
        np.testing.assert_array_equal(gb[b, h], ref["buckets"], err_msg=f"buckets b{b} h{h}")
        rel_check(gfo[b, h], ref["out"], tol, f"fused end-to-end b{b} h{h}")
        lse_check(gfl[b, h], ref["lse"], f"fused end-to-end lse b{b} h{h}")


REDUCED = [
    ("single_head_fp32", dict(), 1),
    ("single_head_fp32", dict(), 3),
    ("mlm_small_512", dict(B=2, H=2), 4),
    ("causal_lm_4k", dict(B=1, H=2, L=1024), 4),
    ("peaked_vmf_16k", dict(B=1, H=1, L=2048), 8),
]


@pytest.mark.parametrize("sb,dd", VARIANTS, ids=VIDS)
@pytest.mark.parametrize("name,shape,n_h", REDUCED, ids=[f"{n}-h{h}" for n, _, h in REDUCED])
def test_variants_match_oracle(gpu_lib, name, shape, n_h, sb, dd):
    inp = I.make_inputs(name, n_hashes=n_h, **shape)
    w = inp.workload
    B, H, L, _ = inp.qk.values.shape
    say(f"case {name} B{B} H{H} L{L} n_b{w.n_buckets} n_h{n_h} causal={w.causal} {w.dtype} sb={sb} dd={dd}")
    qk, v, rot = upload(inp)
    rot64 = None if inp.rot is None else inp.rot.values.astype(np.float64)
    check_problem_set(inp.qk.values, inp.v.values, rot64, w.n_buckets, n_h, w.causal, w.dtype, qk, v, rot, sb, dd)


# One chunk per round (L = 64), two chunks per round, a single round whose
# look-back wraps onto itself, and one or two buckets (with one bucket the
# same-bucket mask keeps only the query's round).
EDGE = [(64, 1), (64, 3), (128, 1), (128, 2), (192, 5)]


@pytest.mark.parametrize("n_b", [1, 2])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("L,n_h", EDGE, ids=[f"L{l}-h{h}" for l, h in EDGE])
def test_variant_edge_shapes(gpu_lib, L, n_h, causal, n_b):
    x = I.gaussian(9100 + L + n_h, (2, 1, L, 64), "f32")
    vv = I.gaussian(9200 + L + n_h, (2, 1, L, 64), "f32")
    r = I.rotations(9300 + n_h, n_h, 64, n_b, "f32")
    rot64 = None if r is None else r.values.astype(np.float64)
    for sb, dd in VARIANTS:
        say(f"edge L{L} n_h{n_h} causal={causal} n_b{n_b} sb={sb} dd={dd}")
        check_problem_set(x.values, vv.values, rot64, n_b, n_h, causal, "f32", to_device(x), to_device(vv),
                          to_device(r), sb, dd, e2e=((0, 0), (1, 0)))


def test_attend_zero_is_the_base_call(gpu_lib):
    """lsh_chunk_attn_ex with attend = 0 runs the base kernel: bit-identical
    results, with the variant inputs ignored (NULL)."""
    inp = I.make_inputs("mlm_small_512", n_hashes=4, B=1, H=2)
    qk, v, rot = upload(inp)
    w = inp.workload
    buckets = bd.lsh_hash(qk, rot, w.n_buckets, 4)
    sidx, undo = bd.lsh_sort(buckets, w.n_buckets)
    o0, l0 = bd.lsh_chunk_attn(qk, v, sidx, 4, 64, w.causal)
    o1, l1 = torch.empty_like(o0), torch.empty_like(l0)
    B, H, L, D = qk.shape
    st = gpu_lib.lsh_chunk_attn_ex(qk.data_ptr(), v.data_ptr(), sidx.data_ptr(), None, None, o1.data_ptr(),
                                   l1.data_ptr(), B, H, L, D, 4, 64, int(w.causal), 0, bd.LSH_BF16, None, 0,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


FULL = [("long_seq_64k", 8), ("causal_lm_4k", 4)]


@pytest.mark.parametrize("sb,dd", VARIANTS, ids=VIDS)
@pytest.mark.parametrize("name,n_h", FULL, ids=[f"{n}-h{h}" for n, h in FULL])
def test_variant_full_size(gpu_lib, name, n_h, sb, dd):
    """At the workload's full size: fused vs staged everywhere, sampled chunks
    of the attention stage and sampled tokens of the output vs the oracle."""
    inp = I.make_inputs(name, n_hashes=n_h)
    w = inp.workload
    B, H, L, D = inp.qk.values.shape
    n_b, causal, tol = w.n_buckets, w.causal, TOL[w.dtype]
    say(f"full {name} B{B} H{H} L{L} n_b{n_b} n_h{n_h} causal={causal} sb={sb} dd={dd}")
    qk, v, rot = upload(inp)
    out_f, lse_f = bd.reformer_lsh_attn_fwd(qk, v, rot, n_b, n_h, 64, causal, same_bucket=sb, dedup=dd)
    buckets = bd.lsh_hash(qk, rot, n_b, n_h)
    sidx, undo = bd.lsh_sort(buckets, n_b)
    o_s, l_s = bd.lsh_chunk_attn(qk, v, sidx, n_h, 64, causal, buckets=buckets, undo_idx=undo, same_bucket=sb,
                                 dedup=dd)
    out, lse = bd.lsh_unsort_combine(o_s, l_s, undo)
    torch.cuda.synchronize()
    rel_check(f64(out_f), f64(out), tol, "fused vs staged")
    gb, gs, gu = buckets.cpu().numpy(), sidx.cpu().numpy(), undo.cpu().numpy()
    rng = np.random.default_rng(77)
    n_chunks = n_h * L // 64
    b, h = int(rng.integers(0, B)), int(rng.integers(0, H))
    x = inp.qk.values[b, h].astype(np.float64)
    vv = inp.v.values[b, h].astype(np.float64)
    chunks = sorted(set(rng.integers(0, n_chunks, 6).tolist()) | {0, n_chunks - 1})
    rows = np.concatenate([np.arange(c * 64, c * 64 + 64) for c in chunks])
    toks = sorted(set(rng.integers(0, L, 12).tolist()) | {0, L - 1})
    need = set(gs[b, h][rows].tolist()) | set(toks)
    codes, mult = oracle_tables(gb[b, h], gs[b, h], gu[b, h], causal, sb, dd, tokens=need)
    oo, ol = O.chunk_attention(x, vv, gs[b, h].astype(np.int64), 64, causal, chunks=chunks, codes=codes, mult=mult)
    ti = torch.as_tensor(rows, device="cuda")
    rel_check(f64(o_s[b, h, ti]), oo[rows], tol, f"o_sorted b{b} h{h}")
    lse_check(f64(l_s[b, h, ti]), ol[rows], f"lse_sorted b{b} h{h}")
    ref_o = np.empty((len(toks), D))
    ref_l = np.empty(len(toks))
    for k, i in enumerate(toks):
        ref_o[k], ref_l[k] = O.token_output(x, vv, gs[b, h].astype(np.int64), gu[b, h].astype(np.int64), 64, causal,
                                            i, codes=codes, mult=mult)
    tt = torch.as_tensor(toks, device="cuda")
    rel_check(f64(out_f[b, h, tt]), ref_o, tol, f"fused out b{b} h{h}")
    lse_check(f64(lse_f[b, h, tt]), ref_l, f"fused lse b{b} h{h}")
    say(f"  sampled chunks {chunks} and {len(toks)} tokens within tolerance")
