"""Backward pass of the HIP path vs the float64 autograd oracle, through the C
ABI.  The GPU backward takes the GPU forward's permutation, per-round lse and
output, as a training step would; the oracle differentiates its own forward
with that same permutation (no gradient flows through hashing or sorting)."""
import numpy as np
import pytest
import torch

from _helpers import TOL, f64, rel_check, to_device, upload
from lsh_attention_amd import binding as bd
from lsh_attention_amd import inputs as I
from oracle import lsh_backward as OB

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-backward]", *a, flush=True)


def gpu_forward(qk, v, rot, n_b, n_h, causal):
    buckets = bd.lsh_hash(qk, rot, n_b, n_h)
    sidx, undo = bd.lsh_sort(buckets, n_b)
    o_s, l_s = bd.lsh_chunk_attn(qk, v, sidx, n_h, 64, causal)
    out, lse = bd.lsh_unsort_combine(o_s, l_s, undo)
    return sidx, undo, l_s, out, lse


def grads_inputs(seed, shape, dtype):
    dout = I.gaussian(seed, shape, dtype)
    dlse = I.gaussian(seed + 1, shape[:3], "f32")
    return dout, dlse


def check_backward(xv, vv, rot, n_b, n_h, causal, dtype, qk, v, rot_d, seed, with_dlse=True, problems=None):
    B, H, L, D = xv.shape
    sidx, undo, l_s, out, lse = gpu_forward(qk, v, rot_d, n_b, n_h, causal)
    dout_t, dlse_t = grads_inputs(seed, (B, H, L, D), dtype)
    dout = to_device(dout_t)
    dlse = to_device(dlse_t) if with_dlse else None
    dqk, dv = bd.lsh_attn_bwd(qk, v, sidx, undo, l_s, out, dout, dlse, n_h, 64, causal)
    torch.cuda.synchronize()
    gs, gu = sidx.cpu().numpy().astype(np.int64), undo.cpu().numpy().astype(np.int64)
    gdx, gdv = f64(dqk), f64(dv)
    tol = TOL[dtype]
    for b, h in (problems or [(b, h) for b in range(B) for h in range(H)]):
        ox, ov = OB.backward_problem(xv[b, h].astype(np.float64), vv[b, h].astype(np.float64), gs[b, h], gu[b, h],
                                     64, causal, dout_t.values[b, h].astype(np.float64),
                                     dlse_t.values[b, h].astype(np.float64) if with_dlse else None)
        rel_check(gdx[b, h], ox, tol, f"dqk b{b} h{h}")
        rel_check(gdv[b, h], ov, tol, f"dv b{b} h{h}")
    return gdx, gdv


REDUCED = [
    ("single_head_fp32", dict(), 1),
    ("single_head_fp32", dict(), 3),
    ("mlm_small_512", dict(B=2, H=2), 4),
    ("causal_lm_4k", dict(B=1, H=2, L=1024), 4),
    ("peaked_vmf_16k", dict(B=1, H=1, L=1024), 8),
]


@pytest.mark.parametrize("name,shape,n_h", REDUCED, ids=[f"{n}-h{h}" for n, _, h in REDUCED])
def test_backward_matches_oracle(gpu_lib, name, shape, n_h):
    inp = I.make_inputs(name, n_hashes=n_h, **shape)
    w = inp.workload
    B, H, L, _ = inp.qk.values.shape
    say(f"case {name} B{B} H{H} L{L} n_b{w.n_buckets} n_h{n_h} causal={w.causal} {w.dtype}")
    qk, v, rot = upload(inp)
    rot64 = None if inp.rot is None else inp.rot.values.astype(np.float64)
    check_backward(inp.qk.values, inp.v.values, rot64, w.n_buckets, n_h, w.causal, w.dtype, qk, v, rot,
                   seed=7000 + n_h)


EDGE = [(64, 1), (64, 3), (128, 1), (128, 2), (192, 5), (576, 2)]


@pytest.mark.parametrize("n_b", [1, 2])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("L,n_h", EDGE, ids=[f"L{l}-h{h}" for l, h in EDGE])
def test_backward_edge_shapes(gpu_lib, L, n_h, causal, n_b):
    """One chunk per round (the window is the chunk twice), two chunks per
    round, a run of 8 chunks that ends in the middle of a round (L = 576, two
    rounds: 18 chunks, 3 blocks, the last one short), one or two buckets."""
    x = I.gaussian(9400 + L + n_h, (2, 1, L, 64), "f32")
    vv = I.gaussian(9500 + L + n_h, (2, 1, L, 64), "f32")
    r = I.rotations(9600 + n_h, n_h, 64, n_b, "f32")
    say(f"edge L{L} n_h{n_h} causal={causal} n_b{n_b}")
    check_backward(x.values, vv.values, None, n_b, n_h, causal, "f32", to_device(x), to_device(vv), to_device(r),
                   seed=9700 + L + n_h)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_without_lse_gradient(gpu_lib, dtype):
    x = I.gaussian(9800, (1, 2, 256, 64), dtype)
    vv = I.gaussian(9801, (1, 2, 256, 64), dtype)
    r = I.rotations(9802, 2, 64, 8, dtype)
    say(f"no dlse {dtype}")
    check_backward(x.values, vv.values, None, 8, 2, True, dtype, to_device(x), to_device(vv), to_device(r),
                   seed=9803, with_dlse=False)


FULL = [("long_seq_64k", 8), ("causal_lm_4k", 4), ("peaked_vmf_16k", 8)]


@pytest.mark.parametrize("name,n_h", FULL, ids=[f"{n}-h{h}" for n, h in FULL])
def test_backward_full_size(gpu_lib, name, n_h):
    """Full size: sum_j dv_j = sum_i dout_i per problem (each token's combined
    weights sum to one), and sampled tokens' gradients vs the oracle's
    single-token form."""
    inp = I.make_inputs(name, n_hashes=n_h)
    w = inp.workload
    B, H, L, D = inp.qk.values.shape
    say(f"full {name} B{B} H{H} L{L} n_b{w.n_buckets} n_h{n_h} causal={w.causal}")
    qk, v, rot = upload(inp)
    sidx, undo, l_s, out, lse = gpu_forward(qk, v, rot, w.n_buckets, n_h, w.causal)
    dout_t, dlse_t = grads_inputs(8100, (B, H, L, D), w.dtype)
    dout, dlse = to_device(dout_t), to_device(dlse_t)
    dqk, dv = bd.lsh_attn_bwd(qk, v, sidx, undo, l_s, out, dout, dlse, n_h, 64, w.causal)
    torch.cuda.synchronize()
    tol = TOL[w.dtype]
    sum_dv = dv.float().sum(dim=2).double().cpu().numpy()
    sum_do = dout_t.values.astype(np.float64).sum(axis=2)
    rel_check(sum_dv, sum_do, tol, "sum of dv vs sum of dout")
    rng = np.random.default_rng(55)
    b, h = int(rng.integers(0, B)), int(rng.integers(0, H))
    gs, gu = sidx[b, h].cpu().numpy().astype(np.int64), undo[b, h].cpu().numpy().astype(np.int64)
    x64 = inp.qk.values[b, h].astype(np.float64)
    v64 = inp.v.values[b, h].astype(np.float64)
    d64 = dout_t.values[b, h].astype(np.float64)
    l64 = dlse_t.values[b, h].astype(np.float64)
    toks = sorted(set(rng.integers(0, L, 3).tolist()) | {0, L - 1})
    gdx, gdv = f64(dqk[b, h]), f64(dv[b, h])
    ref_x = np.empty((len(toks), D))
    ref_v = np.empty((len(toks), D))
    for k, j in enumerate(toks):
        ref_x[k], ref_v[k] = OB.token_grads(x64, v64, gs, gu, 64, w.causal, d64, l64, j)
    rel_check(gdx[toks], ref_x, tol, f"dqk sampled b{b} h{h}")
    rel_check(gdv[toks], ref_v, tol, f"dv sampled b{b} h{h}")
    say(f"  tokens {toks} within tolerance")


def test_backward_is_deterministic_and_train_forward_matches(gpu_lib):
    """No atomics: repeated backward calls give identical bits.  The training
    forward returns the plain fused forward's output and lse, and the staged
    calls' permutation and per-round lse, exactly."""
    inp = I.make_inputs("causal_lm_4k", n_hashes=4, B=2, H=2, L=1024)
    w = inp.workload
    qk, v, rot = upload(inp)
    out_t, lse_t, sidx, undo, l_s = bd.reformer_lsh_attn_fwd_train(qk, v, rot, w.n_buckets, 4, 64, w.causal)
    out_f, lse_f = bd.reformer_lsh_attn_fwd(qk, v, rot, w.n_buckets, 4, 64, w.causal)
    s_sidx, s_undo, s_ls, _, _ = gpu_forward(qk, v, rot, w.n_buckets, 4, w.causal)
    torch.cuda.synchronize()
    assert torch.equal(out_t, out_f) and torch.equal(lse_t, lse_f)
    assert torch.equal(sidx, s_sidx) and torch.equal(undo, s_undo)
    # the staged attention computes its own key scales from the rows: same to rounding
    rel_check(f64(l_s), f64(s_ls), 1e-5, "per-round lse, fused vs staged")
    dout_t, dlse_t = grads_inputs(123, tuple(qk.shape), w.dtype)
    dout, dlse = to_device(dout_t), to_device(dlse_t)
    first = bd.lsh_attn_bwd(qk, v, sidx, undo, l_s, out_t, dout, dlse, 4, 64, w.causal)
    for _ in range(3):
        again = bd.lsh_attn_bwd(qk, v, sidx, undo, l_s, out_t, dout, dlse, 4, 64, w.causal)
        torch.cuda.synchronize()
        assert torch.equal(first[0], again[0]) and torch.equal(first[1], again[1])
