"""The allocation-free forward (reformer_lsh_attn_fwd_noalloc: the library's
fixed device scratch in place of a workspace) against the workspace form
reformer_lsh_attn_fwd, through the C ABI, on two calls in a row: a first call
whose problems need more than the scratch in total (processed in groups), then
a smaller one that reuses the scratch.  The kernels are the same and every
problem is computed independently, so the results must be bit-identical."""
import numpy as np
import pytest
import torch

from _helpers import upload
from lsh_attention_amd import binding as bd
from lsh_attention_amd import inputs as I

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-noalloc]", *a, flush=True)


def _same(a, b, what):
    if a is None or b is None:
        assert a is None and b is None, what
        return
    assert a.shape == b.shape and a.dtype == b.dtype, what
    ab, bb = a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)
    n = int((ab != bb).sum())
    assert n == 0, f"{what}: {n} bytes differ"


CASES = [
    # (workload, B, H, L, n_h): the first needs two scratch groups (about 319 MB of
    # workspace for 1024 problems), the second is smaller and fits in one
    ("mlm_small_512", None, None, None, 4),
    ("causal_lm_4k", 2, 4, 1024, 4),
]


def test_noalloc_matches_the_workspace_forward(gpu_lib):
    for name, B, H, L, n_h in CASES:
        kw = {k: v for k, v in (("B", B), ("H", H), ("L", L)) if v is not None}
        inp = I.make_inputs(name, n_hashes=n_h, **kw)
        w = inp.workload
        Bq, Hq, Lq, D = inp.qk.values.shape
        dt = bd.LSH_BF16 if w.dtype == "bf16" else bd.LSH_F32
        need = bd.fwd_workspace_bytes(Bq, Hq, Lq, D, w.n_buckets, n_h, 64, dt)
        say(f"case {name} B{Bq} H{Hq} L{Lq} n_b{w.n_buckets} n_h{n_h} causal={w.causal} {w.dtype}: "
            f"workspace {need / 2**20:.1f} MiB against the {256} MiB scratch")
        qk, v, rot = upload(inp)
        ref_out, ref_lse = bd.reformer_lsh_attn_fwd(qk, v, rot, w.n_buckets, n_h, 64, w.causal)
        out, lse = bd.reformer_lsh_attn_fwd_noalloc(qk, v, rot, w.n_buckets, n_h, 64, w.causal)
        torch.cuda.synchronize()
        _same(out, ref_out, f"{name} out")
        _same(lse, ref_lse, f"{name} lse")
        # without lse_out, into caller buffers
        out2 = torch.empty_like(qk)
        out2b, none = bd.reformer_lsh_attn_fwd_noalloc(qk, v, rot, w.n_buckets, n_h, 64, w.causal, out=out2,
                                                       want_lse=False)
        torch.cuda.synchronize()
        assert none is None and out2b.data_ptr() == out2.data_ptr()
        _same(out2, ref_out, f"{name} out without lse")
        assert torch.isfinite(out.float()).all()
        say(f"  bit-identical to reformer_lsh_attn_fwd ({'two groups' if need > 256 << 20 else 'one group'})")


def test_noalloc_rejects_a_problem_beyond_the_scratch(gpu_lib):
    """fp32, one problem of 65536 tokens with 16 rounds needs about 296 MiB: the
    call fails with LSH_ERR_TOO_LARGE and enqueues nothing (the outputs keep
    their contents)."""
    qk = torch.zeros((1, 1, 65536, 64), dtype=torch.float32, device="cuda")
    rot = torch.zeros((16, 64, 2048), dtype=torch.float32, device="cuda")
    out = torch.full_like(qk, 7.0)
    with pytest.raises(bd.LshError) as ei:
        bd.reformer_lsh_attn_fwd_noalloc(qk, qk.clone(), rot, 4096, 16, 64, False, out=out)
    assert ei.value.status == -8
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    np.testing.assert_equal(bd.lib().lsh_status_string(-8).decode().startswith("one (batch, head) problem"), True)
