"""The fused forward's permutation (the training forward returns it) must be
the one the staged calls give (lsh_hash, then lsh_sort), bit for bit: several
sort tiles per (problem, round), a ragged last tile, few and many buckets, and
near-tie tokens that only the fixup decides."""
import numpy as np
import pytest
import torch

from _helpers import to_device, upload
from lsh_attention_amd import binding as bd
from lsh_attention_amd import inputs as I

pytestmark = pytest.mark.gpu

CASES = [
    # (workload, B, H, L, n_h): sort tiles per (problem, round) > 1 where L allows
    ("long_seq_64k", 1, 2, 3 * 8192 + 64 * 5, 4),   # n_b 1024: tiles of fewer waves, ragged tail
    ("peaked_vmf_16k", 1, 2, 16384, 8),              # clustered rows, many near ties
    ("causal_lm_4k", 2, 2, 4096, 4),
    ("mlm_small_512", 8, 2, 512, 4),                 # few buckets, one tile
]


@pytest.mark.parametrize("name,B,H,L,n_h", CASES)
def test_fused_permutation_matches_staged_sort(gpu_lib, name, B, H, L, n_h):
    inp = I.make_inputs(name, n_hashes=n_h, B=B, H=H, L=L)
    w = inp.workload
    print(f"[fused sort] {name} B{B} H{H} L{L} n_b{w.n_buckets} n_h{n_h}", flush=True)
    qk, v, rot = upload(inp)
    _, _, sidx, undo, _ = bd.reformer_lsh_attn_fwd_train(qk, v, rot, w.n_buckets, n_h, 64, w.causal)
    buckets = bd.lsh_hash(qk, rot, w.n_buckets, n_h)
    s_sidx, s_undo = bd.lsh_sort(buckets, w.n_buckets)
    torch.cuda.synchronize()
    assert torch.equal(sidx, s_sidx), "sorted index differs from the staged sort"
    assert torch.equal(undo, s_undo), "unsort index differs from the staged sort"


def test_fused_permutation_with_fixup_decisions(gpu_lib):
    """Rotation columns in pairs one fp32 ulp apart (coordinate 0), so every
    decision between a pair is a near tie that only the fixup settles.  Two sort
    tiles per (problem, round), the second ragged."""
    rng = np.random.default_rng(31)
    half, n_h, L = 64, 2, 8192 + 192
    base = rng.standard_normal((n_h, 64, half // 2)).astype(np.float32)
    base[:, 0, :] = np.where(base[:, 0, :] >= 0, 1, -1) * np.maximum(np.abs(base[:, 0, :]), 0.25)
    rot = np.repeat(base, 2, axis=2)
    rot[:, 0, 1::2] = np.nextafter(rot[:, 0, 1::2], np.float32(np.inf))
    x = I.gaussian(32, (1, 2, L, 64), "f32").values.copy()
    x[..., 0] = np.where(x[..., 0] >= 0, 1, -1) * np.maximum(np.abs(x[..., 0]), 0.5)
    v = I.gaussian(33, (1, 2, L, 64), "f32").values
    qk_d, v_d, rot_d = (to_device(I.Tensor(np.ascontiguousarray(a, dtype=np.float32))) for a in (x, v, rot))
    n_b = 2 * half
    print(f"[fused sort] one-ulp column pairs fp32 L{L} n_b{n_b} n_h{n_h}", flush=True)
    ws = torch.empty(bd.fwd_workspace_bytes(1, 2, L, 64, n_b, n_h, 64, bd.LSH_F32), dtype=torch.uint8,
                     device="cuda")
    _, _, sidx, undo, _ = bd.reformer_lsh_attn_fwd_train(qk_d, v_d, rot_d, n_b, n_h, 64, False, workspace=ws)
    unc = bd.hash_uncertified(ws, 1, 2, L, n_b, n_h, torch.float32)
    buckets = bd.lsh_hash(qk_d, rot_d, n_b, n_h)
    s_sidx, s_undo = bd.lsh_sort(buckets, n_b)
    torch.cuda.synchronize()
    print(f"  {unc} of {2 * n_h * L} token-rounds decided by the fixup", flush=True)
    assert unc > L  # most decisions are near ties
    assert torch.equal(sidx, s_sidx) and torch.equal(undo, s_undo)
