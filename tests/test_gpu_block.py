"""Reversible block (attention sublayer + chunked feed-forward) of the HIP path
vs the float64 block oracle, through the C ABI.

Each stage of a staged GPU run (LayerNorm, projections, LSH attention, output
projection, LayerNorm, feed-forward) is checked against the oracle applied to
the GPU's own previous stage, so that a bucket decision taken on the GPU's
bf16 projections is checked on the same values; the fused block call must
equal the staged run bit for bit (same kernels, row chunking included)."""
import numpy as np
import pytest
import torch

import oracle as O
from _helpers import TOL, f64, rel_check, to_device
from lsh_attention_amd import binding as bd
from lsh_attention_amd import inputs as I
from oracle import lsh_block as OBk

pytestmark = pytest.mark.gpu
TOLB = TOL["bf16"]


def say(*a):
    print("[gpu-block]", *a, flush=True)


def upload_block(bi):
    P = {k: to_device(t) for k, t in bi.params.items()}
    return to_device(bi.x1), to_device(bi.x2), to_device(bi.rot), P


def staged(x1, x2, rot, P, n_b, n_h, causal):
    h1 = bd.lsh_layer_norm(x2, P["ln1_g"], P["ln1_b"])
    qk = bd.lsh_linear_heads(h1, P["w_qk"])
    v = bd.lsh_linear_heads(h1, P["w_v"])
    att, _ = bd.reformer_lsh_attn_fwd(qk, v, rot, n_b, n_h, 64, causal)
    y1 = bd.lsh_linear(att, P["w_o"], resid=x1, a_heads=True)
    h2 = bd.lsh_layer_norm(y1, P["ln2_g"], P["ln2_b"])
    hid = bd.lsh_linear(h2, P["w1"], bias=P["b1"], gelu=True)
    y2 = bd.lsh_linear(hid, P["w2"], bias=P["b2"], resid=x2)
    torch.cuda.synchronize()
    return dict(h1=h1, qk=qk, v=v, att=att, y1=y1, h2=h2, hid=hid, y2=y2)


def heads_to_rows(a):  # [B, H, L, 64] -> [B, L, 64 H]
    B, H, L, _ = a.shape
    return a.transpose(0, 2, 1, 3).reshape(B, L, H * 64) if isinstance(a, np.ndarray) else \
        a.permute(0, 2, 1, 3).reshape(B, L, H * 64)


REDUCED = [
    ("mlm_small_512", dict(B=2, L=256, heads=2), 4, 0),
    ("mlm_small_512", dict(B=1, L=192, heads=2), 2, 100),   # M = 192: a half row tile; ragged chunks
    ("causal_lm_4k", dict(B=1, L=512, heads=4), 2, 64),
    ("long_seq_64k", dict(B=1, L=1024, heads=2), 8, 384),
]


@pytest.mark.parametrize("name,shape,n_h,chunk_rows", REDUCED,
                         ids=[f"{n}-L{s['L']}-H{s['heads']}-h{h}-c{c}" for n, s, h, c in REDUCED])
def test_block_stages_match_oracle(gpu_lib, name, shape, n_h, chunk_rows):
    bi = I.make_block_inputs(name, n_hashes=n_h, **shape)
    w = bi.workload
    B, L, dim = bi.x1.values.shape
    say(f"case {name} B{B} L{L} dim{dim} n_b{w.n_buckets} n_h{n_h} causal={w.causal} chunk_rows={chunk_rows}")
    x1, x2, rot, P = upload_block(bi)
    st = staged(x1, x2, rot, P, w.n_buckets, n_h, w.causal)
    y1f, y2f = bd.reformer_block_fwd(x1, x2, rot, P, w.n_buckets, n_h, w.causal, chunk_rows=chunk_rows)
    torch.cuda.synchronize()
    assert torch.equal(y1f, st["y1"]) and torch.equal(y2f, st["y2"]), "fused block differs from the staged run"
    p = bi.params_math()
    rot64 = None if bi.rot is None else bi.rot.values.astype(np.float64)
    g = {k: f64(t) for k, t in st.items()}
    x1v, x2v = bi.x1.values.astype(np.float64), bi.x2.values.astype(np.float64)
    rel_check(g["h1"], OBk.layer_norm(x2v, p["ln1_g"], p["ln1_b"]), TOLB, "LayerNorm 1")
    rows_qk = g["h1"] @ p["w_qk"]
    rows_v = g["h1"] @ p["w_v"]
    rel_check(heads_to_rows(g["qk"]), rows_qk, TOLB, "shared-QK projection")
    rel_check(heads_to_rows(g["v"]), rows_v, TOLB, "V projection")
    ref_att, _ = O.forward(g["qk"], g["v"], rot64, w.n_buckets, n_h, 64, w.causal)
    rel_check(g["att"], ref_att, TOLB, "LSH attention")
    rel_check(g["y1"], x1v + heads_to_rows(g["att"]) @ p["w_o"], TOLB, "output projection + residual")
    rel_check(g["h2"], OBk.layer_norm(g["y1"], p["ln2_g"], p["ln2_b"]), TOLB, "LayerNorm 2")
    rel_check(g["hid"], OBk.gelu(g["h2"] @ p["w1"] + p["b1"]), TOLB, "Linear 1 + GELU")
    rel_check(g["y2"], x2v + g["hid"] @ p["w2"] + p["b2"], TOLB, "Linear 2 + residual")
    # the oracle's whole feed-forward (float64 hidden) from the GPU's y1
    ffn = np.stack([OBk.feed_forward(g["y1"][b], p, chunk_rows or None) for b in range(B)])
    rel_check(g["y2"], x2v + ffn, TOLB, "feed-forward sublayer")


@pytest.mark.parametrize("epi", ["plain", "bias_gelu", "resid", "bias_resid"])
def test_linear_epilogues_and_layouts(gpu_lib, epi):
    rng = np.random.default_rng(5)
    B, L, K, N = 1, 192, 128, 256

    def bf(a):
        return to_device(I._store(np.asarray(a, dtype=np.float32), "bf16"))

    a = bf(rng.standard_normal((B, L, K)))
    wt = bf(rng.standard_normal((N, K)) / np.sqrt(K))
    bias = bf(rng.standard_normal(N))
    res = bf(rng.standard_normal((B, L, N)))
    A, W, BI, R = f64(a), f64(wt), f64(bias), f64(res)
    kw = {}
    ref = A @ W.T
    if epi in ("bias_gelu", "bias_resid"):
        kw["bias"] = bias
        ref = ref + BI
    if epi == "bias_gelu":
        kw["gelu"] = True
        ref = OBk.gelu(ref)
    if epi in ("resid", "bias_resid"):
        kw["resid"] = res
        ref = ref + R
    rel_check(f64(bd.lsh_linear(a, wt, **kw)), ref, TOLB, f"rows -> rows {epi}")
    if epi == "plain":
        hm = bd.lsh_linear_heads(a, wt)  # [B, H, L, 64]
        rel_check(heads_to_rows(f64(hm)), A @ W.T, TOLB, "rows -> heads")
        w2 = bf(rng.standard_normal((N, N)) / np.sqrt(N))
        rel_check(f64(bd.lsh_linear(hm, w2, a_heads=True)), heads_to_rows(f64(hm)) @ f64(w2).T, TOLB,
                  "heads -> rows")


@pytest.mark.parametrize("epi", ["plain", "bias_gelu", "resid", "bias_resid"])
def test_linear_large_tiles(gpu_lib, epi):
    """The GEMM at a long shape: M = 32832 rows (257 row tiles, the last one
    partial), K = 192 (three K-stages), N = 512; every element against float64,
    every epilogue, and both head-major layouts."""
    rng = np.random.default_rng(7)
    B, L, K, N = 1, 32832, 192, 512
    say(f"case long linear {epi} M{L} K{K} N{N}")

    def bf(a):
        return to_device(I._store(np.asarray(a, dtype=np.float32), "bf16"))

    a = bf(rng.standard_normal((B, L, K)))
    wt = bf(rng.standard_normal((N, K)) / np.sqrt(K))
    bias = bf(rng.standard_normal(N))
    res = bf(rng.standard_normal((B, L, N)))
    A, W, BI, R = f64(a), f64(wt), f64(bias), f64(res)
    kw = {}
    ref = A @ W.T
    if epi in ("bias_gelu", "bias_resid"):
        kw["bias"] = bias
        ref = ref + BI
    if epi == "bias_gelu":
        kw["gelu"] = True
        ref = OBk.gelu(ref)
    if epi in ("resid", "bias_resid"):
        kw["resid"] = res
        ref = ref + R
    rel_check(f64(bd.lsh_linear(a, wt, **kw)), ref, TOLB, f"large tiles rows -> rows {epi}")
    if epi == "plain":
        hm = bd.lsh_linear_heads(a, wt)  # [B, H, L, 64]
        rel_check(heads_to_rows(f64(hm)), A @ W.T, TOLB, "large tiles rows -> heads")
        w2 = bf(rng.standard_normal((N, N)) / np.sqrt(N))
        rel_check(f64(bd.lsh_linear(hm, w2, a_heads=True)), heads_to_rows(f64(hm)) @ f64(w2).T, TOLB,
                  "large tiles heads -> rows")


@pytest.mark.parametrize("dim", [128, 512, 1024])
def test_layer_norm(gpu_lib, dim):
    rng = np.random.default_rng(dim)

    def bf(a):
        return to_device(I._store(np.asarray(a, dtype=np.float32), "bf16"))

    x = bf(3.0 + 2.0 * rng.standard_normal((100, dim)))
    g = bf(1.0 + 0.1 * rng.standard_normal(dim))
    b = bf(0.1 * rng.standard_normal(dim))
    rel_check(f64(bd.lsh_layer_norm(x, g, b)), OBk.layer_norm(f64(x), f64(g), f64(b)), TOLB, f"LayerNorm dim {dim}")


def test_block_full_size(gpu_lib):
    """long_seq_64k as one block (B1 L65536, 8 heads -> dim 512, 1024 buckets, 8
    rounds, causal): the fused block equals the staged run bit for bit, and
    sampled rows of every stage match the oracle (the attention on two heads,
    from the GPU's projections)."""
    bi = I.make_block_inputs("long_seq_64k")
    w = bi.workload
    B, L, dim = bi.x1.values.shape
    n_h = bi.n_hashes
    say(f"full long_seq_64k B{B} L{L} dim{dim} n_b{w.n_buckets} n_h{n_h} causal={w.causal}")
    x1, x2, rot, P = upload_block(bi)
    st = staged(x1, x2, rot, P, w.n_buckets, n_h, w.causal)
    y1f, y2f = bd.reformer_block_fwd(x1, x2, rot, P, w.n_buckets, n_h, w.causal, chunk_rows=8192)
    torch.cuda.synchronize()
    assert torch.equal(y1f, st["y1"]) and torch.equal(y2f, st["y2"]), "fused block differs from the staged run"
    say("  fused equals staged")
    p = bi.params_math()
    rot64 = bi.rot.values.astype(np.float64)
    rng = np.random.default_rng(31)
    rows = np.array(sorted(set(rng.integers(0, L, 24).tolist()) | {0, L - 1}))
    ti = torch.as_tensor(rows, device="cuda")
    x1v, x2v = bi.x1.values[0].astype(np.float64), bi.x2.values[0].astype(np.float64)
    h1 = f64(st["h1"][0, ti])
    rel_check(h1, OBk.layer_norm(x2v[rows], p["ln1_g"], p["ln1_b"]), TOLB, "LayerNorm 1 rows")
    rel_check(f64(st["qk"][0][:, ti]).transpose(1, 0, 2).reshape(len(rows), dim), h1 @ p["w_qk"], TOLB,
              "shared-QK projection rows")
    qk_all, v_all = f64(st["qk"][0]), f64(st["v"][0])
    att = f64(st["att"][0])
    for hd in (0, 5):
        q64, v64 = qk_all[hd], v_all[hd]
        bk, _ = O.hash_buckets(q64, rot64, w.n_buckets)
        sidx, undo = O.sort_by_bucket(bk)
        ref = np.stack([O.token_output(q64, v64, sidx, undo, 64, w.causal, int(i))[0] for i in rows])
        rel_check(att[hd][rows], ref, TOLB, f"LSH attention rows head {hd}")
    att_rows = att[:, rows].transpose(1, 0, 2).reshape(len(rows), dim)
    y1 = f64(st["y1"][0, ti])
    rel_check(y1, x1v[rows] + att_rows @ p["w_o"], TOLB, "output projection rows")
    h2 = f64(st["h2"][0, ti])
    rel_check(h2, OBk.layer_norm(y1, p["ln2_g"], p["ln2_b"]), TOLB, "LayerNorm 2 rows")
    rel_check(f64(st["y2"][0, ti]), x2v[rows] + OBk.feed_forward(y1, p), TOLB, "feed-forward rows")
    say(f"  {len(rows)} sampled rows within tolerance at every stage")
