"""The C-ABI library loads, exports every declared symbol, and rejects invalid
arguments on the host before touching the GPU (no compute is launched here)."""
import ctypes
import os

import pytest

from lsh_attention_amd import binding as bd

OK, NULL, SHAPE, BUCKETS, UNSUPPORTED, WORKSPACE, ALIAS, HIPERR = 0, -1, -2, -3, -4, -5, -6, -7
F32, BF16 = 0, 1
# Distinct fake device addresses: validation must reject the call before any
# pointer is dereferenced or any HIP call is made.
P1, P2, P3, P4, P5 = (0x10000000 * k for k in range(1, 6))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bd.library_path()):
        pytest.fail("liblsh_attn.so is not built; run `python -m lsh_attention_amd.build`")
    return bd.lib()


def test_every_declared_symbol_is_exported(L):
    names = bd.header_functions()
    assert "reformer_lsh_attn_fwd" in names and len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert set(bd._SIGS) == set(names)


def test_status_strings(L):
    for s in (OK, NULL, SHAPE, BUCKETS, UNSUPPORTED, WORKSPACE, ALIAS, HIPERR, 99):
        assert isinstance(L.lsh_status_string(s), bytes) and L.lsh_status_string(s)


def _ws(fn, *args):
    n = ctypes.c_size_t()
    st = getattr(bd.lib(), fn)(*args, ctypes.byref(n))
    return st, n.value


def test_workspace_sizes(L):
    st, n1 = _ws("lsh_fwd_workspace_bytes", 1, 8, 65536, 64, 1024, 8, 64, BF16)
    assert st == OK
    # buckets, sorted, undo (int32) + o_sorted (bf16) + lse (fp32) per slot at least
    assert n1 >= 8 * 8 * 65536 * (3 * 4 + 64 * 2 + 4)
    st, n2 = _ws("lsh_fwd_workspace_bytes", 1, 8, 65536, 64, 1024, 8, 64, F32)
    assert st == OK and n2 > n1
    st, h = _ws("lsh_hash_workspace_bytes", 1, 8, 65536, 64, 1024, 8, BF16)
    assert st == OK and h >= 8 * 512 * 64 * 2
    st, s = _ws("lsh_sort_workspace_bytes", 1, 8, 65536, 1024, 8)
    assert st == OK and s >= 8 * 8 * 1024 * (65536 // 8192) * 4  # histogram per (problem, round, 8192-token tile)
    assert L.lsh_fwd_workspace_bytes(1, 1, 64, 64, 2, 1, 64, BF16, None) == NULL


@pytest.mark.parametrize("args,expect", [
    ((-1, 1, 64, 64, 2, 1, 64, BF16), SHAPE),
    ((1, 1, -64, 64, 2, 1, 64, BF16), SHAPE),
    ((1, 1, 100, 64, 2, 1, 64, BF16), SHAPE),       # L not a multiple of 64
    ((1, 1, 64, 32, 2, 1, 64, BF16), UNSUPPORTED),  # D != 64
    ((1, 1, 64, 64, 2, 1, 32, BF16), UNSUPPORTED),  # chunk_len != 64
    ((1, 1, 64, 64, 2, 1, 0, BF16), SHAPE),
    ((1, 1, 64, 64, 3, 1, 64, BF16), BUCKETS),      # odd n_b
    ((1, 1, 64, 64, 0, 1, 64, BF16), BUCKETS),
    ((1, 1, 64, 64, 8192, 1, 64, BF16), BUCKETS),
    ((1, 1, 64, 64, 2, 17, 64, BF16), UNSUPPORTED), # n_h > 16
    ((1, 1, 64, 64, 2, 0, 64, BF16), SHAPE),
    ((1, 1, 64, 64, 2, 1, 64, 7), UNSUPPORTED),     # dtype
    ((1024, 1024, 4096, 64, 2, 1, 64, BF16), SHAPE),  # B*H*n_h*L overflows int32
    ((1, 1, 64, 64, 1, 1, 64, F32), OK),
    ((1, 1, 64, 64, 4096, 16, 64, BF16), OK),
])
def test_shape_validation(L, args, expect):
    st, _ = _ws("lsh_fwd_workspace_bytes", *args)
    assert st == expect


def test_fused_call_rejects_before_launch(L):
    st, need = _ws("lsh_fwd_workspace_bytes", 1, 2, 128, 64, 8, 2, 64, BF16)
    assert st == OK
    f = L.reformer_lsh_attn_fwd
    # NULL inputs
    assert f(None, P2, P3, 8, 2, 64, 0, 1, 2, 128, 64, BF16, P4, None, P5, need, None, None) == NULL
    assert f(P1, P2, None, 8, 2, 64, 0, 1, 2, 128, 64, BF16, P4, None, P5, need, None, None) == NULL
    assert f(P1, P2, P3, 8, 2, 64, 0, 1, 2, 128, 64, BF16, None, None, P5, need, None, None) == NULL
    # rot may be NULL with one bucket only
    assert f(P1, P2, None, 1, 2, 64, 0, 1, 2, 128, 64, BF16, P4, None, None, 0, None, None) == WORKSPACE
    # workspace
    assert f(P1, P2, P3, 8, 2, 64, 0, 1, 2, 128, 64, BF16, P4, None, None, need, None, None) == WORKSPACE
    assert f(P1, P2, P3, 8, 2, 64, 0, 1, 2, 128, 64, BF16, P4, None, P5, need - 1, None, None) == WORKSPACE
    # aliasing: out == qk, out inside the workspace, lse on top of v
    assert f(P1, P2, P3, 8, 2, 64, 0, 1, 2, 128, 64, BF16, P1, None, P5, need, None, None) == ALIAS
    assert f(P1, P2, P3, 8, 2, 64, 0, 1, 2, 128, 64, BF16, P5 + 256, None, P5, need, None, None) == ALIAS
    assert f(P1, P2, P3, 8, 2, 64, 0, 1, 2, 128, 64, BF16, P4, P2, P5, need, None, None) == ALIAS
    # shape errors win over pointer errors
    assert f(None, None, None, 8, 2, 64, 0, 1, 2, 100, 64, BF16, None, None, None, 0, None, None) == SHAPE


def test_stage_calls_reject_before_launch(L):
    st, hws = _ws("lsh_hash_workspace_bytes", 1, 1, 256, 64, 16, 2, BF16)
    assert L.lsh_hash(P1, P2, None, 1, 1, 256, 64, 16, 2, BF16, P4, hws, None) == NULL
    assert L.lsh_hash(P1, P2, P3, 1, 1, 256, 64, 16, 2, BF16, P4, hws - 1, None) == WORKSPACE
    assert L.lsh_hash(P1, P2, P1, 1, 1, 256, 64, 16, 2, BF16, P4, hws, None) == ALIAS
    assert L.lsh_hash(P1, P2, P3, 1, 1, 256, 64, 15, 2, BF16, P4, hws, None) == BUCKETS
    st, sws = _ws("lsh_sort_workspace_bytes", 1, 1, 256, 16, 2)
    assert L.lsh_sort(P1, P2, P3, 1, 1, 256, 16, 2, P4, sws - 4, None) == WORKSPACE
    assert L.lsh_sort(P1, P1, P3, 1, 1, 256, 16, 2, P4, sws, None) == ALIAS
    assert L.lsh_sort(P1, P2, P2, 1, 1, 256, 16, 2, P4, sws, None) == ALIAS
    assert L.lsh_chunk_attn(P1, P2, P3, P4, None, 1, 1, 256, 64, 2, 64, 0, BF16, None) == NULL
    assert L.lsh_chunk_attn(P1, P2, P3, P1, P5, 1, 1, 256, 64, 2, 64, 0, BF16, None) == ALIAS
    assert L.lsh_chunk_attn(P1, P2, P3, P4, P5, 1, 1, 256, 64, 2, 128, 0, BF16, None) == UNSUPPORTED
    assert L.lsh_unsort_combine(P1, P2, P3, None, None, 1, 1, 256, 64, 2, BF16, None) == NULL
    assert L.lsh_unsort_combine(P1, P2, P3, P1, None, 1, 1, 256, 64, 2, BF16, None) == ALIAS
    assert L.lsh_unsort_combine(P1, P2, P3, P4, P4, 1, 1, 256, 64, 2, BF16, None) == ALIAS
    assert L.lsh_event_create(None) == NULL
    assert L.lsh_event_elapsed_ms(None, None, None) == NULL


def test_uncertified_count_rejects_before_copy(L):
    n = ctypes.c_int(7)
    st, hws = _ws("lsh_hash_workspace_bytes", 1, 1, 256, 64, 16, 2, BF16)
    assert st == OK
    assert L.lsh_hash_uncertified(P1, hws, 1, 1, 256, 16, 2, BF16, None, None) == NULL
    assert L.lsh_hash_uncertified(P1, hws - 1, 1, 1, 256, 16, 2, BF16, ctypes.byref(n), None) == WORKSPACE
    assert L.lsh_hash_uncertified(None, hws, 1, 1, 256, 16, 2, BF16, ctypes.byref(n), None) == WORKSPACE
    assert L.lsh_hash_uncertified(P1, hws, 1, 1, 256, 15, 2, BF16, ctypes.byref(n), None) == BUCKETS
    assert L.lsh_hash_uncertified(P1, hws, 1, 1, 256, 16, 0, BF16, ctypes.byref(n), None) == SHAPE
    assert L.lsh_hash_uncertified(P1, hws, 1, 1, 256, 16, 2, 9, ctypes.byref(n), None) == UNSUPPORTED
    # nothing is hashed for one bucket or an empty problem: the count is 0 and no
    # workspace is read
    assert L.lsh_hash_uncertified(None, 0, 1, 1, 256, 1, 2, BF16, ctypes.byref(n), None) == OK and n.value == 0
    n.value = 7
    assert L.lsh_hash_uncertified(None, 0, 0, 1, 256, 16, 2, BF16, ctypes.byref(n), None) == OK and n.value == 0
    # the forward workspace starts with the hashing part, so it always suffices
    st, fws = _ws("lsh_fwd_workspace_bytes", 1, 1, 256, 64, 16, 2, 64, BF16)
    assert st == OK and fws >= hws


def test_clock_measurement_rejects_before_launch(L):
    mhz = ctypes.c_double(0.0)
    assert L.lsh_measure_clock(None, 100, ctypes.byref(mhz), None) == NULL
    assert L.lsh_measure_clock(P1, 100, None, None) == NULL
    assert L.lsh_measure_clock(P1, 0, ctypes.byref(mhz), None) == SHAPE
    assert L.lsh_measure_clock(P1, 100001, ctypes.byref(mhz), None) == SHAPE
    assert bd.CLOCK_TICKS_BYTES == 2 * 2048 * 8


@pytest.mark.parametrize("B,H,n", [(0, 1, 64), (1, 0, 64), (1, 1, 0), (0, 0, 0)])
def test_empty_problems_are_no_ops(L, B, H, n):
    # Zero-sized problems succeed without touching any pointer (all NULL here)
    # and need no workspace; the other arguments are still validated.
    for fn, args in [("lsh_fwd_workspace_bytes", (B, H, n, 64, 8, 2, 64, BF16)),
                     ("lsh_hash_workspace_bytes", (B, H, n, 64, 8, 2, BF16)),
                     ("lsh_sort_workspace_bytes", (B, H, n, 8, 2))]:
        st, nbytes = _ws(fn, *args)
        assert st == OK and nbytes == 0, fn
    assert L.reformer_lsh_attn_fwd(None, None, None, 8, 2, 64, 1, B, H, n, 64, BF16, None, None, None, 0, None,
                                   None) == OK
    assert L.lsh_hash(None, None, None, B, H, n, 64, 8, 2, BF16, None, 0, None) == OK
    assert L.lsh_sort(None, None, None, B, H, n, 8, 2, None, 0, None) == OK
    assert L.lsh_chunk_attn(None, None, None, None, None, B, H, n, 64, 2, 64, 1, BF16, None) == OK
    assert L.lsh_unsort_combine(None, None, None, None, None, B, H, n, 64, 2, BF16, None) == OK
    # still validated: bucket count, chunk length, dtype
    assert L.reformer_lsh_attn_fwd(None, None, None, 7, 2, 64, 1, B, H, n, 64, BF16, None, None, None, 0, None,
                                   None) == BUCKETS
    assert L.lsh_chunk_attn(None, None, None, None, None, B, H, n, 64, 2, 32, 1, BF16, None) == UNSUPPORTED
    assert L.lsh_unsort_combine(None, None, None, None, None, B, H, n, 64, 2, 9, None) == UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        bd.reformer_lsh_attn_fwd(x, x, None, 1, 1)


def test_variant_calls_reject_before_launch(L):
    SB, DD = bd.LSH_ATTEND_SAME_BUCKET, bd.LSH_ATTEND_DEDUP
    P6, P7, P8 = 0x60000000, 0x70000000, 0x80000000
    st, need = _ws("lsh_chunk_attn_ex_workspace_bytes", 1, 1, 256, 2, DD)
    assert st == OK and need >= 256 * 2 * 4
    assert _ws("lsh_chunk_attn_ex_workspace_bytes", 1, 1, 256, 2, SB) == (OK, 0)
    assert _ws("lsh_chunk_attn_ex_workspace_bytes", 1, 1, 256, 2, 4)[0] == UNSUPPORTED
    assert _ws("lsh_chunk_attn_ex_workspace_bytes", 0, 1, 256, 2, DD) == (OK, 0)
    ex = L.lsh_chunk_attn_ex
    # args: qk, v, sorted_idx, buckets, undo_idx, o, lse, B, H, L, D, n_h, C, causal, attend, dt, ws, ws_bytes, stream
    assert ex(P1, P2, P3, None, None, P6, P7, 1, 1, 256, 64, 2, 64, 0, SB, BF16, None, 0, None) == NULL  # buckets
    assert ex(P1, P2, P3, None, None, P6, P7, 1, 1, 256, 64, 2, 64, 0, DD, BF16, P8, need, None) == NULL  # undo
    assert ex(P1, P2, P3, P4, None, P6, P7, 1, 1, 256, 64, 2, 64, 0, SB | DD, BF16, P8, need, None) == NULL
    assert ex(P1, P2, P3, None, P5, P6, P7, 1, 1, 256, 64, 2, 64, 0, DD, BF16, None, 0, None) == WORKSPACE
    assert ex(P1, P2, P3, None, P5, P6, P7, 1, 1, 256, 64, 2, 64, 0, DD, BF16, P8, need - 1, None) == WORKSPACE
    assert ex(P1, P2, P3, P4, P5, P6, P7, 1, 1, 256, 64, 2, 64, 0, 4, BF16, P8, need, None) == UNSUPPORTED
    assert ex(P1, P2, P3, P4, P5, P6, P7, 1, 1, 256, 64, 2, 64, 0, -1, BF16, P8, need, None) == UNSUPPORTED
    # outputs or workspace on top of the variant's inputs; an unread input may alias
    assert ex(P1, P2, P3, P4, None, P4, P7, 1, 1, 256, 64, 2, 64, 0, SB, BF16, None, 0, None) == ALIAS
    assert ex(P1, P2, P3, None, P5, P6, P5, 1, 1, 256, 64, 2, 64, 0, DD, BF16, P8, need, None) == ALIAS
    assert ex(P1, P2, P3, None, P5, P6, P7, 1, 1, 256, 64, 2, 64, 0, DD, BF16, P5 + 64, need, None) == ALIAS
    assert ex(P1, P2, P3, None, P5, P6, P7, 1, 1, 256, 64, 2, 64, 0, DD, BF16, P6, need, None) == ALIAS
    assert ex(None, None, None, None, None, None, None, 0, 1, 256, 64, 2, 64, 0, SB | DD, BF16, None, 0, None) == OK
    assert ex(None, None, None, None, None, None, None, 1, 1, 100, 64, 2, 64, 0, SB, BF16, None, 0, None) == SHAPE
    st, need = _ws("lsh_fwd_workspace_bytes", 1, 2, 128, 64, 8, 2, 64, BF16)
    f = L.reformer_lsh_attn_fwd_ex
    # args: qk, v, rot, n_b, n_h, C, causal, attend, B, H, L, D, dt, out, lse, ws, ws_bytes, stream, events
    assert f(P1, P2, P3, 8, 2, 64, 0, 8, 1, 2, 128, 64, BF16, P4, None, P5, need, None, None) == UNSUPPORTED
    assert f(P1, P2, P3, 8, 2, 64, 0, SB | DD, 1, 2, 128, 64, BF16, P4, None, P5, need - 1, None, None) == WORKSPACE
    assert f(P1, P2, P3, 8, 2, 64, 0, DD, 1, 2, 128, 64, BF16, P1, None, P5, need, None, None) == ALIAS
    assert f(None, P2, P3, 8, 2, 64, 0, SB, 1, 2, 128, 64, BF16, P4, None, P5, need, None, None) == NULL
    assert f(None, None, None, 8, 2, 64, 0, SB, 1, 0, 128, 64, BF16, None, None, None, 0, None, None) == OK


def test_block_calls_reject_before_launch(L):
    BF = BF16
    P6, P7 = 0x60000000, 0x70000000
    ln = L.lsh_layer_norm
    assert ln(P1, P2, P3, P4, 10, 512, F32, None) == UNSUPPORTED
    assert ln(P1, P2, P3, P4, 10, 2048, BF, None) == UNSUPPORTED
    assert ln(P1, P2, P3, P1, 10, 512, BF, None) == ALIAS
    assert ln(None, P2, P3, P4, 10, 512, BF, None) == NULL
    assert ln(None, None, None, None, 0, 512, BF, None) == OK
    lin = L.lsh_linear
    # args: a, a_layout, w, bias, resid, c, c_layout, M, N, K, L, heads, epilogue, dt, stream
    assert lin(P1, 0, P2, None, None, P3, 0, 128, 100, 64, 1, 1, 0, BF, None) == UNSUPPORTED   # N % 128
    assert lin(P1, 0, P2, None, None, P3, 0, 128, 128, 60, 1, 1, 0, BF, None) == UNSUPPORTED   # K % 64
    assert lin(P1, 0, P2, None, None, P3, 0, 128, 128, 64, 1, 1, 2, BF, None) == UNSUPPORTED   # GELU alone
    assert lin(P1, 0, P2, None, None, P3, 0, 128, 128, 64, 1, 1, 1, BF, None) == UNSUPPORTED   # bias alone
    assert lin(P1, 1, P2, None, None, P3, 1, 128, 128, 128, 64, 2, 0, BF, None) == UNSUPPORTED  # heads -> heads
    assert lin(P1, 0, P2, None, P4, P3, 1, 128, 128, 64, 64, 2, 4, BF, None) == UNSUPPORTED    # resid with heads out
    assert lin(P1, 1, P2, None, None, P3, 0, 128, 128, 128, 64, 3, 0, BF, None) == SHAPE       # K != 64 heads
    assert lin(P1, 0, P2, None, None, P3, 0, 128, 128, 64, 1, 1, 0, F32, None) == UNSUPPORTED
    assert lin(P1, 0, P2, None, None, P1, 0, 128, 128, 64, 1, 1, 0, BF, None) == ALIAS
    assert lin(P1, 0, P2, None, None, None, 0, 128, 128, 64, 1, 1, 0, BF, None) == NULL
    assert lin(P1, 0, P2, None, None, P3, 0, 128, 128, 64, 1, 1, 5, BF, None) == NULL          # bias|resid missing
    assert lin(None, 0, None, None, None, None, 0, 0, 128, 64, 1, 1, 0, BF, None) == OK
    st, need = _ws("reformer_block_workspace_bytes", 1, 256, 2, 8, 2, 64, 100, BF)
    assert st == OK and need > 256 * 128 * 2 * 6
    assert _ws("reformer_block_workspace_bytes", 1, 256, 3, 8, 2, 64, 0, BF)[0] == UNSUPPORTED  # odd heads
    assert _ws("reformer_block_workspace_bytes", 1, 256, 2, 8, 2, 64, 0, F32)[0] == UNSUPPORTED
    assert _ws("reformer_block_workspace_bytes", 1, 256, 2, 8, 2, 64, -1, BF)[0] == SHAPE
    params = (ctypes.c_void_p * 11)(*[0x1000000 * (k + 200) for k in range(11)])
    pp = ctypes.cast(params, ctypes.c_void_p)
    f = L.reformer_block_fwd
    # args: x1, x2, rot, params, B, L, heads, n_b, n_h, C, causal, chunk_rows, dt, y1, y2, ws, ws_bytes, stream, ev
    assert f(P1, P2, P3, pp, 1, 256, 2, 8, 2, 64, 0, 100, BF, P4, P5, P6, need - 1, None, None) == WORKSPACE
    assert f(P1, P2, P3, pp, 1, 256, 2, 8, 2, 64, 0, 100, BF, P1, P5, P6, need, None, None) == ALIAS
    assert f(P1, P2, P3, pp, 1, 256, 2, 8, 2, 64, 0, 100, BF, P4, P4, P6, need, None, None) == ALIAS
    assert f(P1, P2, P3, None, 1, 256, 2, 8, 2, 64, 0, 100, BF, P4, P5, P6, need, None, None) == NULL
    params[7] = None
    assert f(P1, P2, P3, pp, 1, 256, 2, 8, 2, 64, 0, 100, BF, P4, P5, P6, need, None, None) == NULL
    assert f(None, None, None, None, 1, 0, 2, 8, 2, 64, 0, 100, BF, None, None, None, 0, None, None) == OK


TOO_LARGE = -8


def test_noalloc_forward_rejects_on_the_host(L):
    """The allocation-free forward validates like reformer_lsh_attn_fwd and
    rejects a problem whose workspace exceeds its fixed scratch before it looks
    up the scratch or enqueues anything (no GPU is used here)."""
    f = L.reformer_lsh_attn_fwd_noalloc
    # fp32, one problem of 65536 tokens with 16 rounds: about 296 MiB of workspace
    big = bd.fwd_workspace_bytes(1, 1, 65536, 64, 4096, 16, 64, F32)
    assert big > 256 << 20
    assert f(P1, P2, P3, 4096, 16, 64, 0, 1, 1, 65536, 64, F32, P4, P5, None) == TOO_LARGE
    # the largest bf16 problem the header names fits (2^20 token-rounds)
    assert bd.fwd_workspace_bytes(1, 1, 65536, 64, 4096, 16, 64, BF16) <= 256 << 20
    assert bd.fwd_workspace_bytes(1, 1, 65536, 64, 4096, 8, 64, F32) <= 256 << 20
    assert f(None, P2, P3, 16, 1, 64, 0, 1, 1, 1024, 64, F32, P4, P5, None) == NULL
    assert f(P1, P2, None, 16, 1, 64, 0, 1, 1, 1024, 64, F32, P4, P5, None) == NULL
    assert f(P1, P2, P3, 16, 1, 64, 0, 1, 1, 1000, 64, F32, P4, P5, None) == SHAPE
    assert f(P1, P2, P3, 15, 1, 64, 0, 1, 1, 1024, 64, F32, P4, P5, None) == BUCKETS
    assert f(P1, P2, P3, 16, 1, 32, 0, 1, 1, 1024, 64, F32, P4, P5, None) == UNSUPPORTED
    assert f(P1, P2, P3, 16, 1, 64, 0, 1, 1, 1024, 64, 7, P4, P5, None) == UNSUPPORTED
    # out overlapping qk
    assert f(P1, P2, P3, 16, 1, 64, 0, 1, 1, 1024, 64, F32, P1 + 64, P5, None) == ALIAS
    # empty problems are no-op successes that touch no pointer
    assert f(None, None, None, 16, 1, 64, 0, 0, 1, 1024, 64, F32, None, None, None) == OK
    assert L.lsh_status_string(TOO_LARGE) != L.lsh_status_string(99)
