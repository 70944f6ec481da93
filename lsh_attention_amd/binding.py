"""Thin ctypes binding of the C ABI in include/lsh_attn.h.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs and workspaces are allocated with torch (device memory
plumbing), and the C entry point of the same name is called on torch's
current HIP stream.  Every step of the method runs in the library's gfx950
kernels; there is no fallback, and a missing library or GPU raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblsh_attn.so")
_HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lsh_attn.h")
_lib = None

LSH_F32, LSH_BF16 = 0, 1
LSH_ATTEND_SAME_BUCKET, LSH_ATTEND_DEDUP = 1, 2
N_KERNELS = 7
N_EVENTS = N_KERNELS + 1
KERNEL_NAMES = ["prep", "hash", "fixup", "sort_hist", "sort_scatter", "chunk_attn", "combine"]
BWD_N_KERNELS = 3
BWD_N_EVENTS = BWD_N_KERNELS + 1
BWD_KERNEL_NAMES = ["bwd_prep", "attn_bwd", "bwd_reduce"]

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
_SIGS = {
    "lsh_status_string": (ctypes.c_char_p, [_c_int]),
    "lsh_hash_workspace_bytes": (_c_int, [_c_int] * 7 + [ctypes.POINTER(_c_size)]),
    "lsh_hash": (_c_int, [_vp, _vp, _vp] + [_c_int] * 7 + [_vp, _c_size, _vp]),
    "lsh_hash_uncertified": (_c_int, [_vp, _c_size] + [_c_int] * 6 + [ctypes.POINTER(_c_int), _vp]),
    "lsh_sort_workspace_bytes": (_c_int, [_c_int] * 5 + [ctypes.POINTER(_c_size)]),
    "lsh_sort": (_c_int, [_vp, _vp, _vp] + [_c_int] * 5 + [_vp, _c_size, _vp]),
    "lsh_chunk_attn": (_c_int, [_vp] * 5 + [_c_int] * 8 + [_vp]),
    "reformer_lsh_attn_fwd_noalloc": (_c_int, [_vp, _vp, _vp] + [_c_int] * 9 + [_vp, _vp, _vp]),
    "lsh_chunk_attn_ex_workspace_bytes": (_c_int, [_c_int] * 5 + [ctypes.POINTER(_c_size)]),
    "lsh_chunk_attn_ex": (_c_int, [_vp] * 7 + [_c_int] * 9 + [_vp, _c_size, _vp]),
    "lsh_unsort_combine": (_c_int, [_vp] * 5 + [_c_int] * 6 + [_vp]),
    "lsh_fwd_workspace_bytes": (_c_int, [_c_int] * 8 + [ctypes.POINTER(_c_size)]),
    "reformer_lsh_attn_fwd": (_c_int, [_vp] * 3 + [_c_int] * 9 + [_vp, _vp, _vp, _c_size, _vp, _vp]),
    "reformer_lsh_attn_fwd_ex": (_c_int, [_vp] * 3 + [_c_int] * 10 + [_vp, _vp, _vp, _c_size, _vp, _vp]),
    "lsh_attn_bwd_workspace_bytes": (_c_int, [_c_int] * 7 + [ctypes.POINTER(_c_size)]),
    "lsh_attn_bwd": (_c_int, [_vp] * 10 + [_c_int] * 8 + [_vp, _c_size, _vp, _vp]),
    "reformer_lsh_attn_fwd_train": (_c_int, [_vp] * 3 + [_c_int] * 9 + [_vp] * 6 + [_c_size, _vp, _vp]),
    "lsh_layer_norm": (_c_int, [_vp] * 4 + [_c_int] * 3 + [_vp]),
    "lsh_linear": (_c_int, [_vp, _c_int, _vp, _vp, _vp, _vp] + [_c_int] * 8 + [_vp]),
    "reformer_block_workspace_bytes": (_c_int, [_c_int] * 8 + [ctypes.POINTER(_c_size)]),
    "reformer_block_fwd": (_c_int, [_vp] * 4 + [_c_int] * 9 + [_vp, _vp, _vp, _c_size, _vp, _vp]),
    "lsh_event_create": (_c_int, [ctypes.POINTER(_vp)]),
    "lsh_event_destroy": (_c_int, [_vp]),
    "lsh_event_record": (_c_int, [_vp, _vp]),
    "lsh_event_elapsed_ms": (_c_int, [_vp, _vp, ctypes.POINTER(ctypes.c_float)]),
    "lsh_measure_clock": (_c_int, [_vp, _c_int, ctypes.POINTER(ctypes.c_double), _vp]),
}


class LshError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().lsh_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def header_functions() -> list:
    """Names of the functions declared in include/lsh_attn.h."""
    text = open(_HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\*|int)\s+(\w+)\s*\(", text, flags=re.M)))


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m lsh_attention_amd.build`")
        h = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype, f.argtypes = res, args
        _lib = h
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise LshError(fn, status)


def _dtype_code_of(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return LSH_BF16
    if dtype == torch.float32:
        return LSH_F32
    raise TypeError(f"unsupported dtype {dtype} (float32 or bfloat16)")


def _dtype_code(t: torch.Tensor) -> int:
    return _dtype_code_of(t.dtype)


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU (the HIP path has no CPU fallback)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def hash_workspace_bytes(B, H, L, D, n_buckets, n_hashes, dtype_code) -> int:
    n = _c_size()
    _check("lsh_hash_workspace_bytes", lib().lsh_hash_workspace_bytes(B, H, L, D, n_buckets, n_hashes, dtype_code,
                                                                     ctypes.byref(n)))
    return n.value


def sort_workspace_bytes(B, H, L, n_buckets, n_hashes) -> int:
    n = _c_size()
    _check("lsh_sort_workspace_bytes", lib().lsh_sort_workspace_bytes(B, H, L, n_buckets, n_hashes, ctypes.byref(n)))
    return n.value


def fwd_workspace_bytes(B, H, L, D, n_buckets, n_hashes, chunk_len, dtype_code) -> int:
    n = _c_size()
    _check("lsh_fwd_workspace_bytes", lib().lsh_fwd_workspace_bytes(B, H, L, D, n_buckets, n_hashes, chunk_len,
                                                                   dtype_code, ctypes.byref(n)))
    return n.value


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def lsh_hash(qk: torch.Tensor, rot: torch.Tensor | None, n_buckets: int, n_hashes: int,
             buckets: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """qk [B,H,L,D], rot [n_h,D,n_b/2] (or None when n_b == 1) -> buckets int32 [B,H,n_h,L].
    `workspace` (uint8, at least hash_workspace_bytes) may be passed in, e.g. to read
    hash_uncertified afterwards."""
    _dev(qk, rot, buckets, workspace)
    B, H, L, D = qk.shape
    dt = _dtype_code(qk)
    if rot is not None and rot.dtype != qk.dtype:
        raise TypeError("rot must have the dtype of qk")
    if buckets is None:
        buckets = torch.empty((B, H, n_hashes, L), dtype=torch.int32, device=qk.device)
    ws = workspace if workspace is not None else _workspace(
        hash_workspace_bytes(B, H, L, D, n_buckets, n_hashes, dt), qk.device)
    _check("lsh_hash", lib().lsh_hash(qk.data_ptr(), _ptr(rot), buckets.data_ptr(), B, H, L, D, n_buckets, n_hashes,
                                      dt, ws.data_ptr(), ws.numel(), _stream(qk.device)))
    return buckets


def hash_uncertified(workspace: torch.Tensor, B: int, H: int, L: int, n_buckets: int, n_hashes: int,
                     dtype: torch.dtype) -> int:
    """Token-rounds the last hashing on `workspace` (of lsh_hash or the fused forward,
    same shapes) re-decided from float64 sums because fp32 could not certify them."""
    _dev(workspace)
    n = _c_int(0)
    _check("lsh_hash_uncertified", lib().lsh_hash_uncertified(
        workspace.data_ptr(), workspace.numel(), B, H, L, n_buckets, n_hashes, _dtype_code_of(dtype), ctypes.byref(n),
        _stream(workspace.device)))
    return int(n.value)


CLOCK_TICKS_BYTES = 2 * 2048 * 8  # LSH_CLOCK_TICKS_BYTES


def measure_clock_mhz(spin_us: int = 200, device="cuda") -> float:
    """Shader clock in MHz under a full-chip FMA spin of about spin_us microseconds
    (shader-cycle counter against the constant-rate real-time counter)."""
    ticks = torch.empty(CLOCK_TICKS_BYTES, dtype=torch.uint8, device=device)
    mhz = ctypes.c_double(0.0)
    _check("lsh_measure_clock", lib().lsh_measure_clock(ticks.data_ptr(), spin_us, ctypes.byref(mhz),
                                                        _stream(ticks.device)))
    return float(mhz.value)


def lsh_sort(buckets: torch.Tensor, n_buckets: int):
    """buckets int32 [B,H,n_h,L] -> (sorted_idx int32 [B,H,n_h*L], undo_idx int32 [B,H,n_h,L])."""
    _dev(buckets)
    if buckets.dtype != torch.int32:
        raise TypeError("buckets must be int32")
    B, H, n_h, L = buckets.shape
    sorted_idx = torch.empty((B, H, n_h * L), dtype=torch.int32, device=buckets.device)
    undo_idx = torch.empty((B, H, n_h, L), dtype=torch.int32, device=buckets.device)
    ws = _workspace(sort_workspace_bytes(B, H, L, n_buckets, n_h), buckets.device)
    _check("lsh_sort", lib().lsh_sort(buckets.data_ptr(), sorted_idx.data_ptr(), undo_idx.data_ptr(), B, H, L,
                                      n_buckets, n_h, ws.data_ptr(), ws.numel(), _stream(buckets.device)))
    return sorted_idx, undo_idx


def attend_flags(same_bucket: bool = False, dedup: bool = False) -> int:
    """The `attend` argument of the *_ex entry points."""
    return (LSH_ATTEND_SAME_BUCKET if same_bucket else 0) | (LSH_ATTEND_DEDUP if dedup else 0)


def lsh_chunk_attn(qk: torch.Tensor, v: torch.Tensor, sorted_idx: torch.Tensor, n_hashes: int, chunk_len: int,
                   causal: bool, buckets: torch.Tensor | None = None, undo_idx: torch.Tensor | None = None,
                   same_bucket: bool = False, dedup: bool = False):
    """-> (o_sorted [B,H,n_h*L,D] in qk's dtype, lse_sorted float32 [B,H,n_h*L]).
    With `same_bucket` (needs `buckets` [B,H,n_h,L]) or `dedup` (needs `undo_idx`
    [B,H,n_h,L]) the attended-set variant of lsh_chunk_attn_ex runs."""
    _dev(qk, v, sorted_idx, buckets, undo_idx)
    B, H, L, D = qk.shape
    dt = _dtype_code(qk)
    if v.shape != qk.shape or v.dtype != qk.dtype:
        raise ValueError("v must match qk in shape and dtype")
    if sorted_idx.dtype != torch.int32 or sorted_idx.shape != (B, H, n_hashes * L):
        raise ValueError("sorted_idx must be int32 [B,H,n_h*L]")
    for name, t, need in (("buckets", buckets, same_bucket), ("undo_idx", undo_idx, dedup)):
        if need and t is None:
            raise ValueError(f"{name} is required for this variant")
        if t is not None and (t.dtype != torch.int32 or t.shape != (B, H, n_hashes, L)):
            raise ValueError(f"{name} must be int32 [B,H,n_h,L]")
    o_sorted = torch.empty((B, H, n_hashes * L, D), dtype=qk.dtype, device=qk.device)
    lse_sorted = torch.empty((B, H, n_hashes * L), dtype=torch.float32, device=qk.device)
    attend = attend_flags(same_bucket, dedup)
    if attend == 0:
        _check("lsh_chunk_attn", lib().lsh_chunk_attn(qk.data_ptr(), v.data_ptr(), sorted_idx.data_ptr(),
                                                      o_sorted.data_ptr(), lse_sorted.data_ptr(), B, H, L, D,
                                                      n_hashes, chunk_len, int(bool(causal)), dt, _stream(qk.device)))
    else:
        n = ctypes.c_size_t()
        _check("lsh_chunk_attn_ex_workspace_bytes",
               lib().lsh_chunk_attn_ex_workspace_bytes(B, H, L, n_hashes, attend, ctypes.byref(n)))
        ws = _workspace(n.value, qk.device) if n.value else None
        _check("lsh_chunk_attn_ex", lib().lsh_chunk_attn_ex(
            qk.data_ptr(), v.data_ptr(), sorted_idx.data_ptr(), _ptr(buckets), _ptr(undo_idx), o_sorted.data_ptr(),
            lse_sorted.data_ptr(), B, H, L, D, n_hashes, chunk_len, int(bool(causal)), attend, dt, _ptr(ws),
            0 if ws is None else ws.numel(), _stream(qk.device)))
    return o_sorted, lse_sorted


def lsh_unsort_combine(o_sorted: torch.Tensor, lse_sorted: torch.Tensor, undo_idx: torch.Tensor,
                       want_lse: bool = True):
    """-> (out [B,H,L,D] in o_sorted's dtype, lse float32 [B,H,L] or None)."""
    _dev(o_sorted, lse_sorted, undo_idx)
    B, H, n_h, L = undo_idx.shape
    D = o_sorted.shape[-1]
    dt = _dtype_code(o_sorted)
    out = torch.empty((B, H, L, D), dtype=o_sorted.dtype, device=o_sorted.device)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=o_sorted.device) if want_lse else None
    _check("lsh_unsort_combine", lib().lsh_unsort_combine(o_sorted.data_ptr(), lse_sorted.data_ptr(),
                                                          undo_idx.data_ptr(), out.data_ptr(), _ptr(lse), B, H, L,
                                                          D, n_h, dt, _stream(o_sorted.device)))
    return out, lse


def reformer_lsh_attn_fwd(qk: torch.Tensor, v: torch.Tensor, rot: torch.Tensor | None, n_buckets: int,
                          n_hashes: int, chunk_len: int = 64, causal: bool = False, want_lse: bool = True,
                          out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None, stage_events=None, same_bucket: bool = False,
                          dedup: bool = False):
    """The fused forward pass.  Returns (out [B,H,L,D], lse float32 [B,H,L] or None).
    `workspace` (uint8, at least fwd_workspace_bytes) and `out`/`lse` may be passed
    in to avoid allocation; `stage_events` is an EventSet for per-kernel timing.
    `same_bucket` / `dedup` select the attended-set variants (reformer_lsh_attn_fwd_ex)."""
    _dev(qk, v, rot, out, lse, workspace)
    B, H, L, D = qk.shape
    dt = _dtype_code(qk)
    if v.shape != qk.shape or v.dtype != qk.dtype:
        raise ValueError("v must match qk in shape and dtype")
    if rot is not None and rot.dtype != qk.dtype:
        raise TypeError("rot must have the dtype of qk")
    if out is None:
        out = torch.empty_like(qk)
    if lse is None and want_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=qk.device)
    if workspace is None:
        workspace = _workspace(fwd_workspace_bytes(B, H, L, D, n_buckets, n_hashes, chunk_len, dt), qk.device)
    ev = None if stage_events is None else stage_events.array()
    attend = attend_flags(same_bucket, dedup)
    if attend == 0:
        _check("reformer_lsh_attn_fwd", lib().reformer_lsh_attn_fwd(
            qk.data_ptr(), v.data_ptr(), _ptr(rot), n_buckets, n_hashes, chunk_len, int(bool(causal)), B, H, L, D,
            dt, out.data_ptr(), _ptr(lse), workspace.data_ptr(), workspace.numel(), _stream(qk.device), ev))
    else:
        _check("reformer_lsh_attn_fwd_ex", lib().reformer_lsh_attn_fwd_ex(
            qk.data_ptr(), v.data_ptr(), _ptr(rot), n_buckets, n_hashes, chunk_len, int(bool(causal)), attend, B, H,
            L, D, dt, out.data_ptr(), _ptr(lse), workspace.data_ptr(), workspace.numel(), _stream(qk.device), ev))
    return out, lse


def reformer_lsh_attn_fwd_noalloc(qk: torch.Tensor, v: torch.Tensor, rot: torch.Tensor | None, n_buckets: int,
                                  n_hashes: int, chunk_len: int = 64, causal: bool = False,
                                  out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                                  want_lse: bool = True):
    """The fused forward pass on the library's fixed device scratch (no workspace).
    Returns (out, lse or None); pass `out` / `lse` to allocate nothing here either."""
    _dev(qk, v, rot, out, lse)
    B, H, L, D = qk.shape
    dt = _dtype_code(qk)
    if v.shape != qk.shape or v.dtype != qk.dtype:
        raise ValueError("v must match qk in shape and dtype")
    if rot is not None and rot.dtype != qk.dtype:
        raise TypeError("rot must have the dtype of qk")
    if out is None:
        out = torch.empty_like(qk)
    if lse is None and want_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=qk.device)
    _check("reformer_lsh_attn_fwd_noalloc", lib().reformer_lsh_attn_fwd_noalloc(
        qk.data_ptr(), v.data_ptr(), _ptr(rot), n_buckets, n_hashes, chunk_len, int(bool(causal)), B, H, L, D, dt,
        out.data_ptr(), _ptr(lse), _stream(qk.device)))
    return out, lse


def lsh_attn_bwd(qk: torch.Tensor, v: torch.Tensor, sorted_idx: torch.Tensor, undo_idx: torch.Tensor,
                 lse_sorted: torch.Tensor, out: torch.Tensor, dout: torch.Tensor, dlse: torch.Tensor | None,
                 n_hashes: int, chunk_len: int = 64, causal: bool = False, dqk: torch.Tensor | None = None,
                 dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stage_events=None):
    """Gradients (dqk, dv) of sum(dout * out) + sum(dlse * lse) through the forward pass
    whose permutation (sorted_idx, undo_idx) and per-round lse (lse_sorted) are given.
    `stage_events`: an EventSet of BWD_N_EVENTS events for per-kernel timing."""
    _dev(qk, v, sorted_idx, undo_idx, lse_sorted, out, dout, dlse, dqk, dv, workspace)
    B, H, L, D = qk.shape
    dt = _dtype_code(qk)
    for name, t in (("v", v), ("out", out), ("dout", dout)):
        if t.shape != qk.shape or t.dtype != qk.dtype:
            raise ValueError(f"{name} must match qk in shape and dtype")
    if sorted_idx.dtype != torch.int32 or sorted_idx.shape != (B, H, n_hashes * L):
        raise ValueError("sorted_idx must be int32 [B,H,n_h*L]")
    if undo_idx.dtype != torch.int32 or undo_idx.shape != (B, H, n_hashes, L):
        raise ValueError("undo_idx must be int32 [B,H,n_h,L]")
    if lse_sorted.dtype != torch.float32 or lse_sorted.shape != (B, H, n_hashes * L):
        raise ValueError("lse_sorted must be float32 [B,H,n_h*L]")
    if dlse is not None and (dlse.dtype != torch.float32 or dlse.shape != (B, H, L)):
        raise ValueError("dlse must be float32 [B,H,L]")
    dqk = torch.empty_like(qk) if dqk is None else dqk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        n = ctypes.c_size_t()
        _check("lsh_attn_bwd_workspace_bytes",
               lib().lsh_attn_bwd_workspace_bytes(B, H, L, D, n_hashes, chunk_len, dt, ctypes.byref(n)))
        workspace = _workspace(n.value, qk.device)
    _check("lsh_attn_bwd", lib().lsh_attn_bwd(
        qk.data_ptr(), v.data_ptr(), sorted_idx.data_ptr(), undo_idx.data_ptr(), lse_sorted.data_ptr(),
        out.data_ptr(), dout.data_ptr(), _ptr(dlse), dqk.data_ptr(), dv.data_ptr(), B, H, L, D, n_hashes, chunk_len,
        int(bool(causal)), dt, _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(qk.device),
        None if stage_events is None else stage_events.array()))
    return dqk, dv


def bwd_workspace_bytes(B: int, H: int, L: int, D: int, n_hashes: int, chunk_len: int, dt: int) -> int:
    n = ctypes.c_size_t()
    _check("lsh_attn_bwd_workspace_bytes",
           lib().lsh_attn_bwd_workspace_bytes(B, H, L, D, n_hashes, chunk_len, dt, ctypes.byref(n)))
    return n.value


def reformer_lsh_attn_fwd_train(qk: torch.Tensor, v: torch.Tensor, rot: torch.Tensor | None, n_buckets: int,
                                n_hashes: int, chunk_len: int = 64, causal: bool = False, out=None, lse=None,
                                sorted_idx=None, undo_idx=None, lse_sorted=None, workspace=None, stage_events=None):
    """The fused forward that also returns the state the backward reuses:
    (out, lse, sorted_idx [B,H,n_h*L], undo_idx [B,H,n_h,L], lse_sorted [B,H,n_h*L])."""
    _dev(qk, v, rot, out, lse, sorted_idx, undo_idx, lse_sorted, workspace)
    B, H, L, D = qk.shape
    dt = _dtype_code(qk)
    if v.shape != qk.shape or v.dtype != qk.dtype:
        raise ValueError("v must match qk in shape and dtype")
    if rot is not None and rot.dtype != qk.dtype:
        raise TypeError("rot must have the dtype of qk")
    dev = qk.device
    out = torch.empty_like(qk) if out is None else out
    lse = torch.empty((B, H, L), dtype=torch.float32, device=dev) if lse is None else lse
    n_slots = n_hashes * L
    sorted_idx = torch.empty((B, H, n_slots), dtype=torch.int32, device=dev) if sorted_idx is None else sorted_idx
    undo_idx = torch.empty((B, H, n_hashes, L), dtype=torch.int32, device=dev) if undo_idx is None else undo_idx
    lse_sorted = torch.empty((B, H, n_slots), dtype=torch.float32, device=dev) if lse_sorted is None else lse_sorted
    if workspace is None:
        workspace = _workspace(fwd_workspace_bytes(B, H, L, D, n_buckets, n_hashes, chunk_len, dt), dev)
    ev = None if stage_events is None else stage_events.array()
    _check("reformer_lsh_attn_fwd_train", lib().reformer_lsh_attn_fwd_train(
        qk.data_ptr(), v.data_ptr(), _ptr(rot), n_buckets, n_hashes, chunk_len, int(bool(causal)), B, H, L, D, dt,
        out.data_ptr(), lse.data_ptr(), sorted_idx.data_ptr(), undo_idx.data_ptr(), lse_sorted.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream(dev), ev))
    return out, lse, sorted_idx, undo_idx, lse_sorted


LAYOUT_ROWS, LAYOUT_HEADS = 0, 1
EPI_BIAS, EPI_GELU, EPI_RESID = 1, 2, 4
BLOCK_PARAMS = ["ln1_g", "ln1_b", "w_qk", "w_v", "w_o", "ln2_g", "ln2_b", "w1", "b1", "w2", "b2"]
BLOCK_N_STAGES = 6
BLOCK_N_EVENTS = BLOCK_N_STAGES + 1
BLOCK_STAGE_NAMES = ["ln1", "qkv_proj", "attention", "out_proj", "ln2", "ffn"]


def lsh_layer_norm(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, out: torch.Tensor | None = None):
    """LayerNorm over the last dimension (bf16)."""
    _dev(x, gamma, beta, out)
    dim = x.shape[-1]
    rows = x.numel() // dim
    out = torch.empty_like(x) if out is None else out
    _check("lsh_layer_norm", lib().lsh_layer_norm(x.data_ptr(), gamma.data_ptr(), beta.data_ptr(), out.data_ptr(),
                                                  rows, dim, _dtype_code(x), _stream(x.device)))
    return out


def lsh_linear(a: torch.Tensor, w: torch.Tensor, bias=None, resid=None, gelu: bool = False, a_heads: bool = False,
               out=None):
    """epilogue(a . w^T) with w [N, K] (bf16), as rows [..., N].  a is rows [..., K],
    or head-major [B, H, L, 64] (a_heads; the result is then [B, L, N])."""
    _dev(a, w, bias, resid, out)
    N, K = w.shape
    if a_heads:
        B, H, L, _ = a.shape
        M, shape, Ld, Hd = B * L, (B, L, N), L, H
    else:
        M, shape, Ld, Hd = a.numel() // K, tuple(a.shape[:-1]) + (N,), 1, 1
    epi = (EPI_BIAS if bias is not None else 0) | (EPI_GELU if gelu else 0) | (EPI_RESID if resid is not None else 0)
    out = torch.empty(shape, dtype=a.dtype, device=a.device) if out is None else out
    _check("lsh_linear", lib().lsh_linear(a.data_ptr(), LAYOUT_HEADS if a_heads else LAYOUT_ROWS, w.data_ptr(),
                                          _ptr(bias), _ptr(resid), out.data_ptr(), LAYOUT_ROWS, M, N, K, Ld, Hd, epi,
                                          _dtype_code(a), _stream(a.device)))
    return out


def lsh_linear_heads(a: torch.Tensor, w: torch.Tensor, out=None):
    """a [B, L, K] rows . w^T -> [B, H, L, 64] head-major, H = N / 64 (no epilogue)."""
    _dev(a, w, out)
    N, K = w.shape
    B, L, _ = a.shape
    H = N // 64
    out = torch.empty((B, H, L, 64), dtype=a.dtype, device=a.device) if out is None else out
    _check("lsh_linear", lib().lsh_linear(a.data_ptr(), LAYOUT_ROWS, w.data_ptr(), None, None, out.data_ptr(),
                                          LAYOUT_HEADS, B * L, N, K, L, H, 0, _dtype_code(a), _stream(a.device)))
    return out


def block_workspace_bytes(B, L, heads, n_buckets, n_hashes, chunk_len=64, chunk_rows=0, dt=LSH_BF16) -> int:
    n = ctypes.c_size_t()
    _check("reformer_block_workspace_bytes", lib().reformer_block_workspace_bytes(
        B, L, heads, n_buckets, n_hashes, chunk_len, chunk_rows, dt, ctypes.byref(n)))
    return n.value


def reformer_block_fwd(x1: torch.Tensor, x2: torch.Tensor, rot, params: dict, n_buckets: int, n_hashes: int,
                       causal: bool = False, chunk_rows: int = 0, chunk_len: int = 64, y1=None, y2=None,
                       workspace=None, stage_events=None):
    """One reversible block: (y1, y2) = (x1 + F(x2), x2 + G(y1)).  x1, x2 [B, L, dim] bf16;
    params: the BLOCK_PARAMS tensors (weights [out, in])."""
    plist = [params[k] for k in BLOCK_PARAMS]
    _dev(x1, x2, rot, y1, y2, workspace, *plist)
    B, L, dim = x1.shape
    heads = dim // 64
    dt = _dtype_code(x1)
    y1 = torch.empty_like(x1) if y1 is None else y1
    y2 = torch.empty_like(x2) if y2 is None else y2
    if workspace is None:
        workspace = _workspace(block_workspace_bytes(B, L, heads, n_buckets, n_hashes, chunk_len, chunk_rows, dt),
                               x1.device)
    parr = (_vp * len(plist))(*[t.data_ptr() for t in plist])
    ev = None if stage_events is None else stage_events.array()
    _check("reformer_block_fwd", lib().reformer_block_fwd(
        x1.data_ptr(), x2.data_ptr(), _ptr(rot), ctypes.cast(parr, _vp), B, L, heads, n_buckets, n_hashes,
        chunk_len, int(bool(causal)), chunk_rows, dt, y1.data_ptr(), y2.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream(x1.device), ev))
    return y1, y2


class EventSet:
    """N_EVENTS hipEvents created by the library, recorded by the fused call
    around each kernel; `durations_ms()` gives the per-kernel times.  With
    `only`, just those indices get an event (the others stay NULL and are not
    recorded): `only=(k, k + 1)` times kernel k alone."""

    def __init__(self, n: int = N_EVENTS, only=None):
        self._ev = (_vp * n)()
        for i in (range(n) if only is None else only):
            if not 0 <= i < n:
                raise ValueError(f"event index {i} outside 0..{n - 1}")
            h = _vp()
            _check("lsh_event_create", lib().lsh_event_create(ctypes.byref(h)))
            self._ev[i] = h
        self.n = n

    def array(self):
        return ctypes.cast(self._ev, _vp)

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        _check("lsh_event_elapsed_ms", lib().lsh_event_elapsed_ms(self._ev[i], self._ev[j], ctypes.byref(ms)))
        return ms.value

    def durations_ms(self) -> list:
        return [self.elapsed_ms(i, i + 1) for i in range(self.n - 1)]

    def record(self, i: int, device=None):
        _check("lsh_event_record", lib().lsh_event_record(self._ev[i], _stream(device)))

    def close(self):
        for i in range(self.n):
            if self._ev[i]:
                lib().lsh_event_destroy(self._ev[i])
                self._ev[i] = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
