"""Thin ctypes binding of libpkv.so (see include/pkv.h for the operations).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's kernels.  The
library must have been built (``python -m paged_kv_cache_02_amd.build``);
importing this module without it raises ``ImportError`` -- there is no other
implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

(PKV_OK, PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP,
 PKV_ERR_SCRATCH) = range(7)
NOALLOC_SCRATCH_BYTES = 32 << 20
PKV_F32, PKV_BF16 = 0, 1

# name -> (restype, argtypes), in the order of include/pkv.h
_P, _I32, _I64, _SZ, _F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                           ctypes.c_float)
SIGNATURES = {
    "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_version": (ctypes.c_int, []),
    "pkv_reshape_and_cache": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I64, _I64, _I32, _I32,
                                             _I32, _I32, ctypes.c_int, _P]),
    "pkv_rope_cos_sin": (ctypes.c_int, [_P, _I32, _I32, _F, _I32, _F, _I32, _P]),
    "pkv_rope_apply": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32,
                                      ctypes.c_int, _P]),
    "pkv_reshape_and_cache_rope": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I64,
                                                  _I32, _I32, _I32, _I32, _I32, _I32,
                                                  ctypes.c_int, _P]),
    "pkv_paged_decode_workspace_bytes": (ctypes.c_size_t, [_I32] * 5),
    "pkv_paged_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                        _I32, _I32, _I32, _I32, _F, _I32, _P, _I32, _P, _SZ,
                                        ctypes.c_int, _P]),
    "pkv_paged_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                                _I32, _I32, _I32, _I32, _I32, _F, _I32, _P, _I32,
                                                ctypes.c_int, _P]),
    "pkv_paged_decode_append": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32,
                                               _I32, _I32, _I32, _I32, _I32, _I32, _I32, _F,
                                               _I32, _P, _P, _I32, _I32, _I32, _P, _SZ,
                                               ctypes.c_int, _P]),
    "pkv_paged_decode_stage": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                              _I32, _I32, _I32, _F, _I32, _P, _P, _SZ,
                                              ctypes.c_int, _P]),
    "pkv_paged_decode_finish": (ctypes.c_int, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _SZ,
                                               ctypes.c_int, _P]),
    "pkv_paged_decode_partitions": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                                   _I32, _I32, _I32, _I32, _I32, _F, _I32, _P,
                                                   _I32, _I32, ctypes.c_int, _P]),
    "pkv_merge_partitions": (ctypes.c_int, [_P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I32,
                                            _I32, ctypes.c_int, _P]),
    "pkv_vertical_slash_blocks": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                                 _I32, _I32, _P]),
    "pkv_sparse_prefill": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32,
                                          _I32, _I32, _I32, _I32, _F, _P, ctypes.c_int, _P]),
    "pkv_varlen_prefill": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P,
                                          _P, _I32, _I32, _I32, _I32, _I32, _I32, _F, _I32,
                                          _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _SZ,
                                          ctypes.c_int, _P]),
    "pkv_varlen_prefill_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I32,
                                                             ctypes.c_int]),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m paged_kv_cache_02_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


# Entry points that enqueue GPU work (prepare() records these instead of
# running them).
_LAUNCHES = {
    "pkv_reshape_and_cache", "pkv_reshape_and_cache_rope", "pkv_rope_apply", "pkv_rope_cos_sin",
    "pkv_paged_decode", "pkv_paged_decode_noalloc", "pkv_paged_decode_append",
    "pkv_paged_decode_stage", "pkv_paged_decode_finish", "pkv_paged_decode_partitions",
    "pkv_merge_partitions", "pkv_varlen_prefill", "pkv_vertical_slash_blocks",
    "pkv_sparse_prefill",
}
_recording = None          # while prepare() runs: [(function, args, name)], and the tensors kept
_keep = None


class _Library:
    """The loaded library.  Attribute access gives its functions; while
    prepare() records a call, the launching ones are noted with their
    marshalled arguments instead of being run."""

    def __init__(self, cdll):
        self._cdll = cdll

    def __getattr__(self, name):
        fn = getattr(self._cdll, name)
        if name in _LAUNCHES:
            def call(*args, _fn=fn, _name=name):
                if _recording is not None:
                    _recording.append((_fn, args, _name))
                    return PKV_OK
                return _fn(*args)
            fn = call
        setattr(self, name, fn)
        return fn


lib = _Library(load_library())


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib.pkv_status_string(status).decode()} (status {status})")


def _check(status: int, what: str):
    if status != PKV_OK:
        raise PkvError(status, what)


def _dt(t: torch.Tensor, *same: Optional[torch.Tensor]) -> int:
    """The library's dtype code for t; every tensor in same (None skipped)
    must have t's dtype, since the kernels read them all as that type."""
    for u in same:
        if u is not None and u.dtype != t.dtype:
            raise ValueError(f"dtype mismatch: {u.dtype} where {t.dtype} is expected")
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float32:
        return PKV_F32
    raise ValueError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if _keep is not None:
        _keep.append(t)
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32")
    return t


def _f32(t: Optional[torch.Tensor], name: str) -> Optional[torch.Tensor]:
    if t is not None and t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32")
    return t


def _rope_table(cos_sin: torch.Tensor, rotary_dim: int) -> torch.Tensor:
    """The kernels step through the table rotary_dim floats per row and the C
    ABI does not take its width: it must be a contiguous float32
    [positions, rotary_dim] tensor, or a row would be read from the wrong
    place (or past the end of the table)."""
    if cos_sin.dtype != torch.float32 or cos_sin.dim() != 2:
        raise ValueError("cos_sin must be a float32 [positions, rotary_dim] table")
    if cos_sin.shape[1] != rotary_dim:
        raise ValueError(f"cos_sin has {cos_sin.shape[1]} columns, rotary_dim is {rotary_dim}")
    if not cos_sin.is_contiguous():
        raise ValueError("cos_sin must be contiguous")
    return cos_sin


def _row_stride(t: torch.Tensor, name: str) -> int:
    """Elements between tokens of t [T, H, D], whose per-token [H, D] blocks
    must be contiguous (the tokens themselves may be strided)."""
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if t.dim() != 3 or (t.shape[0] > 0 and not t[0].is_contiguous()):
        raise ValueError(f"{name}: each token's [heads, head_dim] block must be contiguous")
    return t.stride(0)


def _raw_ptr(t: torch.Tensor) -> int:
    """Address of a GPU tensor whose rows may be strided (checked by the caller)."""
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if _keep is not None:
        _keep.append(t)
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def version() -> int:
    return lib.pkv_version()


def prepare(fn, *args, **kwargs):
    """Run the binding call fn(*args, **kwargs) up to its library launches,
    which are recorded rather than run, and return a callable that issues
    those launches with the same marshalled arguments, skipping the Python
    checks (for timing loops and tight serving loops).  Every tensor the
    call passed to the library, including buffers it allocated, is kept
    alive by the callable; the launches go to the stream that was current
    when the call was prepared."""
    global _recording, _keep
    rec, keep = [], []
    _recording, _keep = rec, keep
    try:
        result = fn(*args, **kwargs)
    finally:
        _recording, _keep = None, None

    def run(_rec=rec, _keep_alive=(keep, result)):
        for f, a, name in _rec:
            status = f(*a)
            if status != PKV_OK:
                raise PkvError(status, name)
    return run


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping):
    """Store rows key/value [T, Hkv, D] into the caches at slot_mapping [T]."""
    T, Hkv, D = key.shape
    NB, bs = k_cache.shape[0], k_cache.shape[1]
    ks, vs = _row_stride(key, "key"), _row_stride(value, "value")
    _check(lib.pkv_reshape_and_cache(
        _raw_ptr(key), _raw_ptr(value), _ptr(k_cache), _ptr(v_cache),
        _ptr(_i32(slot_mapping, "slot_mapping")), T, ks, vs, Hkv, D, bs, NB,
        _dt(key, value, k_cache, v_cache), _stream()), "reshape_and_cache")


def rope_cos_sin(num_positions: int, rotary_dim: int, base: float = 10000.0, scaling: int = 0,
                 factor: float = 1.0, max_position: int = 0, device="cuda"):
    """Rotary table [num_positions, rotary_dim] float32 (cos, then sin) built on the GPU;
    scaling 0 none, 1 linear, 2 dynamic (see pkv_rope_cos_sin)."""
    t = torch.empty((num_positions, rotary_dim), dtype=torch.float32, device=device)
    _check(lib.pkv_rope_cos_sin(_ptr(t), num_positions, rotary_dim, float(base), scaling,
                                float(factor), max_position, _stream()), "rope_cos_sin")
    return t


def rope_apply(x, positions, cos_sin, rotary_dim: int, neox: bool = True):
    """Rotate x [T, H, D] (rows may be strided, e.g. q or k of a fused QKV
    buffer) in place by positions [T]."""
    _rope_table(cos_sin, rotary_dim)
    T, H, D = x.shape
    xs = _row_stride(x, "x")
    _check(lib.pkv_rope_apply(_raw_ptr(x), _ptr(_i32(positions, "positions")),
                              _ptr(cos_sin), T, H, D, xs, rotary_dim,
                              int(bool(neox)), _dt(x), _stream()), "rope_apply")
    return x


def reshape_and_cache_rope(key, value, k_cache, v_cache, slot_mapping, positions, cos_sin,
                           rotary_dim: int, neox: bool = True):
    """reshape_and_cache with each key row rotated by positions [T] as it is stored."""
    _rope_table(cos_sin, rotary_dim)
    T, Hkv, D = key.shape
    NB, bs = k_cache.shape[0], k_cache.shape[1]
    ks, vs = _row_stride(key, "key"), _row_stride(value, "value")
    _check(lib.pkv_reshape_and_cache_rope(
        _raw_ptr(key), _raw_ptr(value), _ptr(k_cache), _ptr(v_cache),
        _ptr(_i32(slot_mapping, "slot_mapping")), _ptr(_i32(positions, "positions")),
        _ptr(cos_sin), T, ks, vs, Hkv, D, bs, NB,
        rotary_dim, int(bool(neox)), _dt(key, value, k_cache, v_cache), _stream()),
        "reshape_and_cache_rope")


def decode_workspace_bytes(B, num_q_heads, head_dim, max_seqlen_k, partition_size=0) -> int:
    """Workspace bytes for a decode of these sizes (any kv-head count, dtype
    and block size; see pkv_paged_decode_workspace_bytes)."""
    n = lib.pkv_paged_decode_workspace_bytes(B, num_q_heads, head_dim, max_seqlen_k,
                                             partition_size)
    if n == ctypes.c_size_t(-1).value:
        raise PkvError(PKV_ERR_SHAPE, "paged_decode_workspace_bytes")
    return n


def paged_decode(q, k_cache, v_cache, block_table, cache_seqlens, sm_scale: float, sink=None,
                 window_left: int = -1, partition_size: int = 0,
                 max_seqlen_k: Optional[int] = None, out=None, lse=None, workspace=None,
                 alibi_slopes=None):
    """out [B,Hq,D] for q [B,Hq,D] over k/v_cache [NB,bs,Hkv,D].

    partition_size: 0 the balanced schedule (bf16: a stage launch and a merge
    launch), -1 the same in one launch with the merge fused in, > 0 fixed
    partitions of that many keys (see pkv_paged_decode).
    `workspace`: at least decode_workspace_bytes(...) bytes, reusable across
    calls (see pkv_paged_decode); without one, a buffer is allocated for this
    call."""
    B, Hq, D = q.shape
    NB, bs, Hkv, _ = k_cache.shape
    if max_seqlen_k is None:
        max_seqlen_k = int(cache_seqlens.max().item()) if B else 0
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_bytes(B, Hq, D, max_seqlen_k, partition_size)
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    _check(lib.pkv_paged_decode(
        _ptr(out), _ptr(_f32(lse, "lse")), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(_i32(block_table, "block_table")), _ptr(_i32(cache_seqlens, "cache_seqlens")),
        _ptr(_f32(sink, "sink")), B, Hq, Hkv, D, bs, NB, block_table.shape[1], max_seqlen_k,
        float(sm_scale), window_left, _ptr(_f32(alibi_slopes, "alibi_slopes")), partition_size,
        _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _dt(q, k_cache, v_cache, out),
        _stream()), "paged_decode")
    return out


def paged_decode_noalloc(q, k_cache, v_cache, block_table, cache_seqlens, sm_scale: float,
                         sink=None, window_left: int = -1, partition_size: int = 0,
                         max_seqlen_k: Optional[int] = None, out=None, lse=None,
                         alibi_slopes=None):
    """paged_decode with the library's static device scratch as its workspace
    (pkv_paged_decode_noalloc): allocates nothing beyond `out` when the
    caller passes it.  Raises PkvError (PKV_ERR_SCRATCH) for calls that need
    more than NOALLOC_SCRATCH_BYTES."""
    B, Hq, D = q.shape
    NB, bs, Hkv, _ = k_cache.shape
    if max_seqlen_k is None:
        max_seqlen_k = int(cache_seqlens.max().item()) if B else 0
    if out is None:
        out = torch.empty_like(q)
    _check(lib.pkv_paged_decode_noalloc(
        _ptr(out), _ptr(_f32(lse, "lse")), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(_i32(block_table, "block_table")), _ptr(_i32(cache_seqlens, "cache_seqlens")),
        _ptr(_f32(sink, "sink")), B, Hq, Hkv, D, bs, NB, block_table.shape[1], max_seqlen_k,
        float(sm_scale), window_left, _ptr(_f32(alibi_slopes, "alibi_slopes")), partition_size,
        _dt(q, k_cache, v_cache, out), _stream()), "paged_decode_noalloc")
    return out


def paged_decode_append(q, k_new, v_new, k_cache, v_cache, block_table, cache_seqlens,
                        sm_scale: float, sink=None, window_left: int = -1,
                        max_seqlen_k: Optional[int] = None, out=None, lse=None, workspace=None,
                        alibi_slopes=None, rope_cos_sin=None, rotary_dim: int = 0,
                        rope_neox: bool = True):
    """Store k_new/v_new [B,Hkv,D] at position cache_seqlens[b] of each sequence and
    attend q [B,Hq,D] to keys 0..cache_seqlens[b]; cache_seqlens is not changed.
    With rope_cos_sin, q and k_new are rotated by that position in the call.

    The bf16 path needs a workspace of decode_workspace_bytes(B, Hq, D,
    max_seqlen_k + 1) bytes (allocated for this call when none is given);
    fp32 needs none."""
    B, Hq, D = q.shape
    NB, bs, Hkv, _ = k_cache.shape
    if max_seqlen_k is None:
        max_seqlen_k = int(cache_seqlens.max().item()) if B else 0
    if rope_cos_sin is not None:
        _rope_table(rope_cos_sin, rotary_dim)
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_bytes(B, Hq, D, max_seqlen_k + 1)
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    _check(lib.pkv_paged_decode_append(
        _ptr(out), _ptr(_f32(lse, "lse")), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
        _ptr(v_cache), _ptr(_i32(block_table, "block_table")),
        _ptr(_i32(cache_seqlens, "cache_seqlens")), _ptr(_f32(sink, "sink")), B, Hq, Hkv, D, bs,
        NB, block_table.shape[1], max_seqlen_k, float(sm_scale), window_left,
        _ptr(_f32(alibi_slopes, "alibi_slopes")), _ptr(rope_cos_sin),
        0 if rope_cos_sin is None else rope_cos_sin.shape[0], rotary_dim, int(bool(rope_neox)),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _dt(q, k_new, v_new, k_cache, v_cache, out),
        _stream()), "paged_decode_append")
    return out


def paged_decode_stage(q, k_cache, v_cache, block_table, cache_seqlens, sm_scale: float,
                       max_seqlen_k: int, workspace, window_left: int = -1, alibi_slopes=None):
    """First stage of automatic bf16 decode: balanced partial results into workspace."""
    B, Hq, D = q.shape
    NB, bs, Hkv, _ = k_cache.shape
    _check(lib.pkv_paged_decode_stage(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(_i32(block_table, "block_table")),
        _ptr(_i32(cache_seqlens, "cache_seqlens")), B, Hq, Hkv, D, bs, NB, block_table.shape[1],
        max_seqlen_k, float(sm_scale), window_left, _ptr(_f32(alibi_slopes, "alibi_slopes")),
        _ptr(workspace),
        workspace.numel() * workspace.element_size(), _dt(q, k_cache, v_cache), _stream()),
        "paged_decode_stage")


def paged_decode_finish(out, workspace, num_kv_heads: int, sink=None, lse=None):
    """Second stage: merge the workspace pieces (with the sink) into out [B,Hq,D]."""
    B, Hq, D = out.shape
    _check(lib.pkv_paged_decode_finish(
        _ptr(out), _ptr(_f32(lse, "lse")), _ptr(_f32(sink, "sink")), B, Hq, num_kv_heads, D,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _dt(out), _stream()),
        "paged_decode_finish")
    return out


def paged_decode_partitions(q, k_cache, v_cache, block_table, cache_seqlens, sm_scale: float,
                            partition_size: int, max_seqlen_k: int, window_left: int = -1,
                            part_out=None, part_lse=None, alibi_slopes=None):
    """Per-partition results (sink excluded): part_out [B,Hq,P,D], part_lse [B,Hq,P]."""
    B, Hq, D = q.shape
    NB, bs, Hkv, _ = k_cache.shape
    P = max(1, (max_seqlen_k + partition_size - 1) // partition_size)
    if part_out is None:
        part_out = torch.empty((B, Hq, P, D), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((B, Hq, P), dtype=torch.float32, device=q.device)
    _check(lib.pkv_paged_decode_partitions(
        _ptr(_f32(part_out, "part_out")), _ptr(_f32(part_lse, "part_lse")), _ptr(q),
        _ptr(k_cache), _ptr(v_cache), _ptr(_i32(block_table, "block_table")),
        _ptr(_i32(cache_seqlens, "cache_seqlens")), B, Hq, Hkv, D, bs, NB, block_table.shape[1],
        max_seqlen_k, float(sm_scale), window_left, _ptr(_f32(alibi_slopes, "alibi_slopes")),
        partition_size, part_out.shape[2], _dt(q, k_cache, v_cache),
        _stream()), "paged_decode_partitions")
    return part_out, part_lse


def merge_partitions(part_out, part_lse, cache_seqlens, partition_size: int, sink=None,
                     out_dtype=torch.bfloat16, out=None, lse=None):
    """out [B,Hq,D] from part_out [B,Hq,P,D] / part_lse [B,Hq,P] (float32)."""
    B, Hq, P, D = part_out.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=part_out.device)
    _check(lib.pkv_merge_partitions(
        _ptr(out), _ptr(_f32(lse, "lse")), _ptr(_f32(part_out, "part_out")),
        _ptr(_f32(part_lse, "part_lse")), _ptr(_i32(cache_seqlens, "cache_seqlens")),
        partition_size, _ptr(_f32(sink, "sink")), B, Hq, D, P, _dt(out), _stream()),
        "merge_partitions")
    return out


def varlen_prefill(q, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                   sm_scale: float, num_kv_heads: Optional[int] = None, k=None, v=None,
                   k_cache=None, v_cache=None, block_table=None, sink=None,
                   window_left: int = -1, out=None, lse=None, alibi_slopes=None,
                   rope_cos_sin=None, rotary_dim: int = 0, rope_neox: bool = True,
                   causal: bool = True, rope_k: bool = False, workspace=None):
    """Varlen prefill: out [sum Lq, Hq, D].  causal=False lets every query
    row see every key of its request (a window still bounds the left side).
    With rope_cos_sin, q is rotated by its position; rope_k=True rotates the
    contiguous keys by theirs too (k is not modified).  bfloat16 rope_k
    rotates the keys once into `workspace` (at least
    varlen_prefill_workspace_bytes(...) bytes; allocated when None), or,
    with workspace=False, inside the attention kernel."""
    if rope_cos_sin is not None:
        _rope_table(rope_cos_sin, rotary_dim)
    T, Hq, D = q.shape
    B = cu_seqlens_q.shape[0] - 1
    if k is not None:
        Hkv = k.shape[1]
        bs = NB = MB = 0
    else:
        NB, bs, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
        MB = block_table.shape[1]
    if num_kv_heads is not None and num_kv_heads != Hkv:
        raise ValueError("num_kv_heads does not match the K/V tensors")
    if out is None:
        out = torch.empty_like(q)
    dt = _dt(q, k, v, k_cache, v_cache, out)
    if workspace is False:
        workspace = None
    elif workspace is None and rope_k:
        need = varlen_prefill_workspace_bytes(B, max_seqlen_k, Hkv, D, rope_k, q.dtype)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib.pkv_varlen_prefill(
        _ptr(out), _ptr(_f32(lse, "lse")), _ptr(q), _ptr(k), _ptr(v), _ptr(k_cache),
        _ptr(v_cache), _ptr(None if block_table is None else _i32(block_table, "block_table")),
        bs, NB, MB, _ptr(_i32(cu_seqlens_q, "cu_seqlens_q")),
        _ptr(_i32(cu_seqlens_k, "cu_seqlens_k")), B, int(max_seqlen_q), int(max_seqlen_k), Hq,
        Hkv, D, float(sm_scale), int(bool(causal)), window_left, _ptr(_f32(alibi_slopes, "alibi_slopes")),
        _ptr(rope_cos_sin),
        0 if rope_cos_sin is None else rope_cos_sin.shape[0], rotary_dim, int(bool(rope_neox)),
        int(bool(rope_k)), _ptr(_f32(sink, "sink")), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), dt,
        _stream()), "varlen_prefill")
    return out


def varlen_prefill_workspace_bytes(B: int, max_seqlen_k: int, num_kv_heads: int, head_dim: int,
                                   rope_k: bool, dtype: torch.dtype) -> int:
    """Workspace bytes varlen_prefill needs to rotate the keys once (see
    pkv_varlen_prefill_workspace_bytes); 0 when it needs none."""
    code = PKV_BF16 if dtype == torch.bfloat16 else PKV_F32
    n = lib.pkv_varlen_prefill_workspace_bytes(int(B), int(max_seqlen_k), int(num_kv_heads),
                                               int(head_dim), int(bool(rope_k)), code)
    if n == ctypes.c_size_t(-1).value:
        raise PkvError(PKV_ERR_SHAPE, "varlen_prefill_workspace_bytes")
    return int(n)


SPARSE_BLOCK = 64


def vertical_slash_blocks(vertical_indices, slash_indices, cu_seqlens, max_seqlen: int):
    """Block form of vertical [B,H,NV] / slash [B,H,NS] indices per 64-row block:
    ``(block_count [B,H,NM], block_offset [B,H,NM,NM], column_count [B,H,NM],
    column_index [B,H,NM,NV])``, NM = ceil(max_seqlen / 64); entries past a
    count are left as -1."""
    B, H, NV = vertical_indices.shape
    NS = slash_indices.shape[2]
    if slash_indices.shape[:2] != (B, H) or cu_seqlens.shape[0] != B + 1:
        raise ValueError("vertical / slash / cu_seqlens shapes disagree")
    NM = (int(max_seqlen) + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    dev = vertical_indices.device
    bc = torch.zeros((B, H, NM), dtype=torch.int32, device=dev)
    bo = torch.full((B, H, NM, NM), -1, dtype=torch.int32, device=dev)
    cc = torch.zeros((B, H, NM), dtype=torch.int32, device=dev)
    ci = torch.full((B, H, NM, NV), -1, dtype=torch.int32, device=dev)
    _check(lib.pkv_vertical_slash_blocks(
        _ptr(bc), _ptr(bo), _ptr(cc), _ptr(ci), _ptr(_i32(vertical_indices, "vertical_indices")),
        _ptr(_i32(slash_indices, "slash_indices")), _ptr(_i32(cu_seqlens, "cu_seqlens")), B, H,
        NV, NS, int(max_seqlen), _stream()), "vertical_slash_blocks")
    return bc, bo, cc, ci


def sparse_prefill(q, k, v, cu_seqlens, max_seqlen: int, blocks, sm_scale: float, sink=None,
                   out=None, lse=None):
    """Block-sparse prefill (bf16) over ``blocks`` from vertical_slash_blocks:
    q [sum L, Hq, D], k / v [sum L, Hkv, D]; returns out like q."""
    bc, bo, cc, ci = blocks
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    B = cu_seqlens.shape[0] - 1
    NM = (int(max_seqlen) + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    if tuple(bc.shape) != (B, Hq, NM) or tuple(bo.shape) != (B, Hq, NM, NM) \
            or tuple(cc.shape) != (B, Hq, NM) or ci.shape[:3] != (B, Hq, NM):
        raise ValueError("block lists do not match the request shape")
    if out is None:
        out = torch.empty_like(q)
    _check(lib.pkv_sparse_prefill(
        _ptr(out), _ptr(_f32(lse, "lse")), _ptr(q), _ptr(k), _ptr(v),
        _ptr(_i32(cu_seqlens, "cu_seqlens")), _ptr(_i32(bc, "block_count")),
        _ptr(_i32(bo, "block_offset")), _ptr(_i32(cc, "column_count")),
        _ptr(_i32(ci, "column_index")), B, int(max_seqlen), Hq, Hkv, D, ci.shape[3],
        float(sm_scale), _ptr(_f32(sink, "sink")), _dt(q, k, v, out), _stream()),
        "sparse_prefill")
    return out
