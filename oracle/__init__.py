"""fp64 CPU oracle for attention over a paged KV cache -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it imports nothing
from the product package.

The arithmetic lives in ``oracle.c`` (plain C, fp64, two-pass softmax over an
explicit visible-key list); this module only builds it with gcc and marshals
numpy / torch CPU arrays into it.  Every function returns float64 numpy
arrays.  See ``oracle.c`` for the definition it follows and the passages it
cites.

Parity pins (what holds this oracle to something other than itself) live in
``tests/oracle_pins.py`` (run by ``tests/test_oracle_pins.py``), and
``tests/test_oracle_mutations.py`` shows that each plausible mistake in this
package fails one of them.

Parity unpinned: the dynamic (NTK-aware) branch of ``rope_cos_sin``.  The
vLLM page names a "dynamic" rope_scaling type but prints no formula; the
base-raising rule used here is the common reading, and its only check
restates that rule.  Every other function here is pinned.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def compile_source(src: str, out: str) -> str:
    """gcc -O2, no fast-math, no FMA contraction: fp64 as written."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                           "-ffp-contract=off", "-fno-fast-math", src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` when it is missing or stale."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def use_library(path: Optional[str]):
    """Point this module at another build of ``oracle.c`` (``None``: the
    default one).  Used by the tests that plant mistakes in a copy of the
    oracle to show the pins catch them."""
    global _lib, _override
    _override = path
    _lib = None


_override: Optional[str] = None


def _load():
    global _lib
    if _lib is None:
        path = _override
        if path is None:
            path = build()
        lib = ctypes.CDLL(path)
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.oracle_paged_decode.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, D, I, I,
                                            I, I, P, I, I]
        lib.oracle_varlen_prefill.argtypes = [P, P, P, P, P, P, P, P, I, I, P, P, I, I, I, I, D,
                                              I, I, P, P, I, P, I, I]
        lib.oracle_merge.argtypes = [P, P, P, P, P, P, I, I, I, I]
        lib.oracle_reshape_and_cache.argtypes = [P, P, P, P, P, I, I, I, I, I, I]
        lib.oracle_token_request.argtypes = [P, I, I, P]
        lib.oracle_slot_of.argtypes = [P, I, I]
        lib.oracle_slot_of.restype = ctypes.c_longlong
        lib.oracle_vertical_slash_blocks.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I]
        lib.oracle_masked_prefill.argtypes = [P, P, P, P, P, P, I, I, I, I, D, P, I, P, I, P, I,
                                              I]
        _lib = lib
    return _lib


def _np(t) -> Optional[np.ndarray]:
    """Contiguous numpy view of a CPU tensor/array (bf16 as its uint16 bits)."""
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()
    return np.ascontiguousarray(t)


def _dtype_code(t) -> int:
    if isinstance(t, torch.Tensor):
        if t.dtype == torch.bfloat16:
            return BF16
        if t.dtype == torch.float32:
            return F32
    elif isinstance(t, np.ndarray) and t.dtype == np.float32:
        return F32
    raise TypeError(f"oracle inputs must be float32 or bfloat16, got {getattr(t, 'dtype', t)}")


def _ptr(a) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _threads(n: Optional[int]) -> int:
    """Worker threads: n, else OMP_NUM_THREADS, else the host's cores (at most 16)."""
    if n:
        return n
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(16, os.cpu_count() or 1))


def token_request(cu: Sequence[int], T: Optional[int] = None) -> np.ndarray:
    """Request index of every packed token (varlen cumulative-length map)."""
    cu = np.asarray(cu, dtype=np.int32)
    B = len(cu) - 1
    T = int(cu[-1] - cu[0]) if T is None else T
    out = np.empty(max(T, 1), dtype=np.int32)
    _load().oracle_token_request(_ptr(cu), B, T, _ptr(out))
    return out[:T]


def slot_of(block_table_row: Sequence[int], pos: int, block_size: int) -> int:
    row = np.asarray(block_table_row, dtype=np.int32)
    return int(_load().oracle_slot_of(_ptr(row), pos, block_size))


def paged_decode(q, k_cache, v_cache, block_table, cache_seqlens, sink, sm_scale: float,
                 window_left: int = -1, partition_size: int = 0,
                 units: Optional[Sequence[int]] = None, nthreads: Optional[int] = None,
                 alibi=None):
    """Decode over a paged cache (``alibi``: per-query-head slopes, or None).

    Returns ``(out [B,Hq,D], lse [B,Hq])`` for ``partition_size == 0``, else
    the per-partition results ``(out [B,Hq,P,D], lse [B,Hq,P])`` with the
    sink left out.  ``units`` restricts the work to flat ids
    ``(b*Hq + h) * P + p``; other entries are left NaN."""
    dt = _dtype_code(q)
    qn, kn, vn = _np(q), _np(k_cache), _np(v_cache)
    bt = _np(block_table).astype(np.int32, copy=False)
    sl = _np(cache_seqlens).astype(np.int32, copy=False)
    sk = None if sink is None else _np(sink).astype(np.float32, copy=False)
    al = None if alibi is None else _np(alibi).astype(np.float32, copy=False)
    B, Hq, D = qn.shape
    NB, bs, Hkv, D2 = kn.shape
    assert D2 == D and tuple(vn.shape) == tuple(kn.shape)
    if partition_size > 0:
        P = max(1, (int(sl.max(initial=0)) + partition_size - 1) // partition_size)
        out = np.full((B, Hq, P, D), np.nan)
        lse = np.full((B, Hq, P), np.nan)
    else:
        P = 1
        out = np.full((B, Hq, D), np.nan)
        lse = np.full((B, Hq), np.nan)
    un = None if units is None else np.ascontiguousarray(units, dtype=np.int32)
    rc = _load().oracle_paged_decode(
        _ptr(out), _ptr(lse), _ptr(qn), _ptr(kn), _ptr(vn), _ptr(bt), _ptr(sl), _ptr(sk), _ptr(al),
        B, Hq, Hkv, D, bs, bt.shape[1], float(sm_scale), int(window_left), int(partition_size),
        P, dt, _ptr(un), 0 if un is None else len(un), _threads(nthreads))
    assert rc == 0
    return out, lse


def varlen_prefill(q, cu_seqlens_q, cu_seqlens_k, sink, sm_scale: float, num_kv_heads: int,
                   k=None, v=None, k_cache=None, v_cache=None, block_table=None,
                   block_size: int = 0, window_left: int = -1,
                   units: Optional[Sequence[int]] = None, nthreads: Optional[int] = None,
                   alibi=None, causal: bool = True):
    """Varlen prefill; returns ``(out [sum Lq,Hq,D], lse [sum Lq,Hq])``.
    ``units`` restricts the work to flat ids ``t*Hq + h``; ``alibi``: per-query-head
    slopes, or None; ``causal=False`` drops the upper bound on the visible keys
    (a window then bounds only the left side)."""
    dt = _dtype_code(q)
    qn = _np(q)
    T, Hq, D = qn.shape
    cq = _np(cu_seqlens_q).astype(np.int32, copy=False)
    ck = _np(cu_seqlens_k).astype(np.int32, copy=False)
    B = len(cq) - 1
    kn, vn = _np(k), _np(v)
    kc, vc = _np(k_cache), _np(v_cache)
    bt = None if block_table is None else _np(block_table).astype(np.int32, copy=False)
    assert (kn is None) != (kc is None), "exactly one of contiguous or paged K/V"
    sk = None if sink is None else _np(sink).astype(np.float32, copy=False)
    al = None if alibi is None else _np(alibi).astype(np.float32, copy=False)
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    un = None if units is None else np.ascontiguousarray(units, dtype=np.int32)
    rc = _load().oracle_varlen_prefill(
        _ptr(out), _ptr(lse), _ptr(qn), _ptr(kn), _ptr(vn), _ptr(kc), _ptr(vc), _ptr(bt),
        int(block_size), 0 if bt is None else bt.shape[1], _ptr(cq), _ptr(ck), B, Hq,
        int(num_kv_heads), D, float(sm_scale), int(bool(causal)), int(window_left), _ptr(sk),
        _ptr(al), dt, _ptr(un),
        0 if un is None else len(un), _threads(nthreads))
    assert rc == 0
    return out, lse


# ---------------------------------------------------------------------------
# Vertical + slash sparse prefill (nano-vllm "minference.py" page,
# MInferencePolicy.estimate_pattern / sparse_prefill_attention, 64 x 64
# blocks).  The block form is the reading stated in oracle.c: key block n is a
# slash block of row block m when a diagonal of the head meets it within m's
# rows; vertical columns outside those blocks are listed one by one.
# ---------------------------------------------------------------------------

SPARSE_BLOCK = 64


def vertical_slash_blocks(vertical, slash, cu_seqlens, max_seqlen: int):
    """Block lists of every (request, head, 64-row block).  vertical [B,H,NV]
    key positions (ascending), slash [B,H,NS] diagonal offsets i - j.  Returns
    ``(block_count [B,H,NM], block_offset [B,H,NM,NM], column_count [B,H,NM],
    column_index [B,H,NM,NV])``, NM = ceil(max_seqlen / 64); entries past a
    count are -1."""
    V = np.ascontiguousarray(vertical, dtype=np.int32)
    S = np.ascontiguousarray(slash, dtype=np.int32)
    cu = np.ascontiguousarray(_np(cu_seqlens), dtype=np.int32)
    B, H, NV = V.shape
    NS = S.shape[2]
    assert S.shape[:2] == (B, H) and len(cu) == B + 1
    NM = (int(max_seqlen) + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    bc = np.zeros((B, H, NM), dtype=np.int32)
    bo = np.full((B, H, NM, NM), -1, dtype=np.int32)
    cc = np.zeros((B, H, NM), dtype=np.int32)
    ci = np.full((B, H, NM, NV), -1, dtype=np.int32)
    rc = _load().oracle_vertical_slash_blocks(_ptr(bc), _ptr(bo), _ptr(cc), _ptr(ci), _ptr(V),
                                              _ptr(S), _ptr(cu), B, H, NV, NS, NM)
    assert rc == 0
    return bc, bo, cc, ci


def block_sparse_mask(block_count, block_offset, column_count, column_index, cu_seqlens,
                      num_heads: int, units: Optional[Sequence[int]] = None) -> np.ndarray:
    """The explicit key mask the block lists describe: row i of request r
    (64-row block m = i // 64) of head h sees key j iff j <= i and j lies in
    one of m's 64-key blocks or is one of m's columns.  One row of W =
    ceil(max L / 64) uint64 words per unit (t * Hq + h), bit j % 64 of word
    j // 64; all units, or those listed."""
    cu = np.asarray(_np(cu_seqlens), dtype=np.int64)
    B = len(cu) - 1
    T = int(cu[-1])
    Lmax = int((cu[1:] - cu[:-1]).max()) if B else 0
    W = max(1, (Lmax + 63) // 64)
    ids = np.arange(T * num_heads) if units is None else np.asarray(units, dtype=np.int64)
    req = token_request(cu.astype(np.int32), T)
    out = np.zeros((len(ids), W), dtype=np.uint64)
    cache = {}
    for n, uid in enumerate(ids.tolist()):
        t, h = divmod(uid, num_heads)
        r = int(req[t])
        i = t - int(cu[r])
        m = i // SPARSE_BLOCK
        key = (r, h, m)
        if key not in cache:
            vis = np.zeros(W * 64, dtype=bool)
            for k in range(int(block_count[r, h, m])):
                off = int(block_offset[r, h, m, k])
                vis[off:off + SPARSE_BLOCK] = True
            for k in range(int(column_count[r, h, m])):
                vis[int(column_index[r, h, m, k])] = True
            cache = {key: vis}
        row = cache[key].copy()
        row[i + 1:] = False
        out[n] = np.packbits(row, bitorder="little").view(np.uint64)[:W]
    return out


def masked_prefill(q, k, v, cu_seqlens, mask, sink, sm_scale: float, num_kv_heads: int,
                   units: Optional[Sequence[int]] = None, nthreads: Optional[int] = None):
    """Self-attention prefill (Lq = Lk per request) under an explicit mask:
    unit n (``t * Hq + h``, all or ``units``) sees exactly the keys whose bit
    is set in ``mask[n]`` (uint64 words, as block_sparse_mask).  Returns
    ``(out [T,Hq,D], lse [T,Hq])`` with NaN for units not computed."""
    dt = _dtype_code(q)
    qn, kn, vn = _np(q), _np(k), _np(v)
    T, Hq, D = qn.shape
    cu = np.ascontiguousarray(_np(cu_seqlens), dtype=np.int32)
    mk = np.ascontiguousarray(mask, dtype=np.uint64)
    un = None if units is None else np.ascontiguousarray(units, dtype=np.int32)
    assert mk.shape[0] == (T * Hq if un is None else len(un))
    sk = None if sink is None else _np(sink).astype(np.float32, copy=False)
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    rc = _load().oracle_masked_prefill(
        _ptr(out), _ptr(lse), _ptr(qn), _ptr(kn), _ptr(vn), _ptr(cu), len(cu) - 1, Hq,
        int(num_kv_heads), D, float(sm_scale), _ptr(mk), mk.shape[1], _ptr(sk), dt, _ptr(un),
        0 if un is None else len(un), _threads(nthreads))
    assert rc == 0
    return out, lse


def sparse_prefill(q, k, v, cu_seqlens, vertical, slash, sink, sm_scale: float,
                   num_kv_heads: int, units: Optional[Sequence[int]] = None,
                   nthreads: Optional[int] = None):
    """Vertical + slash sparse prefill: block lists, their mask, attention."""
    cu = np.asarray(_np(cu_seqlens), dtype=np.int64)
    Lmax = int((cu[1:] - cu[:-1]).max()) if len(cu) > 1 else 0
    lists = vertical_slash_blocks(vertical, slash, cu_seqlens, Lmax)
    mask = block_sparse_mask(*lists, cu_seqlens, _np(q).shape[1], units)
    return masked_prefill(q, k, v, cu_seqlens, mask, sink, sm_scale, num_kv_heads, units,
                          nthreads)


def merge(part_out, part_lse, nparts_per_seq, sink):
    """Split-KV merge of partition results ``[B,Hq,P,D]`` / ``[B,Hq,P]``."""
    po = np.ascontiguousarray(np.asarray(part_out, dtype=np.float64))
    pl = np.ascontiguousarray(np.asarray(part_lse, dtype=np.float64))
    npb = np.ascontiguousarray(nparts_per_seq, dtype=np.int32)
    sk = None if sink is None else _np(sink).astype(np.float32, copy=False)
    B, Hq, P, D = po.shape
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    _load().oracle_merge(_ptr(out), _ptr(lse), _ptr(po), _ptr(pl), _ptr(npb), _ptr(sk), B, Hq,
                         D, P)
    return out, lse


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping):
    """Returns new (k_cache, v_cache) CPU tensors with the rows scattered."""
    kc = k_cache.detach().cpu().clone().contiguous()
    vc = v_cache.detach().cpu().clone().contiguous()
    key = key.detach().cpu().contiguous()
    value = value.detach().cpu().contiguous()
    sm = _np(slot_mapping).astype(np.int32, copy=False)
    T, Hkv, D = key.shape
    NB, bs = kc.shape[0], kc.shape[1]
    rc = _load().oracle_reshape_and_cache(
        key.data_ptr(), value.data_ptr(), kc.data_ptr(), vc.data_ptr(), _ptr(sm), T, Hkv, D, bs,
        NB, key.element_size())
    assert rc == 0, "slot out of range"
    return kc, vc


def decode_append(q, k_new, v_new, k_cache, v_cache, block_table, cache_seqlens, sink,
                  sm_scale: float, window_left: int = -1,
                  units: Optional[Sequence[int]] = None, nthreads: Optional[int] = None,
                  alibi=None):
    """Decode with the new token appended in the same call (Transformers
    "Paged attention" doc, decode path: the kvcache kernel writes k and v
    into the cache at index cache_seqlens[b], updating it in place, and the
    query attends to the cache including them).  Written as its two steps:
    row b of k_new / v_new goes to the slot of position cache_seqlens[b]
    (reshape_and_cache), then decode over cache_seqlens[b] + 1 keys with the
    query at that position (paged_decode).  Returns ``(out, lse, k_cache
    after, v_cache after)``."""
    sl = _np(cache_seqlens).astype(np.int32, copy=False)
    bt = _np(block_table).astype(np.int32, copy=False)
    bs = k_cache.shape[1]
    slots = np.array([slot_of(bt[b], int(sl[b]), bs) for b in range(len(sl))], dtype=np.int32)
    kc, vc = reshape_and_cache(k_new, v_new, k_cache, v_cache, torch.from_numpy(slots))
    out, lse = paged_decode(q, kc, vc, block_table, torch.from_numpy(sl + 1), sink, sm_scale,
                            window_left=window_left, units=units, nthreads=nthreads, alibi=alibi)
    return out, lse, kc, vc



# ---------------------------------------------------------------------------
# Rotary position embedding.  The vLLM "attention.py" page (PagedAttentionWithRoPE)
# applies a rotary embedding to query and key before attention, parameterised
# by head size, rotary_dim, max_position, base, is_neox_style and an optional
# rope_scaling {"type": "linear" | "dynamic", "factor"}; the rotation itself is
# not printed on the pages.  These functions take the standard rotary
# embedding as the reading: frequency i < rotary_dim / 2 turns at
# base^(-2i / rotary_dim) per position; neox style pairs dimension d with
# d + rotary_dim / 2, the other style pairs 2i with 2i + 1; dimensions from
# rotary_dim on are left alone.  Linear scaling divides the position by the
# factor; dynamic (NTK-aware) scaling raises the base for a table longer than
# max_position.  All in float64 numpy.
# ---------------------------------------------------------------------------

ROPE_NONE, ROPE_LINEAR, ROPE_DYNAMIC = 0, 1, 2


def rope_cos_sin(num_positions: int, rotary_dim: int, base: float, scaling: int = ROPE_NONE,
                 factor: float = 1.0, max_position: int = 0) -> np.ndarray:
    """Table [num_positions, rotary_dim]: cos of the angles, then sin.
    The dynamic branch is parity unpinned (see the module docstring)."""
    half = rotary_dim // 2
    b = float(base)
    if scaling == ROPE_DYNAMIC and num_positions > max_position:
        b = b * ((factor * num_positions / max_position) - (factor - 1.0)) ** (
            rotary_dim / (rotary_dim - 2))
    inv_freq = b ** (-(2.0 * np.arange(half)) / rotary_dim)
    t = np.arange(num_positions, dtype=np.float64)
    if scaling == ROPE_LINEAR:
        t = t / factor
    ang = np.outer(t, inv_freq)
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def _values64(t) -> np.ndarray:
    """Values (not storage bits) of a tensor or array as float64."""
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def rope_apply(x, positions, cos_sin, rotary_dim: int, neox: bool) -> np.ndarray:
    """Rows x [T, H, D] rotated by their positions [T]; float64 copy."""
    y = _values64(x).copy()
    pos = np.asarray(_np(positions)).astype(np.int64)
    tab = _values64(cos_sin)
    assert pos.size == 0 or (pos.min() >= 0 and pos.max() < tab.shape[0]), "position outside the table"
    half = rotary_dim // 2
    c = tab[pos, :half][:, None, :]           # [T, 1, half]
    s = tab[pos, half:rotary_dim][:, None, :]
    if neox:
        a, b = y[..., :half].copy(), y[..., half:rotary_dim].copy()
        y[..., :half] = a * c - b * s
        y[..., half:rotary_dim] = b * c + a * s
    else:
        a, b = y[..., 0:rotary_dim:2].copy(), y[..., 1:rotary_dim:2].copy()
        y[..., 0:rotary_dim:2] = a * c - b * s
        y[..., 1:rotary_dim:2] = b * c + a * s
    return y


def query_positions(cu_seqlens_q, cu_seqlens_k) -> np.ndarray:
    """Position of every packed query row: Lk - Lq + i within its request
    (FlashInfer page, sink_attention_unified, varlen branch: the queries are
    the last qo_len positions of the request's keys)."""
    cq = _np(cu_seqlens_q).astype(np.int64)
    ck = _np(cu_seqlens_k).astype(np.int64)
    out = []
    for r in range(len(cq) - 1):
        Lq, Lk = cq[r + 1] - cq[r], ck[r + 1] - ck[r]
        out.append(Lk - Lq + np.arange(Lq))
    return np.concatenate(out) if out else np.zeros(0, np.int64)
