"""Host-side checks of the index data the kernels read on the device.

The C ABI does not validate device-resident index arrays (block tables,
sequence lengths, cumulative lengths, slots): that would need a copy to the
host on every call.  Reading outside a block pool or past a table row is then
undefined behaviour on the GPU.  These functions check the same contracts on
host copies (numpy arrays or CPU tensors) and raise ``ValueError`` with the
first violation; call them where the index data is built, or in tests.

Contracts (include/pkv.h):
  decode        0 <= cache_seqlens[b] <= max_seqlen_k
                  <= max_blocks_per_seq * block_size (one more token with an
                  append); the first ceil(L_b / block_size) entries of row b
                  (ceil((L_b + 1) / block_size) with an append) are block ids
                  in [0, num_blocks); with an append, the new tokens' slots
                  are distinct across sequences.
  varlen        cu_seqlens_q/k start at 0 and are nondecreasing; every
                  length is <= max_seqlen_q / max_seqlen_k; paged K/V: the
                  decode contract for the key lengths.
  slots         every slot_mapping entry is < num_blocks * block_size;
                  non-negative entries are distinct (negative = padding).
"""

from __future__ import annotations

from typing import Optional

import numpy as np


def _host(a, name) -> np.ndarray:
    if a is None:
        raise ValueError(f"{name} is missing")
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    a = np.asarray(a)
    if a.dtype.kind not in "iu":
        raise ValueError(f"{name} must hold integers, not {a.dtype}")
    return a.astype(np.int64)


def check_block_table(block_table, lengths, num_blocks: int, block_size: int,
                      what: str = "sequence") -> None:
    """The first ceil(L_b / block_size) entries of row b are valid block ids."""
    bt = _host(block_table, "block_table")
    L = _host(lengths, "lengths")
    if bt.ndim != 2 or bt.shape[0] != L.shape[0]:
        raise ValueError(f"block_table must be [B, max_blocks_per_seq] with B = {L.shape[0]}")
    need = (L + block_size - 1) // block_size
    if (need > bt.shape[1]).any():
        b = int(np.argmax(need > bt.shape[1]))
        raise ValueError(f"{what} {b}: {int(L[b])} tokens need {int(need[b])} blocks, the table "
                         f"row has {bt.shape[1]}")
    cols = np.arange(bt.shape[1])[None, :]
    used = cols < need[:, None]
    bad = used & ((bt < 0) | (bt >= num_blocks))
    if bad.any():
        b, j = (int(x) for x in np.argwhere(bad)[0])
        raise ValueError(f"{what} {b}: block_table[{b}][{j}] = {int(bt[b, j])} is not a block "
                         f"id in [0, {num_blocks})")


def check_decode(block_table, cache_seqlens, num_blocks: int, block_size: int,
                 max_seqlen_k: int, append: bool = False) -> None:
    """Index contract of pkv_paged_decode (append=False) and of
    pkv_paged_decode_append (append=True: one more token per sequence, at
    position cache_seqlens[b], whose slots must be distinct)."""
    L = _host(cache_seqlens, "cache_seqlens")
    bt = _host(block_table, "block_table")
    if (L < 0).any():
        raise ValueError(f"cache_seqlens[{int(np.argmax(L < 0))}] is negative")
    if (L > max_seqlen_k).any():
        b = int(np.argmax(L > max_seqlen_k))
        raise ValueError(f"cache_seqlens[{b}] = {int(L[b])} exceeds max_seqlen_k = {max_seqlen_k}")
    total = L + (1 if append else 0)
    if max_seqlen_k + (1 if append else 0) > bt.shape[1] * block_size:
        raise ValueError("max_seqlen_k does not fit max_blocks_per_seq * block_size")
    check_block_table(bt, total, num_blocks, block_size)
    if append and L.size:
        rows = np.arange(L.size)
        slots = bt[rows, L // block_size] * block_size + L % block_size
        if np.unique(slots).size != slots.size:
            raise ValueError("two sequences append their new token to the same cache slot")


def check_cu_seqlens(cu, max_len: int, name: str) -> np.ndarray:
    """cu starts at 0, is nondecreasing, and every length is <= max_len;
    returns the lengths."""
    c = _host(cu, name)
    if c.ndim != 1 or c.size < 1:
        raise ValueError(f"{name} must be [B + 1]")
    if c[0] != 0:
        raise ValueError(f"{name}[0] = {int(c[0])}, must be 0")
    lens = np.diff(c)
    if (lens < 0).any():
        r = int(np.argmax(lens < 0))
        raise ValueError(f"{name} decreases at request {r}")
    if (lens > max_len).any():
        r = int(np.argmax(lens > max_len))
        raise ValueError(f"request {r} has {int(lens[r])} tokens in {name}, more than the "
                         f"maximum {max_len}")
    return lens


def check_varlen(cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                 block_table=None, num_blocks: Optional[int] = None,
                 block_size: Optional[int] = None, num_k_rows: Optional[int] = None) -> None:
    """Index contract of pkv_varlen_prefill.  With block_table, the keys are
    paged; otherwise num_k_rows (rows of the contiguous k / v) bounds
    cu_seqlens_k[-1]."""
    lq = check_cu_seqlens(cu_seqlens_q, max_seqlen_q, "cu_seqlens_q")
    lk = check_cu_seqlens(cu_seqlens_k, max_seqlen_k, "cu_seqlens_k")
    if lq.size != lk.size:
        raise ValueError("cu_seqlens_q and cu_seqlens_k describe different batch sizes")
    if block_table is not None:
        if num_blocks is None or block_size is None:
            raise ValueError("paged K/V: num_blocks and block_size are needed")
        check_block_table(block_table, lk, num_blocks, block_size, what="request")
    elif num_k_rows is not None and int(lk.sum()) > num_k_rows:
        raise ValueError(f"cu_seqlens_k covers {int(lk.sum())} keys, k has {num_k_rows} rows")


def check_slots(slot_mapping, num_blocks: int, block_size: int) -> None:
    """Index contract of pkv_reshape_and_cache: slots below the pool size,
    non-negative ones distinct (a negative slot marks a padding token)."""
    s = _host(slot_mapping, "slot_mapping")
    if (s >= num_blocks * block_size).any():
        t = int(np.argmax(s >= num_blocks * block_size))
        raise ValueError(f"slot_mapping[{t}] = {int(s[t])} is past the pool of "
                         f"{num_blocks * block_size} slots")
    live = s[s >= 0]
    if np.unique(live).size != live.size:
        raise ValueError("two tokens share a cache slot")
