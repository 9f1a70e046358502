"""Seeded generators for the five attention workloads and for the tests.

Every array is drawn from numpy's PCG64 (``numpy.random.default_rng(seed)``)
as float32 N(0, 1); bf16 workloads round those draws to bfloat16 with
round-to-nearest-even (torch's CPU conversion) and both the kernels and the
oracle consume the rounded values.  Large pools are drawn in fixed-size chunks,
each from its own child stream of ``SeedSequence(seed)``, so the values do not
depend on how many threads draw them.

Layouts (token-major, like the packed ``[tokens, heads, head_dim]``
activations of the pages):

* decode query            ``q [B, Hq, D]``
* packed prefill tensors  ``q [sum Lq, Hq, D]``, ``k/v [sum Lk, Hkv, D]``
* paged caches            ``k_cache/v_cache [num_blocks, block_size, Hkv, D]``
* ``block_table [B, max_blocks_per_seq]`` int32, ``-1`` for unused entries
* ``cache_seqlens [B]`` int32, ``cu_seqlens [B + 1]`` int32

Blocks a request does not own, and slots past the last token of its final
block, can be filled with NaN ("poisoned") so that any read outside the
visible range shows up in the result.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = [
    "DecodeCase",
    "PrefillCase",
    "normal",
    "to_dtype",
    "pool_from_lengths",
    "decode_case",
    "prefill_case",
    "paged_prefill_case",
    "cu_from_lengths",
    "slots_for_tokens",
    "config1_decode",
    "config1_prefill",
    "config2_decode",
    "config3_lengths",
    "config3_prefill",
    "config4_chunked",
    "config5_split_decode",
    "random_partials",
    "vertical_slash_pattern",
    "sparse_prefill_workload",
]

CHUNK = 1 << 22  # values per independent child stream for large draws


def _threads() -> int:
    return max(1, min(16, torch.get_num_threads()))


def normal(seed: int, shape, stream: int = 0) -> np.ndarray:
    """float32 N(0,1) of ``shape`` from child stream ``stream`` of ``seed``.

    Values are drawn in ``CHUNK``-sized pieces, piece ``i`` from the ``i``-th
    spawned child of ``SeedSequence([seed, stream])``; the result is therefore
    independent of the number of worker threads."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, (n + CHUNK - 1) // CHUNK)
    children = np.random.SeedSequence([seed, stream]).spawn(nchunks)

    def fill(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(children[i]))
        out[lo:hi] = g.standard_normal(hi - lo, dtype=np.float32)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def to_dtype(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """float32 numpy -> torch CPU tensor of ``dtype`` (bf16: round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t if dtype == torch.float32 else t.to(dtype)


def cu_from_lengths(lengths) -> torch.Tensor:
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    assert cu[-1] < 2**31
    return torch.from_numpy(cu.astype(np.int32))


def pool_from_lengths(rng: np.random.Generator, lengths, block_size: int,
                      spare_blocks: int = 0, shuffle: bool = True,
                      max_blocks_per_seq: Optional[int] = None):
    """Block table for requests of ``lengths`` tokens over a pool of
    ``sum(ceil(L/bs)) + spare_blocks`` blocks.

    With ``shuffle`` the pool is a seeded permutation and row ``b`` takes the
    next ``ceil(L_b/bs)`` entries of it; otherwise blocks are handed out in
    order (the identity table over a contiguous pool).  Returns
    ``(block_table int32 [B, MB], num_blocks)``."""
    nblk = [(int(L) + block_size - 1) // block_size for L in lengths]
    total = sum(nblk) + spare_blocks
    order = rng.permutation(total) if shuffle else np.arange(total)
    mb = max(max(nblk, default=0), 1) if max_blocks_per_seq is None else max_blocks_per_seq
    bt = np.full((len(lengths), mb), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = order[off:off + n]
        off += n
    return torch.from_numpy(bt), total


def slots_for_tokens(block_table: torch.Tensor, positions, block_size: int) -> torch.Tensor:
    """Cache slot of logical position ``positions[b]`` of request ``b``:
    the physical block from the table times the block size plus the offset."""
    bt = block_table.numpy()
    out = np.empty(len(positions), dtype=np.int32)
    for b, p in enumerate(positions):
        out[b] = bt[b, p // block_size] * block_size + p % block_size
    return torch.from_numpy(out)


def _poison(cache: torch.Tensor, block_table: torch.Tensor, lengths, block_size: int):
    """NaN in every slot that no request's visible range covers."""
    used = torch.zeros(cache.shape[0] * block_size, dtype=torch.bool)
    bt = block_table.numpy()
    for b, L in enumerate(lengths):
        for j0 in range(0, int(L), block_size):
            blk = int(bt[b, j0 // block_size])
            n = min(block_size, int(L) - j0)
            used[blk * block_size: blk * block_size + n] = True
    flat = cache.view(cache.shape[0] * block_size, -1)
    flat[~used] = float("nan")


def _fill_pool(seed, stream, block_table, lengths, num_blocks, block_size, Hkv, D, dtype,
               poison: bool):
    """Cache pool whose used slots hold the request's tokens in logical order.

    Token ``j`` of request ``b`` takes the ``j``-th row of that request's own
    draw, so the same request gets the same K/V whatever the table is."""
    cache = torch.zeros((num_blocks, block_size, Hkv, D), dtype=dtype)
    flat = cache.view(num_blocks * block_size, Hkv, D)
    bt = block_table.numpy()
    for b, L in enumerate(lengths):
        L = int(L)
        if L == 0:
            continue
        rows = to_dtype(normal(seed, (L, Hkv, D), stream=stream * 100003 + b), dtype)
        nb = (L + block_size - 1) // block_size
        phys = torch.from_numpy(bt[b, :nb].astype(np.int64))
        slot = (phys[:, None] * block_size + torch.arange(block_size)[None, :]).reshape(-1)[:L]
        flat[slot] = rows
    if poison:
        _poison(cache, block_table, lengths, block_size)
    return cache


@dataclass
class DecodeCase:
    q: torch.Tensor                 # [B, Hq, D]
    k_cache: torch.Tensor           # [NB, bs, Hkv, D]
    v_cache: torch.Tensor
    block_table: torch.Tensor       # [B, MB] int32
    cache_seqlens: torch.Tensor     # [B] int32
    sink: Optional[torch.Tensor]    # [Hq] float32 or None
    block_size: int
    sm_scale: float
    window_left: int = -1
    meta: dict = field(default_factory=dict)

    @property
    def B(self): return self.q.shape[0]
    @property
    def Hq(self): return self.q.shape[1]
    @property
    def Hkv(self): return self.k_cache.shape[2]
    @property
    def D(self): return self.q.shape[2]
    @property
    def num_blocks(self): return self.k_cache.shape[0]
    @property
    def max_blocks_per_seq(self): return self.block_table.shape[1]
    @property
    def max_seqlen_k(self): return int(self.cache_seqlens.max()) if self.B else 0


@dataclass
class PrefillCase:
    q: torch.Tensor                       # [sum Lq, Hq, D]
    cu_seqlens_q: torch.Tensor            # [B+1] int32
    cu_seqlens_k: torch.Tensor            # [B+1] int32
    sink: Optional[torch.Tensor]
    sm_scale: float
    window_left: int
    Hkv: int
    k: Optional[torch.Tensor] = None      # contiguous [sum Lk, Hkv, D]
    v: Optional[torch.Tensor] = None
    k_cache: Optional[torch.Tensor] = None  # paged [NB, bs, Hkv, D]
    v_cache: Optional[torch.Tensor] = None
    block_table: Optional[torch.Tensor] = None
    block_size: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def B(self): return self.cu_seqlens_q.shape[0] - 1
    @property
    def Hq(self): return self.q.shape[1]
    @property
    def D(self): return self.q.shape[2]
    @property
    def q_lens(self): return (self.cu_seqlens_q[1:] - self.cu_seqlens_q[:-1]).tolist()
    @property
    def k_lens(self): return (self.cu_seqlens_k[1:] - self.cu_seqlens_k[:-1]).tolist()
    @property
    def max_seqlen_q(self): return max(self.q_lens, default=0)
    @property
    def max_seqlen_k(self): return max(self.k_lens, default=0)
    @property
    def paged(self): return self.k is None


def _sink(seed, Hq, with_sink):
    return torch.from_numpy(normal(seed, (Hq,), stream=7).copy()) if with_sink else None


def decode_case(seed: int, lengths, Hq: int, Hkv: int, D: int, block_size: int,
                dtype=torch.bfloat16, with_sink: bool = True, window_left: int = -1,
                sm_scale: Optional[float] = None, spare_blocks: int = 2, shuffle: bool = True,
                poison: bool = True, max_blocks_per_seq: Optional[int] = None) -> DecodeCase:
    rng = np.random.default_rng(seed)
    bt, nb = pool_from_lengths(rng, lengths, block_size, spare_blocks, shuffle, max_blocks_per_seq)
    B = len(lengths)
    q = to_dtype(normal(seed, (B, Hq, D), stream=1), dtype)
    kc = _fill_pool(seed, 2, bt, lengths, nb, block_size, Hkv, D, dtype, poison)
    vc = _fill_pool(seed, 3, bt, lengths, nb, block_size, Hkv, D, dtype, poison)
    return DecodeCase(q, kc, vc, bt, torch.tensor(list(lengths), dtype=torch.int32),
                      _sink(seed, Hq, with_sink), block_size,
                      (1.0 / math.sqrt(D)) if sm_scale is None else sm_scale, window_left)


def prefill_case(seed: int, q_lens, k_lens, Hq: int, Hkv: int, D: int,
                 dtype=torch.bfloat16, with_sink: bool = True, window_left: int = -1,
                 sm_scale: Optional[float] = None) -> PrefillCase:
    """Packed contiguous prefill: ``q [sum Lq,Hq,D]``, ``k/v [sum Lk,Hkv,D]``."""
    cq, ck = cu_from_lengths(q_lens), cu_from_lengths(k_lens)
    tq, tk = int(cq[-1]), int(ck[-1])
    q = to_dtype(normal(seed, (tq, Hq, D), stream=1), dtype)
    k = to_dtype(normal(seed, (tk, Hkv, D), stream=2), dtype)
    v = to_dtype(normal(seed, (tk, Hkv, D), stream=3), dtype)
    return PrefillCase(q, cq, ck, _sink(seed, Hq, with_sink),
                       (1.0 / math.sqrt(D)) if sm_scale is None else sm_scale, window_left, Hkv,
                       k=k, v=v)


def paged_prefill_case(seed: int, q_lens, k_lens, Hq: int, Hkv: int, D: int, block_size: int,
                       dtype=torch.bfloat16, with_sink: bool = True, window_left: int = -1,
                       sm_scale: Optional[float] = None, spare_blocks: int = 2,
                       shuffle: bool = True, poison: bool = True) -> PrefillCase:
    """Prefill whose K/V (all ``Lk`` tokens, including the chunk's own) sit in
    a paged pool reached through ``block_table``; ``cu_seqlens_k`` carries
    the per-request key counts."""
    rng = np.random.default_rng(seed)
    bt, nb = pool_from_lengths(rng, k_lens, block_size, spare_blocks, shuffle)
    cq, ck = cu_from_lengths(q_lens), cu_from_lengths(k_lens)
    q = to_dtype(normal(seed, (int(cq[-1]), Hq, D), stream=1), dtype)
    kc = _fill_pool(seed, 2, bt, k_lens, nb, block_size, Hkv, D, dtype, poison)
    vc = _fill_pool(seed, 3, bt, k_lens, nb, block_size, Hkv, D, dtype, poison)
    return PrefillCase(q, cq, ck, _sink(seed, Hq, with_sink),
                       (1.0 / math.sqrt(D)) if sm_scale is None else sm_scale, window_left, Hkv,
                       k_cache=kc, v_cache=vc, block_table=bt, block_size=block_size)


# --------------------------------------------------------------------------
# The five workloads.  Seeds 0..4 for workloads 1..5.
# --------------------------------------------------------------------------

def config1_decode(seed: int = 0) -> DecodeCase:
    """Tiny fp32 decode exactly as the worked example on the paged-attention
    doc page (decode path): cache_seqlens [30,32,70], block size 32,
    block_table [[2,-1,-1,-1],[0,1,-1,-1],[3,5,6,-1]] over 8 blocks (4 and 7
    unused); 4 q heads / 2 kv heads, head_dim 64, sm_scale 1/8, N(0,1) sink."""
    bt = torch.tensor([[2, -1, -1, -1], [0, 1, -1, -1], [3, 5, 6, -1]], dtype=torch.int32)
    lengths = [30, 32, 70]
    q = to_dtype(normal(seed, (3, 4, 64), stream=1), torch.float32)
    kc = _fill_pool(seed, 2, bt, lengths, 8, 32, 2, 64, torch.float32, True)
    vc = _fill_pool(seed, 3, bt, lengths, 8, 32, 2, 64, torch.float32, True)
    return DecodeCase(q, kc, vc, bt, torch.tensor(lengths, dtype=torch.int32),
                      _sink(seed, 4, True), 32, 1.0 / 8.0, -1)


def config1_prefill(seed: int = 0) -> PrefillCase:
    """Tiny fp32 varlen causal prefill: q_len = kv_len = [10,3,1]
    (cu_seqlens [0,10,13,14]), 4/2 heads, head_dim 64, sm_scale 1/8, the
    decode case's sink."""
    c = prefill_case(seed, [10, 3, 1], [10, 3, 1], 4, 2, 64, torch.float32, True, -1, 1.0 / 8.0)
    c.sink = _sink(seed, 4, True)
    return c


def config2_decode(seed: int = 1, spare_blocks: int = 0, poison: bool = False) -> DecodeCase:
    """bf16 decode: 64 sequences, cache_seqlens ~ U[512, 4096], 32/8 heads,
    head_dim 128, block size 16, shuffled pool, no sink, no window."""
    rng = np.random.default_rng([seed, 11])
    lengths = rng.integers(512, 4096, size=64, endpoint=True).tolist()
    return decode_case(seed, lengths, 32, 8, 128, 16, torch.bfloat16, with_sink=False,
                       spare_blocks=spare_blocks, poison=poison)


def config3_lengths(seed: int = 2):
    rng = np.random.default_rng([seed, 11])
    return rng.integers(256, 4096, size=8, endpoint=True).tolist()


def config3_prefill(seed: int = 2) -> PrefillCase:
    """bf16 varlen causal prefill: 8 requests, q_len = kv_len ~ U[256, 4096],
    32/8 heads, head_dim 128, N(0,1) sink, no window."""
    L = config3_lengths(seed)
    return prefill_case(seed, L, L, 32, 8, 128, torch.bfloat16, True, -1)


def config4_chunked(seed: int = 3, poison: bool = True, spare_blocks: int = 2) -> PrefillCase:
    """bf16 chunked prefill: 4 requests, a 512-token query chunk after 8192
    cached tokens (8704 keys, the chunk's own K/V already in the cache),
    paged blocks of 16, causal with window_left 128, 64/8 heads,
    head_dim 64, N(0,1) sink."""
    return paged_prefill_case(seed, [512] * 4, [8704] * 4, 64, 8, 64, 16, torch.bfloat16,
                              True, 128, spare_blocks=spare_blocks, poison=poison)


def config5_split_decode(seed: int = 4, batch: int = 16, seqlen: int = 131072,
                         poison: bool = False) -> DecodeCase:
    """bf16 long-context decode: 16 sequences of 131072 cached tokens,
    32/8 heads, head_dim 128, block size 64, shuffled pool, N(0,1) sink;
    split into 512-token partitions."""
    return decode_case(seed, [seqlen] * batch, 32, 8, 128, 64, torch.bfloat16, with_sink=True,
                       spare_blocks=0, poison=poison)


def random_partials(seed: int, B: int, Hq: int, P: int, D: int, nparts) -> tuple:
    """Partition results for merge tests: ``part_out [B,Hq,P,D]`` ~ N(0,1),
    ``part_lse [B,Hq,P]`` ~ 3*N(0,1), with ``-inf`` in a seeded subset of the
    valid partitions (an empty partition) and NaN past ``nparts[b]``."""
    po = normal(seed, (B, Hq, P, D), stream=1)
    pl = 3.0 * normal(seed, (B, Hq, P), stream=2)
    rng = np.random.default_rng([seed, 5])
    empty = rng.random((B, Hq, P)) < 0.1
    pl[empty] = -np.inf
    po[empty] = 0.0
    for b, n in enumerate(nparts):
        po[b, :, n:, :] = np.nan
        pl[b, :, n:] = np.nan
    return torch.from_numpy(po), torch.from_numpy(pl)


def vertical_slash_pattern(seed: int, lengths, H: int, budget: float = 0.3,
                           num_sink: int = 30, num_recent: int = 100, band: int = 64):
    """Synthetic vertical + slash index sets shaped like the nano-vllm
    minference.py page's estimate_pattern output (which needs a trained
    model's attention to mean anything): per request and head, with the
    page's adaptive budget (vertical = max(num_sink + 1, 0.2 budget L), slash
    = max(num_recent + 1, 0.8 budget L)), vertical = the first num_sink keys
    plus distinct random keys, ascending; slash = diagonals 0 .. num_recent-1
    plus runs of `band` consecutive diagonals at random offsets.  Returns
    int32 ``vertical [B,H,NV]`` and ``slash [B,H,NS]`` padded with -1 (ignored
    entries) to the longest request's sizes."""
    rng = np.random.default_rng([seed, 2594])
    Lmax = max(lengths)
    def sizes(L):
        b = int(L * budget)
        return (min(L, max(num_sink + 1, int(b * 0.2))), min(L, max(num_recent + 1, int(b * 0.8))))
    NV, NS = sizes(Lmax)
    V = np.full((len(lengths), H, NV), -1, dtype=np.int32)
    S = np.full((len(lengths), H, NS), -1, dtype=np.int32)
    for r, L in enumerate(lengths):
        nv, ns = sizes(L)
        for h in range(H):
            sink = np.arange(min(num_sink, L))
            rest = rng.choice(np.arange(len(sink), L), size=max(0, nv - len(sink)), replace=False)
            V[r, h, :nv] = np.sort(np.concatenate([sink, rest]))[:nv]
            diags = set(range(min(num_recent, L)))
            while len(diags) < ns:
                start = int(rng.integers(0, L))
                diags.update(range(start, min(L, start + band)))
            S[r, h, :ns] = np.array(sorted(diags)[:ns], dtype=np.int32)[rng.permutation(ns)]
    return torch.from_numpy(V), torch.from_numpy(S)


def sparse_prefill_workload(seed: int = 6, L: int = 32768, Hq: int = 32, Hkv: int = 8,
                            D: int = 128):
    """A long-context vertical + slash sparse prefill: one request of 32768
    tokens, 32/8 heads, head_dim 128, bf16, no sink (the minference.py page
    attends without one), with the page's default pattern knobs (budget 0.3,
    30 sink columns, 100 recent diagonals)."""
    c = prefill_case(seed, [L], [L], Hq, Hkv, D, torch.bfloat16, False)
    V, S = vertical_slash_pattern(seed, [L], Hq)
    return c, V, S
