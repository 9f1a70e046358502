"""The host validator of device-resident index data (paged_kv_cache_02_amd.validate):
it accepts the index data of every synthetic workload and of the pages'
worked examples, and rejects each kind of contract violation with a
ValueError (no GPU needed)."""

import numpy as np
import pytest
import torch

import synth
from paged_kv_cache_02_amd import validate as V


def test_workloads_pass():
    c1 = synth.config1_decode()
    V.check_decode(c1.block_table, c1.cache_seqlens, c1.num_blocks, 32, 70)
    # the page's new tokens at 30 / 32 / 70 fit blocks 2, 1 and 6
    V.check_decode(c1.block_table, c1.cache_seqlens, c1.num_blocks, 32, 70, append=True)
    p1 = synth.config1_prefill()
    V.check_varlen(p1.cu_seqlens_q, p1.cu_seqlens_k, 10, 10, num_k_rows=p1.k.shape[0])
    # the varlen example: q lengths [10, 3, 1] over k lengths [0, 1, 7]
    V.check_varlen([0, 10, 13, 14], [0, 0, 1, 8], 10, 7, num_k_rows=8)
    c2 = synth.config2_decode()
    V.check_decode(c2.block_table, c2.cache_seqlens, c2.num_blocks, 16, c2.max_seqlen_k)
    c4 = synth.config4_chunked(poison=False, spare_blocks=0)
    V.check_varlen(c4.cu_seqlens_q, c4.cu_seqlens_k, 512, 8704, c4.block_table,
                   c4.k_cache.shape[0], 16)
    # config 5: only the index data (the pool itself is 8.6 GB)
    bt, nb = synth.pool_from_lengths(np.random.default_rng(4), [131072] * 16, 64)
    V.check_decode(bt, torch.full((16,), 131072, dtype=torch.int32), nb, 64, 131072)
    L = synth.config3_lengths()
    bt3, nb3 = synth.pool_from_lengths(np.random.default_rng(7), L, 16)
    slots = torch.cat([synth.slots_for_tokens(bt3[r:r + 1].expand(n, -1).contiguous(),
                                              list(range(n)), 16) for r, n in enumerate(L)])
    V.check_slots(slots, nb3, 16)


def _decode_table():
    bt = torch.tensor([[2, -1, -1, -1], [0, 1, -1, -1], [3, 5, 6, -1]], dtype=torch.int32)
    return bt, torch.tensor([30, 32, 70], dtype=torch.int32)


@pytest.mark.parametrize("mutate,match", [
    (lambda bt, L: L.__setitem__(0, -1), "negative"),
    (lambda bt, L: L.__setitem__(2, 71), "exceeds max_seqlen_k"),
    (lambda bt, L: bt.__setitem__((2, 2), 8), "not a block id"),        # past the 8-block pool
    (lambda bt, L: bt.__setitem__((2, 2), -1), "not a block id"),       # a used entry is -1
])
def test_decode_violations(mutate, match):
    bt, L = _decode_table()
    mutate(bt, L)
    with pytest.raises(ValueError, match=match):
        V.check_decode(bt, L, 8, 32, 70)


def test_decode_append_violations():
    bt, L = _decode_table()
    # sequence 1 appends at position 32: its second block is needed
    bt[1, 1] = -1
    with pytest.raises(ValueError, match="not a block id"):
        V.check_decode(bt, L, 8, 32, 70, append=True)
    bt, L = _decode_table()
    with pytest.raises(ValueError, match="does not fit"):
        V.check_decode(bt[:, :3].contiguous(), L, 8, 32, 96, append=True)
    # two sequences appending into one slot
    bt = torch.tensor([[0, 1], [0, 2]], dtype=torch.int32)
    with pytest.raises(ValueError, match="same cache slot"):
        V.check_decode(bt, torch.tensor([5, 5], dtype=torch.int32), 4, 16, 5, append=True)


@pytest.mark.parametrize("cu_q,cu_k,match", [
    ([1, 10, 13, 14], [0, 0, 1, 8], "must be 0"),
    ([0, 10, 9, 14], [0, 0, 1, 8], "decreases"),
    ([0, 11, 13, 14], [0, 0, 1, 8], "more than the maximum"),
    ([0, 10, 13, 14], [0, 0, 1, 9], "more than the maximum"),
    ([0, 10, 13], [0, 0, 1, 8], "different batch sizes"),
])
def test_varlen_violations(cu_q, cu_k, match):
    with pytest.raises(ValueError, match=match):
        V.check_varlen(cu_q, cu_k, 10, 7)


def test_varlen_key_rows_and_paged():
    with pytest.raises(ValueError, match="rows"):
        V.check_varlen([0, 10, 13, 14], [0, 0, 1, 8], 10, 7, num_k_rows=7)
    bt = torch.tensor([[-1], [0], [3]], dtype=torch.int32)
    V.check_varlen([0, 10, 13, 14], [0, 0, 1, 8], 10, 7, bt, 4, 8)
    with pytest.raises(ValueError, match="not a block id"):
        V.check_varlen([0, 10, 13, 14], [0, 0, 1, 8], 10, 7, bt, 3, 8)
    with pytest.raises(ValueError, match="need"):
        V.check_varlen([0, 10, 13, 14], [0, 0, 1, 8], 10, 7, bt, 4, 4)


def test_slot_violations():
    V.check_slots(torch.tensor([3, -1, 0, -1, 7], dtype=torch.int32), 2, 4)
    with pytest.raises(ValueError, match="past the pool"):
        V.check_slots(torch.tensor([3, 8], dtype=torch.int32), 2, 4)
    with pytest.raises(ValueError, match="share"):
        V.check_slots(torch.tensor([3, 3], dtype=torch.int32), 2, 4)
    with pytest.raises(ValueError, match="integers"):
        V.check_slots(torch.tensor([3.0]), 2, 4)
