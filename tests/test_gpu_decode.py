"""Paged decode (and its split-KV merge) on the GPU against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, banner, check_decode_case, dev, oracle_decode, run_decode

pytestmark = pytest.mark.gpu


def test_config1_worked_example_fp32():
    """The doc page's decode example as configured: 3 sequences of 30/32/70
    keys, block size 32, block_table [[2,-1,-1,-1],[0,1,-1,-1],[3,5,6,-1]],
    fp32, 4/2 heads, D 64, sink; unused blocks 4 and 7 and block tails NaN."""
    banner("config1 decode")
    c = synth.config1_decode()
    assert torch.isnan(c.k_cache[4]).all() and torch.isnan(c.k_cache[7]).all()
    out, lse = run_decode(c)
    o, l = oracle_decode(c)
    assert_close(out, o, torch.float32, "config1 out")
    assert_close(lse, l, torch.float32, "config1 lse", lse=True)
    for P in (32, 64):
        out2, lse2 = run_decode(c, partition_size=P)
        assert_close(out2, o, torch.float32, f"config1 split {P}")
        assert_close(lse2, l, torch.float32, "config1 split lse", lse=True)


def _one_hot_case(dtype, D, bs, G):
    """Every query row selects exactly one logical key: q = 30 e_0, K(j*)[0] = 30
    and 0 elsewhere, so with sm_scale 1/8 the margin is 112.5 and o = V(j*)
    bit for bit.  V rows encode (sequence, position, kv head) as small integers."""
    lengths = [1, 17, 40, 64]
    Hkv = 2
    c = synth.decode_case(5, lengths, G * Hkv, Hkv, D, bs, dtype, with_sink=False,
                          sm_scale=1.0 / 8.0, poison=True)
    B = len(lengths)
    rng = np.random.default_rng(3)
    targets = [int(rng.integers(0, L)) for L in lengths]
    c.q.zero_()
    c.q[:, :, 0] = 30.0
    flat_k = c.k_cache.view(-1, Hkv, D)
    flat_v = c.v_cache.view(-1, Hkv, D)
    bt = c.block_table.tolist()
    for b, L in enumerate(lengths):
        for j in range(L):
            s = bt[b][j // bs] * bs + j % bs
            flat_k[s] = 0.0
            flat_k[s, :, 0] = 30.0 if j == targets[b] else 0.0
            for g in range(Hkv):
                flat_v[s, g] = 0.0
                flat_v[s, g, :3] = torch.tensor([b, j, g], dtype=dtype)
                flat_v[s, g, 3:] = float(j % 7)
    return c, targets


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D,bs,G", [(128, 16, 4), (64, 32, 2), (128, 64, 1), (64, 16, 8)])
def test_one_hot_gather_bitwise(dtype, D, bs, G):
    banner(f"one-hot gather {dtype} D={D} bs={bs} G={G}")
    c, targets = _one_hot_case(dtype, D, bs, G)
    for P in (0, 32):
        out, _ = run_decode(c, partition_size=P if P % bs == 0 else 0)
        out = out.float().cpu()
        for b, j in enumerate(targets):
            for h in range(c.Hq):
                g = h // G
                want = torch.zeros(D)
                want[:3] = torch.tensor([b, j, g], dtype=torch.float32)
                want[3:] = float(j % 7)
                if not torch.equal(out[b, h], want):
                    d = (out[b, h] - want).abs()
                    i = int(d.argmax())
                    raise AssertionError(f"P={P} b={b} h={h} d={i}: got {out[b, h, i].item()!r} "
                                         f"want {want[i].item()!r} ({int((d > 0).sum())} differ)")


CASES = [
    # lengths, Hq, Hkv, D, bs, sink, window
    ([0, 1, 15, 16, 17, 100], 8, 2, 128, 16, True, -1),
    ([33, 64, 65, 250, 1000], 32, 8, 128, 16, False, -1),
    ([5, 128, 300, 777], 16, 8, 64, 32, True, -1),
    ([70, 129, 513, 1030], 8, 8, 128, 64, True, 50),
    ([1, 2, 200, 600], 16, 2, 64, 16, True, 0),
    ([300, 301, 2048], 4, 1, 128, 128, True, 700),
    ([47, 1500], 16, 4, 64, 16, False, 3),
    # block size 8: every 16-token tile spans two blocks
    ([0, 1, 7, 8, 9, 15, 16, 17, 100, 333], 8, 2, 128, 8, True, -1),
    ([40, 1500, 63], 16, 4, 64, 8, False, 20),
    # head counts that are not a multiple of what one merge wave takes (2 heads
    # of 128 dims, 4 of 64): the merge falls back to fewer heads per wave
    ([3, 90, 400, 2000], 3, 1, 128, 16, True, -1),
    ([10, 200, 1300], 6, 2, 64, 16, False, -1),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_vs_oracle(case, dtype):
    lengths, Hq, Hkv, D, bs, sink, window = case
    banner(f"decode {dtype} {case}")
    c = synth.decode_case(11 + len(lengths), lengths, Hq, Hkv, D, bs, dtype, with_sink=sink,
                          window_left=window, poison=True)
    o, l = oracle_decode(c)
    for P in (0, -1, max(16, bs), 2 * max(16, bs), 256 if 256 % bs == 0 else bs, 512):
        out, lse = run_decode(c, partition_size=P)
        assert_close(out, o, dtype, f"out P={P}")
        assert_close(lse, l, dtype, f"lse P={P}", lse=True)


def test_decode_deterministic_and_permutation_invariant():
    banner("decode determinism / pool permutation")
    lengths = [100, 513, 2000]
    a = synth.decode_case(21, lengths, 32, 8, 128, 16, torch.bfloat16, with_sink=True,
                          shuffle=True, poison=True)
    b = synth.decode_case(21, lengths, 32, 8, 128, 16, torch.bfloat16, with_sink=True,
                          shuffle=False, poison=True)
    # same logical keys, different physical pools
    assert torch.equal(a.q, b.q)
    for P in (0, -1, 256):
        o1, l1 = run_decode(a, P)
        o2, l2 = run_decode(a, P)
        o3, l3 = run_decode(b, P)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "run-to-run"
        assert torch.equal(o1, o3) and torch.equal(l1, l3), "block permutation"
    # the balanced schedule folds the same pieces in the same order whether
    # the merge is its own launch (0) or fused into the stream (-1)
    o0, l0 = run_decode(a, 0)
    o1, l1 = run_decode(a, -1)
    assert torch.equal(o0, o1) and torch.equal(l0, l1), "two launches vs one"


def _decode_poisoned(c, P):
    from paged_kv_cache_02_amd import pkv
    check_decode_case(c)
    out = torch.full((c.B, c.Hq, c.D), float("nan"), dtype=c.q.dtype, device="cuda")
    lse = torch.full((c.B, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_decode(dev(c.q), dev(c.k_cache), dev(c.v_cache), dev(c.block_table),
                     dev(c.cache_seqlens), c.sm_scale, sink=dev(c.sink), window_left=c.window_left,
                     partition_size=P, max_seqlen_k=c.max_seqlen_k, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def test_config2_full_size():
    """bf16 decode at full size (64 seqs, 512..4096 keys, 32/8 heads, D 128,
    bs 16), in the launch configuration the benchmark times (the balanced
    schedule, stage and merge launches), and in one launch with the merge
    fused; every element against the oracle, the output poisoned with NaN
    first."""
    banner("config2 full size")
    c = synth.config2_decode(poison=True, spare_blocks=4)
    o, l = oracle_decode(c)
    for P in (0, -1):
        out, lse = _decode_poisoned(c, P)
        assert_close(out, o, torch.bfloat16, f"config2 P={P} out")
        assert_close(lse, l, torch.bfloat16, f"config2 P={P} lse", lse=True)


@pytest.mark.slow
def test_config5_long_context():
    """Long-context split decode at full size: 16 x 131072 keys, bs 64, sink;
    partitions of 512 merged by log-sum-exp (the configured split), and the
    automatic balanced schedule (two launches); every element of out and lse
    against the oracle.  The partition stage alone is compared too: its
    part_out / part_lse against the oracle's partition mode."""
    banner("config5 full size (generating 8.6 GB of K/V)")
    from paged_kv_cache_02_amd import pkv
    c = synth.config5_split_decode()
    o, l = oracle_decode(c)
    for P in (512, 0):
        banner(f"config5 P={P}")
        out, lse = _decode_poisoned(c, P)
        assert_close(out, o, torch.bfloat16, f"config5 P={P} out")
        assert_close(lse, l, torch.bfloat16, f"config5 P={P} lse", lse=True)
    banner("config5 partitions of 512")
    po, pl = pkv.paged_decode_partitions(dev(c.q), dev(c.k_cache), dev(c.v_cache),
                                         dev(c.block_table), dev(c.cache_seqlens), c.sm_scale,
                                         512, c.max_seqlen_k)
    torch.cuda.synchronize()
    wo, wl = oracle.paged_decode(c.q, c.k_cache, c.v_cache, c.block_table, c.cache_seqlens, None,
                                 c.sm_scale, partition_size=512)
    assert_close(po, wo, torch.bfloat16, "config5 part_out")
    assert_close(pl, wl, torch.bfloat16, "config5 part_lse", lse=True)


@pytest.mark.parametrize("case", [CASES[0], CASES[3], CASES[4], CASES[6]],
                         ids=["short", "window50", "window0", "window3"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_partitions_vs_oracle(case, dtype):
    """The first stage of split-KV decode on its own (vLLM page, the
    partitioned path's tmp_output / exp_sums): part_out / part_lse of every
    (sequence, head, partition) against the oracle's partition mode, at
    partition sizes of one block and 512 keys.  Sequences shorter than the
    longest have empty trailing partitions, and windows empty the leading
    ones; those must read out = 0 and lse = -inf."""
    from paged_kv_cache_02_amd import pkv
    lengths, Hq, Hkv, D, bs, sink, window = case
    banner(f"partitions {dtype} {case}")
    c = synth.decode_case(71 + len(lengths), lengths, Hq, Hkv, D, bs, dtype, with_sink=sink,
                          window_left=window, poison=True)
    for P in sorted({bs, 512}):
        po, pl = pkv.paged_decode_partitions(dev(c.q), dev(c.k_cache), dev(c.v_cache),
                                             dev(c.block_table), dev(c.cache_seqlens), c.sm_scale,
                                             P, c.max_seqlen_k, c.window_left)
        torch.cuda.synchronize()
        wo, wl = oracle.paged_decode(c.q, c.k_cache, c.v_cache, c.block_table, c.cache_seqlens,
                                     None, c.sm_scale, c.window_left, partition_size=P)
        assert po.shape == wo.shape, (po.shape, wo.shape)
        assert np.isneginf(wl).any(), "the case should have empty partitions"
        assert_close(po, wo, dtype, f"part_out P={P}")
        assert_close(pl, wl, dtype, f"part_lse P={P}", lse=True)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_merge_vs_oracle(dtype):
    banner(f"merge {dtype}")
    from paged_kv_cache_02_amd import pkv
    B, Hq, P, D, psz = 5, 8, 9, 128, 64
    seqlens = torch.tensor([0, 1, 64, 65, 570], dtype=torch.int32)
    nparts = [(int(L) + psz - 1) // psz for L in seqlens]
    po, pl = synth.random_partials(9, B, Hq, P, D, nparts)
    for with_sink in (False, True):
        sink = torch.from_numpy(synth.normal(4, (Hq,), 3)) if with_sink else None
        lse = torch.empty(B, Hq, device="cuda")
        out = pkv.merge_partitions(dev(po.float()), dev(pl.float()), dev(seqlens), psz,
                                   sink=dev(sink), out_dtype=dtype, lse=lse)
        torch.cuda.synchronize()
        o, l = oracle.merge(po.numpy(), pl.numpy(), nparts, sink)
        assert_close(out, o, dtype, "merge out")
        assert_close(lse, l, dtype, "merge lse", lse=True)


def test_decode_equals_paged_prefill_single_row():
    """Decode over cache_seqlens keys equals paged prefill with Lq = 1 over
    the same block table (same definition, different kernel)."""
    banner("decode == paged prefill Lq=1")
    from paged_kv_cache_02_amd import pkv
    c = synth.decode_case(31, [50, 300, 1200], 16, 4, 128, 16, torch.bfloat16, with_sink=True)
    out, _ = run_decode(c)
    cu_q = torch.arange(c.B + 1, dtype=torch.int32)
    cu_k = synth.cu_from_lengths(c.cache_seqlens.tolist())
    pre = pkv.varlen_prefill(dev(c.q), dev(cu_q), dev(cu_k), 1, c.max_seqlen_k, c.sm_scale,
                             c.Hkv, k_cache=dev(c.k_cache), v_cache=dev(c.v_cache),
                             block_table=dev(c.block_table), sink=dev(c.sink))
    torch.cuda.synchronize()
    o, _ = oracle_decode(c)
    assert_close(pre, o, torch.bfloat16, "prefill Lq=1 vs oracle")
    assert_close(out, pre.float().cpu().numpy(), torch.bfloat16, "decode vs prefill")


def test_fused_merge_workspace_reuse():
    """The one-launch balanced decode counts the pieces of each (sequence,
    head group) in 64-bit epoch-tagged counters at the start of the
    workspace and leaves them zero: one workspace serves consecutive calls
    with different batches; each result matches the oracle and a repeated
    call is bitwise identical."""
    banner("fused merge: workspace reuse")
    from paged_kv_cache_02_amd import pkv
    cases = [
        synth.decode_case(41, [0, 3, 700, 1500, 16, 2100], 32, 8, 128, 16, torch.bfloat16,
                          with_sink=True, poison=True),
        synth.decode_case(42, [90, 4000, 1], 32, 8, 128, 16, torch.bfloat16, with_sink=False,
                          window_left=300, poison=True),
    ]
    need = max(pkv.decode_workspace_bytes(c.B, c.Hq, c.D, c.max_seqlen_k) for c in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    first = None
    for rep, c in enumerate(cases + cases[:1]):
        lse = torch.empty(c.B, c.Hq, dtype=torch.float32, device="cuda")
        out = pkv.paged_decode(dev(c.q), dev(c.k_cache), dev(c.v_cache), dev(c.block_table),
                               dev(c.cache_seqlens), c.sm_scale, sink=dev(c.sink),
                               window_left=c.window_left, partition_size=-1,
                               max_seqlen_k=c.max_seqlen_k, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        counters = ws[:4096 * c.Hq * 8].view(torch.int64)
        assert int((counters != 0).sum()) == 0, f"call {rep}: counters left non-zero"
        o, l = oracle_decode(c)
        assert_close(out, o, torch.bfloat16, f"call {rep} out")
        assert_close(lse, l, torch.bfloat16, f"call {rep} lse", lse=True)
        if rep == 0:
            first = (out.clone(), lse.clone())
        elif rep == 2:
            assert torch.equal(out, first[0]) and torch.equal(lse, first[1]), "repeat differs"


def test_dirty_workspace_still_correct():
    """A workspace left dirty must not change the result: (1) fixed partitions,
    then the balanced schedule in both forms, on one buffer never re-zeroed
    (the partition results sit after the counter region); (2) counters
    holding stale counts of another epoch (what an interrupted call leaves)
    and NaN everywhere else, under the one-launch form that uses them.  Every
    call matches the oracle; the one-launch calls leave the counters zero."""
    banner("dirty workspace")
    from paged_kv_cache_02_amd import pkv
    c = synth.decode_case(43, [5, 700, 1500, 2100, 16, 3000, 1], 32, 8, 128, 16, torch.bfloat16,
                          with_sink=True, poison=True)
    o, l = oracle_decode(c)
    need = max(pkv.decode_workspace_bytes(c.B, c.Hq, c.D, c.max_seqlen_k, P) for P in (0, 256))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    args = (dev(c.q), dev(c.k_cache), dev(c.v_cache), dev(c.block_table), dev(c.cache_seqlens),
            c.sm_scale)
    for P in (256, 0, -1):
        lse = torch.empty(c.B, c.Hq, dtype=torch.float32, device="cuda")
        out = pkv.paged_decode(*args, sink=dev(c.sink), partition_size=P,
                               max_seqlen_k=c.max_seqlen_k, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        assert_close(out, o, torch.bfloat16, f"partition {P} then balanced: out")
        assert_close(lse, l, torch.bfloat16, f"partition {P} lse", lse=True)
    nc = 4096 * c.Hq
    ws.view(torch.uint8)[nc * 8:].view(torch.float32)[:] = float("nan")
    stale = (0x5EEDF00D << 32) | 3
    ws[:nc * 8].view(torch.int64)[:] = stale
    lse = torch.empty(c.B, c.Hq, dtype=torch.float32, device="cuda")
    out = pkv.paged_decode(*args, sink=dev(c.sink), partition_size=-1,
                           max_seqlen_k=c.max_seqlen_k, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    assert_close(out, o, torch.bfloat16, "stale counters: out")
    assert_close(lse, l, torch.bfloat16, "stale counters: lse", lse=True)
    # counter (b, head group) sits at b * (Hq / 4) + group: those the call counted
    # on are zero again, the others (sequences held by one wave) keep the stale value
    used = ws[:nc * 8].view(torch.int64)[:c.B * (c.Hq // 4)].cpu()
    assert bool(((used == 0) | (used == stale)).all()), "counter neither reset nor untouched"
    assert int((used == 0).sum()) > 0, "no counter was used"


@pytest.mark.parametrize("case", CASES[:4], ids=[str(i) for i in range(4)])
def test_two_launch_decode_vs_oracle(case):
    """The balanced schedule as two launches (pieces, then the merge kernel)."""
    lengths, Hq, Hkv, D, bs, sink, window = case
    banner(f"two-launch decode {case}")
    from paged_kv_cache_02_amd import pkv
    c = synth.decode_case(51 + len(lengths), lengths, Hq, Hkv, D, bs, torch.bfloat16,
                          with_sink=sink, window_left=window, poison=True)
    ws = torch.empty(pkv.decode_workspace_bytes(c.B, Hq, D, c.max_seqlen_k), dtype=torch.uint8, device="cuda")
    out = torch.empty(c.B, Hq, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(c.B, Hq, dtype=torch.float32, device="cuda")
    pkv.paged_decode_stage(dev(c.q), dev(c.k_cache), dev(c.v_cache), dev(c.block_table),
                           dev(c.cache_seqlens), c.sm_scale, c.max_seqlen_k, ws, c.window_left)
    pkv.paged_decode_finish(out, ws, Hkv, sink=dev(c.sink), lse=lse)
    torch.cuda.synchronize()
    o, l = oracle_decode(c)
    assert_close(out, o, torch.bfloat16, "two-launch out")
    assert_close(lse, l, torch.bfloat16, "two-launch lse", lse=True)


@pytest.mark.parametrize("D,Hq,Hkv,window,B,bs", [(128, 32, 8, -1, 300, 16),
                                                   (64, 16, 2, 9, 1200, 16),
                                                   (128, 8, 2, -1, 500, 8)])
def test_decode_many_short_sequences(D, Hq, Hkv, window, B, bs):
    """Hundreds of 1..40-key sequences: each wave's range of the balanced
    schedule crosses several sequences, so the Q of the second sequence
    (preloaded) and of later ones (loaded at the change) are both used;
    one launch and two launches against the oracle."""
    banner(f"many short sequences D={D} window={window}")
    from paged_kv_cache_02_amd import pkv
    rng = np.random.default_rng(61)
    lengths = rng.integers(1, 40, size=B, endpoint=True).tolist()
    c = synth.decode_case(62, lengths, Hq, Hkv, D, bs, torch.bfloat16, with_sink=True,
                          window_left=window, poison=True)
    o, l = oracle_decode(c)
    out, lse = run_decode(c, partition_size=-1)
    assert_close(out, o, torch.bfloat16, "one launch out")
    assert_close(lse, l, torch.bfloat16, "one launch lse", lse=True)
    ws = torch.empty(pkv.decode_workspace_bytes(c.B, Hq, D, c.max_seqlen_k), dtype=torch.uint8, device="cuda")
    out2 = torch.empty(c.B, Hq, D, dtype=torch.bfloat16, device="cuda")
    lse2 = torch.empty(c.B, Hq, dtype=torch.float32, device="cuda")
    pkv.paged_decode_stage(dev(c.q), dev(c.k_cache), dev(c.v_cache), dev(c.block_table),
                           dev(c.cache_seqlens), c.sm_scale, c.max_seqlen_k, ws, c.window_left)
    pkv.paged_decode_finish(out2, ws, Hkv, sink=dev(c.sink), lse=lse2)
    torch.cuda.synchronize()
    assert_close(out2, o, torch.bfloat16, "two launches out")
    assert_close(lse2, l, torch.bfloat16, "two launches lse", lse=True)


@pytest.mark.parametrize("bs", [16, 8])
def test_decode_large_batch(bs):
    """More sequences than the balanced schedule takes (B > 4096): bf16 decode
    runs one workgroup per (sequence, head group, partition), unsplit and
    with 64-token partitions merged afterwards."""
    banner(f"large batch bs={bs}")
    rng = np.random.default_rng(63)
    lengths = rng.integers(0, 80, size=4100, endpoint=True).tolist()
    c = synth.decode_case(64, lengths, 8, 2, 128, bs, torch.bfloat16, with_sink=True,
                          poison=True)
    o, l = oracle_decode(c)
    for P in (0, 64):
        out, lse = run_decode(c, partition_size=P)
        assert_close(out, o, torch.bfloat16, f"out P={P}")
        assert_close(lse, l, torch.bfloat16, f"lse P={P}", lse=True)


def test_prepared_launches_match_direct_calls():
    """pkv.prepare records a binding call's launches with their marshalled
    arguments; running the prepared launcher (twice) gives bit for bit what
    the direct call gives (decode through the balanced schedule, and a
    varlen prefill)."""
    from paged_kv_cache_02_amd import pkv
    banner("prepared launches")
    c = synth.decode_case(65, [5, 300, 1000, 2048], 32, 8, 128, 16, torch.bfloat16, True)
    q, kc, vc, bt, sl = dev(c.q), dev(c.k_cache), dev(c.v_cache), dev(c.block_table), \
        dev(c.cache_seqlens)
    ws = torch.empty(pkv.decode_workspace_bytes(c.B, c.Hq, c.D, c.max_seqlen_k), dtype=torch.uint8,
                     device="cuda")
    want = pkv.paged_decode(q, kc, vc, bt, sl, c.sm_scale, sink=dev(c.sink), workspace=ws,
                            max_seqlen_k=c.max_seqlen_k)
    out = torch.full_like(want, float("nan"))
    run = pkv.prepare(pkv.paged_decode, q, kc, vc, bt, sl, c.sm_scale, sink=dev(c.sink),
                      workspace=ws, max_seqlen_k=c.max_seqlen_k, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all(), "prepare must not launch"
    for _ in range(2):
        run()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16))
    p = synth.prefill_case(66, [100, 333], [100, 333], 8, 2, 64, torch.bfloat16, True)
    args = (dev(p.q), dev(p.cu_seqlens_q), dev(p.cu_seqlens_k), p.max_seqlen_q, p.max_seqlen_k,
            p.sm_scale, p.Hkv)
    kw = dict(k=dev(p.k), v=dev(p.v), sink=dev(p.sink))
    want = pkv.varlen_prefill(*args, **kw)
    out = torch.empty_like(want)
    pkv.prepare(pkv.varlen_prefill, *args, out=out, **kw)()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))


def _repage(kc, bt, lengths, bs, seed):
    """The same logical keys in a pool of block size bs with a shuffled
    block table (built on the GPU from a paged cache kc / table bt)."""
    bs0 = kc.shape[1]
    rows = []
    for b, L in enumerate(lengths):
        nb0 = (L + bs0 - 1) // bs0
        rows.append(kc[bt[b, :nb0].long()].reshape(nb0 * bs0, *kc.shape[2:])[:L])
    nbs = [(L + bs - 1) // bs for L in lengths]
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(sum(nbs))).cuda()
    pool = torch.zeros((sum(nbs), bs) + tuple(kc.shape[2:]), dtype=kc.dtype, device="cuda")
    table = torch.zeros((len(lengths), max(nbs)), dtype=torch.int32, device="cuda")
    o = 0
    for b, L in enumerate(lengths):
        ids = perm[o:o + nbs[b]]
        flat = torch.zeros((nbs[b] * bs,) + tuple(kc.shape[2:]), dtype=kc.dtype, device="cuda")
        flat[:L] = rows[b]
        pool[ids] = flat.reshape(nbs[b], bs, *kc.shape[2:])
        table[b, :nbs[b]] = ids.int()
        o += nbs[b]
    return pool, table


def test_long_ranges_block_sizes_bitwise():
    """Ranges of more than two 64-tile batches per wave (about 136 tiles), so
    each wave reads block ids from both LDS slots of its batch double buffer:
    the same logical cache paged with block sizes 8, 16 and 64 gives the same
    bits in every decode form (the schedule's tiles are 16 tokens whatever
    the block size), and two sequences match the oracle."""
    banner("long ranges, block sizes 8 / 16 / 64")
    from paged_kv_cache_02_amd import pkv
    lengths = [70001, 69000, 71234, 68500]
    c = synth.decode_case(71, lengths, 32, 8, 128, 16, torch.bfloat16, with_sink=True,
                          poison=False, spare_blocks=0)
    q, kc, vc, bt, sl = dev(c.q), dev(c.k_cache), dev(c.v_cache), dev(c.block_table), \
        dev(c.cache_seqlens)
    sink = dev(c.sink)
    results = {}
    for bs in (16, 8, 64):
        if bs == 16:
            k2, v2, t2 = kc, vc, bt
        else:
            k2, t2 = _repage(kc, bt, lengths, bs, 72 + bs)
            v2, _ = _repage(vc, bt, lengths, bs, 72 + bs)    # same seed: the same table
        for P in (0, -1, 512):
            lse = torch.empty(c.B, c.Hq, dtype=torch.float32, device="cuda")
            out = pkv.paged_decode(q, k2, v2, t2, sl, c.sm_scale, sink=sink, partition_size=P,
                                   max_seqlen_k=max(lengths), lse=lse)
            torch.cuda.synchronize()
            results[(bs, P)] = (out, lse)
        del k2, v2
    ref_out, ref_lse = results[(16, 0)]
    for key, (out, lse) in results.items():
        if key[1] == 512:
            continue            # fixed partitions fold in another order
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"bs/P {key} differs"
    for bs in (8, 64):
        assert torch.equal(results[(bs, 512)][0], results[(16, 512)][0]), f"bs {bs} P 512 differs"
    # two sequences against the oracle
    sub = synth.DecodeCase(c.q[:2], c.k_cache, c.v_cache, c.block_table[:2],
                           c.cache_seqlens[:2], c.sink, c.block_size, c.sm_scale, c.window_left)
    o, l = oracle_decode(sub)
    assert_close(ref_out[:2], o, torch.bfloat16, "long ranges out")
    assert_close(ref_lse[:2], l, torch.bfloat16, "long ranges lse", lse=True)


@pytest.mark.parametrize("P", [0, -1, 64])
def test_all_sequences_empty(P):
    """No sequence has a key: with a positive max_seqlen_k the balanced
    schedule runs with an empty tile list (every wave's range is empty, the
    merge sees no piece), and with max_seqlen_k 0 no schedule is needed.
    out is 0 and lse the sink (or -inf), as the oracle gives."""
    banner(f"all sequences empty P={P}")
    from paged_kv_cache_02_amd import pkv
    for with_sink in (True, False):
        c = synth.decode_case(81, [0, 0, 0, 0, 0], 32, 8, 128, 16, torch.bfloat16,
                              with_sink=with_sink, poison=True, max_blocks_per_seq=4)
        o, l = oracle_decode(c)
        for msk in (64, 0):
            if msk == 0 and P == 64:
                continue
            out = torch.full((c.B, c.Hq, c.D), float("nan"), dtype=c.q.dtype, device="cuda")
            lse = torch.full((c.B, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
            pkv.paged_decode(dev(c.q), dev(c.k_cache), dev(c.v_cache), dev(c.block_table),
                             dev(c.cache_seqlens), c.sm_scale, sink=dev(c.sink),
                             partition_size=P, max_seqlen_k=msk, out=out, lse=lse)
            torch.cuda.synchronize()
            assert_close(out, o, torch.bfloat16, f"empty out msk={msk} sink={with_sink}")
            assert_close(lse, l, torch.bfloat16, f"empty lse msk={msk} sink={with_sink}", lse=True)
