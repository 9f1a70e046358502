"""ALiBi (per-head slope times key position minus query position, added to the
scaled logits) on every attention path, on the GPU against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, banner, dev

pytestmark = pytest.mark.gpu


def slopes(Hq):
    """The usual geometric ALiBi slopes 2^(-8 (h + 1) / Hq)."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=torch.float32)


DECODE = [
    # lengths, Hq, Hkv, D, bs, sink, window
    ([1, 17, 300, 2000], 32, 8, 128, 16, True, -1),
    ([64, 1000, 5], 8, 2, 64, 32, False, 100),
    ([129, 700], 12, 4, 128, 16, True, -1),
]


@pytest.mark.parametrize("case", DECODE, ids=[str(i) for i in range(len(DECODE))])
@pytest.mark.parametrize("mode", ["auto", "one_launch", "two_launch", "partitions", "fp32"])
def test_decode_alibi(case, mode):
    from paged_kv_cache_02_amd import pkv
    lens, Hq, Hkv, D, bs, sink, window = case
    dtype = torch.float32 if mode == "fp32" else torch.bfloat16
    banner(f"decode alibi {mode} {case}")
    c = synth.decode_case(400 + len(lens), lens, Hq, Hkv, D, bs, dtype, sink, window_left=window)
    al = slopes(Hq)
    q, kc, vc, bt, sl = (dev(t) for t in (c.q, c.k_cache, c.v_cache, c.block_table,
                                          c.cache_seqlens))
    msk = int(c.cache_seqlens.max())
    lse = torch.empty(c.B, Hq, dtype=torch.float32, device="cuda")
    if mode == "two_launch":
        nb = pkv.decode_workspace_bytes(c.B, Hq, D, msk)
        ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        pkv.paged_decode_stage(q, kc, vc, bt, sl, c.sm_scale, msk, ws, window, alibi_slopes=dev(al))
        out = torch.empty_like(q)
        pkv.paged_decode_finish(out, ws, Hkv, sink=dev(c.sink), lse=lse)
    else:
        out = pkv.paged_decode(q, kc, vc, bt, sl, c.sm_scale, sink=dev(c.sink), window_left=window,
                               partition_size={"partitions": 64, "one_launch": -1}.get(mode, 0),
                               max_seqlen_k=msk, lse=lse, alibi_slopes=dev(al))
    torch.cuda.synchronize()
    o, l = oracle.paged_decode(c.q, c.k_cache, c.v_cache, c.block_table, c.cache_seqlens, c.sink,
                               c.sm_scale, window_left=window, alibi=al)
    assert_close(out, o, dtype, "decode alibi out")
    assert_close(lse, l, dtype, "decode alibi lse", lse=True)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_append_alibi(dtype):
    from paged_kv_cache_02_amd import pkv
    banner(f"decode append alibi {dtype}")
    lens, Hq, Hkv, D, bs = [0, 16, 250, 1500], 32, 8, 128, 16
    c = synth.decode_case(410, [L + 1 for L in lens], Hq, Hkv, D, bs, dtype, True)
    L = torch.tensor(lens, dtype=torch.int32)
    kn = synth.to_dtype(synth.normal(410, (len(lens), Hkv, D), stream=11), dtype)
    vn = synth.to_dtype(synth.normal(410, (len(lens), Hkv, D), stream=12), dtype)
    al = slopes(Hq)
    kc, vc = dev(c.k_cache), dev(c.v_cache)
    lse = torch.empty(len(lens), Hq, dtype=torch.float32, device="cuda")
    out = pkv.paged_decode_append(dev(c.q), dev(kn), dev(vn), kc, vc, dev(c.block_table), dev(L),
                                  c.sm_scale, sink=dev(c.sink), max_seqlen_k=int(L.max()),
                                  lse=lse, alibi_slopes=dev(al))
    torch.cuda.synchronize()
    o, l, _, _ = oracle.decode_append(c.q, kn, vn, c.k_cache, c.v_cache, c.block_table, L,
                                      c.sink, c.sm_scale, alibi=al)
    assert_close(out, o, dtype, "append alibi out")
    assert_close(lse, l, dtype, "append alibi lse", lse=True)


PREFILL = [
    # q_lens, k_lens, Hq, Hkv, D, sink, window, paged block size (0: contiguous)
    ([1, 100, 300], None, 32, 8, 128, True, -1, 0),
    ([64, 257], None, 8, 2, 64, True, 50, 0),
    ([33, 200], [500, 200], 12, 4, 128, False, -1, 0),
    ([90, 7], [300, 64], 16, 2, 128, True, -1, 16),
    ([129, 40], [129, 300], 8, 8, 64, True, 31, 32),
]


@pytest.mark.parametrize("case", PREFILL, ids=[str(i) for i in range(len(PREFILL))])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_alibi(case, dtype):
    from paged_kv_cache_02_amd import pkv
    q_lens, k_lens, Hq, Hkv, D, sink, window, bs = case
    banner(f"prefill alibi {dtype} {case}")
    k_lens = k_lens or q_lens
    if bs:
        c = synth.paged_prefill_case(420 + len(q_lens), q_lens, k_lens, Hq, Hkv, D, bs, dtype, sink,
                                     window_left=window)
    else:
        c = synth.prefill_case(420 + len(q_lens), q_lens, k_lens, Hq, Hkv, D, dtype, sink,
                               window_left=window)
    al = slopes(Hq)
    T = c.q.shape[0]
    lse = torch.empty(T, Hq, dtype=torch.float32, device="cuda")
    out = pkv.varlen_prefill(dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q,
                             c.max_seqlen_k, c.sm_scale, c.Hkv, k=dev(c.k), v=dev(c.v),
                             k_cache=dev(c.k_cache), v_cache=dev(c.v_cache),
                             block_table=dev(c.block_table), sink=dev(c.sink),
                             window_left=window, lse=lse, alibi_slopes=dev(al))
    torch.cuda.synchronize()
    o, l = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, c.sm_scale, c.Hkv,
                                 k=c.k, v=c.v, k_cache=c.k_cache, v_cache=c.v_cache,
                                 block_table=c.block_table, block_size=c.block_size,
                                 window_left=window, alibi=al)
    assert_close(out, o, dtype, "prefill alibi out")
    assert_close(lse, l, dtype, "prefill alibi lse", lse=True)


@pytest.mark.parametrize("case", [PREFILL[1], PREFILL[3]], ids=["window", "paged"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_alibi_noncausal(case, dtype):
    """ALiBi with causal=False: keys after the query position get a positive
    bias (slope times key minus query position)."""
    from paged_kv_cache_02_amd import pkv
    q_lens, k_lens, Hq, Hkv, D, sink, window, bs = case
    banner(f"prefill alibi non-causal {dtype} {case}")
    k_lens = k_lens or q_lens
    if bs:
        c = synth.paged_prefill_case(440 + len(q_lens), q_lens, k_lens, Hq, Hkv, D, bs, dtype, sink,
                                     window_left=window)
    else:
        c = synth.prefill_case(440 + len(q_lens), q_lens, k_lens, Hq, Hkv, D, dtype, sink,
                               window_left=window)
    al = slopes(Hq)
    T = c.q.shape[0]
    lse = torch.empty(T, Hq, dtype=torch.float32, device="cuda")
    out = pkv.varlen_prefill(dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q,
                             c.max_seqlen_k, c.sm_scale, c.Hkv, k=dev(c.k), v=dev(c.v),
                             k_cache=dev(c.k_cache), v_cache=dev(c.v_cache),
                             block_table=dev(c.block_table), sink=dev(c.sink),
                             window_left=window, lse=lse, alibi_slopes=dev(al), causal=False)
    torch.cuda.synchronize()
    o, l = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, c.sm_scale, c.Hkv,
                                 k=c.k, v=c.v, k_cache=c.k_cache, v_cache=c.v_cache,
                                 block_table=c.block_table, block_size=c.block_size,
                                 window_left=window, alibi=al, causal=False)
    assert_close(out, o, dtype, "prefill alibi non-causal out")
    assert_close(lse, l, dtype, "prefill alibi non-causal lse", lse=True)


def test_alibi_zero_slopes_equal_plain():
    """Slopes of zero give exactly the results of a call without slopes
    (bf16 prefill: the ALiBi instantiation reorders no arithmetic that
    matters beyond rounding, so compare within the bf16 bar; decode: the
    engine adds 0 to the scaled logit, so it is bitwise)."""
    from paged_kv_cache_02_amd import pkv
    banner("alibi zero slopes")
    c = synth.decode_case(430, [100, 999], 32, 8, 128, 16, torch.bfloat16, True)
    args = (dev(c.q), dev(c.k_cache), dev(c.v_cache), dev(c.block_table), dev(c.cache_seqlens),
            c.sm_scale)
    o1 = pkv.paged_decode(*args, sink=dev(c.sink))
    o2 = pkv.paged_decode(*args, sink=dev(c.sink), alibi_slopes=torch.zeros(32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    p = synth.prefill_case(431, [300], [300], 32, 8, 128, torch.bfloat16, True)
    pa = (dev(p.q), dev(p.cu_seqlens_q), dev(p.cu_seqlens_k), p.max_seqlen_q, p.max_seqlen_k,
          p.sm_scale, p.Hkv)
    r1 = pkv.varlen_prefill(*pa, k=dev(p.k), v=dev(p.v), sink=dev(p.sink))
    r2 = pkv.varlen_prefill(*pa, k=dev(p.k), v=dev(p.v), sink=dev(p.sink),
                            alibi_slopes=torch.zeros(32, device="cuda"))
    torch.cuda.synchronize()
    assert_close(r2, r1.float().cpu().double().numpy(), torch.bfloat16, "zero slopes prefill")
