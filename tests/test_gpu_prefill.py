"""Varlen prefill, causal and non-causal (contiguous and paged K/V), on the GPU
against the fp64 oracle."""

import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_close, banner, check_prefill_case, dev, oracle_prefill, run_prefill

pytestmark = pytest.mark.gpu


def test_config1_prefill_fp32():
    banner("config1 prefill")
    c = synth.config1_prefill()
    out, lse = run_prefill(c)
    o, l = oracle_prefill(c)
    assert_close(out, o, torch.float32, "config1 prefill")
    assert_close(lse, l, torch.float32, "config1 lse", lse=True)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_page_example_lengths(dtype):
    """The doc's varlen example lengths: q [10,3,1] over k [0,1,7]; rows
    that see no key give 0 (lse = sink)."""
    banner(f"page varlen example {dtype}")
    c = synth.prefill_case(3, [10, 3, 1], [0, 1, 7], 4, 2, 64, dtype, True)
    out, lse = run_prefill(c)
    o, l = oracle_prefill(c)
    assert (out.float().cpu()[:12] == 0).all()
    assert_close(out, o, dtype, "page example")
    assert_close(lse, l, dtype, "page example lse", lse=True)


def test_request_tag_probe():
    """q = 0 gives uniform weights over the visible keys; V = 2^r for every
    key of request r, so each output is 2^r and names the request whose keys
    were read (cu_seqlens_k indexing); no sink."""
    banner("request tag probe")
    lens = [37, 1, 130, 64, 200]
    c = synth.prefill_case(4, lens, lens, 8, 2, 128, torch.bfloat16, False)
    c.q.zero_()
    cu = c.cu_seqlens_k.tolist()
    for r in range(len(lens)):
        c.v[cu[r]:cu[r + 1]] = float(2 ** r)
    out, _ = run_prefill(c, with_lse=False)
    out = out.float().cpu()
    for r in range(len(lens)):
        assert (out[cu[r]:cu[r + 1]] == float(2 ** r)).all(), r


CASES = [
    # q_lens, k_lens, Hq, Hkv, D, sink, window
    ([1, 5, 128, 129, 300], None, 8, 2, 128, True, -1),
    ([64, 255, 256, 257], None, 32, 8, 128, False, -1),
    ([100, 513], None, 16, 16, 64, True, -1),
    ([200, 77, 400], None, 8, 1, 64, True, 31),
    ([130, 20], [500, 20], 8, 4, 128, True, -1),           # chunk: queries at the end
    ([0, 33, 1], [10, 40, 1000], 4, 2, 128, True, 64),
    ([300], None, 4, 4, 128, True, 0),
    ([1, 63, 64, 65, 129, 192, 257], None, 8, 4, 64, True, -1),   # D 64: 1 to 5 key tiles
    # GQA groups that set the workgroup shape: heads per workgroup x positions
    ([70, 333], None, 12, 4, 128, True, -1),       # G 3: 1 head x 128, three head subgroups
    ([129, 40, 260], None, 12, 2, 64, True, 50),   # G 6: 2 heads x 64, three subgroups, window
    ([300, 17], None, 16, 1, 128, False, -1),      # G 16: 4 heads x 32, four subgroups
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_contiguous_vs_oracle(case, dtype):
    q_lens, k_lens, Hq, Hkv, D, sink, window = case
    banner(f"prefill contiguous {dtype} {case}")
    c = synth.prefill_case(40 + len(q_lens), q_lens, k_lens or q_lens, Hq, Hkv, D, dtype, sink,
                           window_left=window)
    out, lse = run_prefill(c)
    o, l = oracle_prefill(c)
    assert_close(out, o, dtype, "out")
    assert_close(lse, l, dtype, "lse", lse=True)


PAGED = [
    ([64, 100], [64 + 300, 100], 16, 8, 64, 16, True, 128),
    ([512, 3], [1000, 700], 8, 2, 128, 32, True, -1),
    ([129, 1], [129, 2000], 8, 8, 128, 64, False, 17),
    ([40, 1, 200], [40 + 150, 70, 200 + 64], 8, 2, 64, 16, False, -1),   # D 64 ring, no window
    ([90, 200], [300, 200], 16, 2, 128, 16, True, -1),                   # G 8: two head subgroups
    ([64, 100], [364, 100], 16, 8, 64, 8, True, 128),                    # block size 8
    ([90, 200], [300, 200], 8, 2, 128, 8, True, -1),
]


@pytest.mark.parametrize("case", PAGED, ids=[str(i) for i in range(len(PAGED))])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_paged_vs_oracle(case, dtype):
    q_lens, k_lens, Hq, Hkv, D, bs, sink, window = case
    banner(f"prefill paged {dtype} {case}")
    c = synth.paged_prefill_case(60 + len(q_lens), q_lens, k_lens, Hq, Hkv, D, bs, dtype, sink,
                                 window_left=window, poison=True)
    out, lse = run_prefill(c)
    o, l = oracle_prefill(c)
    assert_close(out, o, dtype, "out")
    assert_close(lse, l, dtype, "lse", lse=True)


NONCAUSAL = [
    # q_lens, k_lens, Hq, Hkv, D, sink, window, paged block size (0: contiguous)
    ([1, 5, 128, 129, 300], None, 8, 2, 128, True, -1, 0),
    ([130, 20], [500, 20], 8, 4, 128, True, -1, 0),          # queries fewer than keys
    ([10, 3, 1], [0, 1, 7], 4, 2, 64, True, -1, 0),           # more queries than keys, Lk = 0
    ([200, 77, 400], None, 8, 1, 64, True, 31, 0),            # left-only window
    ([300], None, 4, 4, 128, False, 0, 0),                    # window 0: from p on
    ([129, 40, 260], None, 12, 2, 64, True, 3, 0),            # G 6, small window
    ([64, 100], [364, 100], 16, 8, 64, True, 128, 16),
    ([129, 1], [129, 2000], 8, 8, 128, False, 17, 64),
    ([1000], [70], 16, 2, 64, True, 17, 32),                  # Lq > Lk with a window
    ([40, 1, 200], [190, 70, 264], 8, 2, 64, False, -1, 16),
]


@pytest.mark.parametrize("case", NONCAUSAL, ids=[str(i) for i in range(len(NONCAUSAL))])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_noncausal_vs_oracle(case, dtype):
    """causal=False (the FlashInfer page's non-causal branches): every key of
    the request, a window bounding only the left side."""
    q_lens, k_lens, Hq, Hkv, D, sink, window, bs = case
    banner(f"prefill non-causal {dtype} {case}")
    k_lens = k_lens or q_lens
    if bs:
        c = synth.paged_prefill_case(90 + len(q_lens), q_lens, k_lens, Hq, Hkv, D, bs, dtype,
                                     sink, window_left=window, poison=True)
    else:
        c = synth.prefill_case(90 + len(q_lens), q_lens, k_lens, Hq, Hkv, D, dtype, sink,
                               window_left=window)
    out, lse = run_prefill(c, causal=False)
    o, l = oracle_prefill(c, causal=False)
    assert_close(out, o, dtype, "out")
    assert_close(lse, l, dtype, "lse", lse=True)


def test_prefill_noncausal_differs_from_causal():
    """The flag reaches the kernel: a non-causal call equals the oracle's
    non-causal result and not its causal one."""
    banner("prefill non-causal vs causal")
    c = synth.prefill_case(99, [200, 70], [200, 70], 8, 2, 128, torch.bfloat16, True)
    out, _ = run_prefill(c, causal=False)
    o_nc, _ = oracle_prefill(c, causal=False)
    o_c, _ = oracle_prefill(c, causal=True)
    assert_close(out, o_nc, torch.bfloat16, "non-causal")
    assert (out.float().cpu() - torch.as_tensor(o_c).float()).abs().max() > 0.1


@pytest.mark.parametrize("heads", [(4, 4), (8, 4), (12, 4), (8, 2), (12, 2), (16, 2), (16, 1)],
                         ids=lambda x: f"{x[0]}q{x[1]}kv")
def test_prefill_every_row_written(heads):
    """Every (row, head) of out and lse is written exactly by the grid: both
    start as NaN, and lengths straddle the 32-row blocks and 128-row tiles
    that the GQA group size arranges into workgroups."""
    from paged_kv_cache_02_amd import pkv
    Hq, Hkv = heads
    banner(f"prefill coverage {Hq}/{Hkv}")
    lens = [1, 31, 32, 33, 95, 128, 161, 255]
    c = synth.prefill_case(80, lens, lens, Hq, Hkv, 64, torch.bfloat16, True)
    T = c.q.shape[0]
    out = torch.full((T, Hq, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, Hq), float("nan"), dtype=torch.float32, device="cuda")
    pkv.varlen_prefill(dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q,
                       c.max_seqlen_k, c.sm_scale, c.Hkv, k=dev(c.k), v=dev(c.v), sink=dev(c.sink),
                       window_left=c.window_left, lse=lse, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
    o, l = oracle_prefill(c)
    assert_close(out, o, torch.bfloat16, "out")
    assert_close(lse, l, torch.bfloat16, "lse", lse=True)


def test_prefill_deterministic():
    banner("prefill determinism")
    c = synth.prefill_case(70, [300, 1000], [300, 1000], 32, 8, 128, torch.bfloat16, True)
    o1, l1 = run_prefill(c)
    o2, l2 = run_prefill(c)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_config3_full_size():
    """bf16 varlen causal prefill at full size, in the launch configuration the
    benchmark times: 8 requests of 256..4096 tokens, 32/8 heads, D 128, sink;
    every output element and every lse compared with the oracle (all host
    cores), the output poisoned with NaN first so an unwritten row shows."""
    banner("config3 full size")
    c = synth.config3_prefill()
    check_prefill_case(c)
    T = c.q.shape[0]
    out = torch.full((T, c.Hq, c.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
    from paged_kv_cache_02_amd import pkv
    pkv.varlen_prefill(dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q,
                       c.max_seqlen_k, c.sm_scale, c.Hkv, k=dev(c.k), v=dev(c.v),
                       sink=dev(c.sink), lse=lse, out=out)
    torch.cuda.synchronize()
    o, l = oracle_prefill(c)
    assert_close(out, o, torch.bfloat16, "config3 out")
    assert_close(lse, l, torch.bfloat16, "config3 lse", lse=True)


def test_config4_full_size():
    """bf16 chunked prefill at full size: 4 x (512 queries after 8192 cached
    keys), paged bs 16, window 128, 64/8 heads, D 64, sink; every element
    against the oracle, output poisoned with NaN first."""
    banner("config4 full size")
    c = synth.config4_chunked()
    check_prefill_case(c)
    T = c.q.shape[0]
    from paged_kv_cache_02_amd import pkv
    out = torch.full((T, c.Hq, c.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
    pkv.varlen_prefill(dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q,
                       c.max_seqlen_k, c.sm_scale, c.Hkv, k_cache=dev(c.k_cache),
                       v_cache=dev(c.v_cache), block_table=dev(c.block_table), sink=dev(c.sink),
                       window_left=c.window_left, lse=lse, out=out)
    torch.cuda.synchronize()
    o, l = oracle_prefill(c)
    assert_close(out, o, torch.bfloat16, "config4 out")
    assert_close(lse, l, torch.bfloat16, "config4 lse", lse=True)
