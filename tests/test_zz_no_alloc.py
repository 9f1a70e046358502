"""pkv_paged_decode_noalloc (the decode entry point that allocates nothing,
its workspace a static device array) against pkv_paged_decode with a
caller-allocated workspace: the same outputs on two calls in a row, the
second with a smaller batch, in the balanced schedule (two launches, and one
launch with the merge fused, which counts pieces in the static array) and
with fixed partitions; and both against the oracle."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_close, banner, check_decode_case, dev, oracle_decode

pytestmark = pytest.mark.gpu


def _noalloc(c, P, out, lse):
    """Call the entry point through the C ABI directly."""
    from paged_kv_cache_02_amd import pkv
    st = pkv.lib.pkv_paged_decode_noalloc(
        out.data_ptr(), lse.data_ptr(), c.q_d.data_ptr(), c.kc_d.data_ptr(), c.vc_d.data_ptr(),
        c.bt_d.data_ptr(), c.sl_d.data_ptr(), None if c.sink is None else c.sink_d.data_ptr(),
        c.B, c.Hq, c.Hkv, c.D, c.block_size, c.num_blocks, c.max_blocks_per_seq, c.max_seqlen_k,
        ctypes.c_float(c.sm_scale), c.window_left, None, P, pkv.PKV_BF16,
        torch.cuda.current_stream().cuda_stream)
    return st


def _with_workspace(c, P):
    from paged_kv_cache_02_amd import pkv
    out = torch.full((c.B, c.Hq, c.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((c.B, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(pkv.decode_workspace_bytes(c.B, c.Hq, c.D, c.max_seqlen_k, P), 256),
                     dtype=torch.uint8, device="cuda")
    pkv.paged_decode(c.q_d, c.kc_d, c.vc_d, c.bt_d, c.sl_d, c.sm_scale, sink=c.sink_d,
                     window_left=c.window_left, partition_size=P, max_seqlen_k=c.max_seqlen_k,
                     out=out, lse=lse, workspace=ws)
    return out, lse


@pytest.mark.parametrize("P", [0, -1, 256])
def test_noalloc_matches_workspace_entry(P):
    from paged_kv_cache_02_amd import pkv
    big = synth.decode_case(91, np.random.default_rng(91).integers(1, 3000, 48).tolist(), 32, 8,
                            128, 16, torch.bfloat16, with_sink=True, poison=True)
    small = synth.decode_case(92, [0, 5, 700, 33, 1290], 32, 8, 128, 16, torch.bfloat16,
                              with_sink=True, window_left=400, poison=True)
    for step, c in enumerate((big, small)):
        banner(f"noalloc P={P} call {step}: B={c.B}")
        check_decode_case(c)
        c.q_d, c.kc_d, c.vc_d = dev(c.q), dev(c.k_cache), dev(c.v_cache)
        c.bt_d, c.sl_d, c.sink_d = dev(c.block_table), dev(c.cache_seqlens), dev(c.sink)
        out = torch.full((c.B, c.Hq, c.D), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((c.B, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
        st = _noalloc(c, P, out, lse)
        assert st == pkv.PKV_OK, pkv.lib.pkv_status_string(st)
        ref_out, ref_lse = _with_workspace(c, P)
        torch.cuda.synchronize()
        # same kernels, same schedule: the same bits as the workspace entry point
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "out differs"
        assert torch.equal(lse, ref_lse), "lse differs"
        o, l = oracle_decode(c)
        assert_close(out, o, torch.bfloat16, f"noalloc call {step} out")
        assert_close(lse, l, torch.bfloat16, f"noalloc call {step} lse", lse=True)
