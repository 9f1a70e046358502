"""Decode with the new token appended in the same call (pkv_paged_decode_append)
on the GPU against the fp64 oracle: outputs, and the caches bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, banner, dev
from paged_kv_cache_02_amd import validate

pytestmark = pytest.mark.gpu


def make_case(seed, lens, Hq, Hkv, D, bs, dtype, sink, window=-1):
    """A paged pool with room for L + 1 tokens per sequence; the slot of
    position L (where the new token goes) is set to NaN, so a read of the
    old row instead of the appended one cannot go unnoticed."""
    c = synth.decode_case(seed, [L + 1 for L in lens], Hq, Hkv, D, bs, dtype, sink,
                          window_left=window)
    L = torch.tensor(lens, dtype=torch.int32)
    for b, Lb in enumerate(lens):
        blk, off = int(c.block_table[b, Lb // bs]), Lb % bs
        c.k_cache[blk, off] = float("nan")
        c.v_cache[blk, off] = float("nan")
    kn = synth.to_dtype(synth.normal(seed, (len(lens), Hkv, D), stream=11), dtype)
    vn = synth.to_dtype(synth.normal(seed, (len(lens), Hkv, D), stream=12), dtype)
    return c, L, kn, vn


def run_append(c, L, kn, vn, workspace=None):
    from paged_kv_cache_02_amd import pkv
    validate.check_decode(c.block_table, L, c.num_blocks, c.block_size, int(L.max()), append=True)
    kc, vc = dev(c.k_cache), dev(c.v_cache)
    # outputs poisoned with NaN: a row the call does not write shows up
    lse = torch.full((c.q.shape[0], c.q.shape[1]), float("nan"), dtype=torch.float32,
                     device="cuda")
    out = torch.full_like(dev(c.q), float("nan"))
    pkv.paged_decode_append(dev(c.q), dev(kn), dev(vn), kc, vc, dev(c.block_table), dev(L),
                            c.sm_scale, sink=dev(c.sink), window_left=c.window_left,
                            max_seqlen_k=int(L.max()), lse=lse, workspace=workspace, out=out)
    torch.cuda.synchronize()
    return out, lse, kc, vc


def check(c, L, kn, vn, out, lse, kc, vc, dtype, units=None):
    o, l, okc, ovc = oracle.decode_append(c.q, kn, vn, c.k_cache, c.v_cache, c.block_table, L,
                                          c.sink, c.sm_scale, c.window_left, units=units)
    if units is None:
        assert_close(out, o, dtype, "append out")
        assert_close(lse, l, dtype, "append lse", lse=True)
    else:
        b, h = np.asarray(units) // c.q.shape[1], np.asarray(units) % c.q.shape[1]
        assert_close(out.float().cpu()[b, h], o[b, h], dtype, "append out (sampled)")
        assert_close(lse.cpu()[b, h], l[b, h], dtype, "append lse (sampled)", lse=True)
    # the caches: the new rows at their slots, every other byte unchanged
    # (NaN == NaN bitwise: compare the raw bits)
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(kc.cpu().view(bits), okc.view(bits)), "k_cache"
    assert torch.equal(vc.cpu().view(bits), ovc.view(bits)), "v_cache"


CASES = [
    # lengths already cached, Hq, Hkv, D, block size, sink, window
    ([0, 1, 15, 16, 17, 31, 32, 33, 100, 257], 8, 2, 128, 16, True, -1),
    ([5, 64, 300, 1000], 32, 8, 128, 16, True, 127),
    ([40, 0, 63, 64], 16, 16, 64, 32, False, -1),
    ([77, 200, 15], 16, 2, 128, 64, True, 0),          # window 0: only the new token
    ([1000, 3, 48], 64, 8, 128, 16, True, -1),          # G 8: two head groups per kv head
    ([129, 7], 12, 4, 64, 16, True, 20),                # G 3
    ([0, 7, 8, 15, 16, 100], 8, 2, 128, 8, True, -1),   # block size 8: tiles over two blocks
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_append_vs_oracle(case, dtype):
    lens, Hq, Hkv, D, bs, sink, window = case
    banner(f"decode append {dtype} {case}")
    c, L, kn, vn = make_case(300 + len(lens), lens, Hq, Hkv, D, bs, dtype, sink, window)
    out, lse, kc, vc = run_append(c, L, kn, vn)
    check(c, L, kn, vn, out, lse, kc, vc, dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_page_example_fused_append(dtype):
    """The page's decode example (lengths 30 / 32 / 70, block size 32, the
    doc's block table): the new tokens land at slots 94, 32 and 198."""
    banner(f"page example fused append {dtype}")
    c = synth.config1_decode()
    c.q, c.k_cache, c.v_cache = (t.to(dtype) for t in (c.q, c.k_cache, c.v_cache))
    L = c.cache_seqlens.clone()
    kn = synth.to_dtype(synth.normal(8, (3, c.Hkv, c.D), stream=11), dtype)
    vn = synth.to_dtype(synth.normal(8, (3, c.Hkv, c.D), stream=12), dtype)
    out, lse, kc, vc = run_append(c, L, kn, vn)
    flat_k, flat_v = kc.cpu().view(-1, c.Hkv, c.D), vc.cpu().view(-1, c.Hkv, c.D)
    for b, slot in enumerate([94, 32, 198]):
        assert torch.equal(flat_k[slot], kn[b]) and torch.equal(flat_v[slot], vn[b])
    check(c, L, kn, vn, out, lse, kc, vc, dtype)


def test_append_many_short_sequences():
    """Hundreds of short sequences: a wave's range holds the last tiles of
    many sequences, so the owning wave stores many new rows."""
    banner("append many short sequences")
    lens = np.random.default_rng(62).integers(0, 40, size=300).tolist()
    c, L, kn, vn = make_case(310, lens, 32, 8, 128, 16, torch.bfloat16, True)
    out, lse, kc, vc = run_append(c, L, kn, vn)
    check(c, L, kn, vn, out, lse, kc, vc, torch.bfloat16)


def test_append_workspace_reuse():
    """Two appends in a row with one workspace, then a plain decode with the
    same workspace: the arrival counters are left zero by each call."""
    from paged_kv_cache_02_amd import pkv
    banner("append workspace reuse")
    c, L, kn, vn = make_case(311, [100, 333, 2000, 1], 32, 8, 128, 16, torch.bfloat16, True)
    nb = pkv.decode_workspace_bytes(4, 32, 128, int(L.max()) + 1)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    out1, lse1, kc, vc = run_append(c, L, kn, vn, workspace=ws)
    out2, lse2, _, _ = run_append(c, L, kn, vn, workspace=ws)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    check(c, L, kn, vn, out1, lse1, kc, vc, torch.bfloat16)
    # the same caches, now holding the new tokens, decoded over L + 1 keys
    out3 = pkv.paged_decode(dev(c.q), kc, vc, dev(c.block_table), dev(L + 1), c.sm_scale,
                            sink=dev(c.sink), max_seqlen_k=int(L.max()) + 1, workspace=ws)
    torch.cuda.synchronize()
    assert_close(out3, oracle.decode_append(c.q, kn, vn, c.k_cache, c.v_cache, c.block_table, L,
                                            c.sink, c.sm_scale)[0], torch.bfloat16, "decode after")


def test_append_config2_full_size():
    """The headline decode shape (64 sequences of 512..4096 cached tokens,
    32/8 heads, D 128, block size 16, sink) with the new token appended;
    every output element and lse against the oracle, and the caches
    compared in full on the GPU."""
    banner("append config2 full size")
    c2 = synth.config2_decode()
    lens = (c2.cache_seqlens - 1).tolist()          # the last cached token becomes the new one
    c, L, kn, vn = make_case(312, lens, c2.Hq, c2.Hkv, c2.D, c2.block_size, torch.bfloat16, True)
    kc0, vc0 = dev(c.k_cache).clone(), dev(c.v_cache).clone()
    out, lse, kc, vc = run_append(c, L, kn, vn)
    o, l, _, _ = oracle.decode_append(c.q, kn, vn, c.k_cache, c.v_cache, c.block_table, L,
                                      c.sink, c.sm_scale)
    assert_close(out, o, torch.bfloat16, "config2 append out")
    assert_close(lse, l, torch.bfloat16, "config2 append lse", lse=True)
    bs = c.block_size
    slots = torch.tensor([int(c.block_table[i, Lb // bs]) * bs + Lb % bs
                          for i, Lb in enumerate(lens)], device="cuda")
    for got, before, new in ((kc, kc0, kn), (vc, vc0, vn)):
        want = before.view(-1, c.Hkv, c.D).clone()
        want[slots] = dev(new)
        assert torch.equal(got.view(-1, c.Hkv, c.D).view(torch.int16), want.view(torch.int16))


ROPE = [
    # lengths already cached, Hq, Hkv, D, block size, window, rotary_dim, neox
    ([0, 1, 15, 16, 17, 31, 32, 33, 100, 257], 8, 2, 128, 16, -1, 128, True),
    ([5, 64, 300, 1000], 32, 8, 128, 16, 127, 64, False),
    ([40, 0, 63, 64], 16, 16, 64, 32, -1, 32, True),
    ([77, 200, 15], 12, 4, 128, 64, 20, 96, True),      # G 3, a quarter of the dims pass through
]


@pytest.mark.parametrize("case", ROPE, ids=[str(i) for i in range(len(ROPE))])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_append_rope(case, dtype):
    """q and k_new rotated by the new token's position inside the append
    call (vLLM page, PagedAttentionWithRoPE.forward: rotate, then attend).
    The oracle rotates with its own table, rounds to the storage type as
    the kernel does, and runs its decode_append; q itself is unchanged, the
    cache receives the rotated key, and every other cache byte is unchanged."""
    from paged_kv_cache_02_amd import pkv
    lens, Hq, Hkv, D, bs, window, rd, neox = case
    banner(f"append rope {dtype} {case}")
    c, L, kn, vn = make_case(330 + len(lens), lens, Hq, Hkv, D, bs, dtype, True, window)
    n_pos = int(L.max()) + 1
    tab = pkv.rope_cos_sin(n_pos, rd, 10000.0)
    otab = oracle.rope_cos_sin(n_pos, rd, 10000.0)      # the oracle's own table
    validate.check_decode(c.block_table, L, c.num_blocks, c.block_size, int(L.max()), append=True)
    q, kc, vc = dev(c.q), dev(c.k_cache), dev(c.v_cache)
    q0 = q.clone()
    lse = torch.empty((c.q.shape[0], Hq), dtype=torch.float32, device="cuda")
    out = pkv.paged_decode_append(q, dev(kn), dev(vn), kc, vc, dev(c.block_table), dev(L),
                                  c.sm_scale, sink=dev(c.sink), window_left=window,
                                  max_seqlen_k=int(L.max()), lse=lse, rope_cos_sin=tab,
                                  rotary_dim=rd, rope_neox=neox)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(q.view(bits), q0.view(bits)), "q modified"
    pos = L.numpy().astype(np.int32)
    qr = synth.to_dtype(oracle.rope_apply(c.q, pos, otab, rd, neox).astype(np.float32), dtype)
    kr = synth.to_dtype(oracle.rope_apply(kn, pos, otab, rd, neox).astype(np.float32), dtype)
    o, l, okc, ovc = oracle.decode_append(qr, kr, vn, c.k_cache, c.v_cache, c.block_table, L,
                                          c.sink, c.sm_scale, window)
    assert_close(out, o, dtype, "append rope out")
    assert_close(lse, l, dtype, "append rope lse", lse=True)
    assert torch.equal(vc.cpu().view(bits), ovc.view(bits)), "v_cache"
    # the rotated keys at the new slots (the kernel rotates in float32, the
    # oracle in float64: one unit in the last place apart at most), every
    # other slot bit for bit
    slots = [int(c.block_table[b, Lb // bs]) * bs + Lb % bs for b, Lb in enumerate(lens)]
    got = kc.cpu().view(-1, Hkv, D)
    want = okc.view(-1, Hkv, D)
    rest = np.setdiff1d(np.arange(got.shape[0]), slots)
    assert torch.equal(got[rest].view(bits), want[rest].view(bits)), "k_cache outside the new slots"
    g, w = got[slots].double(), want[slots].double()
    rtol = 2.0 ** -7 if dtype == torch.bfloat16 else 1e-6
    assert ((g - w).abs() <= 1e-6 + rtol * w.abs()).all(), float((g - w).abs().max())
