"""Rotary position embedding on the GPU against the fp64 oracle: the table, the
in-place rotation, the rotated cache store and q rotated inside prefill."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, banner, dev

pytestmark = pytest.mark.gpu

TABLES = [
    # num_positions, rotary_dim, base, scaling, factor, max_position
    (512, 128, 10000.0, 0, 1.0, 0),
    (300, 64, 500000.0, 1, 4.0, 0),
    (4096, 128, 10000.0, 2, 2.0, 1024),
    (64, 32, 10000.0, 2, 2.0, 1024),            # dynamic, table within max_position
]


@pytest.mark.parametrize("case", TABLES, ids=[str(i) for i in range(len(TABLES))])
def test_rope_table(case):
    from paged_kv_cache_02_amd import pkv
    n, rd, base, scaling, factor, maxp = case
    banner(f"rope table {case}")
    t = pkv.rope_cos_sin(n, rd, base, scaling, factor, maxp)
    torch.cuda.synchronize()
    want = oracle.rope_cos_sin(n, rd, base, scaling, factor, maxp)
    got = t.cpu().double().numpy()
    assert np.abs(got - want).max() <= 2e-7, np.abs(got - want).max()


APPLY = [
    # T, H, D, rotary_dim, neox
    (37, 8, 128, 128, True),
    (37, 8, 128, 64, False),
    (50, 4, 64, 32, True),
    (50, 4, 64, 64, False),
]


@pytest.mark.parametrize("case", APPLY, ids=[str(i) for i in range(len(APPLY))])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rope_apply(case, dtype):
    """Rows of a fused QKV-style buffer (strided tokens) rotated in place;
    the columns past each row's head block are untouched."""
    from paged_kv_cache_02_amd import pkv
    T, H, D, rd, neox = case
    banner(f"rope apply {dtype} {case}")
    buf = synth.to_dtype(synth.normal(500, (T, 3 * H, D), stream=1), dtype).cuda()
    x = buf[:, H:2 * H]                            # the middle third: strided rows
    before = buf.clone()
    pos = torch.from_numpy(np.random.default_rng(5).integers(0, 512, size=T).astype(np.int32))
    tab = pkv.rope_cos_sin(512, rd, 10000.0)
    pkv.rope_apply(x, pos.cuda(), tab, rd, neox)
    torch.cuda.synchronize()
    want = oracle.rope_apply(before[:, H:2 * H].cpu(), pos, oracle.rope_cos_sin(512, rd, 10000.0),
                             rd, neox)
    assert_close(x, want, dtype, "rope apply")
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(buf[:, :H].view(bits), before[:, :H].view(bits))
    assert torch.equal(buf[:, 2 * H:].view(bits), before[:, 2 * H:].view(bits))
    assert torch.equal(x[..., rd:].contiguous().view(bits),
                       before[:, H:2 * H, rd:].contiguous().view(bits))


@pytest.mark.parametrize("neox", [True, False])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_reshape_and_cache_rope(neox, dtype):
    """Keys rotated as they are stored, values stored unchanged, padding slots
    skipped, every other slot untouched."""
    from paged_kv_cache_02_amd import pkv
    banner(f"reshape_and_cache_rope {dtype} neox={neox}")
    T, Hkv, D, bs, NB, rd = 41, 4, 128, 16, 8, 64
    key = synth.to_dtype(synth.normal(501, (T, Hkv, D), stream=1), dtype)
    val = synth.to_dtype(synth.normal(501, (T, Hkv, D), stream=2), dtype)
    slots = np.random.default_rng(6).permutation(NB * bs)[:T].astype(np.int32)
    slots[[3, 17]] = -1
    pos = np.random.default_rng(7).integers(0, 1000, size=T).astype(np.int32)
    kc = torch.full((NB, bs, Hkv, D), -3.0, dtype=dtype)
    vc = torch.full((NB, bs, Hkv, D), -5.0, dtype=dtype)
    tab = pkv.rope_cos_sin(1000, rd, 10000.0)
    gk, gv = kc.cuda(), vc.cuda()
    pkv.reshape_and_cache_rope(key.cuda(), val.cuda(), gk, gv, torch.from_numpy(slots).cuda(),
                               torch.from_numpy(pos).cuda(), tab, rd, neox)
    torch.cuda.synchronize()
    krot = oracle.rope_apply(key, pos, oracle.rope_cos_sin(1000, rd, 10000.0), rd, neox)
    fk, fv = gk.cpu().view(-1, Hkv, D), gv.cpu().view(-1, Hkv, D)
    live = slots >= 0
    assert_close(fk[slots[live]], krot[live], dtype, "rotated keys")
    assert torch.equal(fv[slots[live]], val[torch.from_numpy(live)])
    untouched = np.setdiff1d(np.arange(NB * bs), slots[live])
    assert (fk[untouched] == -3.0).all() and (fv[untouched] == -5.0).all()


PREFILL = [
    # q_lens, k_lens, Hq, Hkv, D, rotary_dim, neox, paged block size (0: contiguous)
    ([1, 100, 300], None, 32, 8, 128, 128, True, 0),
    ([64, 257], None, 8, 2, 64, 32, False, 0),
    ([33, 200], [500, 200], 12, 4, 128, 64, True, 0),
    ([90, 7], [300, 64], 16, 2, 128, 96, True, 16),
    ([129, 40], [129, 300], 8, 8, 64, 64, False, 32),
]


@pytest.mark.parametrize("case", PREFILL, ids=[str(i) for i in range(len(PREFILL))])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_rope(case, dtype):
    """q rotated by its position (Lk - Lq + i) inside the prefill; the keys
    are rotated beforehand (by the oracle for contiguous K, by
    reshape_and_cache_rope for the paged pool)."""
    from paged_kv_cache_02_amd import pkv
    q_lens, k_lens, Hq, Hkv, D, rd, neox, bs = case
    banner(f"prefill rope {dtype} {case}")
    k_lens = k_lens or q_lens
    c = synth.prefill_case(510 + len(q_lens), q_lens, k_lens, Hq, Hkv, D, dtype, True)
    n_pos = max(k_lens)
    tab = pkv.rope_cos_sin(n_pos, rd, 10000.0)
    otab = oracle.rope_cos_sin(n_pos, rd, 10000.0)      # the oracle's own table
    kpos = np.concatenate([np.arange(L) for L in k_lens]).astype(np.int32)
    krot = synth.to_dtype(oracle.rope_apply(c.k, kpos, otab, rd, neox).astype(np.float32),
                          dtype)
    kw = dict(k=dev(krot), v=dev(c.v))
    if bs:
        rng = np.random.default_rng(8)
        bt, nb = synth.pool_from_lengths(rng, k_lens, bs)
        slots = torch.cat([synth.slots_for_tokens(bt[r:r + 1].expand(L, -1).contiguous(),
                                                  list(range(L)), bs)
                           for r, L in enumerate(k_lens)]).cuda()
        kc = torch.zeros((nb, bs, Hkv, D), dtype=dtype, device="cuda")
        vc = torch.zeros_like(kc)
        pkv.reshape_and_cache_rope(dev(c.k), dev(c.v), kc, vc, slots,
                                   torch.from_numpy(kpos).cuda(), tab, rd, neox)
        kw = dict(k_cache=kc, v_cache=vc, block_table=bt.cuda())
    T = c.q.shape[0]
    lse = torch.empty(T, Hq, dtype=torch.float32, device="cuda")
    out = pkv.varlen_prefill(dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q,
                             c.max_seqlen_k, c.sm_scale, Hkv, sink=dev(c.sink), lse=lse,
                             rope_cos_sin=tab, rotary_dim=rd, rope_neox=neox, **kw)
    torch.cuda.synchronize()
    qpos = oracle.query_positions(c.cu_seqlens_q, c.cu_seqlens_k)
    qrot = torch.from_numpy(oracle.rope_apply(c.q, qpos, otab, rd, neox)).float()
    o, l = oracle.varlen_prefill(qrot, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, c.sm_scale, Hkv,
                                 k=krot.float(), v=c.v.float())
    assert_close(out, o, dtype, "prefill rope out")
    assert_close(lse, l, dtype, "prefill rope lse", lse=True)


@pytest.mark.parametrize("case", [
    ([33, 200], [500, 200], 12, 4, 128, 64, True),
    ([100, 5], [40, 5], 8, 2, 64, 64, False),         # rows 0..59 of request 0 at p < 0
], ids=["chunk", "lq_gt_lk"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_rope_noncausal(case, dtype):
    """q rotated inside a non-causal prefill.  Rows at a negative position
    (more queries than keys) have no table row: they are not rotated, and
    (non-causal) still see every key."""
    from paged_kv_cache_02_amd import pkv
    q_lens, k_lens, Hq, Hkv, D, rd, neox = case
    banner(f"prefill rope non-causal {dtype} {case}")
    c = synth.prefill_case(540 + len(q_lens), q_lens, k_lens, Hq, Hkv, D, dtype, True)
    n_pos = max(k_lens)
    tab = pkv.rope_cos_sin(n_pos, rd, 10000.0)
    otab = oracle.rope_cos_sin(n_pos, rd, 10000.0)
    kpos = np.concatenate([np.arange(L) for L in k_lens]).astype(np.int32)
    krot = synth.to_dtype(oracle.rope_apply(c.k, kpos, otab, rd, neox).astype(np.float32),
                          dtype)
    T = c.q.shape[0]
    lse = torch.empty(T, Hq, dtype=torch.float32, device="cuda")
    out = pkv.varlen_prefill(dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q,
                             c.max_seqlen_k, c.sm_scale, Hkv, k=dev(krot), v=dev(c.v),
                             sink=dev(c.sink), lse=lse, rope_cos_sin=tab, rotary_dim=rd,
                             rope_neox=neox, causal=False)
    torch.cuda.synchronize()
    qpos = oracle.query_positions(c.cu_seqlens_q, c.cu_seqlens_k)
    at = qpos >= 0
    qrot = c.q.double().numpy().copy()
    qrot[at] = oracle.rope_apply(c.q[torch.from_numpy(at)], qpos[at], otab, rd, neox)
    o, l = oracle.varlen_prefill(torch.from_numpy(qrot).float(), c.cu_seqlens_q, c.cu_seqlens_k,
                                 c.sink, c.sm_scale, Hkv, k=krot.float(), v=c.v.float(),
                                 causal=False)
    assert_close(out, o, dtype, "prefill rope non-causal out")
    assert_close(lse, l, dtype, "prefill rope non-causal lse", lse=True)


ROPE_K = [
    # q_lens, k_lens, Hq, Hkv, D, rotary_dim, neox, window, causal
    ([1, 100, 300], None, 32, 8, 128, 128, True, -1, True),
    ([64, 257], None, 8, 2, 64, 32, False, -1, True),
    ([33, 200], [500, 200], 12, 4, 128, 64, True, -1, True),     # chunks after cached keys
    ([300, 77, 513], None, 8, 2, 128, 128, True, 50, True),       # window: runs of blocks
    ([90, 7], [300, 64], 16, 4, 64, 64, True, -1, False),         # non-causal
    ([129, 1000], [129, 1000], 16, 2, 128, 96, False, -1, True),
]


# float32 rotates the keys in registers, with or without a workspace: one case
ROPE_K_PATHS = [("workspace", torch.bfloat16), ("in_kernel", torch.bfloat16),
                ("registers", torch.float32)]


@pytest.mark.parametrize("case", ROPE_K, ids=[str(i) for i in range(len(ROPE_K))])
@pytest.mark.parametrize("keys,dtype", ROPE_K_PATHS, ids=[k for k, _ in ROPE_K_PATHS])
def test_prefill_rope_k(case, keys, dtype):
    """rope_k: contiguous keys rotated by their positions, q by its own;
    bf16 rotates the keys once into a workspace (NaN-filled beforehand) or,
    without one, inside the attention kernel as it loads them; against the
    oracle fed q and k rotated with its own table (k rounded to the storage
    type, as the kernels round it)."""
    from paged_kv_cache_02_amd import pkv
    q_lens, k_lens, Hq, Hkv, D, rd, neox, window, causal = case
    banner(f"prefill rope_k {dtype} {keys} {case}")
    k_lens = k_lens or q_lens
    c = synth.prefill_case(560 + len(q_lens), q_lens, k_lens, Hq, Hkv, D, dtype, True,
                           window_left=window)
    n_pos = max(k_lens)
    tab = pkv.rope_cos_sin(n_pos, rd, 10000.0)
    otab = oracle.rope_cos_sin(n_pos, rd, 10000.0)
    k0 = dev(c.k)
    k_before = k0.clone()
    T = c.q.shape[0]
    lse = torch.empty(T, Hq, dtype=torch.float32, device="cuda")
    ws = False
    if keys != "in_kernel":
        need = pkv.varlen_prefill_workspace_bytes(len(q_lens), c.max_seqlen_k, Hkv, D, True, dtype)
        ws = torch.full((max(need, 1) // 2,), float("nan"), dtype=torch.bfloat16,
                        device="cuda").view(torch.uint8) if need else None
    out = pkv.varlen_prefill(dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q,
                             c.max_seqlen_k, c.sm_scale, Hkv, k=k0, v=dev(c.v), sink=dev(c.sink),
                             lse=lse, window_left=window, causal=causal, rope_cos_sin=tab,
                             rotary_dim=rd, rope_neox=neox, rope_k=True, workspace=ws)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(k0.view(bits), k_before.view(bits)), "k modified"
    kpos = np.concatenate([np.arange(L) for L in k_lens]).astype(np.int32)
    krot = synth.to_dtype(oracle.rope_apply(c.k, kpos, otab, rd, neox).astype(np.float32), dtype)
    qpos = oracle.query_positions(c.cu_seqlens_q, c.cu_seqlens_k)
    at = qpos >= 0
    qrot = c.q.double().numpy().copy()
    qrot[at] = oracle.rope_apply(c.q[torch.from_numpy(at)], qpos[at], otab, rd, neox)
    o, l = oracle.varlen_prefill(torch.from_numpy(qrot).float(), c.cu_seqlens_q, c.cu_seqlens_k,
                                 c.sink, c.sm_scale, Hkv, k=krot.float(), v=c.v.float(),
                                 window_left=window, causal=causal)
    assert_close(out, o, dtype, "prefill rope_k out")
    assert_close(lse, l, dtype, "prefill rope_k lse", lse=True)


def test_prefill_rejects_mixed_dtypes():
    """K or V of another dtype than q is refused before any launch (the
    kernels would read its bytes as q's type)."""
    from paged_kv_cache_02_amd import pkv
    banner("prefill mixed dtypes")
    c = synth.prefill_case(520, [40], [40], 8, 2, 64, torch.float32, True)
    args = (dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q, c.max_seqlen_k,
            c.sm_scale, c.Hkv)
    with pytest.raises(ValueError, match="dtype mismatch"):
        pkv.varlen_prefill(*args, k=dev(c.k).double(), v=dev(c.v))
    with pytest.raises(ValueError, match="dtype mismatch"):
        pkv.varlen_prefill(*args, k=dev(c.k), v=dev(c.v).bfloat16())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_with_rope(dtype):
    """A decode step with rotary embedding: the cached keys stored by
    reshape_and_cache_rope at positions 0 .. L-1, q rotated in place by
    rope_apply at its position L - 1, then paged_decode.  The oracle takes the
    rotated keys and q, each rounded to the storage type as the GPU stores
    them, scattered into a pool through the same slots."""
    from paged_kv_cache_02_amd import pkv
    banner(f"decode with rope {dtype}")
    lens, Hq, Hkv, D, bs, rd = [1, 40, 300], 16, 4, 128, 16, 128
    bt, nb = synth.pool_from_lengths(np.random.default_rng(9), lens, bs)
    T, B = sum(lens), len(lens)
    key = synth.to_dtype(synth.normal(530, (T, Hkv, D), stream=1), dtype)
    val = synth.to_dtype(synth.normal(530, (T, Hkv, D), stream=2), dtype)
    q = synth.to_dtype(synth.normal(530, (B, Hq, D), stream=3), dtype)
    sink = torch.from_numpy(synth.normal(530, (Hq,), stream=7).copy())
    kpos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    qpos = np.array([L - 1 for L in lens], dtype=np.int32)
    slots = torch.cat([synth.slots_for_tokens(bt[r:r + 1].expand(L, -1).contiguous(),
                                              list(range(L)), bs) for r, L in enumerate(lens)])
    tab = pkv.rope_cos_sin(max(lens), rd)
    kc = torch.zeros((nb, bs, Hkv, D), dtype=dtype, device="cuda")
    vc = torch.zeros_like(kc)
    pkv.reshape_and_cache_rope(key.cuda(), val.cuda(), kc, vc, slots.cuda(),
                               torch.from_numpy(kpos).cuda(), tab, rd)
    qg = q.cuda()
    pkv.rope_apply(qg, torch.from_numpy(qpos).cuda(), tab, rd)
    sl = torch.tensor(lens, dtype=torch.int32)
    sm = 1.0 / np.sqrt(D)
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
    out = pkv.paged_decode(qg, kc, vc, bt.cuda(), sl.cuda(), sm, sink=sink.cuda(), lse=lse)
    torch.cuda.synchronize()
    otab = oracle.rope_cos_sin(max(lens), rd, 10000.0)    # the oracle's own table
    krot = synth.to_dtype(oracle.rope_apply(key, kpos, otab, rd, True).astype(np.float32),
                          dtype).float()
    qrot = synth.to_dtype(oracle.rope_apply(q, qpos, otab, rd, True).astype(np.float32),
                          dtype).float()
    pk = torch.zeros((nb * bs, Hkv, D), dtype=torch.float32)
    pv = torch.zeros_like(pk)
    pk[slots.long()] = krot
    pv[slots.long()] = val.float()
    o, l = oracle.paged_decode(qrot, pk.view(nb, bs, Hkv, D), pv.view(nb, bs, Hkv, D), bt, sl,
                               sink, sm)
    assert_close(out, o, dtype, "decode rope out")
    assert_close(lse, l, dtype, "decode rope lse", lse=True)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_rope_window_alibi(dtype):
    """q rotated inside the prefill together with a sliding window and ALiBi
    slopes (GQA 4, D 128, one request whose queries start mid-sequence)."""
    from paged_kv_cache_02_amd import pkv
    banner(f"prefill rope + window + alibi {dtype}")
    q_lens, k_lens, Hq, Hkv, D, rd, window = [70, 200], [400, 200], 16, 4, 128, 64, 50
    c = synth.prefill_case(540, q_lens, k_lens, Hq, Hkv, D, dtype, True, window_left=window)
    al = torch.tensor([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=torch.float32)
    tab = pkv.rope_cos_sin(max(k_lens), rd)
    otab = oracle.rope_cos_sin(max(k_lens), rd, 10000.0)  # the oracle's own table
    kpos = np.concatenate([np.arange(L) for L in k_lens]).astype(np.int32)
    krot = synth.to_dtype(oracle.rope_apply(c.k, kpos, otab, rd, True).astype(np.float32),
                          dtype)
    lse = torch.empty(c.q.shape[0], Hq, dtype=torch.float32, device="cuda")
    out = pkv.varlen_prefill(dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q,
                             c.max_seqlen_k, c.sm_scale, Hkv, k=dev(krot), v=dev(c.v),
                             sink=dev(c.sink), window_left=window, lse=lse, alibi_slopes=dev(al),
                             rope_cos_sin=tab, rotary_dim=rd)
    torch.cuda.synchronize()
    qpos = oracle.query_positions(c.cu_seqlens_q, c.cu_seqlens_k)
    qrot = torch.from_numpy(oracle.rope_apply(c.q, qpos, otab, rd, True)).float()
    o, l = oracle.varlen_prefill(qrot, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, c.sm_scale, Hkv,
                                 k=krot.float(), v=c.v.float(), window_left=window, alibi=al)
    assert_close(out, o, dtype, "prefill rope window alibi out")
    assert_close(lse, l, dtype, "prefill rope window alibi lse", lse=True)


def test_prefill_rope_k_alibi_workspace():
    """rope_k with ALiBi slopes and a window (bf16): the keys rotated once
    into the workspace, then the ALiBi kernel; without a workspace the call
    is refused (no in-kernel rotation variant carries ALiBi)."""
    from paged_kv_cache_02_amd import pkv
    banner("prefill rope_k + alibi + window, workspace")
    dtype = torch.bfloat16
    q_lens, k_lens, Hq, Hkv, D, rd, window = [70, 200], [400, 200], 16, 4, 128, 64, 50
    c = synth.prefill_case(541, q_lens, k_lens, Hq, Hkv, D, dtype, True, window_left=window)
    al = torch.tensor([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=torch.float32)
    tab = pkv.rope_cos_sin(max(k_lens), rd)
    otab = oracle.rope_cos_sin(max(k_lens), rd, 10000.0)
    kpos = np.concatenate([np.arange(L) for L in k_lens]).astype(np.int32)
    krot = synth.to_dtype(oracle.rope_apply(c.k, kpos, otab, rd, True).astype(np.float32), dtype)
    lse = torch.empty(c.q.shape[0], Hq, dtype=torch.float32, device="cuda")
    args = (dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q, c.max_seqlen_k,
            c.sm_scale, Hkv)
    kw = dict(k=dev(c.k), v=dev(c.v), sink=dev(c.sink), window_left=window, lse=lse,
              alibi_slopes=dev(al), rope_cos_sin=tab, rotary_dim=rd, rope_k=True)
    out = pkv.varlen_prefill(*args, **kw)
    torch.cuda.synchronize()
    qpos = oracle.query_positions(c.cu_seqlens_q, c.cu_seqlens_k)
    qrot = torch.from_numpy(oracle.rope_apply(c.q, qpos, otab, rd, True)).float()
    o, l = oracle.varlen_prefill(qrot, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, c.sm_scale, Hkv,
                                 k=krot.float(), v=c.v.float(), window_left=window, alibi=al)
    assert_close(out, o, dtype, "prefill rope_k alibi out")
    assert_close(lse, l, dtype, "prefill rope_k alibi lse", lse=True)
    with pytest.raises(pkv.PkvError):
        pkv.varlen_prefill(*args, **kw, workspace=False)


def test_config3_rope_full_size():
    """The 8-request prefill workload (256..4096 tokens, 32/8 heads, D 128,
    sink) as the benchmark times it with RoPE (rotary_dim 128, neox): q
    rotated inside the prefill over contiguous keys that the oracle rotated
    with its own table, every output element and lse against the oracle;
    the same with the unrotated keys rotated inside the same launch;
    and every key stored by reshape_and_cache_rope into a block-16 pool,
    compared in full with the oracle's rotation (values bitwise)."""
    from paged_kv_cache_02_amd import pkv
    banner("config3 rope full size")
    c = synth.config3_prefill()
    rd = 128
    tab = pkv.rope_cos_sin(max(c.k_lens), rd)
    tab_cpu = oracle.rope_cos_sin(max(c.k_lens), rd, 10000.0)   # the oracle's own table
    kpos = np.concatenate([np.arange(L) for L in c.k_lens]).astype(np.int32)
    krot = synth.to_dtype(oracle.rope_apply(c.k, kpos, tab_cpu, rd, True).astype(np.float32),
                          torch.bfloat16)
    T = c.q.shape[0]
    lse = torch.full((T, c.Hq), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((T, c.Hq, c.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    pkv.varlen_prefill(dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q,
                       c.max_seqlen_k, c.sm_scale, c.Hkv, k=dev(krot), v=dev(c.v),
                       sink=dev(c.sink), lse=lse, out=out, rope_cos_sin=tab, rotary_dim=rd)
    bt, nb = synth.pool_from_lengths(np.random.default_rng(7), c.k_lens, 16)
    slots = torch.cat([synth.slots_for_tokens(bt[r:r + 1].expand(L, -1).contiguous(),
                                              list(range(L)), 16)
                       for r, L in enumerate(c.k_lens)]).cuda()
    kc = torch.zeros((nb, 16, c.Hkv, c.D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    pkv.reshape_and_cache_rope(dev(c.k), dev(c.v), kc, vc, slots, torch.from_numpy(kpos).cuda(),
                               tab, rd)
    torch.cuda.synchronize()
    qpos = oracle.query_positions(c.cu_seqlens_q, c.cu_seqlens_k)
    qrot = torch.from_numpy(oracle.rope_apply(c.q, qpos, tab_cpu, rd, True).astype(np.float32))
    o, l = oracle.varlen_prefill(qrot, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, c.sm_scale, c.Hkv,
                                 k=krot.float(), v=c.v.float())
    assert_close(out, o, torch.bfloat16, "config3 rope out")
    assert_close(lse, l, torch.bfloat16, "config3 rope lse", lse=True)
    # the unrotated keys rotated in the same call: once into a workspace, or
    # inside the attention kernel as it loads them
    for ws in (None, False):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        pkv.varlen_prefill(dev(c.q), dev(c.cu_seqlens_q), dev(c.cu_seqlens_k), c.max_seqlen_q,
                           c.max_seqlen_k, c.sm_scale, c.Hkv, k=dev(c.k), v=dev(c.v),
                           sink=dev(c.sink), lse=lse, out=out, rope_cos_sin=tab, rotary_dim=rd,
                           rope_k=True, workspace=ws)
        torch.cuda.synchronize()
        assert_close(out, o, torch.bfloat16, f"config3 rope_k out (workspace {ws})")
        assert_close(lse, l, torch.bfloat16, f"config3 rope_k lse (workspace {ws})", lse=True)
    s = slots.long()
    assert_close(kc.view(-1, c.Hkv, c.D)[s], krot.float().numpy(), torch.bfloat16,
                 "config3 rotated keys")
    assert torch.equal(vc.view(-1, c.Hkv, c.D)[s].cpu().view(torch.int16), c.v.view(torch.int16))
