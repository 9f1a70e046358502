"""Pins that hold the fp64 oracle to facts other than itself.

Each ``pin_*`` function raises ``AssertionError`` when the oracle disagrees
with a value printed on the pages, a hand-derived closed form, a library
routine (torch's CPU scaled-dot-product attention in float64), an invariant of
the definition, or a brute-force mask-matrix evaluation.  ``test_oracle_pins``
runs them against the real oracle; ``test_oracle_mutations`` runs them against
copies of the oracle with planted mistakes and requires each mistake to be
caught.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, atol=1e-10, rtol=1e-10, what=""):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    ok = np.isclose(a, b, atol=atol, rtol=rtol, equal_nan=False) | ((a == b) & np.isinf(a))
    assert ok.all(), f"{what}: max err {np.nanmax(np.abs(a - b))}"


# ---------------------------------------------------------------------------
# The pages' worked examples (bit-exact indexing)
# ---------------------------------------------------------------------------

def pin_varlen_map():
    """Transformers 'Paged attention' doc, Varlen path example."""
    g = _golden("varlen_map.json")
    cq = synth.cu_from_lengths(g["q_lens"]).tolist()
    ck = synth.cu_from_lengths(g["k_lens"]).tolist()
    assert cq == g["cu_seq_lens_q"] and ck == g["cu_seq_lens_k"]
    assert max(g["q_lens"]) == g["max_length_q"] and max(g["k_lens"]) == g["max_length_k"]
    assert cq[-1] == g["q_shape_tokens"] and ck[-1] == g["k_shape_tokens"]
    assert oracle.token_request(cq).tolist() == g["q_request_index"]
    assert oracle.token_request(ck).tolist() == g["k_request_index"]


def pin_query_positions():
    """Query positions on the Transformers doc's varlen example (lengths
    [10,3,1] over [0,1,7]) under the FlashInfer varlen branch's alignment
    (queries are the last qo_len positions), from a hand-written fixture; and
    the prefill oracle's mask agrees with them: with q = 0 every visible key
    gets the same weight, and with V(j) = j in dimension 0 each row's output
    is the mean of 0..p, i.e. p / 2 (0 for a row that sees no key)."""
    g = _golden("varlen_positions.json")
    cq = synth.cu_from_lengths(g["q_lens"])
    ck = synth.cu_from_lengths(g["k_lens"])
    assert oracle.query_positions(cq, ck).tolist() == g["query_positions"]
    D = 4
    q = torch.zeros((int(cq[-1]), 2, D))
    kv = torch.zeros((int(ck[-1]), 1, D))
    v = torch.zeros((int(ck[-1]), 1, D))
    for r, Lk in enumerate(g["k_lens"]):
        v[int(ck[r]):int(ck[r]) + Lk, 0, 0] = torch.arange(Lk, dtype=torch.float32)
        v[int(ck[r]):int(ck[r]) + Lk, 0, 1] = 1.0
    o, _ = oracle.varlen_prefill(q, cq, ck, None, 1.0, 1, k=kv, v=v)
    pos = np.array(g["query_positions"])
    seen = np.array(g["visible_keys_causal"])
    for h in range(2):
        _close(o[:, h, 1], (seen > 0).astype(float), 0, 1e-15, "rows that see a key")
        _close(o[:, h, 0], np.where(seen > 0, pos / 2.0, 0.0), 0, 1e-14, "mean key index")


def pin_decode_block_example():
    """Transformers 'Paged attention' doc, Decode path example."""
    g = _golden("decode_blocks.json")
    bs, bt, L = g["block_size"], g["block_table"], g["cache_seqlens"]
    for b in range(len(L)):
        need = (L[b] + 1 + bs - 1) // bs
        assert need == g["blocks_used_with_new_token"][b]
        assert L[b] // bs == g["new_token_table_entry"][b]
        assert bt[b][L[b] // bs] == g["new_token_block"][b]
        assert all(x == -1 for x in bt[b][need:])
        assert [bt[b][i] for i in range((L[b] + bs - 1) // bs)] == g["blocks_holding_cache"][b]
        assert oracle.slot_of(bt[b], L[b], bs) == g["derived_append_slots"][b]
        # every cached token's slot falls in one of the request's own blocks
        for j in range(L[b]):
            assert oracle.slot_of(bt[b], j, bs) // bs in g["blocks_holding_cache"][b]


# ---------------------------------------------------------------------------
# Hand-derived example (fixture with its derivation)
# ---------------------------------------------------------------------------

def _hand_tensors():
    g = _golden("hand_attention.json")
    q = torch.tensor(g["q"], dtype=torch.float32)[:, None, :]
    k = torch.tensor(g["k"], dtype=torch.float32)[:, None, :]
    v = torch.tensor(g["v"], dtype=torch.float32)[:, None, :]
    sink = torch.tensor([g["sink"]], dtype=torch.float32)
    return g, q, k, v, sink


def pin_hand_prefill():
    g, q, k, v, sink = _hand_tensors()
    cu = torch.tensor([0, 3], dtype=torch.int32)
    for case in g["cases"]:
        o, l = oracle.varlen_prefill(q, cu, cu, sink, g["sm_scale"], 1, k=k, v=v,
                                     window_left=case["window_left"])
        _close(o[:, 0, :], case["out"], 1e-6, 1e-6, f"hand prefill w={case['window_left']}")
        _close(l[:, 0], case["lse"], 1e-6, 1e-6, "hand prefill lse")


def pin_hand_decode_paged():
    """The hand example's keys in a paged pool (block size 2, blocks 3 then 1)."""
    g, q, k, v, sink = _hand_tensors()
    kc = torch.full((4, 2, 1, 2), float("nan"))
    vc = torch.full((4, 2, 1, 2), float("nan"))
    for j, slot in enumerate([6, 7, 2]):     # tokens 0,1 -> block 3; token 2 -> block 1
        kc.view(8, 1, 2)[slot] = k[j]
        vc.view(8, 1, 2)[slot] = v[j]
    bt = torch.tensor([[3, 1]], dtype=torch.int32)
    for case in g["cases"]:
        for L in (3, 2, 1):                     # the decode query sits at L-1: hand row L-1
            o, l = oracle.paged_decode(q[L - 1:L], kc, vc, bt, torch.tensor([L], dtype=torch.int32),
                                       sink, g["sm_scale"], case["window_left"])
            _close(o[0, 0], case["out"][L - 1], 1e-6, 1e-6, f"hand decode L={L}")
            _close(l[0, 0], case["lse"][L - 1], 1e-6, 1e-6, "hand decode lse")


def pin_hand_gqa():
    """Hq=4 over Hkv=2: kv head 1 holds -v, so heads 2,3 (group 1) must see -o."""
    g, q, k, v, sink = _hand_tensors()
    q4 = q.expand(3, 4, 2).contiguous()
    k2 = torch.cat([k, k], dim=1)
    v2 = torch.cat([v, -v], dim=1)
    s4 = sink.expand(4).contiguous()
    cu = torch.tensor([0, 3], dtype=torch.int32)
    o, _ = oracle.varlen_prefill(q4, cu, cu, s4, g["sm_scale"], 2, k=k2, v=v2)
    want = np.asarray(g["cases"][0]["out"])
    for h, sign in enumerate([1, 1, -1, -1]):
        _close(o[:, h, :], sign * want, 1e-6, 1e-6, f"gqa head {h}")


# ---------------------------------------------------------------------------
# Library routine: torch SDPA (float64, CPU) is plain causal softmax attention
# ---------------------------------------------------------------------------

def pin_sdpa_no_sink():
    for seed, (lens, Hq, Hkv, D) in enumerate([([5, 9, 1], 4, 2, 8), ([12, 7], 6, 3, 16),
                                                ([16], 8, 1, 32)]):
        c = synth.prefill_case(100 + seed, lens, lens, Hq, Hkv, D, torch.float32, False,
                               sm_scale=0.3 + 0.1 * seed)
        o, l = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, None, c.sm_scale,
                                     Hkv, k=c.k, v=c.v)
        cu = c.cu_seqlens_q.tolist()
        for r in range(len(lens)):
            qr = c.q[cu[r]:cu[r + 1]].double().transpose(0, 1)[None]
            kr = c.k[cu[r]:cu[r + 1]].double().transpose(0, 1)[None]
            vr = c.v[cu[r]:cu[r + 1]].double().transpose(0, 1)[None]
            ref = F.scaled_dot_product_attention(qr, kr, vr, is_causal=True, scale=c.sm_scale,
                                                 enable_gqa=True)[0].transpose(0, 1)
            _close(o[cu[r]:cu[r + 1]], ref.numpy(), 1e-12, 1e-10, f"sdpa request {r}")
            # lse against torch.logsumexp of the explicit causal logits
            logits = torch.einsum("hqd,hkd->hqk", qr[0],
                                  kr[0].repeat_interleave(Hq // Hkv, 0)) * c.sm_scale
            n = logits.shape[-1]
            logits = logits.masked_fill(torch.ones(n, n).triu(1).bool(), float("-inf"))
            _close(l[cu[r]:cu[r + 1]], torch.logsumexp(logits, -1).T.numpy(), 1e-12, 1e-10,
                   "sdpa lse")


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def pin_sink_closed_form():
    """With sink s: O_s = O_plain * (1 - share), share = e^s / (e^s + Z_plain),
    lse_s = logaddexp(lse_plain, s)."""
    c = synth.prefill_case(7, [9, 4, 13], [9, 4, 13], 4, 2, 16, torch.float32, True,
                           sm_scale=0.25)
    s = c.sink.double().numpy()
    o1, l1 = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, c.sm_scale,
                                   2, k=c.k, v=c.v)
    o0, l0 = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, None, c.sm_scale,
                                   2, k=c.k, v=c.v)
    share = 1.0 / (1.0 + np.exp(l0 - s[None, :]))
    _close(o1, o0 * (1.0 - share)[..., None], 1e-12, 1e-10, "sink output")
    _close(l1, np.logaddexp(l0, s[None, :]), 1e-12, 1e-10, "sink lse")
    # a sink of -inf is no sink
    ninf = torch.full_like(c.sink, float("-inf"))
    o2, l2 = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, ninf, c.sm_scale,
                                   2, k=c.k, v=c.v)
    _close(o2, o0, 0, 0, "sink -inf output")
    _close(l2, l0, 0, 0, "sink -inf lse")


def pin_empty_rows():
    """The varlen example's lengths: q [10,3,1] over k [0,1,7].  With the
    queries at the last Lq positions, r0's rows and r1's first two rows see
    no key; r1's last row sees key 0 only; r2's row sees all 7 keys."""
    g = _golden("varlen_map.json")
    c = synth.prefill_case(11, g["q_lens"], g["k_lens"], 2, 2, 8, torch.float32, True,
                           sm_scale=0.5)
    v = c.v.double().numpy()
    o, l = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, None, 0.5, 2, k=c.k, v=c.v)
    assert (o[:12] == 0).all() and np.isneginf(l[:12]).all()
    assert (o[12] == v[0]).all() and (l[12] != -np.inf).all()   # one visible key: o = V exactly
    # with a sink, an empty row puts all weight on the sink: o = 0, lse = sink
    o, l = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, 0.5, 2,
                                 k=c.k, v=c.v)
    assert (o[:12] == 0).all()
    _close(l[:12], np.broadcast_to(c.sink.double().numpy(), (12, 2)), 0, 0, "empty lse")
    s12 = 0.5 * (c.q[12].double() * c.k[0].double()).sum(-1).numpy()
    w = 1.0 / (1.0 + np.exp(c.sink.double().numpy() - s12))
    _close(o[12], w[:, None] * v[0], 1e-12, 1e-12, "one key with sink")


def pin_window_truncation():
    """Decode with window w over L keys equals plain decode over just the
    last w+1 keys (re-packed into a new pool)."""
    for w in (0, 1, 5, 17):
        L = 40
        c = synth.prefill_case(20 + w, [L], [L], 4, 2, 16, torch.float32, True, sm_scale=0.4)
        keep = list(range(max(0, L - 1 - w), L))
        full = synth.decode_case(0, [L], 4, 2, 16, 8, torch.float32, True, poison=False)
        part = synth.decode_case(0, [len(keep)], 4, 2, 16, 8, torch.float32, True, poison=False)
        _fill_from(full, c.k, c.v, list(range(L)))
        _fill_from(part, c.k, c.v, keep)
        q = c.q[L - 1:L]
        o1, l1 = oracle.paged_decode(q, full.k_cache, full.v_cache, full.block_table,
                                     full.cache_seqlens, c.sink, 0.4, window_left=w)
        o2, l2 = oracle.paged_decode(q, part.k_cache, part.v_cache, part.block_table,
                                     part.cache_seqlens, c.sink, 0.4)
        _close(o1, o2, 1e-12, 1e-12, f"window {w}")
        _close(l1, l2, 1e-12, 1e-12, f"window {w} lse")


def _fill_from(case, k, v, rows):
    """Write logical tokens rows[j] of contiguous k/v into case's pool at position j."""
    bs = case.block_size
    bt = case.block_table.tolist()[0]
    for j, r in enumerate(rows):
        s = bt[j // bs] * bs + j % bs
        case.k_cache.view(-1, *case.k_cache.shape[2:])[s] = k[r]
        case.v_cache.view(-1, *case.v_cache.shape[2:])[s] = v[r]


def pin_window_special_cases():
    c = synth.prefill_case(31, [6, 11], [6, 11], 4, 4, 8, torch.float32, False, sm_scale=0.7)
    args = (c.q, c.cu_seqlens_q, c.cu_seqlens_k)
    o_none, l_none = oracle.varlen_prefill(*args, None, 0.7, 4, k=c.k, v=c.v)
    o_big, l_big = oracle.varlen_prefill(*args, None, 0.7, 4, k=c.k, v=c.v, window_left=10)
    _close(o_big, o_none, 0, 0, "window >= Lk-1")
    o0, _ = oracle.varlen_prefill(*args, None, 0.7, 4, k=c.k, v=c.v, window_left=0)
    _close(o0, c.v.double().numpy(), 0, 0, "window 0 selects the query's own key")


def pin_q_zero_mean():
    c = synth.prefill_case(41, [7, 3], [7, 3], 2, 1, 8, torch.float32, False, sm_scale=1.0)
    o, l = oracle.varlen_prefill(torch.zeros_like(c.q), c.cu_seqlens_q, c.cu_seqlens_k, None,
                                 1.0, 1, k=c.k, v=c.v)
    v = c.v.double().numpy()[:, 0]
    cu = c.cu_seqlens_q.tolist()
    for r in range(2):
        for i in range(cu[r + 1] - cu[r]):
            want = v[cu[r]:cu[r] + i + 1].mean(0)
            for h in range(2):
                _close(o[cu[r] + i, h], want, 1e-14, 1e-12, "uniform weights")
            _close(l[cu[r] + i], np.log(i + 1) * np.ones(2), 1e-14, 1e-12, "lse ln n")


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def _decode_from_prefill(c, L_list, bs, shuffle, seed):
    """Paged decode case whose request b holds the K/V rows of prefill request b."""
    d = synth.decode_case(seed, L_list, c.Hq, c.Hkv, c.D, bs, c.q.dtype, c.sink is not None,
                          shuffle=shuffle, poison=True)
    cu = c.cu_seqlens_k.tolist()
    flat_k = d.k_cache.view(-1, c.Hkv, c.D)
    flat_v = d.v_cache.view(-1, c.Hkv, c.D)
    bt = d.block_table.tolist()
    for b, L in enumerate(L_list):
        for j in range(L):
            s = bt[b][j // bs] * bs + j % bs
            flat_k[s] = c.k[cu[b] + j]
            flat_v[s] = c.v[cu[b] + j]
    return d


def pin_paged_equals_contiguous():
    """Decode over a shuffled paged pool equals the last row of causal
    prefill over the same keys held contiguously, and any two pool orders
    give identical results."""
    lens = [1, 17, 33, 64]
    c = synth.prefill_case(51, lens, lens, 4, 2, 16, torch.float32, True, sm_scale=0.25)
    o_p, l_p = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, 0.25, 2,
                                     k=c.k, v=c.v)
    last = (c.cu_seqlens_q[1:] - 1).long()
    res = []
    for shuffle, seed in ((False, 1), (True, 2), (True, 3)):
        d = _decode_from_prefill(c, lens, 16, shuffle, seed)
        o, l = oracle.paged_decode(c.q[last], d.k_cache, d.v_cache, d.block_table,
                                   d.cache_seqlens, c.sink, 0.25)
        _close(o, o_p[last.numpy()], 1e-13, 1e-12, "decode == last prefill row")
        _close(l, l_p[last.numpy()], 1e-13, 1e-12, "decode lse")
        res.append((o, l))
    _close(res[1][0], res[2][0], 0, 0, "pool order invariance")
    # paged prefill (keys through the table) equals contiguous prefill
    d = _decode_from_prefill(c, lens, 8, True, 4)
    o_pp, l_pp = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, 0.25, 2,
                                       k_cache=d.k_cache, v_cache=d.v_cache,
                                       block_table=d.block_table, block_size=8)
    _close(o_pp, o_p, 0, 0, "paged prefill == contiguous prefill")
    _close(l_pp, l_p, 0, 0, "paged prefill lse")


def pin_chunk_is_tail():
    """A query chunk at the end of a longer KV (bottom-right causal) equals
    the same rows of full causal prefill, with and without a window."""
    L, n = 30, 7
    c = synth.prefill_case(61, [L], [L], 4, 2, 8, torch.float32, True, sm_scale=0.5)
    for w in (-1, 4):
        o_full, l_full = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, 0.5,
                                               2, k=c.k, v=c.v, window_left=w)
        cq = torch.tensor([0, n], dtype=torch.int32)
        o_c, l_c = oracle.varlen_prefill(c.q[L - n:].contiguous(), cq, c.cu_seqlens_k, c.sink,
                                         0.5, 2, k=c.k, v=c.v, window_left=w)
        _close(o_c, o_full[L - n:], 0, 0, f"chunk rows w={w}")
        _close(l_c, l_full[L - n:], 0, 0, "chunk lse")


def pin_gqa_equals_mha():
    c = synth.prefill_case(71, [9, 5], [9, 5], 8, 2, 8, torch.float32, True, sm_scale=0.5)
    o_g, l_g = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, 0.5, 2,
                                     k=c.k, v=c.v)
    k4 = c.k.repeat_interleave(4, dim=1).contiguous()
    v4 = c.v.repeat_interleave(4, dim=1).contiguous()
    o_m, l_m = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, 0.5, 8,
                                     k=k4, v=v4)
    _close(o_g, o_m, 0, 0, "gqa == mha")
    _close(l_g, l_m, 0, 0, "gqa lse")


def pin_split_merge():
    """Merging per-partition results (sink left out of each, added once in
    the merge) equals unsplit decode, for any partition size, with windows."""
    lens = [1, 15, 16, 17, 100, 257]
    for w in (-1, 20):
        d = synth.decode_case(81, lens, 4, 2, 16, 8, torch.float32, True, window_left=w,
                              sm_scale=0.25)
        o, l = oracle.paged_decode(d.q, d.k_cache, d.v_cache, d.block_table, d.cache_seqlens,
                                   d.sink, 0.25, window_left=w)
        for P in (8, 16, 64, 512):
            po, pl = oracle.paged_decode(d.q, d.k_cache, d.v_cache, d.block_table,
                                         d.cache_seqlens, d.sink, 0.25, window_left=w,
                                         partition_size=P)
            npb = [(L + P - 1) // P for L in lens]
            om, lm = oracle.merge(po, pl, npb, d.sink)
            _close(om, o, 1e-13, 1e-11, f"merge P={P} w={w}")
            _close(lm, l, 1e-13, 1e-11, f"merge lse P={P}")
        # one partition covering everything is unsplit attention without the sink
        po, pl = oracle.paged_decode(d.q, d.k_cache, d.v_cache, d.block_table, d.cache_seqlens,
                                     d.sink, 0.25, window_left=w, partition_size=1024)
        o0, l0 = oracle.paged_decode(d.q, d.k_cache, d.v_cache, d.block_table,
                                     d.cache_seqlens, None, 0.25, window_left=w)
        _close(po[:, :, 0], o0, 0, 0, "P >= L")
        _close(pl[:, :, 0], l0, 0, 0, "P >= L lse")


def pin_merge_associative():
    """Merging in two stages (pairs of partitions without the sink, then the
    pair results with the sink) equals a one-stage merge."""
    B, Hq, P, D = 3, 2, 6, 8
    po, pl = synth.random_partials(5, B, Hq, P, D, [6, 6, 6])
    sink = torch.tensor([0.3, -1.2])
    o1, l1 = oracle.merge(po, pl, [6] * B, sink)
    stage_o = np.zeros((B, Hq, 3, D))
    stage_l = np.zeros((B, Hq, 3))
    for k in range(3):
        so, sl = oracle.merge(po[:, :, 2 * k:2 * k + 2].numpy(), pl[:, :, 2 * k:2 * k + 2].numpy(),
                              [2] * B, None)
        stage_o[:, :, k], stage_l[:, :, k] = so, sl
    o2, l2 = oracle.merge(stage_o, stage_l, [3] * B, sink)
    _close(o1, o2, 1e-13, 1e-11, "associative merge")
    _close(l1, l2, 1e-13, 1e-11, "associative lse")
    # every partition empty and no sink: zero output, -inf lse
    o3, l3 = oracle.merge(np.zeros((1, 1, 2, 4)), np.full((1, 1, 2), -np.inf), [2], None)
    assert (o3 == 0).all() and np.isneginf(l3).all()


# ---------------------------------------------------------------------------
# Brute force: an independently written numpy mask-matrix evaluation,
# following the reference's own recipe (explicit mask, sink appended as an
# extra column of the logits, softmax, sink column dropped).
# ---------------------------------------------------------------------------

def _numpy_reference(q, k, v, cu_q, cu_k, sink, sm_scale, Hkv, window, alibi=None, causal=True):
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    Hq = q.shape[1]
    G = Hq // Hkv
    out = np.zeros(q.shape)
    for r in range(len(cu_q) - 1):
        qs, ks = slice(cu_q[r], cu_q[r + 1]), slice(cu_k[r], cu_k[r + 1])
        Lq, Lk = cu_q[r + 1] - cu_q[r], cu_k[r + 1] - cu_k[r]
        rows = (Lk - Lq + np.arange(Lq))[:, None]
        cols = np.arange(Lk)[None, :]
        mask = cols <= rows if causal else np.ones((Lq, Lk), bool)
        if window >= 0:
            mask &= cols >= rows - window
        for h in range(Hq):
            kk, vv = k[ks, h // G], v[ks, h // G]
            bias = 0.0 if alibi is None else float(alibi[h]) * (cols - rows)
            logits = np.where(mask, sm_scale * q[qs, h] @ kk.T + bias, -np.inf)
            col = np.full((Lq, 1), -np.inf if sink is None else float(sink[h]))
            full = np.concatenate([logits, col], axis=1)
            mx = full.max(axis=1, keepdims=True)
            mx[np.isneginf(mx)] = 0.0
            e = np.exp(full - mx)
            den = e.sum(axis=1, keepdims=True)
            p = np.divide(e, den, out=np.zeros_like(e), where=den > 0)[:, :-1]
            out[qs, h] = p @ vv
    return out


def pin_brute_force():
    rng = np.random.default_rng(1234)
    for trial in range(24):
        G = [1, 2, 4][trial % 3]
        Hkv = 1 + trial % 2
        B = 1 + trial % 3
        q_lens = rng.integers(0, 9, size=B).tolist()
        k_lens = [ql + int(rng.integers(0, 6)) for ql in q_lens]
        if trial % 5 == 0:
            k_lens[0] = 0
        w = [-1, 0, 1, 5, 100][trial % 5]
        with_sink = trial % 2 == 0
        # every third trial adds ALiBi slopes (vLLM page, PagedAttentionWithALiBi)
        al = (torch.from_numpy(rng.uniform(0.01, 1.0, size=G * Hkv).astype(np.float32))
              if trial % 3 == 1 else None)
        c = synth.prefill_case(500 + trial, q_lens, k_lens, G * Hkv, Hkv, 8, torch.float32,
                               with_sink, window_left=w, sm_scale=0.6)
        o, _ = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, 0.6, Hkv,
                                     k=c.k, v=c.v, window_left=w, alibi=al)
        ref = _numpy_reference(c.q, c.k, c.v, c.cu_seqlens_q.tolist(), c.cu_seqlens_k.tolist(),
                               None if c.sink is None else c.sink.numpy(), 0.6, Hkv, w,
                               None if al is None else al.numpy())
        _close(o, ref, 1e-12, 1e-10, f"brute force trial {trial}")


def pin_noncausal_brute_force():
    """Non-causal prefill (FlashInfer page, sink_attention_unified, the
    non-causal branches: every key is a candidate; a window only bounds the
    left side, query_position - window_left <= key) against the mask-matrix
    reference, queries shorter and longer than the keys, with sinks and ALiBi."""
    rng = np.random.default_rng(4321)
    for trial in range(18):
        G = [1, 2, 4][trial % 3]
        Hkv = 1 + trial % 2
        B = 1 + trial % 3
        q_lens = rng.integers(0, 9, size=B).tolist()
        k_lens = [max(0, ql + int(rng.integers(-3, 6))) for ql in q_lens]
        w = [-1, 0, 2, 5, 100, 3][trial % 6]
        with_sink = trial % 2 == 1
        al = (torch.from_numpy(rng.uniform(0.01, 1.0, size=G * Hkv).astype(np.float32))
              if trial % 4 == 3 else None)
        c = synth.prefill_case(700 + trial, q_lens, k_lens, G * Hkv, Hkv, 8, torch.float32,
                               with_sink, window_left=w, sm_scale=0.7)
        o, _ = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, 0.7, Hkv,
                                     k=c.k, v=c.v, window_left=w, alibi=al, causal=False)
        ref = _numpy_reference(c.q, c.k, c.v, c.cu_seqlens_q.tolist(), c.cu_seqlens_k.tolist(),
                               None if c.sink is None else c.sink.numpy(), 0.7, Hkv, w,
                               None if al is None else al.numpy(), causal=False)
        _close(o, ref, 1e-12, 1e-10, f"non-causal brute force trial {trial}")


def pin_noncausal_sdpa():
    """Non-causal prefill without a window or sink is textbook attention over
    all of the request's keys: torch's float64 SDPA with no mask (GQA by
    repeated kv heads), for queries fewer and more than the keys; with one
    query it equals decode over the same keys (a causal query at the last
    position sees them all)."""
    for seed, (q_lens, k_lens, Hq, Hkv, D) in enumerate([([5, 9, 1], [7, 3, 4], 4, 2, 8),
                                                         ([12], [20], 6, 3, 16)]):
        c = synth.prefill_case(800 + seed, q_lens, k_lens, Hq, Hkv, D, torch.float32, False,
                               sm_scale=0.25 + 0.1 * seed)
        o, l = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, None, c.sm_scale,
                                     Hkv, k=c.k, v=c.v, causal=False)
        cq, ck = c.cu_seqlens_q.tolist(), c.cu_seqlens_k.tolist()
        for r in range(len(q_lens)):
            qr = c.q[cq[r]:cq[r + 1]].double().transpose(0, 1)[None]
            kr = c.k[ck[r]:ck[r + 1]].double().transpose(0, 1)[None]
            vr = c.v[ck[r]:ck[r + 1]].double().transpose(0, 1)[None]
            ref = F.scaled_dot_product_attention(qr, kr, vr, scale=c.sm_scale,
                                                 enable_gqa=True)[0].transpose(0, 1)
            _close(o[cq[r]:cq[r + 1]], ref.numpy(), 1e-12, 1e-10, f"non-causal sdpa request {r}")
    # one query per request, non-causal == decode over the request's keys
    dc = synth.decode_case(810, [1, 9, 30], 8, 2, 16, 4, torch.float32, with_sink=True,
                           sm_scale=0.4, shuffle=True)
    od, ld = oracle.paged_decode(dc.q, dc.k_cache, dc.v_cache, dc.block_table, dc.cache_seqlens,
                                 dc.sink, 0.4)
    cu_q = torch.arange(dc.B + 1, dtype=torch.int32)
    cu_k = synth.cu_from_lengths(dc.cache_seqlens.tolist())
    op, lp = oracle.varlen_prefill(dc.q, cu_q, cu_k, dc.sink, 0.4, dc.Hkv, k_cache=dc.k_cache,
                                   v_cache=dc.v_cache, block_table=dc.block_table, block_size=4,
                                   causal=False)
    _close(op, od, 1e-13, 1e-12, "non-causal Lq = 1 vs decode")
    _close(lp, ld, 1e-13, 1e-12, "non-causal Lq = 1 vs decode lse")


def pin_alibi_closed_form():
    """ALiBi (vLLM page "attention.py", PagedAttentionWithALiBi.set_attn_bias:
    bias[i][j] = slope_h * (j - i), key position minus query position, added
    to the scaled logits).  With every key equal, the logits differ only by
    the bias, so the weights of the query at position p are the geometric
    sequence r^(j - p), r = e^slope, normalised (with the sink e^sigma in the
    denominator); one-hot value rows read each weight out.  The decode of the
    same rows (query at the last position) gives the last row of the prefill."""
    Lk, D, slopes = 6, 8, [0.5, 0.125]
    q = torch.zeros((Lk, 2, D))
    k = torch.ones((Lk, 1, D))
    v = torch.zeros((Lk, 1, D))
    for j in range(Lk):
        v[j, 0, j] = 1.0
    al = torch.tensor(slopes)
    sink = torch.tensor([0.25, -1.0])
    cu = torch.tensor([0, Lk], dtype=torch.int32)
    o, lse = oracle.varlen_prefill(q, cu, cu, sink, 1.0, 1, k=k, v=v, alibi=al)
    for h, m in enumerate(slopes):
        for p in range(Lk):
            w = np.array([np.exp(m * (j - p)) for j in range(p + 1)])
            z = w.sum() + np.exp(float(sink[h]))
            want = np.zeros(D)
            want[:p + 1] = w / z
            _close(o[p, h], want, 1e-14, 1e-12, f"alibi closed form h {h} p {p}")
            _close(lse[p, h], np.log(z), 1e-14, 1e-12, "alibi lse")
    bt = torch.tensor([[0, 1]], dtype=torch.int32)
    kc, vc = torch.zeros((2, 4, 1, D)), torch.zeros((2, 4, 1, D))
    kc.view(-1, 1, D)[:Lk] = k
    vc.view(-1, 1, D)[:Lk] = v
    od, _ = oracle.paged_decode(q[:1], kc, vc, bt, torch.tensor([Lk], dtype=torch.int32), sink,
                                1.0, alibi=al)
    _close(od[0], o[Lk - 1], 1e-14, 1e-12, "alibi decode == last prefill row")


def pin_rope():
    """Rotary embedding (the reading of the vLLM page's PagedAttentionWithRoPE,
    whose rotation is not printed): position 0 is the identity; each rotated
    pair keeps its norm; dimensions past rotary_dim are untouched; the dot
    product of a rotated query and key depends only on their distance (both
    pairings); the neox pairing equals the interleaved one under the
    dimension permutation; linear scaling is the unscaled table at pos /
    factor; and hand-computed angles for the plain and dynamic tables."""
    rng = np.random.default_rng(31)
    rd, D, base = 8, 12, 10000.0
    tab = oracle.rope_cos_sin(64, rd, base)
    # hand values: rotary_dim 2 turns at 1 rad per position
    t2 = oracle.rope_cos_sin(5, 2, base)
    _close(t2[3], np.array([np.cos(3.0), np.sin(3.0)]), 1e-15, 1e-15, "rope rd 2")
    _close(tab[5, 1], np.cos(5 * base ** -0.25), 1e-15, 1e-15, "rope freq 1")
    for neox in (True, False):
        x = rng.normal(size=(4, 3, D))
        y0 = oracle.rope_apply(x, np.zeros(4, int), tab, rd, neox)
        _close(y0, x, 0, 0, "rope pos 0")
        pos = np.array([1, 7, 20, 63])
        y = oracle.rope_apply(x, pos, tab, rd, neox)
        _close(y[..., rd:], x[..., rd:], 0, 0, "rope pass-through dims")
        if neox:
            pairs = [(i, i + rd // 2) for i in range(rd // 2)]
        else:
            pairs = [(2 * i, 2 * i + 1) for i in range(rd // 2)]
        for a, b in pairs:
            _close(np.hypot(y[..., a], y[..., b]), np.hypot(x[..., a], x[..., b]), 1e-12, 1e-12,
                   "rope pair norm")
        q, k = rng.normal(size=(1, 1, D)), rng.normal(size=(1, 1, D))
        dots = []
        for m, n in [(10, 3), (17, 10), (40, 33)]:
            qm = oracle.rope_apply(q, np.array([m]), tab, rd, neox)[0, 0]
            kn = oracle.rope_apply(k, np.array([n]), tab, rd, neox)[0, 0]
            dots.append(qm @ kn)
        _close(np.array(dots[1:]), np.array([dots[0]] * 2), 1e-12, 1e-12, "rope relative")
    # neox pairing == interleaved pairing under the permutation (i, i+rd/2) -> (2i, 2i+1)
    perm = np.concatenate([np.array([[i, i + rd // 2] for i in range(rd // 2)]).ravel(),
                           np.arange(rd, D)])
    x = rng.normal(size=(2, 1, D))
    pos = np.array([3, 50])
    yn = oracle.rope_apply(x, pos, tab, rd, True)
    yg = oracle.rope_apply(x[..., perm], pos, tab, rd, False)
    _close(yg, yn[..., perm], 1e-13, 1e-13, "rope neox vs interleaved")
    # linear scaling: row f*p of the linear table is row p of the plain one
    lin = oracle.rope_cos_sin(64, rd, base, oracle.ROPE_LINEAR, 4.0, 16)
    _close(lin[0:64:4], tab[0:16], 1e-15, 1e-15, "rope linear")
    # dynamic: no change within max_position; beyond it base' = base * (f L / M - (f - 1))^(rd/(rd-2))
    dyn_short = oracle.rope_cos_sin(8, 4, base, oracle.ROPE_DYNAMIC, 2.0, 8)
    _close(dyn_short, oracle.rope_cos_sin(8, 4, base), 0, 0, "rope dynamic short")
    dyn = oracle.rope_cos_sin(32, 4, base, oracle.ROPE_DYNAMIC, 2.0, 8)
    # base' = 10000 * (2*32/8 - 1)^2 = 490000, frequency 1 = 490000^-0.5 = 1/700
    _close(dyn[7, [1, 3]], np.array([np.cos(0.01), np.sin(0.01)]), 1e-15, 1e-13, "rope dynamic")


def pin_bf16_inputs_read_exactly():
    """bf16 storage is read as its exact value: the oracle on bf16 tensors
    equals the oracle on the same values widened to fp32."""
    c = synth.prefill_case(91, [13, 6], [13, 6], 4, 2, 16, torch.bfloat16, True, sm_scale=0.25)
    o1, l1 = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, 0.25, 2,
                                   k=c.k, v=c.v)
    o2, l2 = oracle.varlen_prefill(c.q.float(), c.cu_seqlens_q, c.cu_seqlens_k, c.sink, 0.25, 2,
                                   k=c.k.float(), v=c.v.float())
    _close(o1, o2, 0, 0, "bf16 == widened fp32")
    _close(l1, l2, 0, 0, "bf16 lse")


def pin_reshape_and_cache():
    """Scatter then gather back through the slots returns the input bitwise;
    negative slots are skipped; untouched slots keep their sentinel.  The
    decode example's append slots [94, 32, 198] land in blocks 2, 1, 6."""
    for dtype in (torch.float32, torch.bfloat16):
        T, Hkv, D, bs, NB = 11, 2, 8, 4, 6
        key = synth.to_dtype(synth.normal(3, (T, Hkv, D), 1), dtype)
        val = synth.to_dtype(synth.normal(3, (T, Hkv, D), 2), dtype)
        rng = np.random.default_rng(9)
        slots = rng.permutation(NB * bs)[:T].astype(np.int32)
        slots[[2, 7]] = -1
        kc0 = torch.full((NB, bs, Hkv, D), -7.0, dtype=dtype)
        vc0 = torch.full((NB, bs, Hkv, D), -9.0, dtype=dtype)
        kc, vc = oracle.reshape_and_cache(key, val, kc0, vc0, torch.from_numpy(slots))
        fk, fv = kc.view(-1, Hkv, D), vc.view(-1, Hkv, D)
        for t, s in enumerate(slots):
            if s >= 0:
                assert torch.equal(fk[s], key[t]) and torch.equal(fv[s], val[t])
        untouched = np.setdiff1d(np.arange(NB * bs), slots[slots >= 0])
        assert (fk[untouched] == -7.0).all() and (fv[untouched] == -9.0).all()
    g = _golden("decode_blocks.json")
    c = synth.config1_decode()
    new_k = synth.to_dtype(synth.normal(5, (3, 2, 64), 1), torch.float32)
    slots = torch.tensor([oracle.slot_of(c.block_table[b].tolist(), int(c.cache_seqlens[b]), 32)
                          for b in range(3)], dtype=torch.int32)
    assert slots.tolist() == g["derived_append_slots"]
    kc, _ = oracle.reshape_and_cache(new_k, new_k, c.k_cache, c.v_cache, slots)
    for b, blk in enumerate(g["new_token_block"]):
        assert torch.equal(kc[blk, int(c.cache_seqlens[b]) % 32], new_k[b])


def pin_decode_append():
    """Decode with the new token appended, against an independent numpy
    evaluation: keys 0..L-1 gathered from the original cache through the
    block table, k_new as key L, window L - w <= j, the sink as one more
    logit.  The returned caches differ from the inputs exactly at the new
    tokens' slots, which hold k_new / v_new; on the page's decode example
    those slots are 94, 32 and 198."""
    rng = np.random.default_rng(77)
    for trial in range(12):
        G = [1, 2, 4][trial % 3]
        Hkv = 1 + trial % 2
        Hq = G * Hkv
        B, D, bs, MB = 3, 8, 4, 6
        NB = B * MB
        lens = rng.integers(0, MB * bs - 1, size=B)
        if trial % 4 == 0:
            lens[0] = 0
        w = [-1, 0, 1, 6][trial % 4]
        sink = None if trial % 2 else torch.from_numpy(rng.normal(size=Hq).astype(np.float32))
        q = torch.from_numpy(rng.normal(size=(B, Hq, D)).astype(np.float32))
        kn = torch.from_numpy(rng.normal(size=(B, Hkv, D)).astype(np.float32))
        vn = torch.from_numpy(rng.normal(size=(B, Hkv, D)).astype(np.float32))
        kc0 = torch.from_numpy(rng.normal(size=(NB, bs, Hkv, D)).astype(np.float32))
        vc0 = torch.from_numpy(rng.normal(size=(NB, bs, Hkv, D)).astype(np.float32))
        bt = torch.from_numpy(rng.permutation(NB).reshape(B, MB).astype(np.int32))
        sl = torch.from_numpy(lens.astype(np.int32))
        out, lse, kc, vc = oracle.decode_append(q, kn, vn, kc0, vc0, bt, sl, sink, 0.7, w)
        for b in range(B):
            L = int(lens[b])
            rows = [int(bt[b, j // bs]) * bs + j % bs for j in range(L)]
            K = np.concatenate([kc0.view(-1, Hkv, D)[rows].numpy(), kn[b:b + 1].numpy()], 0)
            V = np.concatenate([vc0.view(-1, Hkv, D)[rows].numpy(), vn[b:b + 1].numpy()], 0)
            j = np.arange(L + 1)
            vis = (j >= L - w) if w >= 0 else np.ones(L + 1, bool)
            for h in range(Hq):
                lg = np.where(vis, 0.7 * (K[:, h // G].astype(np.float64) @ q[b, h].double().numpy()),
                              -np.inf)
                full = np.append(lg, -np.inf if sink is None else float(sink[h]))
                mx = full.max()
                e = np.exp(full - mx)
                ref = (e[:-1] / e.sum()) @ V[:, h // G].astype(np.float64)
                _close(out[b, h], ref, 1e-12, 1e-10, f"append trial {trial} b {b} h {h}")
                _close(lse[b, h], mx + np.log(e.sum()), 1e-12, 1e-10, "append lse")
        slots = [int(bt[b, int(lens[b]) // bs]) * bs + int(lens[b]) % bs for b in range(B)]
        fk, fv = kc.view(-1, Hkv, D), vc.view(-1, Hkv, D)
        for b, s_ in enumerate(slots):
            assert torch.equal(fk[s_], kn[b]) and torch.equal(fv[s_], vn[b])
        other = np.setdiff1d(np.arange(NB * bs), slots)
        assert torch.equal(fk[other], kc0.view(-1, Hkv, D)[other])
        assert torch.equal(fv[other], vc0.view(-1, Hkv, D)[other])
    g = _golden("decode_blocks.json")
    c = synth.config1_decode()
    kn = synth.to_dtype(synth.normal(6, (3, c.Hkv, c.D), 1), torch.float32)
    _, _, kc, _ = oracle.decode_append(c.q, kn, kn, c.k_cache, c.v_cache, c.block_table,
                                       c.cache_seqlens, c.sink, c.sm_scale)
    fk = kc.view(-1, c.Hkv, c.D)
    for b, s_ in enumerate(g["derived_append_slots"]):
        assert torch.equal(fk[s_], kn[b])


# ---------------------------------------------------------------------------
# Vertical + slash sparse prefill (nano-vllm "minference.py" page: vertical
# key positions and slash diagonal offsets i - j per head, 64 x 64 blocks)
# ---------------------------------------------------------------------------

def _vs_brute(V, S, L):
    """Block lists of one head by enumeration: for every row i of block m and
    diagonal s, the key i - s (when >= 0) marks its 64-key block; vertical
    columns inside the block's rows and outside those blocks are kept."""
    NM = (L + 63) // 64
    out = []
    for m in range(NM):
        rows = range(64 * m, min(64 * m + 64, L))
        sel = set()
        for i in rows:
            for s_ in S:
                if 0 <= s_ < L and i - s_ >= 0:
                    sel.add((i - s_) // 64)
        cols = [v for v in V if 0 <= v < L and v <= rows[-1] and v // 64 not in sel]
        out.append(([64 * n for n in sorted(sel)], cols))
    return out


def _vs_lists(bc, bo, cc, ci, b, h, m):
    return (bo[b, h, m, :bc[b, h, m]].tolist(), ci[b, h, m, :cc[b, h, m]].tolist())


def pin_vertical_slash_brute_force():
    """The oracle's conversion against enumeration over every (row, diagonal)
    pair, on small requests of several row blocks; indices outside [0, L),
    repeated diagonals and unsorted diagonals included."""
    rng = np.random.default_rng(2594)
    for trial in range(30):
        B, H = 1 + trial % 2, 1 + trial % 3
        lens = rng.integers(1, 330, size=B).tolist()
        NV, NS = int(rng.integers(0, 12)), int(rng.integers(0, 12))
        Lmax = max(lens)
        V = np.sort(rng.choice(Lmax + 40, size=(B, H, NV)), axis=-1).astype(np.int32)
        S = rng.integers(-3, Lmax + 20, size=(B, H, NS)).astype(np.int32)
        if NS > 1:
            S[..., 1] = S[..., 0]                            # a repeated diagonal
        cu = synth.cu_from_lengths(lens)
        bc, bo, cc, ci = oracle.vertical_slash_blocks(V, S, cu, Lmax)
        NM = (Lmax + 63) // 64
        for b in range(B):
            for h in range(H):
                want = _vs_brute(V[b, h].tolist(), S[b, h].tolist(), lens[b])
                for m in range(NM):
                    got = _vs_lists(bc, bo, cc, ci, b, h, m)
                    exp = want[m] if m < len(want) else ([], [])
                    assert got == exp, (trial, b, h, m, got, exp)


def pin_vertical_slash_closed_forms():
    """Closed forms of the conversion: every diagonal selects the causal
    triangle of blocks 0..m; diagonal 0 alone selects block m; diagonal 64k
    selects block m - k exactly (the rows of m shifted by a whole block);
    diagonal 1 selects blocks m - 1 and m; no diagonal and every column lists
    keys 0 .. m's last row."""
    L = 300
    cu = [0, L]
    NM = 5
    def lists(V, S):
        V = np.asarray(V, dtype=np.int32).reshape(1, 1, -1)
        S = np.asarray(S, dtype=np.int32).reshape(1, 1, -1)
        r = oracle.vertical_slash_blocks(V, S, cu, L)
        return [_vs_lists(*r, 0, 0, m) for m in range(NM)]
    assert lists([], list(range(L))) == [([64 * n for n in range(m + 1)], []) for m in range(NM)]
    assert lists([], [0]) == [([64 * m], []) for m in range(NM)]
    for k in (1, 2):
        assert lists([], [64 * k]) == [([64 * (m - k)] if m >= k else [], []) for m in range(NM)]
    assert lists([], [1]) == [([0], [])] + [([64 * (m - 1), 64 * m], []) for m in range(1, NM)]
    assert lists(list(range(L)), []) == [([], list(range(min(64 * m + 64, L)))) for m in range(NM)]


def _masked_reference(q, k, v, mask_bool, sink, sm_scale, Hkv):
    """numpy mask-matrix attention for one request: mask_bool [H, L, L]."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    L, Hq, _ = q.shape
    G = Hq // Hkv
    out = np.zeros(q.shape)
    for h in range(Hq):
        logits = np.where(mask_bool[h], sm_scale * q[:, h] @ k[:, h // G].T, -np.inf)
        col = np.full((L, 1), -np.inf if sink is None else float(sink[h]))
        full = np.concatenate([logits, col], axis=1)
        mx = full.max(axis=1, keepdims=True)
        mx[np.isneginf(mx)] = 0.0
        e = np.exp(full - mx)
        den = e.sum(axis=1, keepdims=True)
        p = np.divide(e, den, out=np.zeros_like(e), where=den > 0)[:, :-1]
        out[:, h] = p @ v[:, h // G]
    return out


def _bits(mask_bool):
    """[units, L] bool -> [units, W] uint64 rows (bit j % 64 of word j // 64)."""
    U, L = mask_bool.shape
    W = max(1, (L + 63) // 64)
    padded = np.zeros((U, W * 64), dtype=bool)
    padded[:, :L] = mask_bool
    return np.packbits(padded, axis=1, bitorder="little").view(np.uint64)


def pin_masked_prefill():
    """Attention under an explicit mask: against torch's float64 SDPA with a
    boolean mask (no sink; every row keeps its diagonal key), against the
    mask-matrix reference with a sink and with fully masked rows, and on a
    subset of units."""
    rng = np.random.default_rng(77)
    for trial, (L, Hq, Hkv, D) in enumerate([(37, 4, 2, 8), (70, 2, 2, 16), (9, 6, 3, 8)]):
        c = synth.prefill_case(900 + trial, [L], [L], Hq, Hkv, D, torch.float32, True,
                               sm_scale=0.3)
        mb = rng.random((Hq, L, L)) < 0.4
        mb[:, np.arange(L), np.arange(L)] = True
        units_mask = mb.transpose(1, 0, 2).reshape(L * Hq, L)    # unit t * Hq + h
        o, _ = oracle.masked_prefill(c.q, c.k, c.v, c.cu_seqlens_q, _bits(units_mask), None,
                                     0.3, Hkv)
        ref = F.scaled_dot_product_attention(
            c.q.double().transpose(0, 1)[None], c.k.double().transpose(0, 1)[None],
            c.v.double().transpose(0, 1)[None], attn_mask=torch.from_numpy(mb)[None],
            scale=0.3, enable_gqa=True)[0].transpose(0, 1)
        _close(o, ref.numpy(), 1e-12, 1e-10, f"masked vs sdpa {trial}")
        mb[:, 1, :] = False                                      # a row with no key
        units_mask = mb.transpose(1, 0, 2).reshape(L * Hq, L)
        o, l = oracle.masked_prefill(c.q, c.k, c.v, c.cu_seqlens_q, _bits(units_mask), c.sink,
                                     0.3, Hkv)
        _close(o, _masked_reference(c.q, c.k, c.v, mb, c.sink.numpy(), 0.3, Hkv), 1e-12, 1e-10,
               f"masked vs reference {trial}")
        _close(l[1], c.sink.numpy(), 1e-6, 1e-6, "masked row lse = sink")
        units = [3, L * Hq - 1, Hq + 1]
        ou, _ = oracle.masked_prefill(c.q, c.k, c.v, c.cu_seqlens_q, _bits(units_mask[units]),
                                      c.sink, 0.3, Hkv, units=units)
        for u in units:
            _close(ou[u // Hq, u % Hq], o[u // Hq, u % Hq], 0, 0, "masked units")


def pin_block_sparse_mask():
    """The mask of the block lists is the definition written out: row i of
    block m sees key j <= i when j's block is a slash block of m or j is a
    vertical index; and two limits reduce to plain attention: every diagonal,
    or every column, gives causal prefill; no index gives rows that see
    nothing (output 0, lse = the sink)."""
    rng = np.random.default_rng(31)
    lens = [150, 64, 1]
    cu = synth.cu_from_lengths(lens)
    Hq, Hkv, D = 4, 2, 8
    V = np.stack([np.stack([np.sort(rng.choice(160, 6, replace=False)) for _ in range(Hq)])
                  for _ in lens]).astype(np.int32)
    S = rng.integers(0, 160, size=(3, Hq, 4)).astype(np.int32)
    lists = oracle.vertical_slash_blocks(V, S, cu, max(lens))
    T = int(cu[-1])
    got = oracle.block_sparse_mask(*lists, cu, Hq)
    want = np.zeros((T * Hq, max(lens)), dtype=bool)
    for r, L in enumerate(lens):
        for h in range(Hq):
            bl = _vs_brute(V[r, h].tolist(), S[r, h].tolist(), L)
            for i in range(L):
                blocks, _ = bl[i // 64]
                for j in range(i + 1):
                    if 64 * (j // 64) in blocks or j in V[r, h].tolist():
                        want[(int(cu[r]) + i) * Hq + h, j] = True
    assert (got == _bits(want)).all(), "block-sparse mask differs from the definition"
    c = synth.prefill_case(950, lens, lens, Hq, Hkv, D, torch.float32, True, sm_scale=0.5)
    causal, _ = oracle.varlen_prefill(c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, 0.5, Hkv,
                                      k=c.k, v=c.v)
    all_diag = np.broadcast_to(np.arange(max(lens), dtype=np.int32), (3, Hq, max(lens)))
    none = np.zeros((3, Hq, 0), dtype=np.int32)
    o1, _ = oracle.sparse_prefill(c.q, c.k, c.v, cu, none, all_diag, c.sink, 0.5, Hkv)
    o2, _ = oracle.sparse_prefill(c.q, c.k, c.v, cu, all_diag, none, c.sink, 0.5, Hkv)
    _close(o1, causal, 1e-13, 1e-12, "every diagonal = causal")
    _close(o2, causal, 1e-13, 1e-12, "every column = causal")
    o3, l3 = oracle.sparse_prefill(c.q, c.k, c.v, cu, none, none, c.sink, 0.5, Hkv)
    assert (o3 == 0).all()
    _close(l3, np.broadcast_to(c.sink.numpy(), l3.shape), 1e-6, 1e-6, "no index: lse = sink")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
