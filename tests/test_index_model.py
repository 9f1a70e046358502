"""CPU models of the kernels' work-to-address mappings, checked for bounds.

Each model restates, in numpy, how a kernel turns its launch coordinates
(workgroup, wave, lane) and the device index data (cu_seqlens, cache_seqlens,
block tables) into the rows it reads and writes.  The assertions are facts
the kernels rely on and nothing else checks on the GPU: every query row,
rotary-table row, key/value row, block-table entry, partial-result slot and
output row lies inside its buffer, and every output row is written exactly
once.  The models run over every test shape of the GPU suite, the five
workloads and the edge cases (Lq > Lk, Lk = 0, empty requests), so a change
to a kernel's indexing that breaks a bound fails here, on the CPU, before it
can fault a GPU.  A model must change together with the kernel it models.
"""

import importlib
import math
import os
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

CUS = 256          # compute units the decode schedule is sized for
STREAM_WAVES = 4   # waves per workgroup of the balanced decode schedule
BN = 64            # prefill keys per tile
BM = 128           # prefill positions per workgroup tile


def heads_per_unit(G):
    return 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1


# ---------------------------------------------------------------------------
# prefill_bf16_kernel (csrc/prefill.hip)
# ---------------------------------------------------------------------------

def model_prefill(q_lens, k_lens, Hq, Hkv, D, window=-1, paged_bs=0, rope_rows=None,
                  causal=True):
    """Every access of one prefill launch; returns the number of (workgroup,
    step) blocks that did work.  rope_rows: rows of the rotary table (>= max
    Lk), or None.  With a causal window the launch walks runs of position
    blocks (run_steps blocks per workgroup), otherwise one block per
    workgroup.  Non-causal blocks read keys up to the request's last."""
    B = len(q_lens)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(k_lens)]).astype(np.int64)
    G = Hq // Hkv
    hpw = heads_per_unit(G)
    bm = BM // hpw
    ng = G // hpw
    max_q = max(q_lens, default=0)
    if window >= 0 and causal:
        per_req = (max_q + bm - 1) // bm
        blocks = B * per_req * ng * Hkv
        steps = min(16, max(1, blocks // (2 * CUS)))
        runs = (per_req + steps - 1) // steps
        grid = B * runs * ng * Hkv
        if grid == 0:
            return 0
        bid = np.arange(grid, dtype=np.int64)
        g = bid % Hkv
        rest = bid // Hkv
        hs = rest % ng
        rest = rest // ng
        r = rest % B                       # the last runs of the requests first
        u = runs - 1 - rest // B
        assert (u >= 0).all()
        # one entry per (workgroup, step)
        step = np.tile(np.arange(steps), grid)
        g, hs, u, r = (np.repeat(x, steps) for x in (g, hs, u, r))
        blk_index = u * steps + step
    else:
        max_q_tiles = (max_q + BM - 1) // BM
        grid = B * max_q_tiles * Hq
        if grid == 0:
            return 0
        bid = np.arange(grid, dtype=np.int64)
        p = bid % Hq
        slot = bid // Hq
        g = p % Hkv
        hs = (p // Hkv) % ng
        blk = (hpw - 1 - (p // Hkv) // ng + slot) % hpw
        r = slot % B
        qt = max_q_tiles - 1 - slot // B
        assert (qt >= 0).all()
        blk_index = qt * hpw + blk
    cq0, Lq = cu_q[r], cu_q[r + 1] - cu_q[r]
    live = blk_index * bm < Lq
    g, hs, r, blk_index, cq0, Lq = (x[live] for x in (g, hs, r, blk_index, cq0, Lq))
    ck0, Lk = cu_k[r], cu_k[r + 1] - cu_k[r]
    row0 = blk_index * bm
    nrows = np.minimum(bm, Lq - row0)
    pos0 = Lk - Lq + row0
    pos_last = pos0 + nrows - 1
    kv_lo = np.maximum(0, pos0 - window) if window >= 0 else np.zeros_like(pos0)
    kv_hi = np.minimum(Lk, pos_last + 1) if causal else Lk
    t_begin = kv_lo & ~(BN - 1)
    ntiles = np.where(kv_hi > kv_lo, (kv_hi - t_begin + BN - 1) // BN, 0)
    # K/V tiles: the first and the last tile issued lie inside the request's keys
    has = ntiles > 0
    assert (t_begin[has] >= 0).all()
    t_last = t_begin + (ntiles - 1) * BN
    assert (t_last[has] < Lk[has]).all(), "a K/V tile starts past the request's last key"
    rowbytes = Hkv * D * 2
    if not paged_bs:
        # one buffer per tile whose range (Lk - t0) rows must be positive and fit 32 bits
        assert ((Lk[has] - t_begin[has]) * rowbytes < 2 ** 32).all()
        assert (ck0[has] + t_last[has] < cu_k[-1]).all()
    else:
        bs = paged_bs
        U = D // 8
        RPI = 64 // U                      # key rows per load instruction
        assert bs >= RPI
        nblk = (Lk + bs - 1) // bs         # valid block-table entries of the request
        for k in range(int(ntiles.max(initial=0))):
            sel = k < ntiles
            t0 = t_begin[sel] + k * BN
            lk, nb = Lk[sel], nblk[sel]
            tail = t0 + BN > lk
            for i in range(U):             # load instructions of all four waves
                key0 = np.where(tail, np.minimum(t0 + RPI * i, lk - 1), t0 + RPI * i)
                assert (key0 >= 0).all() and (key0 < lk).all()
                assert ((key0 // bs) < nb).all(), "block-table entry past the request's blocks"
                for lrow in range(RPI):
                    row = np.where(tail, key0 + np.minimum(lrow, lk - 1 - key0), key0 + lrow)
                    assert (row < lk).all(), "a K/V row past the request's keys"
                    assert (row // bs == key0 // bs).all(), "a load instruction crosses a block"
    # waves: query rows, rotary-table rows and output rows
    written = np.zeros((int(cu_q[-1]), Hq), dtype=np.int64)
    for wave in range(4):
        h = g * G + hs * hpw + wave % hpw
        assert (h < Hq).all()
        wrow0 = row0 + 32 * (wave // hpw)
        wrows = np.maximum(0, np.minimum(32, Lq - wrow0))
        wpos0 = Lk - Lq + wrow0
        for lr in range(32):
            ok = lr < wrows
            qrow = cq0 + wrow0 + lr
            assert (qrow[ok] < cq0[ok] + Lq[ok]).all()
            if rope_rows is not None:
                tpos = wpos0 + lr
                trow = np.where(ok & (tpos >= 0), tpos, 0)
                assert (trow >= 0).all() and (trow < rope_rows).all(), "rotary row outside the table"
            np.add.at(written, (qrow[ok], h[ok]), 1)
    assert (written == 1).all(), "an output row written twice or not at all"
    return int(live.sum())


# ---------------------------------------------------------------------------
# decode_stream_kernel (balanced schedule) and decode_part_kernel (csrc/decode.hip)
# ---------------------------------------------------------------------------

def stream_lo(L, w):
    return np.maximum(0, L - 1 - w) if w >= 0 else np.zeros_like(L)


def stream_tiles(L, w):
    return np.where(L <= 0, 0, (L - (stream_lo(L, w) & ~15) + 15) >> 4)


def model_decode_stream(lens, Hq, Hkv, bs, mbps, window=-1, append=False):
    """Every tile of the balanced schedule: its block-table entry, the rows it
    reads, the wave that owns it and the partial-result slot it writes."""
    L = np.asarray(lens, dtype=np.int64) + (1 if append else 0)
    B = L.size
    assert bs >= 8 and (bs % 16 == 0 or bs == 8), "a 16-token tile lies in one block, or two of 8"
    HU = heads_per_unit(Hq // Hkv)
    NHG = Hq // HU
    K = max(1, (CUS * STREAM_WAVES + NHG - 1) // NHG)   # ranges (waves) per head group
    nw = K
    # the grid: ceil(NHG * K / 8) workgroups of 8 waves, head group fastest
    grid = (NHG * K + STREAM_WAVES - 1) // STREAM_WAVES
    gwid = np.arange(grid * STREAM_WAVES)
    assert set(zip((gwid % NHG)[gwid // NHG < K].tolist(), (gwid // NHG)[gwid // NHG < K].tolist())) \
        == {(h, k) for h in range(NHG) for k in range(K)}, "every (head group, range) has one wave"
    tiles = stream_tiles(L, window)
    cum = np.concatenate([[0], np.cumsum(tiles)])
    T = int(cum[-1])
    chunk = max(1, (T + nw - 1) // nw)
    x = np.arange(T, dtype=np.int64)
    b = np.searchsorted(cum, x, side="right") - 1
    assert (b >= 0).all() and (b < B).all()
    t = (stream_lo(L[b], window) & ~15) + 16 * (x - cum[b])
    assert (t >= 0).all() and (t < L[b]).all(), "a tile starts outside its sequence"
    assert ((t >> int(math.log2(bs))) < (L[b] + bs - 1) // bs).all(), "block entry past the sequence"
    assert ((t >> int(math.log2(bs))) < mbps).all()
    if bs >= 16:
        assert (t % bs + 16 <= bs).all()
    else:
        # block size 8: rows 8..15 come from the block of min(t + 8, L - 1),
        # a valid entry of the sequence's row
        t1 = np.minimum(t + 8, L[b] - 1)
        assert (t1 >= t).all() and ((t1 >> 3) < (L[b] + 7) // 8).all()
    gw = x // chunk
    assert (gw < nw).all(), "a tile past the last wave"
    slots = K + B
    assert (gw + b < slots).all(), "partial-result slot past the workspace"
    # the merge reads pieces(b) consecutive slots from first_slot(b)
    has = tiles > 0
    bb = np.arange(B)[has]
    pieces = (cum[bb + 1] - 1) // chunk - cum[bb] // chunk + 1
    first = cum[bb] // chunk + bb
    assert (pieces >= 1).all() and (first + pieces <= slots).all()
    # pieces(b) is exactly the number of waves whose range meets b
    owners = {}
    for xx, bx in zip(gw.tolist(), b.tolist()):
        owners.setdefault(bx, set()).add(xx)
    for k, bx in enumerate(bb.tolist()):
        assert len(owners[bx]) == pieces[k] and min(owners[bx]) + bx == first[k]
    if append:
        # the owner of each sequence's last tile stores row L - 1 (the new token)
        pos = L - 1
        assert ((pos >> int(math.log2(bs))) < mbps).all()
        # with a rotary table each wave rotates the q rows of the sequences
        # its range meets, b_first .. b_last, into q_rot [B, Hq, D], reading
        # table row L - 1 (the table has max(lens) + 1 rows)
        rope_rows = int(L.max()) if B else 0
        for w in np.unique(gw).tolist():
            xs = x[gw == w]
            b_first, b_last = int(b[xs[0]]), int(b[xs[-1]])
            assert 0 <= b_first <= b_last < B
            assert ((L[b_first:b_last + 1] - 1) < rope_rows).all(), "rotary row outside the table"
            assert ((L[b_first:b_last + 1] - 1) >= 0).all()
    return T


def model_block_batches(n, batch=64, plant_slot=False):
    """A wave's block-id batches over its n tiles: batch 0 is loaded into a
    register; batch k >= 1 is copied to LDS slot k % 2 when the wave switches
    to batch k - 1 (batch 1: before the first tile) and read from that slot
    when it switches to batch k.  Checks that every batch read was copied
    into the slot it is read from, at least one batch (64 tiles) earlier,
    and that no copy lands in a slot between the copy and the read of the
    batch it holds.  Returns the number of copies.  plant_slot: copy each
    batch into the slot the wave is reading (a planted mistake)."""
    nb = (n + batch - 1) // batch
    copies, reads = {}, {}                  # batch -> (tile index of the event, slot)
    if n > batch:
        copies[1] = (-1, 1)
    for k in range(1, nb):
        reads[k] = (batch * k, k % 2)
        if batch * (k + 1) < n:
            copies[k + 1] = (batch * k, (k if plant_slot else k + 1) % 2)
    for k, (tr, sr) in reads.items():
        assert k in copies, f"batch {k} read but never copied"
        tc, sc = copies[k]
        assert sc == sr, "batch read from another slot than it was copied to"
        assert tr - tc >= batch or tc == -1, "batch read less than one batch after its copy"
        for j, (tj, sj) in copies.items():
            assert not (j != k and sj == sr and tc < tj <= tr), "slot overwritten before its read"
    assert set(copies) == set(reads)
    return len(copies)


def model_stream_merge(B, Hq, D):
    """The merge launch of the two-launch balanced decode: one wave per
    (sequence, HU heads), HU = 256 / D halved until it divides Hq; every
    (sequence, head) row merged by exactly one wave, 16 bytes (or fewer, with
    fewer heads) of each head row per lane."""
    HU = 256 // D
    while Hq % HU:
        HU //= 2
    NHG = Hq // HU
    waves = B * NHG
    grid = (waves + 3) // 4
    seen = np.zeros((B, Hq), dtype=np.int64)
    for w in range(grid * 4):
        if w >= waves:
            continue
        b, h0 = w // NHG, (w % NHG) * HU
        assert 0 <= b < B and 0 <= h0 and h0 + HU <= Hq
        seen[b, h0:h0 + HU] += 1
    assert (seen == 1).all(), "a row merged twice or never"
    E = HU * D // 64
    assert E in (1, 2, 4) and 64 * E == HU * D


def model_decode_stream_parts(lens, Hq, Hkv, bs, P, max_parts, window=-1):
    """The balanced schedule in partition mode: each wave's range snapped up to
    partition starts.  Every tile belongs to exactly one range, every partition
    with tiles lies wholly in one range, and every part_out row written is
    inside [B, Hq, max_parts]."""
    L = np.asarray(lens, dtype=np.int64)
    B = L.size
    assert P % 16 == 0 and P % bs == 0
    HU = heads_per_unit(Hq // Hkv)
    NHG = Hq // HU
    K = max(1, (CUS * STREAM_WAVES + NHG - 1) // NHG)
    tiles = stream_tiles(L, window)
    cum = np.concatenate([[0], np.cumsum(tiles)])
    T = int(cum[-1])
    chunk = max(1, (T + K - 1) // K)
    lo_al = stream_lo(L, window) & ~15

    def snap(x):
        if x >= T:
            return T
        b = int(np.searchsorted(cum, x, side="right") - 1)
        if x == cum[b]:
            return x
        t = int(lo_al[b]) + 16 * (x - int(cum[b]))
        if t % P == 0:
            return x
        return min(int(cum[b]) + ((t // P + 1) * P - int(lo_al[b])) // 16, int(cum[b + 1]))

    owner = np.full(T, -1)
    for k in range(K):
        x0, x1 = snap(min(T, k * chunk)), snap(min(T, (k + 1) * chunk))
        assert x0 <= x1
        assert (owner[x0:x1] == -1).all(), "two ranges share a tile"
        owner[x0:x1] = k
    assert (owner >= 0).all(), "a tile in no range"
    x = np.arange(T)
    b = np.searchsorted(cum, x, side="right") - 1
    t = lo_al[b] + 16 * (x - cum[b])
    part = t // P
    assert (part < max_parts).all(), "part_out row past max_partitions"
    assert (t < L[b]).all()
    key = b * max_parts + part
    for kk in np.unique(key):
        assert np.unique(owner[key == kk]).size == 1, "a partition split between waves"
    return T


def model_decode_part(lens, Hq, Hkv, bs, part_size, window=-1):
    """Fixed partitions: every (sequence, head group, partition) unit's tiles."""
    L = np.asarray(lens, dtype=np.int64)
    msk = int(L.max(initial=0))
    nparts = max(1, (max(msk, 1) + part_size - 1) // part_size)
    HU = heads_per_unit(Hq // Hkv)
    NHG = Hq // HU
    for pidx in range(nparts):
        start = np.full_like(L, pidx * part_size)
        end = np.minimum(start + part_size, L)
        if window >= 0:
            start = np.maximum(start, L - 1 - window)
        tile0 = start & ~15
        ntiles = np.where(start < end, (end - tile0 + 15) >> 4, 0)
        has = ntiles > 0
        last = tile0 + 16 * (ntiles - 1)
        assert (tile0[has] >= 0).all() and (last[has] < L[has]).all()
        assert ((last[has] // bs) < (L[has] + bs - 1) // bs).all()
        if bs == 8:
            t1 = np.minimum(last + 8, L - 1)
            assert ((t1[has] >> 3) < (L[has] + 7) // 8).all()
    return nparts * NHG * L.size


# ---------------------------------------------------------------------------
# shapes: the GPU suite's cases, the five workloads and edge cases
# ---------------------------------------------------------------------------

def _gpu_module(name):
    return importlib.import_module(name)


def prefill_shapes():
    P = _gpu_module("test_gpu_prefill")
    R = _gpu_module("test_gpu_rope")
    shapes = []
    for q_lens, k_lens, Hq, Hkv, D, sink, window in P.CASES:
        shapes.append((q_lens, k_lens or q_lens, Hq, Hkv, D, window, 0))
    for q_lens, k_lens, Hq, Hkv, D, bs, sink, window in P.PAGED:
        shapes.append((q_lens, k_lens, Hq, Hkv, D, window, bs))
    for q_lens, k_lens, Hq, Hkv, D, sink, window, bs in P.NONCAUSAL:
        shapes.append((q_lens, k_lens or q_lens, Hq, Hkv, D, window, bs))
    for case in R.PREFILL:
        q_lens, k_lens, Hq, Hkv, D, rd, neox, bs = case
        shapes.append((q_lens, k_lens or q_lens, Hq, Hkv, D, -1, bs))
    import synth
    L3 = synth.config3_lengths()
    shapes += [
        ([10, 3, 1], [10, 3, 1], 4, 2, 64, -1, 0),                 # workload 1 (prefill)
        ([10, 3, 1], [0, 1, 7], 4, 2, 64, -1, 0),                  # the varlen example, Lq > Lk
        ([10, 3, 1], [0, 1, 7], 4, 2, 64, -1, 16),
        (L3, L3, 32, 8, 128, -1, 0),                               # workload 3
        ([512] * 4, [8704] * 4, 64, 8, 64, 128, 16),               # workload 4
        ([0, 5, 300], [0, 5, 300], 8, 8, 128, 3, 16),              # empty request, window
        ([129, 1], [0, 0], 12, 4, 128, -1, 0),                     # no keys at all
        ([1000], [70], 16, 2, 64, 17, 32),                         # Lq > Lk with a window
        ([64, 65, 127, 128, 129], [64, 65, 127, 128, 129], 6, 2, 128, 0, 16),
    ]
    return shapes


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window_override", [None, 0, 50])
def test_prefill_mapping_in_bounds(window_override, causal):
    n = 0
    for q_lens, k_lens, Hq, Hkv, D, window, bs in prefill_shapes():
        w = window if window_override is None else window_override
        for paged in sorted({0, bs}):
            n += model_prefill(q_lens, k_lens, Hq, Hkv, D, w, paged,
                               rope_rows=max(max(k_lens, default=0), 1), causal=causal)
    assert n > 0


def model_rope_keys(k_lens, Hkv, D, max_len, rope_rows, ws_rows):
    """rope_keys_kernel (csrc/rope.hip): thread -> (request r, position j,
    kv head h, 16-byte chunk u) over B * max_len * Hkv * D/8 threads; a thread
    with j < L_r reads key row cu[r] + j and table row j and writes the same
    row of the workspace.  Every key row is covered once, and every row read
    or written lies inside k, the table and the workspace."""
    L = np.asarray(k_lens, dtype=np.int64)
    B = L.size
    cu = np.concatenate([[0], np.cumsum(L)])
    cpr = D // 8
    n = B * max_len * Hkv * cpr
    grid = (n + 255) // 256
    idx = np.arange(grid * 256, dtype=np.int64)
    u = idx % cpr
    rest = idx // cpr
    h = rest % Hkv
    rest //= Hkv
    j = rest % max_len
    r = rest // max_len
    live = r < B
    r, j, h, u = r[live], j[live], h[live], u[live]
    act = j < L[r]
    row = cu[r][act] + j[act]
    assert (row < cu[-1]).all() and (row >= 0).all(), "key row outside k"
    assert (row < ws_rows).all(), "row outside the workspace"
    assert (j[act] < rope_rows).all(), "table row outside the table"
    # each (row, head, chunk) exactly once
    key = (row * Hkv + h[act]) * cpr + u[act]
    assert np.unique(key).size == key.size == cu[-1] * Hkv * cpr
    return int(act.sum())


def test_rope_keys_mapping_in_bounds():
    n = 0
    for q_lens, k_lens, Hq, Hkv, D, window, bs in prefill_shapes():
        if not k_lens:
            continue
        mx = max(k_lens)
        # the workspace holds B * max_seqlen_k rows; the table max_seqlen_k rows
        n += model_rope_keys(k_lens, Hkv, D, mx, rope_rows=mx, ws_rows=len(k_lens) * mx)
    assert n > 0
    with pytest.raises(AssertionError):     # a table one row short
        model_rope_keys([5, 9], 2, 64, 9, rope_rows=8, ws_rows=18)


RUN_SLOTS = 4      # tile slots of the LDS ring of a run


def model_run_ring(q_lens, k_lens, Hq, Hkv, window, causal=True, slots=RUN_SLOTS):
    """The tile ring of a run of position blocks (prefill_bf16_kernel, RUN):
    per step, its tile range [tb0, tb1) is taken in chunks (all of it when it
    fits in the ring, else half the ring at a time); a chunk's missing tiles
    are loaded (tile n into slot n % slots), then the next chunk's tiles that
    continue the resident range are prefetched into slots the chunk does not
    read.  Checks, for every run of every request, that each computed tile is
    in its slot when the chunk computes it and that no prefetch refills a slot
    the chunk reads.  Returns the number of tile loads."""
    G = Hq // Hkv
    hpw = heads_per_unit(G)
    bm = BM // hpw
    B = len(q_lens)
    max_q = max(q_lens, default=0)
    per_req = (max_q + bm - 1) // bm
    blocks = B * per_req * (G // hpw) * Hkv
    steps = min(16, max(1, blocks // (2 * CUS)))
    runs = (per_req + steps - 1) // steps

    def keys(row0, Lq, Lk):
        nr = min(bm, Lq - row0)
        p0 = Lk - Lq + row0
        lo = max(0, p0 - window) if window >= 0 else 0
        hi = min(Lk, p0 + nr) if causal else Lk
        tb = lo & ~(BN - 1)
        return tb // BN, ((hi - tb + BN - 1) // BN if hi > lo else 0)

    def chunk_of(nt):
        return slots if nt <= slots else max(1, slots // 2)

    loads = 0
    for Lq, Lk in zip(q_lens, k_lens):
        for u in range(runs):
            slot = [None] * slots
            res_lo = res_hi = 0
            for s in range(steps):
                row0 = (u * steps + s) * bm
                if row0 >= Lq:
                    break
                tb0, nt = keys(row0, Lq, Lk)
                tb1 = tb0 + nt
                has_next = s + 1 < steps and row0 + bm < Lq
                nx_tb, nx_nt = keys(row0 + bm, Lq, Lk) if has_next else (0, 0)
                ch = chunk_of(nt)
                for c0 in range(tb0, tb1, ch):
                    c1 = min(tb1, c0 + ch)
                    if c0 < res_lo or c0 > res_hi:
                        res_lo = res_hi = c0
                    while res_hi < c1:
                        slot[res_hi % slots] = res_hi
                        res_hi += 1
                        loads += 1
                    res_lo = max(res_lo, res_hi - slots)
                    if c1 < tb1:
                        n0, n1 = c1, min(tb1, c1 + ch)
                    elif has_next and nx_nt > 0:
                        n0, n1 = nx_tb, nx_tb + min(nx_nt, chunk_of(nx_nt))
                    else:
                        n0 = n1 = 0
                    pre = []
                    if n1 > n0 and res_lo <= n0 <= res_hi:
                        while res_hi < n1 and res_hi < c0 + slots:
                            assert res_hi % slots not in {t % slots for t in range(c0, c1)}, \
                                "a prefetch refills a slot the chunk reads"
                            pre.append(res_hi)
                            res_hi += 1
                            loads += 1
                        res_lo = max(res_lo, res_hi - slots)
                    for tn in range(c0, c1):
                        assert slot[tn % slots] == tn, "a computed tile is not in its slot"
                    for t in pre:
                        slot[t % slots] = t
    return loads


def test_run_ring_residency():
    import random
    n = 0
    for q_lens, k_lens, Hq, Hkv, D, window, bs in prefill_shapes():
        for w in sorted({window, 0, 50, 128, 300}):
            if w >= 0:
                n += model_run_ring(q_lens, k_lens or q_lens, Hq, Hkv, w)
    rnd = random.Random(5)
    for _ in range(300):               # windows, lengths and GQA shapes the suite does not hold
        Lk = rnd.randint(1, 3000)
        Lq = rnd.randint(1, Lk + 50)
        Hkv = rnd.choice([1, 2, 8])
        Hq = Hkv * rnd.choice([1, 2, 4, 8])
        w = rnd.choice([0, 1, 63, 64, 127, 129, 255, 1000])
        n += model_run_ring([Lq], [Lk], Hq, Hkv, w)
        n += model_run_ring([Lq], [Lk], Hq, Hkv, w, causal=False)
    assert n > 0
    # the chunked workload: 2 steps of 32 positions per run read the same 3 tiles
    assert model_run_ring([512] * 4, [8704] * 4, 64, 8, 128) == 4 * 8 * 3


def decode_shapes():
    Dm = _gpu_module("test_gpu_decode")
    shapes = []
    for lengths, Hq, Hkv, D, bs, sink, window in Dm.CASES:
        shapes.append((lengths, Hq, Hkv, bs, window))
    import synth
    rng = np.random.default_rng([1, 11])
    L2 = rng.integers(512, 4096, size=64, endpoint=True).tolist()
    shapes += [
        ([30, 32, 70], 4, 2, 32, -1),                              # workload 1 (the page example)
        (L2, 32, 8, 16, -1),                                       # workload 2
        ([131072] * 16, 32, 8, 64, -1),                            # workload 5
        ([0, 0, 0], 32, 8, 16, -1),
        (np.random.default_rng(61).integers(1, 40, size=1200).tolist(), 16, 2, 16, 9),
        ([1] * 4096, 32, 8, 16, -1),                               # the largest batch
    ]
    return shapes


def test_decode_stream_mapping_in_bounds():
    for lengths, Hq, Hkv, bs, window in decode_shapes():
        mbps = (max(max(lengths), 1) + 1 + bs - 1) // bs
        model_decode_stream(lengths, Hq, Hkv, bs, mbps, window)
        model_decode_stream(lengths, Hq, Hkv, bs, mbps, window, append=True)
        for D in (64, 128):
            model_stream_merge(len(lengths), Hq, D)


def test_block_batches():
    """The LDS double buffer of block-id batches, for every range length up to
    a few batches past the boundaries, and the C5-sized ranges."""
    for n in list(range(0, 400)) + [1024, 1025, 2047, 131072 // 16 // 128 * 16]:
        copies = model_block_batches(n)
        assert copies == max(0, (n + 63) // 64 - 1)


def test_decode_partition_mapping_in_bounds():
    for lengths, Hq, Hkv, bs, window in decode_shapes():
        if len(lengths) > 512:
            continue
        for P in sorted({bs, 2 * bs, 512 if 512 % bs == 0 else bs}):
            model_decode_part(lengths, Hq, Hkv, bs, P, window)
            if P % 16 == 0:         # bf16 partitions (the balanced stream) are whole tiles
                maxp = max(1, (max(max(lengths), 1) + P - 1) // P)
                model_decode_stream_parts(lengths, Hq, Hkv, bs, P, maxp, window)


def test_models_catch_a_planted_mistake():
    """The models are not vacuous: a prefill whose last tile would start at the
    request's end (ntiles one too many), or a decode table entry one block too
    far, fails their bounds."""
    with pytest.raises(AssertionError):
        # a rotary table one row short of the longest request
        model_prefill([100, 7], [300, 7], 8, 2, 64, -1, 0, rope_rows=299)
    with pytest.raises(AssertionError):
        # a block table one block short for the appended token
        model_decode_stream([16, 31], 8, 2, 16, mbps=1, append=True)
    with pytest.raises(AssertionError):
        # block ids copied into the LDS slot the wave is reading from
        model_block_batches(200, plant_slot=True)


# ---------------------------------------------------------------------------
# vertical_slash_kernel and sparse_prefill_kernel (csrc/sparse.hip)
# ---------------------------------------------------------------------------

def model_sparse(lens, H, Hkv, D, V, S):
    """The block lists (the oracle's conversion, equal to the kernel's by the
    GPU tests) and every access of the conversion and of the sparse prefill:
    bit-set words, list slots, K/V rows, gathered positions, output rows."""
    import oracle
    import synth
    cu = synth.cu_from_lengths(lens).numpy().astype(np.int64)
    Lmax = max(lens)
    NM = (Lmax + 63) // 64
    NMW = (NM + 31) // 32
    NV, NS = V.shape[2], S.shape[2]
    bc, bo, cc, ci = oracle.vertical_slash_blocks(V, S, cu, Lmax)
    rowbytes = Hkv * D * 2
    U = D // 8
    RPI = 64 // U
    for b, L in enumerate(lens):
        for h in range(H):
            for m in range(NM):
                r0 = 64 * m
                if r0 >= L:
                    assert bc[b, h, m] == 0 and cc[b, h, m] == 0
                    continue
                r1 = min(L, r0 + 64)
                # conversion: the bit-set words a diagonal or a column touches
                s = S[b, h]
                s = s[(s >= 0) & (s < L) & (r1 - 1 - s >= 0)]
                hi = (r1 - 1 - s) >> 6
                lo = np.maximum(0, r0 - s) >> 6
                assert (hi >> 5 < NMW).all() and (lo >> 5 < NMW).all()
                v = V[b, h]
                v = v[(v >= 0) & (v < r1)]
                assert (v >> 11 < NMW).all()
                assert bc[b, h, m] <= NM and cc[b, h, m] <= NV
                # prefill: 64-key blocks inside the request, descriptor range
                # positive and within 32 bits; gathered rows inside it
                t0 = bo[b, h, m, :bc[b, h, m]]
                assert (t0 % 64 == 0).all() and (t0 >= 0).all() and (t0 < L).all()
                assert ((L - t0) * rowbytes < 2 ** 32).all()
                cols = ci[b, h, m, :cc[b, h, m]]
                assert (cols >= 0).all() and (cols < L).all()
                for c0 in range(0, int(cc[b, h, m]), 64):
                    for i in range(U):            # load instructions of both waves
                        for lrow in range(RPI):
                            e = c0 + RPI * i + lrow
                            col = cols[e] if e < cc[b, h, m] else cols[c0]
                            assert 0 <= col < L and col * rowbytes + rowbytes <= 2 ** 32
                # output rows of both waves
                for w in range(2):
                    wrow0 = r0 + 32 * w
                    wrows = max(0, min(32, L - wrow0))
                    assert wrows == 0 or wrow0 + wrows <= L
    return int(bc.sum() + cc.sum())


def test_sparse_mapping_in_bounds():
    import synth
    G = _gpu_module("test_gpu_sparse")
    n = 0
    for lens, Hq, Hkv, D, sink, kind in G.SPARSE:
        V, S = G._indices(70 + len(lens), lens, Hq, kind)
        n += model_sparse(lens, Hq, Hkv, D, V.numpy(), S.numpy())
    V, S = synth.vertical_slash_pattern(6, [4096, 100], 4)
    n += model_sparse([4096, 100], 4, 2, 128, V.numpy(), S.numpy())
    assert n > 0
