#!/usr/bin/env python3
"""Benchmark of the paged-KV attention library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--skip-long]

One "step" of the headline workload is one bf16 paged decode over 64
sequences with cache_seqlens ~ U[512, 4096], 32 query / 8 kv heads, head_dim
128, block size 16 and a shuffled block pool: one launch of the balanced
decode kernel, whose last wave per (sequence, head group) merges the pieces
by log-sum-exp, on torch's current stream.
Inputs are resident in HBM before the timed region; K steps are timed
between a synchronize on each side, each kernel with its own pair of HIP
events.  Consecutive steps alternate between two copies of the KV pool so
that no step finds its keys in the 256 MB last-level cache.

The other workloads (varlen prefill with reshape_and_cache, chunked paged
prefill with a window, long-context split decode) are timed the same way and
reported in the same JSON line under "workloads".  The fp64 CPU oracle is
timed on the host cores, at all threads and at one thread, for every workload
("cpu_baseline", bounded samples of the larger ones).

Peaks: HBM3E 8.0 TB/s, dense bf16 MFMA 2.5 PFLOP/s (MI355X public figures).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--only", default="all",
                   choices=["all", "decode", "prefill", "chunked", "longctx", "sparse", "none"])
    p.add_argument("--skip-long", action="store_true", help="skip the 131072-token workload")
    p.add_argument("--spinup", type=float, default=0.3,
                   help="seconds of untimed steps before the warmup steps of each workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--partition-size", type=int, default=0,
                   help="headline decode partition size (0 = automatic balanced schedule)")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="also run a plain device copy of this size (counter calibration)")
    return p.parse_args()


ARGS = parse()
if ARGS.gpus != 1:
    print(f"bench.py runs on one GPU only (asked for --gpus {ARGS.gpus}); the library has no "
          f"multi-GPU path.", file=sys.stderr)
    sys.exit(2)

import numpy as np  # noqa: E402
import torch  # noqa: E402

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import synth  # noqa: E402
from paged_kv_cache_02_amd import pkv  # noqa: E402


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class NoTimer:
    """Passed to a step outside the kernel timing: launches only."""

    def time(self, name, fn):
        return fn()


class Preparer:
    """Passed to a step to collect its launches: each named launch becomes a
    prepared launcher (pkv.prepare: arguments marshalled once, no Python
    checks when it runs), so that a timing loop is not limited by the
    host's call overhead."""

    def __init__(self):
        self.launchers = {}

    def time(self, name, fn):
        self.launchers.setdefault(name, []).append(pkv.prepare(fn))


class KernelTimes:
    def __init__(self, ms):
        self.ms = ms

    def mean_ms(self, name):
        return self.ms[name]

    def names(self):
        return set(self.ms)


# how each kernel's launch time was taken, in the order the kernels were
# timed: "eager" (back-to-back launches from the host) or "graph" (one replay
# of a HIP graph of the same launches)
KERNEL_TIMING = []
GRAPH_BELOW_MS = 0.06      # kernels shorter than this are also timed through a graph
WORKLOAD = ""              # the workload being timed (names the marker ranges)


def _range(label):
    """Push a named range (roctx under ROCm: rocprofv3 --marker-trace records
    it), so that a kernel trace can pick out each timed block of launches."""
    try:
        torch.cuda.nvtx.range_push(label)
        return True
    except Exception:           # noqa: BLE001 - no marker library: nothing to mark
        return False


def _range_end(pushed):
    if pushed:
        torch.cuda.nvtx.range_pop()


def kernel_ms(launchers, steps, warmup, stream, name):
    """Mean duration of one launch: HIP events on the launch stream around
    `steps` back-to-back launches (cycling through the replicas' launchers),
    after `warmup` untimed ones.  A kernel shorter than GRAPH_BELOW_MS is
    issued by the host faster than it runs only barely, if at all (a Python
    call costs tens of µs), so its launches are also captured once in a HIP
    graph and replayed, and the faster of the two timings is kept; the
    method is noted in KERNEL_TIMING.  Longer kernels keep the eager timing
    (graph replays ran them no faster)."""
    with torch.cuda.stream(stream):
        for i in range(warmup):
            launchers[i % len(launchers)]()
    torch.cuda.synchronize()

    def timed(body, kind):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        pushed = _range(f"timed|{WORKLOAD}|{name}|{kind}")
        with torch.cuda.stream(stream):
            e0.record(stream)
            body()
            e1.record(stream)
        e1.synchronize()
        _range_end(pushed)
        return e0.elapsed_time(e1) / steps

    def eager():
        for i in range(steps):
            launchers[i % len(launchers)]()
    ms = timed(eager, "eager")
    method = "eager"
    if ms < GRAPH_BELOW_MS:
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                eager()
            with torch.cuda.stream(stream):   # a graph replays on the current stream
                g.replay()                    # once untimed
            torch.cuda.synchronize()
            gms = timed(g.replay, "graph")
            if gms < ms:
                ms, method = gms, "graph"
        except Exception as exc:              # noqa: BLE001 - capture failed: eager timing
            method = f"eager (graph capture failed: {type(exc).__name__})"
            torch.cuda.synchronize()
    KERNEL_TIMING.append({"workload": WORKLOAD, "kernel": name, "method": method,
                          "ms": round(ms, 4)})
    return ms


def spin_up(step, seconds):
    """Repeat the step until `seconds` of wall time have passed, so the GPU
    runs at its sustained clocks when timing starts (a cold GPU runs the
    prefill kernel ~15 % slower for its first tens of milliseconds)."""
    t_end = time.perf_counter() + seconds
    i = 0
    nt = NoTimer()
    while time.perf_counter() < t_end:
        for _ in range(8):
            step(i, nt)
            i += 1
        torch.cuda.synchronize()


def timed_steps(step, steps, warmup, reps=1):
    """Spin-up, warmup steps, then timed steps (wall clock between two
    synchronizations: ms per step); then each kernel of the step timed on
    its own with HIP events over back-to-back prepared launches of the
    `reps` input replicas.  Returns (ms per step, KernelTimes)."""
    spin_up(step, ARGS.spinup)
    for i in range(warmup):
        step(i, NoTimer())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, NoTimer())
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # the launchers are prepared on a side stream (default priority), which
    # they then launch on and which the graph capture uses
    side = torch.cuda.Stream()
    pr = Preparer()
    with torch.cuda.stream(side):
        for i in range(reps):
            step(i, pr)
    kms = {name: kernel_ms(ls, steps, warmup, side, name) for name, ls in pr.launchers.items()}
    return ms, KernelTimes(kms)


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic.md")
# source files of each kernel whose PMC traffic is recorded in the summary
KERNEL_SOURCES = {
    "decode_c2": ("decode_impl.h", "decode.hip", "decode.h", "common.h", "rope.h"),
    "merge_c2": ("decode_impl.h", "decode.hip", "decode.h", "common.h", "rope.h"),
    "decode_c2_one_launch": ("decode_impl.h", "decode.hip", "decode.h", "common.h", "rope.h"),
    "prefill_c3": ("prefill.hip", "tile.h", "decode.h", "common.h"),
    "prefill_c4": ("prefill.hip", "tile.h", "decode.h", "common.h"),
    "reshape_c3": ("cache.hip", "common.h"),
    "reshape_rope_c3": ("rope.hip", "rope.h", "decode.h", "common.h"),
    "sparse_32k": ("sparse.hip", "tile.h", "decode.h", "common.h"),
}


def sources_digest(key):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[key]:
        with open(os.path.join(ROOT, "paged_kv_cache_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_traffic(key):
    """HBM bytes per launch of one kernel on one workload, from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summary (copy-calibrated); None when the
    summary has no row for it or the kernel's sources changed since."""
    try:
        with open(TRAFFIC_SUMMARY) as fh:
            text = fh.read()
    except OSError:
        return None
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 7 and cells[0] == key:
            if cells[3] != sources_digest(key):
                return None
            return int(cells[6].replace(",", ""))
    return None


def roofline(bound, achieved, peak, unit, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


# ----------------------------------------------------------------------------
# decode workloads
# ----------------------------------------------------------------------------

def decode_bytes(c):
    """Algorithmic bytes of one decode: K and V of every attended token, q,
    the output, the used block-table entries and the sequence lengths."""
    L = c.cache_seqlens.numpy().astype(np.int64)
    kv = int(L.sum()) * c.Hkv * c.D * 2 * 2
    q = c.B * c.Hq * c.D * 2
    table = int(np.sum((L + c.block_size - 1) // c.block_size)) * 4 + c.B * 4
    return kv, q, table


def replicate_pool(c, reps):
    """reps copies of the block pool in one allocation; copy r is reached
    through block_table + r * num_blocks (same values, disjoint memory)."""
    kc = c.k_cache.cuda().repeat(reps, 1, 1, 1)
    vc = c.v_cache.cuda().repeat(reps, 1, 1, 1)
    bt = c.block_table.cuda()
    tables = [torch.where(bt >= 0, bt + r * c.num_blocks, bt).contiguous() for r in range(reps)]
    return kc, vc, tables


def alibi_slopes(Hq):
    """The usual geometric ALiBi slopes 2^(-8 (h + 1) / Hq)."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=torch.float32)


def bench_decode(c, name, steps, warmup, partition_size, reps, traffic_key=None,
                 two_stage=False, alibi=None):
    """partition_size 0: the automatic (balanced) schedule, whose stage and
    merge launches pkv_paged_decode issues one after the other (two_stage:
    the same two launches through their own calls, timed apart); -1: the
    balanced schedule in one launch with the merge fused in; > 0: fixed
    partitions + merge."""
    global WORKLOAD
    WORKLOAD = name
    B, Hq, D = c.B, c.Hq, c.D
    kc, vc, tables = replicate_pool(c, reps)
    q = c.q.cuda()
    sl = c.cache_seqlens.cuda()
    al = None if alibi is None else alibi.cuda()
    sink = None if c.sink is None else c.sink.cuda()
    out = torch.empty_like(q)
    msk = c.max_seqlen_k
    P = partition_size
    ws_bytes = pkv.decode_workspace_bytes(B, Hq, D, msk, P)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    split = P > 0 and P < msk
    nparts = (msk + P - 1) // P if split else 1
    if split:
        part_out = torch.empty((B, Hq, nparts, D), dtype=torch.float32, device="cuda")
        part_lse = torch.empty((B, Hq, nparts), dtype=torch.float32, device="cuda")

    def step(i, kt):
        bt = tables[i % reps]
        if P == 0 and two_stage:
            kt.time("decode", lambda: pkv.paged_decode_stage(q, kc, vc, bt, sl, c.sm_scale, msk,
                                                             ws, c.window_left))
            kt.time("merge", lambda: pkv.paged_decode_finish(out, ws, c.Hkv, sink=sink))
        elif split:
            kt.time("decode", lambda: pkv.paged_decode_partitions(
                q, kc, vc, bt, sl, c.sm_scale, P, msk, c.window_left, part_out, part_lse))
            kt.time("merge", lambda: pkv.merge_partitions(part_out, part_lse, sl, P, sink=sink,
                                                          out=out))
        else:
            kt.time("decode", lambda: pkv.paged_decode(q, kc, vc, bt, sl, c.sm_scale, sink=sink,
                                                       window_left=c.window_left,
                                                       partition_size=P, max_seqlen_k=msk,
                                                       out=out, workspace=ws, alibi_slopes=al))

    ms, kt = timed_steps(step, steps, warmup, reps)
    kv, qb, table = decode_bytes(c)
    step_bytes = kv + 2 * qb + table
    dec_ms = kt.mean_ms("decode")
    two = "merge" in kt.names()
    dec_bytes = kv + qb + table + (0 if two else qb)
    res = {
        "name": name, "value": round(step_bytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "ms_per_step": round(ms, 4), "algorithmic_bytes": step_bytes,
        "schedule": "balanced, stage + merge launches" if P == 0
        else "balanced, one launch (merge fused)" if P == -1
        else (f"partitions of {P}" if split else "unsplit"),
        "kernels_ms": {"decode": round(dec_ms, 4)},
        "roofline": roofline("hbm", dec_bytes / (dec_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                             pmc_traffic(traffic_key) if traffic_key else None),
    }
    if two:
        res["kernels_ms"]["merge"] = round(kt.mean_ms("merge"), 4)
    res["frac_of_hbm_peak_step"] = round(res["value"] / HBM_PEAK_GBS, 4)
    del kc, vc, tables
    torch.cuda.empty_cache()
    return res, out


def bench_decode_append(c, name, steps, warmup, reps):
    """Decode with the new token appended: each sequence's last cached token of
    the workload becomes the token being appended (L = cache_seqlens - 1
    tokens already cached), so the attended keys are those of the plain
    decode.  Timed as one pkv_paged_decode_append launch, and beside it the
    unfused equivalent: reshape_and_cache of the B new rows, then decode."""
    global WORKLOAD
    WORKLOAD = name
    B, Hq, D, bs = c.B, c.Hq, c.D, c.block_size
    kc, vc, tables = replicate_pool(c, reps)
    q = c.q.cuda()
    L = (c.cache_seqlens - 1).cuda()
    L1 = c.cache_seqlens.cuda()
    kn = synth.to_dtype(synth.normal(21, (B, c.Hkv, D), stream=1), q.dtype).cuda()
    vn = synth.to_dtype(synth.normal(21, (B, c.Hkv, D), stream=2), q.dtype).cuda()
    sink = None if c.sink is None else c.sink.cuda()
    out = torch.empty_like(q)
    msk = c.max_seqlen_k
    ws = torch.zeros(max(pkv.decode_workspace_bytes(B, Hq, D, msk), 256),
                     dtype=torch.uint8, device="cuda")
    ar = torch.arange(B, device="cuda")
    slots = [(t[ar, (L // bs).long()] * bs + L % bs).to(torch.int32) for t in tables]

    def fused(i, kt):
        bt = tables[i % reps]
        kt.time("append_decode", lambda: pkv.paged_decode_append(
            q, kn, vn, kc, vc, bt, L, c.sm_scale, sink=sink, window_left=c.window_left,
            max_seqlen_k=msk - 1, out=out, workspace=ws))

    def unfused(i, kt):
        bt = tables[i % reps]
        kt.time("reshape_and_cache", lambda: pkv.reshape_and_cache(kn, vn, kc, vc,
                                                                   slots[i % reps]))
        kt.time("decode", lambda: pkv.paged_decode(q, kc, vc, bt, L1, c.sm_scale, sink=sink,
                                                   window_left=c.window_left, max_seqlen_k=msk,
                                                   out=out, workspace=ws))

    ms, kt = timed_steps(fused, steps, warmup, reps)
    ms_u, kt_u = timed_steps(unfused, steps, warmup, reps)
    kv, qb, table = decode_bytes(c)          # K/V of the L + 1 attended keys, q, table
    new_rows = B * c.Hkv * D * 2 * 2         # the new K/V rows, written into the cache
    step_bytes = kv + 2 * qb + table + new_rows
    k_ms = kt.mean_ms("append_decode")
    res = {
        "name": name, "value": round(step_bytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "ms_per_step": round(ms, 4), "algorithmic_bytes": step_bytes,
        "kernels_ms": {"append_decode": round(k_ms, 4)},
        "roofline": roofline("hbm", step_bytes / (k_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"),
        "unfused_ms_per_step": round(ms_u, 4),
        "unfused_kernels_ms": {"reshape_and_cache": round(kt_u.mean_ms("reshape_and_cache"), 4),
                               "decode": round(kt_u.mean_ms("decode"), 4)},
        "speedup_vs_unfused": round(ms_u / ms, 3),
    }
    del kc, vc, tables
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------
# prefill workloads
# ----------------------------------------------------------------------------

def visible_pairs(q_lens, k_lens, window):
    n = 0
    for Lq, Lk in zip(q_lens, k_lens):
        p = np.arange(Lk - Lq, Lk, dtype=np.int64)
        hi = np.minimum(p, Lk - 1)
        lo = np.zeros_like(p) if window < 0 else np.maximum(0, p - window)
        n += int(np.maximum(0, hi - lo + 1).sum())
    return n


def rope_setup(c, rotary_dim=128, neox=True):
    """Rotary table over the longest request, and the positions of the
    packed queries (Lk - Lq + i) and keys (0 .. Lk - 1)."""
    tab = pkv.rope_cos_sin(max(c.k_lens), rotary_dim)
    qpos = np.concatenate([np.arange(Lk - Lq, Lk) for Lq, Lk in zip(c.q_lens, c.k_lens)])
    kpos = np.concatenate([np.arange(Lk) for Lk in c.k_lens])
    return {"tab": tab, "rd": rotary_dim, "neox": neox,
            "qpos": torch.from_numpy(qpos.astype(np.int32)).cuda(),
            "kpos": torch.from_numpy(kpos.astype(np.int32)).cuda()}


def bench_prefill(c, name, steps, warmup, reps, with_cache_write=False, traffic_key=None,
                  alibi=None, rope=None, rope_unfused=False, rope_k=False, keys_in_kernel=False):
    """rope: from rope_setup; q is then rotated inside the prefill (and K by
    reshape_and_cache_rope when with_cache_write), or, with rope_unfused, by a
    separate rope_apply launch before a plain prefill.  rope_k: the
    contiguous keys are rotated too in the same call, once into a workspace
    (or, keys_in_kernel, inside the attention kernel as it loads them; or,
    unfused, by a rope_apply launch of their own)."""
    global WORKLOAD
    WORKLOAD = name
    T = c.q.shape[0]
    fused = rope is not None and not rope_unfused
    rkw = dict(rope_cos_sin=rope["tab"], rotary_dim=rope["rd"], rope_neox=rope["neox"],
               rope_k=rope_k) if fused else {}
    if fused and rope_k:
        need = pkv.varlen_prefill_workspace_bytes(len(c.q_lens), c.max_seqlen_k, c.Hkv, c.D,
                                                  True, c.q.dtype)
        rkw["workspace"] = False if keys_in_kernel else \
            torch.empty(need, dtype=torch.uint8, device="cuda")
    qs = [c.q.cuda() for _ in range(reps)]
    cq, ck = c.cu_seqlens_q.cuda(), c.cu_seqlens_k.cuda()
    al = None if alibi is None else alibi.cuda()
    sink = None if c.sink is None else c.sink.cuda()
    out = torch.empty_like(qs[0])
    if c.paged:
        kc, vc, tables = replicate_pool(
            synth.DecodeCase(c.q[:1], c.k_cache, c.v_cache, c.block_table,
                             torch.zeros(1, dtype=torch.int32), None, c.block_size, 1.0),
            reps)
        ks = vs = None
    else:
        ks = [c.k.cuda() for _ in range(reps)]
        vs = [c.v.cuda() for _ in range(reps)]
    if with_cache_write:
        # the new K/V go into a shuffled paged pool of block size 16
        rng = np.random.default_rng(7)
        bt, nb = synth.pool_from_lengths(rng, c.k_lens, 16)
        slots = torch.cat([synth.slots_for_tokens(bt[r:r + 1].expand(L, -1).contiguous(),
                                                  list(range(L)), 16)
                           for r, L in enumerate(c.k_lens)]).cuda()
        kcache = torch.zeros((nb, 16, c.Hkv, c.D), dtype=c.q.dtype, device="cuda")
        vcache = torch.zeros_like(kcache)

    def step(i, kt):
        r = i % reps
        if with_cache_write and fused:
            kt.time("reshape_and_cache", lambda: pkv.reshape_and_cache_rope(
                ks[r], vs[r], kcache, vcache, slots, rope["kpos"], rope["tab"], rope["rd"],
                rope["neox"]))
        elif with_cache_write:
            kt.time("reshape_and_cache",
                    lambda: pkv.reshape_and_cache(ks[r], vs[r], kcache, vcache, slots))
        if rope_unfused:
            kt.time("rope_apply", lambda: pkv.rope_apply(qs[r], rope["qpos"], rope["tab"],
                                                         rope["rd"], rope["neox"]))
            if rope_k:
                kt.time("rope_apply_k", lambda: pkv.rope_apply(ks[r], rope["kpos"], rope["tab"],
                                                               rope["rd"], rope["neox"]))
        if c.paged:
            kt.time("prefill", lambda: pkv.varlen_prefill(
                qs[r], cq, ck, c.max_seqlen_q, c.max_seqlen_k, c.sm_scale, c.Hkv,
                k_cache=kc, v_cache=vc, block_table=tables[r], sink=sink,
                window_left=c.window_left, out=out, alibi_slopes=al, **rkw))
        else:
            kt.time("prefill", lambda: pkv.varlen_prefill(
                qs[r], cq, ck, c.max_seqlen_q, c.max_seqlen_k, c.sm_scale, c.Hkv, k=ks[r],
                v=vs[r], sink=sink, window_left=c.window_left, out=out, alibi_slopes=al, **rkw))

    ms, kt = timed_steps(step, steps, warmup, reps)
    pairs = visible_pairs(c.q_lens, c.k_lens, c.window_left)
    flops = 4 * c.D * c.Hq * pairs
    pre_ms = kt.mean_ms("prefill")
    res = {"name": name, "value": round(flops / (pre_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
           "ms_per_step": round(ms, 4), "algorithmic_flops": flops,
           "kernels_ms": {"prefill": round(pre_ms, 4)},
           "roofline": roofline("mfma", flops / (pre_ms * 1e-3) / 1e12, MFMA_BF16_PEAK_TFS,
                                "TFLOP/s", pmc_traffic(traffic_key) if traffic_key else None)}
    # bytes the method must move: q and out, plus K/V of the visible key range
    kv_tokens = 0
    for Lq, Lk in zip(c.q_lens, c.k_lens):
        lo = 0 if c.window_left < 0 else max(0, Lk - Lq - c.window_left)
        kv_tokens += Lk - lo
    byts = 2 * T * c.Hq * c.D * 2 + kv_tokens * c.Hkv * c.D * 2 * 2
    res["algorithmic_bytes"] = byts
    res["hbm_gbs"] = round(byts / (pre_ms * 1e-3) / 1e9, 2)
    if c.window_left >= 0:
        ridge = min(MFMA_BF16_PEAK_TFS * 1e12, flops / byts * HBM_PEAK_GBS * 1e9)
        res["min_roofline_tflops"] = round(ridge / 1e12, 2)
        res["frac_of_min_roofline"] = round(flops / (pre_ms * 1e-3) / ridge, 4)
    if rope_unfused:
        ra_ms = kt.mean_ms("rope_apply")
        res["kernels_ms"]["rope_apply"] = round(ra_ms, 4)
        if rope_k:
            rk_ms = kt.mean_ms("rope_apply_k")
            res["kernels_ms"]["rope_apply_k"] = round(rk_ms, 4)
            ra_ms += rk_ms
        res["prefill_plus_rope_apply_ms"] = round(pre_ms + ra_ms, 4)
    if with_cache_write:
        rc_ms = kt.mean_ms("reshape_and_cache")
        # K and V rows read and written; the rotated form also reads one
        # table row (rotary_dim float32) per token
        rbytes = 2 * sum(c.k_lens) * c.Hkv * c.D * 2 * 2
        if fused:
            rbytes += sum(c.k_lens) * rope["rd"] * 4
        res["reshape_and_cache_rope" if fused else "reshape_and_cache"] = {
            "value": round(rbytes / (rc_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
            "kernel_ms": round(rc_ms, 4), "algorithmic_bytes": rbytes,
            "roofline": roofline("hbm", rbytes / (rc_ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s",
                                 pmc_traffic("reshape_rope_c3" if fused else "reshape_c3"))}
    torch.cuda.empty_cache()
    return res, out


def sparse_pairs(lists, L):
    """Visible (row, key) pairs of every head under the block lists: the keys
    j <= i of each row block's 64-key blocks and columns."""
    bc, bo, cc, ci = lists
    H, NM = bc.shape[1], bc.shape[2]
    per_unit_rows = []
    total = 0
    for h in range(H):
        for m in range(NM):
            r0, r1 = 64 * m, min(L, 64 * m + 64)
            if r0 >= r1:
                continue
            rows = np.arange(r0, r1, dtype=np.int64)
            offs = bo[0, h, m, :bc[0, h, m]].astype(np.int64)      # ascending
            cols = np.sort(ci[0, h, m, :cc[0, h, m]].astype(np.int64))
            # whole blocks before the row's own, the row's own block up to
            # the row, and the columns at or before it
            full = np.searchsorted(offs, rows - 64, side="right")
            own = np.isin(rows & ~63, offs)
            n = 64 * full + own * ((rows & 63) + 1) + np.searchsorted(cols, rows, side="right")
            total += int(n.sum())
            per_unit_rows.append((h, r0, n))
    return total, per_unit_rows


def bench_sparse(steps, warmup):
    """Vertical + slash sparse prefill: the block lists, then the attention,
    on one request of 32768 tokens; the dense causal prefill of the same input
    timed beside it."""
    global WORKLOAD
    WORKLOAD = "sparse_prefill_1x32768_vs"
    c, V, S = synth.sparse_prefill_workload()
    L, Hq, D = c.q.shape
    q, k, v = c.q.cuda(), c.k.cuda(), c.v.cuda()
    cu = c.cu_seqlens_q.cuda()
    Vd, Sd = V.cuda(), S.cuda()
    lists = pkv.vertical_slash_blocks(Vd, Sd, cu, L)
    out = torch.empty_like(q)

    def step(i, kt):
        kt.time("lists", lambda: pkv.vertical_slash_blocks(Vd, Sd, cu, L))
        kt.time("sparse", lambda: pkv.sparse_prefill(q, k, v, cu, L, lists, c.sm_scale,
                                                     out=out))

    def dense(i, kt):
        kt.time("dense", lambda: pkv.varlen_prefill(q, cu, cu, L, L, c.sm_scale, c.Hkv, k=k,
                                                    v=v, out=out))

    ms, kt = timed_steps(step, steps, warmup)
    WORKLOAD = "sparse_prefill_1x32768_vs/dense"
    _, ktd = timed_steps(dense, steps, warmup)
    host = [t.cpu().numpy() for t in lists]
    pairs, _ = sparse_pairs(host, L)
    flops = 4 * D * pairs
    sp_ms, li_ms, de_ms = kt.mean_ms("sparse"), kt.mean_ms("lists"), ktd.mean_ms("dense")
    dense_flops = 4 * D * Hq * visible_pairs([L], [L], -1)
    achieved = flops / (sp_ms * 1e-3) / 1e12
    res = {"name": "sparse_prefill_1x32768_vs", "value": round(achieved, 2), "unit": "TFLOP/s",
           "ms_per_step": round(ms, 4), "algorithmic_flops": flops,
           "density_vs_causal": round(flops / dense_flops, 4),
           "kernels_ms": {"vertical_slash_blocks": round(li_ms, 4), "sparse_prefill": round(sp_ms, 4)},
           "dense_causal_prefill_ms": round(de_ms, 4),
           "speedup_vs_dense": round(de_ms / (sp_ms + li_ms), 3),
           "roofline": roofline("mfma", achieved, MFMA_BF16_PEAK_TFS, "TFLOP/s",
                                pmc_traffic("sparse_32k"))}
    if not ARGS.no_cpu_baseline:
        import oracle  # the CPU-baseline leg is the only bench code that runs the oracle
        n = host_threads()
        units = _sample(L * Hq, 2048, 60)
        t0 = time.perf_counter()
        oracle.sparse_prefill(c.q, c.k, c.v, c.cu_seqlens_q, V.numpy(), S.numpy(), None,
                              c.sm_scale, c.Hkv, units=units.tolist(), nthreads=n)
        dt = time.perf_counter() - t0
        # flops of the sampled units: their rows' visible keys
        _, rows = sparse_pairs(host, L)
        vis = np.zeros((Hq, L), dtype=np.int64)
        for h, r0, nn in rows:
            vis[h, r0:r0 + len(nn)] = nn
        ufl = float(vis[units % Hq, units // Hq].sum()) * 4 * D
        res["cpu_baseline"] = {"kind": "oracle", "unit": "GFLOP/s", "cores": n,
                               "value": round(ufl / dt / 1e9, 4), "seconds": round(dt, 3),
                               "sample": f"{len(units)} of {L * Hq} (token, head) units of the "
                                         f"sparse workload (seeded), block lists, mask and "
                                         f"fp64 masked attention, {n} threads"}
    del q, k, v, out, lists
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------
# oracle parity spot check and CPU baseline
# ----------------------------------------------------------------------------

def host_threads():
    for k in ("OMP_NUM_THREADS",):
        if os.environ.get(k, "").isdigit():
            return int(os.environ[k])
    return min(16, os.cpu_count() or 1)


def _sample(n_units, k, seed):
    """k distinct unit ids out of n_units (all of them when k >= n_units), sorted."""
    if k >= n_units:
        return None
    return np.sort(np.random.default_rng(seed).choice(n_units, k, replace=False))


CPU_MIN_SECONDS = 3.0      # each oracle timing repeats its pass until this much time has run


def _repeat_timed(fn):
    """Run fn() until CPU_MIN_SECONDS have elapsed (at least once, at most 50
    times); return (mean seconds per pass, passes, fn's last result)."""
    total, n, res = 0.0, 0, None
    while n < 50 and (n == 0 or total < CPU_MIN_SECONDS):
        t0 = time.perf_counter()
        res = fn()
        total += time.perf_counter() - t0
        n += 1
    return total / n, n, res


def oracle_decode_rate(c, units, threads):
    """Time the oracle on the (sequence, head) units of a decode workload (None:
    all); return (seconds, GB/s of the algorithmic bytes those units stand for:
    each query head's share, 1 / Hq of its sequence's K/V, q and out rows),
    with the seconds per pass and the number of passes timed."""
    import oracle  # the CPU-baseline leg is the only bench code that runs the oracle
    dt, n, (o, _) = _repeat_timed(lambda: oracle.paged_decode(
        c.q, c.k_cache, c.v_cache, c.block_table, c.cache_seqlens, c.sink, c.sm_scale,
        c.window_left, units=units, nthreads=threads))
    L = c.cache_seqlens.numpy().astype(np.int64)
    u = np.arange(c.B * c.Hq) if units is None else np.asarray(units)
    b = u // c.Hq
    byts = float(np.sum(L[b] * c.Hkv * c.D * 2 * 2 / c.Hq + 2 * c.D * 2))
    return dt, n, byts / dt / 1e9, o


def oracle_prefill_rate(c, units, threads):
    """Time the oracle on (token, head) units of a prefill workload (None: all);
    return (seconds per pass, passes, GFLOP/s of 4 D flops per visible (row, key) pair)."""
    import oracle
    dt, n, _ = _repeat_timed(lambda: oracle.varlen_prefill(
        c.q, c.cu_seqlens_q, c.cu_seqlens_k, c.sink, c.sm_scale, c.Hkv, k=c.k, v=c.v,
        k_cache=c.k_cache, v_cache=c.v_cache, block_table=c.block_table,
        block_size=c.block_size, window_left=c.window_left, units=units, nthreads=threads))
    vis = []
    for Lq, Lk in zip(c.q_lens, c.k_lens):
        pos = np.arange(Lk - Lq, Lk, dtype=np.int64)
        hi = np.minimum(pos, Lk - 1)
        lo = np.zeros_like(pos) if c.window_left < 0 else np.maximum(0, pos - c.window_left)
        vis.append(np.maximum(0, hi - lo + 1))
    vis = np.concatenate(vis)
    u = np.arange(len(vis) * c.Hq) if units is None else np.asarray(units)
    flops = float(np.sum(vis[u // c.Hq])) * 4 * c.D
    return dt, n, flops / dt / 1e9


def cpu_baseline(kind, c, n_all, n_one, seed, what):
    """The oracle as it stands, timed at all host threads and at one thread on
    bounded samples of the workload: kind 'decode' (GB/s) or 'prefill'
    (GFLOP/s).  n_all / n_one: units timed at each thread count (None: all)."""
    n = host_threads()
    units_total = c.B * c.Hq if kind == "decode" else c.q.shape[0] * c.Hq
    res = {"kind": "oracle", "unit": "GB/s" if kind == "decode" else "GFLOP/s", "cores": n}
    out = None
    for label, threads, k, sd in (("all_cores", n, n_all, seed), ("one_thread", 1, n_one, seed + 1)):
        units = None if k is None else _sample(units_total, k, sd)
        if kind == "decode":
            dt, passes, rate, o = oracle_decode_rate(c, units, threads)
            if units is None and label == "all_cores":
                out = o
        else:
            dt, passes, rate = oracle_prefill_rate(c, units, threads)
        res[label] = {"threads": threads, "seconds": round(dt, 5), "passes": passes,
                      "value": round(rate, 4),
                      "units": units_total if units is None else int(len(units))}
    res["value"] = res["all_cores"]["value"]
    res["sample"] = (f"{what}: {res['all_cores']['units']} of {units_total} "
                     f"({'sequence' if kind == 'decode' else 'token'}, head) units at {n} threads, "
                     f"{res['one_thread']['units']} at one thread (seeded), each timing repeated "
                     f"until {CPU_MIN_SECONDS:g} s have run or 50 passes (seconds = mean per pass); "
                     f"fp64 two-pass oracle")
    return res, out


def spot_check(out, want, units, Hq, what):
    b, h = units // Hq, units % Hq
    got = out.float().cpu().numpy()[b, h]
    ref = want[b, h]
    err = np.abs(got - ref)
    ok = bool(np.all(err <= 2e-2 + 1e-2 * np.abs(ref)))
    return {"what": what, "rows": int(len(units)), "max_abs_err": float(err.max()), "pass": ok}


# ----------------------------------------------------------------------------

def main():
    torch.cuda.init()
    dev = torch.cuda.get_device_properties(0)
    log(f"device {dev.name} CUs={dev.multi_processor_count}")
    steps, warmup = ARGS.steps, ARGS.warmup
    workloads = {}

    log("generating decode workload (64 seqs, U[512,4096], 32/8 heads, D 128, bs 16)")
    c2 = synth.config2_decode()
    head = None
    if ARGS.only in ("all", "decode"):
        head, out2 = bench_decode(c2, "decode_64x_U512-4096", steps, warmup,
                                  ARGS.partition_size, reps=2,
                                  traffic_key="decode_c2" if ARGS.partition_size == 0 else None,
                                  two_stage=ARGS.partition_size == 0)
        log(f"decode: {head['value']} GB/s step, kernel {head['roofline']['achieved']} GB/s")
        if ARGS.partition_size == 0:
            r1, _ = bench_decode(c2, "decode_64x_U512-4096_one_launch", steps, warmup, -1,
                                 reps=2)
            workloads["decode_one_launch"] = r1
            log(f"decode in one launch (merge fused): {r1['value']} GB/s step")
            rl, _ = bench_decode(c2, "decode_64x_U512-4096_alibi", steps, warmup, 0, reps=2,
                                 alibi=alibi_slopes(c2.Hq))
            workloads["decode_alibi"] = rl
            log(f"decode with ALiBi slopes: {rl['value']} GB/s step")
            ra = bench_decode_append(c2, "decode_append_64x_U512-4096", steps, warmup, reps=2)
            workloads["decode_append"] = ra
            log(f"decode with the new token appended: {ra['value']} GB/s step, "
                f"{ra['speedup_vs_unfused']}x the unfused reshape_and_cache + decode")

    if ARGS.only in ("all", "prefill"):
        log("prefill workload (8 reqs U[256,4096], 32/8 heads, D 128, sink)")
        c3 = synth.config3_prefill()
        r3, _ = bench_prefill(c3, "varlen_prefill_8x_U256-4096", steps, warmup, reps=2,
                              with_cache_write=True, traffic_key="prefill_c3")
        workloads["varlen_prefill"] = r3
        log(f"prefill: {r3['value']} TFLOP/s")
        if not ARGS.no_cpu_baseline:
            r3["cpu_baseline"], _ = cpu_baseline("prefill", c3, 32768, 4096, 30,
                                                 "the 8-request prefill workload")
        r3a, _ = bench_prefill(c3, "varlen_prefill_8x_U256-4096_alibi", steps, warmup, reps=2,
                               alibi=alibi_slopes(c3.Hq))
        workloads["varlen_prefill_alibi"] = r3a
        log(f"prefill with ALiBi slopes: {r3a['value']} TFLOP/s")
        rp = rope_setup(c3)
        r3r, _ = bench_prefill(c3, "varlen_prefill_8x_U256-4096_rope", steps, warmup, reps=2,
                               with_cache_write=True, rope=rp)
        r3u, _ = bench_prefill(c3, "varlen_prefill_8x_U256-4096_rope_unfused", steps, warmup,
                               reps=2, rope=rp, rope_unfused=True)
        r3r["unfused_prefill_plus_rope_apply_ms"] = r3u["prefill_plus_rope_apply_ms"]
        r3r["speedup_vs_unfused"] = round(r3u["prefill_plus_rope_apply_ms"] /
                                          r3r["kernels_ms"]["prefill"], 3)
        workloads["varlen_prefill_rope"] = r3r
        log(f"prefill with q rotated in the kernel: {r3r['value']} TFLOP/s, "
            f"{r3r['speedup_vs_unfused']}x rope_apply + prefill; reshape_and_cache_rope "
            f"{r3r['reshape_and_cache_rope']['value']} GB/s")
        r3k, _ = bench_prefill(c3, "varlen_prefill_8x_U256-4096_rope_qk", steps, warmup, reps=2,
                               rope=rp, rope_k=True)
        r3ku, _ = bench_prefill(c3, "varlen_prefill_8x_U256-4096_rope_qk_unfused", steps, warmup,
                                reps=2, rope=rp, rope_unfused=True, rope_k=True)
        r3kk, _ = bench_prefill(c3, "varlen_prefill_8x_U256-4096_rope_qk_keys_in_kernel", steps,
                                warmup, reps=2, rope=rp, rope_k=True, keys_in_kernel=True)
        for r in (r3k, r3kk):
            r["unfused_prefill_plus_rope_apply_ms"] = r3ku["prefill_plus_rope_apply_ms"]
            r["speedup_vs_unfused"] = round(r3ku["prefill_plus_rope_apply_ms"] /
                                            r["kernels_ms"]["prefill"], 3)
        workloads["varlen_prefill_rope_qk"] = r3k
        workloads["varlen_prefill_rope_qk_keys_in_kernel"] = r3kk
        log(f"prefill with q and k rotated in the call (keys once into a workspace): "
            f"{r3k['value']} TFLOP/s, {r3k['speedup_vs_unfused']}x rope_apply (q, k) + prefill; "
            f"keys rotated inside the attention kernel: {r3kk['value']} TFLOP/s, "
            f"{r3kk['speedup_vs_unfused']}x")
    if ARGS.only in ("all", "chunked"):
        log("chunked prefill workload (4 x 512 q on 8704 paged keys, window 128, 64/8, D 64)")
        c4 = synth.config4_chunked(poison=False, spare_blocks=0)
        # 48 replicas of q and the pool: ~1 GiB of touched bytes, so no step finds
        # its inputs in the 256 MB last-level cache
        r4, _ = bench_prefill(c4, "chunked_prefill_4x512_on_8704_w128", steps, warmup, reps=48,
                              traffic_key="prefill_c4")
        r4["replicas"] = 48
        workloads["chunked_prefill"] = r4
        if not ARGS.no_cpu_baseline:
            r4["cpu_baseline"], _ = cpu_baseline("prefill", c4, None, 16384, 40,
                                                 "the chunked-prefill workload")
        log(f"chunked: {r4['value']} TFLOP/s, {r4['hbm_gbs']} GB/s")
    if ARGS.only in ("all", "longctx") and not ARGS.skip_long:
        log("long-context decode workload (16 x 131072, bs 64, partitions of 512, sink)")
        c5 = synth.config5_split_decode()
        # the workload asks for 512-token partitions merged by log-sum-exp
        r5, out5 = bench_decode(c5, "split_decode_16x131072_P512", max(3, steps // 4), 2, 512,
                                reps=1)
        workloads["split_decode_long"] = r5
        r5b, _ = bench_decode(c5, "split_decode_16x131072_auto", max(3, steps // 4), 2, 0,
                              reps=1, two_stage=True)
        workloads["split_decode_long_auto"] = r5b
        if not ARGS.no_cpu_baseline:
            r5["cpu_baseline"], _ = cpu_baseline("decode", c5, 256, 16, 50,
                                                 "the long-context decode workload")
        log(f"long decode: {r5['value']} GB/s (P=512), {r5b['value']} GB/s (auto)")
        del c5
    if ARGS.only in ("all", "sparse"):
        log("sparse prefill workload (1 x 32768, 32/8 heads, D 128, vertical + slash, "
            "budget 0.3)")
        rs = bench_sparse(steps, warmup)
        workloads["sparse_prefill"] = rs
        log(f"sparse prefill: {rs['value']} TFLOP/s on {rs['density_vs_causal']} of the causal "
            f"pairs, lists {rs['kernels_ms']['vertical_slash_blocks']} ms, "
            f"{rs['speedup_vs_dense']}x the dense causal prefill")
    if ARGS.copy_calibration_mb:
        n = ARGS.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        workloads["copy_calibration"] = {"bytes_read": n * 4, "bytes_written": n * 4}

    line = {"metric": "decode KV GB/s (% HBM peak); prefill TFLOP/s (% bf16 MFMA peak)",
            "n_gpus": 1, "steps": steps, "warmup": warmup, "spinup_s": ARGS.spinup,
            "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded numpy PCG64, N(0,1) rounded to bf16)"}
    if head is not None:
        line.update({"value": head["value"], "unit": "GB/s", "ms_per_step": head["ms_per_step"],
                     "config": {"workload": "bf16 paged decode: 64 sequences, cache_seqlens "
                                            "U[512,4096], 32 q / 8 kv heads, head_dim 128, "
                                            "block_size 16, shuffled pool, no sink, no window",
                                "global_batch": 64, "seq_len": "U[512,4096]",
                                "parallelism": "single GPU",
                                "schedule": head["schedule"]},
                     "roofline": head["roofline"], "kernels_ms": head["kernels_ms"],
                     "frac_of_hbm_peak_step": head["frac_of_hbm_peak_step"]})
        if not ARGS.no_cpu_baseline:
            log("timing the fp64 oracle on the host cores")
            cb, o2 = cpu_baseline("decode", c2, None, None, 20, "the full headline workload")
            line["cpu_baseline"] = cb
            rng = np.random.default_rng(0)
            units = rng.choice(c2.B * c2.Hq, 64, replace=False)
            line["parity_spot_check"] = spot_check(out2, o2, units, c2.Hq, "decode vs oracle")
    line["workloads"] = workloads
    line["kernel_timing"] = {
        "method": "HIP events on the launch stream around back-to-back prepared launches "
                  "(steps per kernel); kernels under 60 us also through one replay of a HIP "
                  "graph of the same launches, the faster kept",
        "in_order": KERNEL_TIMING}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
