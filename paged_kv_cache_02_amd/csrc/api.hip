// extern "C" entry points of libpkv.so: argument checks on the host, workspace
// sizing, the split-KV choice, and launches on the caller's stream.  The
// operations and their arguments are documented in include/pkv.h.

#include "common.h"
#include "decode.h"

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <unistd.h>

using namespace pkv;

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) { int l = 0; while ((1 << l) < x) ++l; return l; }
bool dtype_ok(pkv_dtype d) { return d == PKV_F32 || d == PKV_BF16; }
int elem_bytes(pkv_dtype d) { return d == PKV_BF16 ? 2 : 4; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

pkv_status check_heads(int32_t Hq, int32_t Hkv, int32_t D) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return PKV_ERR_SHAPE;
    if (D != 64 && D != 128) return PKV_ERR_UNSUPPORTED;
    return PKV_OK;
}

pkv_status check_block_size(int32_t bs) {
    if (bs <= 0) return PKV_ERR_SHAPE;
    if (!is_pow2(bs) || bs < 8 || bs > 512) return PKV_ERR_UNSUPPORTED;
    return PKV_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Logit scale: a positive finite number (the kernels take the row maximum of
// q.k before or after scaling, which is the same only for a positive scale).
bool scale_ok(float s) { return s > 0.f && std::isfinite(s); }

// Epoch of one fused-merge launch: a per-process call counter (never 0),
// started from the clock and the process id so that a workspace a previous
// process left dirty is unlikely to hold a matching epoch either.
uint32_t next_epoch() {
    static std::atomic<uint32_t> counter{
        (uint32_t)std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761u ^
        ((uint32_t)getpid() << 16)};
    uint32_t v;
    do { v = counter.fetch_add(1, std::memory_order_relaxed); } while (v == 0);
    return v;
}

// Compute units of the current device (cached per device; 256 if unknown).
int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Balanced schedule: one workgroup of kStreamWaves waves (two per SIMD) per
// compute unit, the waves of a workgroup on the head groups of one token
// range; K ranges per head group.
int stream_ranges_hu(int Hq, int HU) {
    const int NHG = Hq / HU;
    return std::max(1, (device_cus() * kStreamWaves + NHG - 1) / NHG);
}
int stream_ranges_per_head_group(int Hq, int Hkv) {
    return stream_ranges_hu(Hq, decode_heads_per_unit(Hq / Hkv));
}

// Decode workspace.  Its first counter_bytes(Hq) bytes hold the fused
// merge's 64-bit arrival counters (one per sequence and head group;
// kStreamMaxB * Hq of them whatever B is, so that one workspace serves calls
// with any batch size).  Every other use of the workspace starts after them:
// the balanced schedule's partial results and tile prefix sums, or the fixed
// partitions' part_out / part_lse.  A workspace used for both never has its
// counters overwritten.
size_t counter_bytes(int32_t Hq) { return align256((size_t)kStreamMaxB * Hq * sizeof(uint64_t)); }

struct StreamLayout {
    size_t counters, part_out, part_lse, cum, q_rot, total;
};
StreamLayout stream_layout_hu(int32_t B, int32_t Hq, int HU, int32_t D) {
    const size_t slots = (size_t)stream_ranges_hu(Hq, HU) + B;
    StreamLayout l;
    l.counters = 0;
    l.part_out = counter_bytes(Hq);
    l.part_lse = l.part_out + align256(slots * Hq * D * sizeof(float));
    l.cum = l.part_lse + align256(slots * Hq * sizeof(float));
    l.q_rot = l.cum + align256((size_t)(B + 2) * sizeof(int32_t));
    // q rotated by the append-with-rope call, bf16 [B, Hq, D]
    l.total = l.q_rot + align256((size_t)B * Hq * D * 2);
    return l;
}
StreamLayout stream_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t D) {
    return stream_layout_hu(B, Hq, decode_heads_per_unit(Hq / Hkv), D);
}
// fixed partitions: part_out [B, Hq, P, D] then part_lse [B, Hq, P], after the counters
size_t split_part_lse_offset(int32_t B, int32_t Hq, int32_t D, int32_t nparts) {
    return counter_bytes(Hq) + align256((size_t)B * Hq * nparts * D * sizeof(float));
}
size_t split_bytes(int32_t B, int32_t Hq, int32_t D, int32_t nparts) {
    return split_part_lse_offset(B, Hq, D, nparts) +
           align256((size_t)B * Hq * nparts * sizeof(float));
}
// Arguments of the balanced stream kernel without the fused merge.
StreamArgs stream_args(const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_table, const int32_t *cache_seqlens, int32_t B,
                       int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size, int32_t mbps,
                       float sm_scale, int32_t window_left, const float *alibi,
                       void *workspace) {
    const StreamLayout lay = stream_layout(B, Hq, Hkv, D);
    StreamArgs a{};
    a.part_out = (float *)((char *)workspace + lay.part_out);
    a.part_lse = (float *)((char *)workspace + lay.part_lse);
    a.cum_out = (int32_t *)((char *)workspace + lay.cum);
    a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.block_table = block_table;
    a.seqlens = cache_seqlens; a.B = B; a.Hq = Hq; a.Hkv = Hkv;
    a.G = Hq / Hkv; a.D = D; a.bs_log2 = ilog2(block_size);
    a.mbps = mbps; a.window_left = window_left; a.alibi = alibi;
    a.K = stream_ranges_per_head_group(Hq, Hkv);
    a.scale_log2 = sm_scale * kLog2e;
    a.epoch = next_epoch();
    return a;
}
// Merge launch of the two-launch balanced decode, over the pieces, lse values
// and tile prefix sums that a stage launch left in the workspace.
pkv_status launch_finish(void *out, float *lse, const float *sink, int32_t B, int32_t Hq,
                         int32_t Hkv, int32_t D, const void *workspace, hipStream_t s) {
    const StreamLayout lay = stream_layout(B, Hq, Hkv, D);
    StreamArgs a{};
    a.part_out = (float *)((char *)workspace + lay.part_out);
    a.part_lse = (float *)((char *)workspace + lay.part_lse);
    a.cum_out = (int32_t *)((char *)workspace + lay.cum);
    a.out = out; a.lse = lse; a.sink = sink; a.B = B; a.Hq = Hq; a.D = D;
    return launch_stream_merge(a, s);
}
// The balanced schedule: partition_size 0 (stage launch + merge launch) or
// -1 (one launch, merge fused in).
bool use_stream(pkv_dtype dtype, int32_t B, int32_t partition_size, int32_t max_seqlen_k) {
    return dtype == PKV_BF16 && partition_size <= 0 && B <= kStreamMaxB && max_seqlen_k > 0;
}

struct SplitPlan {
    int32_t part_size;   // tokens per partition (>= max_seqlen_k when not split)
    int32_t nparts;
    bool split;
};

SplitPlan plan_split(int32_t max_seqlen_k, int32_t partition_size) {
    SplitPlan p{};
    const int32_t msk = max_seqlen_k > 0 ? max_seqlen_k : 1;
    if (partition_size <= 0 || partition_size >= msk) {
        p.part_size = msk;
        p.nparts = 1;
        p.split = false;
    } else {
        p.part_size = partition_size;
        p.nparts = (msk + partition_size - 1) / partition_size;
        p.split = p.nparts > 1;
    }
    return p;
}

// Workspace bytes a decode call with these arguments uses (0: none).
size_t decode_need(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_seqlen_k,
                   int32_t partition_size, pkv_dtype dtype) {
    if (B == 0) return 0;
    if (use_stream(dtype, B, partition_size, max_seqlen_k)) return stream_layout(B, Hq, Hkv, D).total;
    const SplitPlan p = plan_split(max_seqlen_k, partition_size);
    return p.split ? split_bytes(B, Hq, D, p.nparts) : 0;
}

// Launch the decode kernel for one plan: the final output (no split) or
// the per-partition results (split).
pkv_status launch_decode_stage(void *out, float *lse, float *part_out, float *part_lse,
                               const void *q, const void *k_cache, const void *v_cache,
                               const int32_t *block_table, const int32_t *cache_seqlens,
                               const float *sink, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                               int32_t block_size, int32_t mbps, float sm_scale,
                               int32_t window_left, const float *alibi, const SplitPlan &plan,
                               pkv_dtype dtype,
                               hipStream_t s)
{
    if (dtype == PKV_BF16 && plan.split && B <= kStreamMaxB) {
        // fixed partitions through the balanced stream: whole partitions per
        // wave, each written straight to part_out / part_lse
        StreamArgs a = stream_args(q, k_cache, v_cache, block_table, cache_seqlens, B, Hq, Hkv, D,
                                   block_size, mbps, sm_scale, window_left, alibi, nullptr);
        a.part_out = part_out; a.part_lse = part_lse; a.cum_out = nullptr;
        a.mode = kStreamParts; a.part_size = plan.part_size; a.max_parts = plan.nparts;
        return launch_decode_stream_bf16(a, s);
    }
    if (dtype == PKV_BF16) {
        DecodeArgs a{};
        a.out = out; a.lse = lse; a.part_out = part_out; a.part_lse = part_lse;
        a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
        a.block_table = block_table; a.seqlens = cache_seqlens; a.sink = sink;
        a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.D = D;
        a.bs_log2 = ilog2(block_size); a.mbps = mbps; a.window_left = window_left;
        a.alibi = alibi;
        a.part_size = plan.part_size; a.nparts = plan.nparts; a.split = plan.split ? 1 : 0;
        a.scale_log2 = sm_scale * kLog2e;
        return launch_decode_bf16(a, s);
    }
    RowArgs a{};
    a.mode = 0; a.out = out; a.lse = lse; a.part_out = part_out; a.part_lse = part_lse;
    a.q = q; a.k_cache = k_cache; a.v_cache = v_cache; a.block_table = block_table;
    a.seqlens = cache_seqlens; a.sink = sink; a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
    a.D = D; a.bs_log2 = ilog2(block_size); a.mbps = mbps; a.window_left = window_left;
    a.alibi = alibi; a.part_size = plan.part_size; a.nparts = plan.nparts; a.split = plan.split ? 1 : 0;
    a.scale_log2 = sm_scale * kLog2e;
    return launch_rows(a, s);
}

}  // namespace

namespace pkv {

pkv_status decode_check(const DecodeCall &c) {
    if (c.B < 0 || c.num_blocks < 0 || c.mbps < 0 || c.max_seqlen_k < 0) return PKV_ERR_SHAPE;
    pkv_status st = check_heads(c.Hq, c.Hkv, c.D);
    if (st != PKV_OK) return st;
    if ((st = check_block_size(c.block_size)) != PKV_OK) return st;
    if (!dtype_ok(c.dtype)) return PKV_ERR_UNSUPPORTED;
    if (c.window_left < -1 || c.partition_size < -1 || !scale_ok(c.sm_scale)) return PKV_ERR_SHAPE;
    if (c.partition_size > 0 && c.partition_size % c.block_size) return PKV_ERR_SHAPE;
    // bf16 partitions hold whole 16-token tiles
    if (c.dtype == PKV_BF16 && c.partition_size > 0 && c.partition_size % 16) return PKV_ERR_SHAPE;
    if ((long long)c.max_seqlen_k > (long long)c.mbps * c.block_size) return PKV_ERR_SHAPE;
    if (c.B == 0) return PKV_OK;
    if (!c.out || !c.q || !c.block_table || !c.cache_seqlens) return PKV_ERR_NULL;
    if (c.max_seqlen_k > 0 && (!c.k_cache || !c.v_cache)) return PKV_ERR_NULL;
    if (c.max_seqlen_k > 0 && c.num_blocks == 0) return PKV_ERR_SHAPE;
    if (!aligned16(c.q) || !aligned16(c.k_cache) || !aligned16(c.v_cache))
        return PKV_ERR_UNSUPPORTED;
    return PKV_OK;
}

size_t decode_workspace_need(const DecodeCall &c) {
    return decode_need(c.B, c.Hq, c.Hkv, c.D, c.max_seqlen_k, c.partition_size, c.dtype);
}

pkv_status decode_launch(const DecodeCall &c, void *workspace) {
    hipStream_t s = (hipStream_t)c.stream;
    if (use_stream(c.dtype, c.B, c.partition_size, c.max_seqlen_k)) {
        StreamArgs a = stream_args(c.q, c.k_cache, c.v_cache, c.block_table, c.cache_seqlens,
                                   c.B, c.Hq, c.Hkv, c.D, c.block_size, c.mbps, c.sm_scale,
                                   c.window_left, c.alibi, workspace);
        if (c.partition_size == 0) {
            // stage launch (pieces, lse, tile prefix sums), then the merge launch
            const pkv_status st = launch_decode_stream_bf16(a, s);
            if (st != PKV_OK) return st;
            return launch_finish(c.out, c.lse, c.sink, c.B, c.Hq, c.Hkv, c.D, workspace, s);
        }
        // one launch: the merge fused in, by the last wave to finish each sequence
        const StreamLayout lay = stream_layout(c.B, c.Hq, c.Hkv, c.D);
        a.counters = (uint64_t *)((char *)workspace + lay.counters);
        a.out = c.out; a.lse = c.lse; a.sink = c.sink;
        a.mode = kStreamFused;
        return launch_decode_stream_bf16(a, s);
    }
    const SplitPlan plan = plan_split(c.max_seqlen_k, c.partition_size);
    float *part_out = plan.split ? (float *)((char *)workspace + counter_bytes(c.Hq)) : nullptr;
    float *part_lse =
        plan.split ? (float *)((char *)workspace + split_part_lse_offset(c.B, c.Hq, c.D, plan.nparts))
                   : nullptr;
    pkv_status st = launch_decode_stage(c.out, c.lse, part_out, part_lse, c.q, c.k_cache,
                                        c.v_cache, c.block_table, c.cache_seqlens, c.sink, c.B,
                                        c.Hq, c.Hkv, c.D, c.block_size, c.mbps, c.sm_scale,
                                        c.window_left, c.alibi, plan, c.dtype, s);
    if (st != PKV_OK || !plan.split) return st;
    MergeArgs m{};
    m.out = c.out; m.lse = c.lse; m.part_out = part_out; m.part_lse = part_lse;
    m.seqlens = c.cache_seqlens; m.sink = c.sink; m.B = c.B; m.Hq = c.Hq; m.D = c.D;
    m.part_size = plan.part_size; m.nparts = plan.nparts; m.dtype = c.dtype;
    return launch_merge(m, s);
}

size_t decode_counter_bytes(int32_t Hq) { return counter_bytes(Hq); }

}  // namespace pkv

extern "C" {

const char *pkv_status_string(pkv_status s) {
    switch (s) {
        case PKV_OK: return "ok";
        case PKV_ERR_NULL: return "required pointer is NULL";
        case PKV_ERR_SHAPE: return "inconsistent or out-of-range sizes";
        case PKV_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, dtype or mode";
        case PKV_ERR_WORKSPACE: return "workspace missing or too small";
        case PKV_ERR_HIP: return "HIP launch failed";
        case PKV_ERR_SCRATCH: return "needs more than the static scratch of the allocation-free entry point";
    }
    return "unknown status";
}

int pkv_version(void) { return kVersion; }

pkv_status pkv_reshape_and_cache(const void *key, const void *value, void *k_cache,
                                 void *v_cache, const int32_t *slot_mapping, int32_t T,
                                 int64_t key_stride, int64_t value_stride, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 pkv_dtype dtype, void *stream)
{
    if (T < 0 || num_kv_heads <= 0 || num_blocks < 0) return PKV_ERR_SHAPE;
    if (!dtype_ok(dtype)) return PKV_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
    pkv_status st = check_block_size(block_size);
    if (st != PKV_OK) return st;
    if (T == 0) return PKV_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PKV_ERR_NULL;
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (key_stride == 0) key_stride = row;
    if (value_stride == 0) value_stride = row;
    if (key_stride < row || value_stride < row) return PKV_ERR_SHAPE;
    if (key_stride % 8 || value_stride % 8) return PKV_ERR_UNSUPPORTED;
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_UNSUPPORTED;
    return launch_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, T, key_stride,
                                    value_stride, num_kv_heads, head_dim, elem_bytes(dtype),
                                    (hipStream_t)stream);
}

pkv_status pkv_rope_cos_sin(float *cos_sin, int32_t num_positions, int32_t rotary_dim,
                           float base, int32_t scaling, float factor, int32_t max_position,
                           void *stream)
{
    if (num_positions < 0 || rotary_dim < 2 || rotary_dim % 2 || !(base > 0.f))
        return PKV_ERR_SHAPE;
    if (scaling < 0 || scaling > 2) return PKV_ERR_UNSUPPORTED;
    if (scaling != 0 && !(factor > 0.f)) return PKV_ERR_SHAPE;
    if (scaling == 2 && (max_position <= 0 || rotary_dim < 4)) return PKV_ERR_SHAPE;
    if (num_positions == 0) return PKV_OK;
    if (!cos_sin) return PKV_ERR_NULL;
    return launch_rope_table(cos_sin, num_positions, rotary_dim, base, scaling, factor,
                             max_position, (hipStream_t)stream);
}

// rotary_dim: a multiple of 16 within the head (the kernels rotate whole
// 16-byte chunks and pair chunk u with chunk u + rotary_dim / 2 / chunk)
static pkv_status check_rope(int32_t rotary_dim, int32_t head_dim) {
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (rotary_dim < 16 || rotary_dim > head_dim || rotary_dim % 16) return PKV_ERR_UNSUPPORTED;
    return PKV_OK;
}

pkv_status pkv_rope_apply(void *x, const int32_t *positions, const float *cos_sin, int32_t T,
                          int32_t num_heads, int32_t head_dim, int64_t row_stride,
                          int32_t rotary_dim, int32_t neox, pkv_dtype dtype, void *stream)
{
    if (T < 0 || num_heads <= 0) return PKV_ERR_SHAPE;
    if (!dtype_ok(dtype)) return PKV_ERR_UNSUPPORTED;
    pkv_status st = check_rope(rotary_dim, head_dim);
    if (st != PKV_OK) return st;
    if (T == 0) return PKV_OK;
    if (!x || !positions || !cos_sin) return PKV_ERR_NULL;
    const int64_t row = (int64_t)num_heads * head_dim;
    if (row_stride == 0) row_stride = row;
    if (row_stride < row) return PKV_ERR_SHAPE;
    if (row_stride % 8 || !aligned16(x)) return PKV_ERR_UNSUPPORTED;
    return launch_rope_apply(x, positions, cos_sin, T, num_heads, head_dim, row_stride,
                             rotary_dim, neox, dtype == PKV_BF16, (hipStream_t)stream);
}

pkv_status pkv_reshape_and_cache_rope(const void *key, const void *value, void *k_cache,
                                      void *v_cache, const int32_t *slot_mapping,
                                      const int32_t *positions, const float *cos_sin, int32_t T,
                                      int64_t key_stride, int64_t value_stride,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int32_t num_blocks, int32_t rotary_dim, int32_t neox,
                                      pkv_dtype dtype, void *stream)
{
    if (T < 0 || num_kv_heads <= 0 || num_blocks < 0) return PKV_ERR_SHAPE;
    if (!dtype_ok(dtype)) return PKV_ERR_UNSUPPORTED;
    pkv_status st = check_rope(rotary_dim, head_dim);
    if (st != PKV_OK) return st;
    if ((st = check_block_size(block_size)) != PKV_OK) return st;
    if (T == 0) return PKV_OK;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping || !positions || !cos_sin)
        return PKV_ERR_NULL;
    const int64_t row = (int64_t)num_kv_heads * head_dim;
    if (key_stride == 0) key_stride = row;
    if (value_stride == 0) value_stride = row;
    if (key_stride < row || value_stride < row) return PKV_ERR_SHAPE;
    if (key_stride % 8 || value_stride % 8) return PKV_ERR_UNSUPPORTED;
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_UNSUPPORTED;
    return launch_rope_cache(key, value, k_cache, v_cache, slot_mapping, positions, cos_sin, T,
                             key_stride, value_stride, num_kv_heads, head_dim, rotary_dim, neox,
                             dtype == PKV_BF16, (hipStream_t)stream);
}

size_t pkv_paged_decode_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t head_dim,
                                        int32_t max_seqlen_k, int32_t partition_size)
{
    if (B < 0 || num_q_heads <= 0 || max_seqlen_k < 0 || partition_size < -1) return (size_t)-1;
    if (head_dim != 64 && head_dim != 128) return (size_t)-1;
    if (B == 0) return 0;
    size_t need = 0;
    if (B <= kStreamMaxB && max_seqlen_k > 0 && partition_size <= 0) {
        // the balanced bf16 schedule, for whichever GQA grouping the call has
        for (int hu = 1; hu <= 4; hu *= 2)
            if (num_q_heads % hu == 0)
                need = std::max(need, stream_layout_hu(B, num_q_heads, hu, head_dim).total);
    }
    const SplitPlan p = plan_split(max_seqlen_k, partition_size);
    if (p.split) need = std::max(need, split_bytes(B, num_q_heads, head_dim, p.nparts));
    return need;
}

pkv_status pkv_paged_decode(void *out, float *lse, const void *q, const void *k_cache,
                            const void *v_cache, const int32_t *block_table,
                            const int32_t *cache_seqlens, const float *sink, int32_t B,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_seqlen_k, float sm_scale, int32_t window_left,
                            const float *alibi_slopes, int32_t partition_size, void *workspace,
                            size_t workspace_bytes, pkv_dtype dtype, void *stream)
{
    const DecodeCall c{out, lse, q, k_cache, v_cache, block_table, cache_seqlens, sink,
                       B, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_seqlen_k, sm_scale, window_left, alibi_slopes,
                       partition_size, dtype, stream};
    pkv_status st = decode_check(c);
    if (st != PKV_OK || B == 0) return st;
    const size_t need = decode_workspace_need(c);
    if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
    if (need > 0 && ((uintptr_t)workspace & 255u)) return PKV_ERR_WORKSPACE;
    return decode_launch(c, workspace);
}

pkv_status pkv_paged_decode_append(void *out, float *lse, const void *q, const void *k_new,
                                   const void *v_new, void *k_cache, void *v_cache,
                                   const int32_t *block_table, const int32_t *cache_seqlens,
                                   const float *sink, int32_t B, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t num_blocks, int32_t max_blocks_per_seq,
                                   int32_t max_seqlen_k, float sm_scale, int32_t window_left,
                                   const float *alibi_slopes, const float *rope_cos_sin,
                                   int32_t rope_positions, int32_t rotary_dim, int32_t rope_neox,
                                   void *workspace, size_t workspace_bytes, pkv_dtype dtype,
                                   void *stream)
{
    if (B < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_seqlen_k < 0)
        return PKV_ERR_SHAPE;
    pkv_status st = check_heads(num_q_heads, num_kv_heads, head_dim);
    if (st != PKV_OK) return st;
    if ((st = check_block_size(block_size)) != PKV_OK) return st;
    if (!dtype_ok(dtype)) return PKV_ERR_UNSUPPORTED;
    if (window_left < -1 || !scale_ok(sm_scale)) return PKV_ERR_SHAPE;
    // the new token goes to position cache_seqlens[b] <= max_seqlen_k
    if ((long long)max_seqlen_k + 1 > (long long)max_blocks_per_seq * block_size)
        return PKV_ERR_SHAPE;
    if (rope_cos_sin) {
        // q and k_new rotated by position cache_seqlens[b]: rotary_dim a
        // multiple of 32 within the head, a table row for every such position
        if (rotary_dim < 32 || rotary_dim > head_dim || rotary_dim % 32)
            return PKV_ERR_UNSUPPORTED;
        if ((long long)rope_positions < (long long)max_seqlen_k + 1) return PKV_ERR_SHAPE;
    }
    if (dtype == PKV_BF16 && B > kStreamMaxB) return PKV_ERR_SHAPE;
    if (B == 0) return PKV_OK;
    if (num_blocks == 0) return PKV_ERR_SHAPE;
    if (!out || !q || !k_new || !v_new || !k_cache || !v_cache || !block_table || !cache_seqlens)
        return PKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
        !aligned16(v_cache))
        return PKV_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    if (dtype == PKV_BF16) {
        const StreamLayout lay = stream_layout(B, num_q_heads, num_kv_heads, head_dim);
        if (!workspace || workspace_bytes < lay.total || ((uintptr_t)workspace & 255u))
            return PKV_ERR_WORKSPACE;
        StreamArgs a = stream_args(q, k_cache, v_cache, block_table, cache_seqlens, B,
                                   num_q_heads, num_kv_heads, head_dim, block_size,
                                   max_blocks_per_seq, sm_scale, window_left, alibi_slopes,
                                   workspace);
        a.k_new = k_new; a.v_new = v_new; a.append = 1;
        a.rope = rope_cos_sin; a.rope_dim = rotary_dim; a.rope_neox = rope_neox != 0;
        a.q_rot = (char *)workspace + lay.q_rot;
        a.mode = kStreamAppend;
        // the stage launch with the new tokens stored and attended, then the
        // merge launch over its pieces (prefix sums counting the new tokens)
        if ((st = launch_decode_stream_bf16(a, s)) != PKV_OK) return st;
        return launch_finish(out, lse, sink, B, num_q_heads, num_kv_heads, head_dim, workspace, s);
    }
    RowArgs a{};
    a.mode = 0; a.out = out; a.lse = lse; a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
    a.block_table = block_table; a.seqlens = cache_seqlens; a.k_new = k_new; a.v_new = v_new;
    a.append = 1; a.sink = sink; a.alibi = alibi_slopes; a.B = B; a.Hq = num_q_heads;
    a.Hkv = num_kv_heads;
    a.G = num_q_heads / num_kv_heads; a.D = head_dim; a.bs_log2 = ilog2(block_size);
    a.mbps = max_blocks_per_seq; a.window_left = window_left;
    a.part_size = max_seqlen_k + 1; a.nparts = 1; a.split = 0;
    a.scale_log2 = sm_scale * kLog2e;
    a.rope = rope_cos_sin; a.rope_dim = rotary_dim; a.rope_neox = rope_neox != 0;
    return launch_rows(a, s);
}

pkv_status pkv_paged_decode_stage(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_table, const int32_t *cache_seqlens,
                                  int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_seqlen_k,
                                  float sm_scale, int32_t window_left,
                                  const float *alibi_slopes, void *workspace,
                                  size_t workspace_bytes, pkv_dtype dtype, void *stream)
{
    if (B < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_seqlen_k < 0)
        return PKV_ERR_SHAPE;
    pkv_status st = check_heads(num_q_heads, num_kv_heads, head_dim);
    if (st != PKV_OK) return st;
    if ((st = check_block_size(block_size)) != PKV_OK) return st;
    if (dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
    if (window_left < -1 || B > kStreamMaxB || !scale_ok(sm_scale)) return PKV_ERR_SHAPE;
    if ((long long)max_seqlen_k > (long long)max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
    if (B == 0) return PKV_OK;
    if (!q || !block_table || !cache_seqlens || !k_cache || !v_cache) return PKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_UNSUPPORTED;
    const StreamLayout lay = stream_layout(B, num_q_heads, num_kv_heads, head_dim);
    if (!workspace || workspace_bytes < lay.total || ((uintptr_t)workspace & 255u))
        return PKV_ERR_WORKSPACE;
    const StreamArgs a = stream_args(q, k_cache, v_cache, block_table, cache_seqlens, B,
                                     num_q_heads, num_kv_heads, head_dim, block_size,
                                     max_blocks_per_seq, sm_scale, window_left, alibi_slopes,
                                   workspace);
    return launch_decode_stream_bf16(a, (hipStream_t)stream);
}

pkv_status pkv_paged_decode_finish(void *out, float *lse, const float *sink, int32_t B,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   const void *workspace, size_t workspace_bytes,
                                   pkv_dtype dtype, void *stream)
{
    if (B < 0) return PKV_ERR_SHAPE;
    pkv_status st = check_heads(num_q_heads, num_kv_heads, head_dim);
    if (st != PKV_OK) return st;
    if (dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
    if (B > kStreamMaxB) return PKV_ERR_SHAPE;
    if (B == 0) return PKV_OK;
    if (!out) return PKV_ERR_NULL;
    const StreamLayout lay = stream_layout(B, num_q_heads, num_kv_heads, head_dim);
    if (!workspace || workspace_bytes < lay.total || ((uintptr_t)workspace & 255u))
        return PKV_ERR_WORKSPACE;
    return launch_finish(out, lse, sink, B, num_q_heads, num_kv_heads, head_dim, workspace,
                         (hipStream_t)stream);
}

pkv_status pkv_paged_decode_partitions(float *part_out, float *part_lse, const void *q,
                                       const void *k_cache, const void *v_cache,
                                       const int32_t *block_table, const int32_t *cache_seqlens,
                                       int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_seqlen_k,
                                       float sm_scale, int32_t window_left,
                                       const float *alibi_slopes, int32_t partition_size, int32_t max_partitions,
                                       pkv_dtype dtype, void *stream)
{
    if (B < 0 || num_blocks < 0 || max_blocks_per_seq < 0 || max_seqlen_k < 0)
        return PKV_ERR_SHAPE;
    pkv_status st = check_heads(num_q_heads, num_kv_heads, head_dim);
    if (st != PKV_OK) return st;
    if ((st = check_block_size(block_size)) != PKV_OK) return st;
    if (!dtype_ok(dtype)) return PKV_ERR_UNSUPPORTED;
    if (window_left < -1 || partition_size <= 0 || partition_size % block_size ||
        (dtype == PKV_BF16 && partition_size % 16) || !scale_ok(sm_scale))
        return PKV_ERR_SHAPE;
    if ((long long)max_seqlen_k > (long long)max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
    const long long need_parts = ((long long)max_seqlen_k + partition_size - 1) / partition_size;
    if (max_partitions <= 0 || max_partitions < need_parts) return PKV_ERR_SHAPE;
    if (B == 0) return PKV_OK;
    if (!part_out || !part_lse || !q || !block_table || !cache_seqlens) return PKV_ERR_NULL;
    if (max_seqlen_k > 0 && (!k_cache || !v_cache)) return PKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_UNSUPPORTED;
    SplitPlan plan{partition_size, max_partitions, true};
    return launch_decode_stage(nullptr, nullptr, part_out, part_lse, q, k_cache, v_cache,
                               block_table, cache_seqlens, nullptr, B, num_q_heads, num_kv_heads,
                               head_dim, block_size, max_blocks_per_seq, sm_scale, window_left,
                               alibi_slopes, plan, dtype, (hipStream_t)stream);
}

pkv_status pkv_merge_partitions(void *out, float *lse, const float *part_out,
                                const float *part_lse, const int32_t *cache_seqlens,
                                int32_t partition_size, const float *sink, int32_t B,
                                int32_t num_q_heads, int32_t head_dim, int32_t max_partitions,
                                pkv_dtype dtype, void *stream)
{
    if (B < 0 || num_q_heads <= 0 || max_partitions <= 0 || partition_size <= 0)
        return PKV_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return PKV_ERR_UNSUPPORTED;
    if (B == 0) return PKV_OK;
    if (!out || !part_out || !part_lse || !cache_seqlens) return PKV_ERR_NULL;
    MergeArgs m{};
    m.out = out; m.lse = lse; m.part_out = part_out; m.part_lse = part_lse;
    m.seqlens = cache_seqlens; m.sink = sink; m.B = B; m.Hq = num_q_heads; m.D = head_dim;
    m.part_size = partition_size; m.nparts = max_partitions; m.dtype = dtype;
    return launch_merge(m, (hipStream_t)stream);
}

size_t pkv_varlen_prefill_workspace_bytes(int32_t B, int32_t max_seqlen_k, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t rope_k, pkv_dtype dtype)
{
    if (B < 0 || max_seqlen_k < 0 || num_kv_heads <= 0 || head_dim <= 0) return (size_t)-1;
    if (!rope_k || dtype != PKV_BF16) return 0;
    return align256((size_t)B * max_seqlen_k * num_kv_heads * head_dim * 2);
}

pkv_status pkv_varlen_prefill(void *out, float *lse, const void *q, const void *k, const void *v,
                              const void *k_cache, const void *v_cache,
                              const int32_t *block_table, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, const int32_t *cu_seqlens_q,
                              const int32_t *cu_seqlens_k, int32_t B, int32_t max_seqlen_q,
                              int32_t max_seqlen_k, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, float sm_scale, int32_t causal,
                              int32_t window_left, const float *alibi_slopes,
                              const float *rope_cos_sin, int32_t rope_positions,
                              int32_t rotary_dim, int32_t rope_neox, int32_t rope_k,
                              const float *sink, void *workspace, size_t workspace_bytes,
                              pkv_dtype dtype, void *stream)
{
    if (B < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return PKV_ERR_SHAPE;
    pkv_status st = check_heads(num_q_heads, num_kv_heads, head_dim);
    if (st != PKV_OK) return st;
    if (!dtype_ok(dtype)) return PKV_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return PKV_ERR_SHAPE;
    if (window_left < -1 || !scale_ok(sm_scale)) return PKV_ERR_SHAPE;
    if (rope_cos_sin) {
        // q rotated in registers: rotary_dim a multiple of 32 within the head,
        // and a table row for every query position (< max_seqlen_k)
        if (rotary_dim < 32 || rotary_dim > head_dim || rotary_dim % 32)
            return PKV_ERR_UNSUPPORTED;
        if (rope_positions < max_seqlen_k) return PKV_ERR_SHAPE;
    }
    const bool contiguous = k != nullptr || v != nullptr;
    const bool paged = k_cache != nullptr || v_cache != nullptr || block_table != nullptr;
    if (contiguous && paged) return PKV_ERR_SHAPE;
    // rotating K as it is loaded: a table, and contiguous keys (cached keys
    // are rotated when they are stored)
    if (rope_k != 0 && rope_k != 1) return PKV_ERR_SHAPE;
    if (rope_k && (!rope_cos_sin || paged)) return PKV_ERR_UNSUPPORTED;
    // bf16 keys rotated once into the workspace, or else inside the attention
    // kernels (which have no variant with ALiBi slopes as well)
    const bool keys_copied = rope_k && dtype == PKV_BF16 && workspace != nullptr;
    if (rope_k && !keys_copied && alibi_slopes) return PKV_ERR_UNSUPPORTED;
    if (keys_copied) {
        const size_t need = pkv_varlen_prefill_workspace_bytes(B, max_seqlen_k, num_kv_heads,
                                                               head_dim, rope_k, dtype);
        if (workspace_bytes < need) return PKV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return PKV_ERR_UNSUPPORTED;
    }
    if (paged) {
        if ((st = check_block_size(block_size)) != PKV_OK) return st;
        if (num_blocks < 0 || max_blocks_per_seq < 0) return PKV_ERR_SHAPE;
        if ((long long)max_seqlen_k > (long long)max_blocks_per_seq * block_size)
            return PKV_ERR_SHAPE;
    }
    if (B == 0 || max_seqlen_q == 0) return PKV_OK;
    if (!out || !q || !cu_seqlens_q || !cu_seqlens_k) return PKV_ERR_NULL;
    if (!contiguous && !paged) return PKV_ERR_NULL;
    if (contiguous && (!k || !v)) return PKV_ERR_NULL;
    if (paged && (!k_cache || !v_cache || !block_table)) return PKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k) || !aligned16(v) ||
        !aligned16(k_cache) || !aligned16(v_cache))
        return PKV_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    const int bs_log2 = paged ? ilog2(block_size) : 0;

    if (dtype == PKV_BF16) {
        // contiguous K/V are read through one 32-bit-ranged buffer per request
        if (contiguous && (unsigned long long)max_seqlen_k * num_kv_heads * head_dim * 2 >= (1ull << 32))
            return PKV_ERR_UNSUPPORTED;
        if (keys_copied) {
            // the keys rotated by their positions into the workspace (same
            // rows), then attended from there as keys already rotated
            if ((st = launch_rope_keys(k, workspace, cu_seqlens_k, rope_cos_sin, B, max_seqlen_k,
                                       num_kv_heads, head_dim, rotary_dim, rope_neox, s)) != PKV_OK)
                return st;
            k = workspace;
            rope_k = 0;
        }
        PrefillArgs a{};
        a.out = out; a.lse = lse; a.q = q; a.k = k; a.v = v; a.k_cache = k_cache;
        a.v_cache = v_cache; a.block_table = block_table; a.cu_q = cu_seqlens_q;
        a.rope = rope_cos_sin; a.rope_dim = rotary_dim; a.rope_neox = rope_neox;
        a.rope_k = rope_k;
        a.cu_k = cu_seqlens_k; a.sink = sink; a.alibi = alibi_slopes; a.B = B;
        a.Hq = num_q_heads; a.Hkv = num_kv_heads;
        a.G = num_q_heads / num_kv_heads; a.D = head_dim; a.bs_log2 = bs_log2;
        a.mbps = max_blocks_per_seq; a.window_left = window_left; a.causal = causal;
        a.hpw = prefill_heads_per_wg(a.G);
        a.max_q_tiles = (max_seqlen_q + prefill_block_m() - 1) / prefill_block_m();
        a.scale_log2 = sm_scale * kLog2e;
        if (window_left >= 0 && causal) {
            // causal sliding window: workgroups walk runs of position blocks
            // (each step's keys overlap the last step's), sized for about two
            // resident workgroups per compute unit
            const int bm = prefill_block_m() / a.hpw;
            const long long per_req = (max_seqlen_q + bm - 1) / bm;
            const long long blocks = (long long)B * per_req * (a.G / a.hpw) * num_kv_heads;
            const long long steps = std::min<long long>(
                16, std::max<long long>(1, blocks / (2LL * device_cus())));
            a.run_steps = (int)steps;
            a.runs = (int)((per_req + steps - 1) / steps);
        }
        return launch_prefill_bf16(a, s);
    }
    // fp32: one wave per (request, row < max_seqlen_q, head)
    RowArgs a{};
    a.mode = 1; a.out = out; a.lse = lse; a.q = q; a.k = k; a.v = v; a.k_cache = k_cache;
    a.v_cache = v_cache; a.block_table = block_table; a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
    a.rope = rope_cos_sin; a.rope_dim = rotary_dim; a.rope_neox = rope_neox; a.rope_k = rope_k;
    a.sink = sink; a.alibi = alibi_slopes; a.B = B; a.Hq = num_q_heads; a.Hkv = num_kv_heads;
    a.G = num_q_heads / num_kv_heads; a.D = head_dim; a.bs_log2 = bs_log2;
    a.mbps = max_blocks_per_seq; a.window_left = window_left; a.scale_log2 = sm_scale * kLog2e;
    a.T = max_seqlen_q; a.causal = causal;
    return launch_rows(a, s);
}

pkv_status pkv_vertical_slash_blocks(int32_t *block_count, int32_t *block_offset,
                                     int32_t *column_count, int32_t *column_index,
                                     const int32_t *vertical_indices,
                                     const int32_t *slash_indices, const int32_t *cu_seqlens,
                                     int32_t B, int32_t num_heads, int32_t num_vertical,
                                     int32_t num_slash, int32_t max_seqlen, void *stream)
{
    if (B < 0 || num_heads <= 0 || num_vertical < 0 || num_slash < 0 || max_seqlen < 0)
        return PKV_ERR_SHAPE;
    const int NM = (max_seqlen + 63) / 64;
    if (B == 0 || NM == 0) return PKV_OK;
    if (!block_count || !block_offset || !column_count || !cu_seqlens) return PKV_ERR_NULL;
    if ((num_vertical > 0 && (!vertical_indices || !column_index)) ||
        (num_slash > 0 && !slash_indices))
        return PKV_ERR_NULL;
    VerticalSlashArgs a{};
    a.block_count = block_count; a.block_offset = block_offset; a.column_count = column_count;
    a.column_index = column_index; a.vertical = vertical_indices; a.slash = slash_indices;
    a.cu = cu_seqlens; a.B = B; a.H = num_heads; a.NV = num_vertical; a.NS = num_slash; a.NM = NM;
    return launch_vertical_slash(a, (hipStream_t)stream);
}

pkv_status pkv_sparse_prefill(void *out, float *lse, const void *q, const void *k, const void *v,
                              const int32_t *cu_seqlens, const int32_t *block_count,
                              const int32_t *block_offset, const int32_t *column_count,
                              const int32_t *column_index, int32_t B, int32_t max_seqlen,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t num_vertical, float sm_scale, const float *sink,
                              pkv_dtype dtype, void *stream)
{
    if (B < 0 || max_seqlen < 0 || num_vertical < 0) return PKV_ERR_SHAPE;
    pkv_status st = check_heads(num_q_heads, num_kv_heads, head_dim);
    if (st != PKV_OK) return st;
    if (dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
    if (!scale_ok(sm_scale)) return PKV_ERR_SHAPE;
    // K/V rows of one request are addressed with 32-bit byte offsets
    if ((unsigned long long)max_seqlen * num_kv_heads * head_dim * 2 >= (1ull << 32))
        return PKV_ERR_UNSUPPORTED;
    const int NM = (max_seqlen + 63) / 64;
    if (B == 0 || NM == 0) return PKV_OK;
    if (!out || !q || !k || !v || !cu_seqlens || !block_count || !block_offset || !column_count)
        return PKV_ERR_NULL;
    if (num_vertical > 0 && !column_index) return PKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(k) || !aligned16(v))
        return PKV_ERR_UNSUPPORTED;
    SparseArgs a{};
    a.out = out; a.lse = lse; a.q = q; a.k = k; a.v = v; a.cu = cu_seqlens;
    a.block_count = block_count; a.block_offset = block_offset; a.column_count = column_count;
    a.column_index = column_index; a.sink = sink; a.B = B; a.Hq = num_q_heads;
    a.Hkv = num_kv_heads; a.G = num_q_heads / num_kv_heads; a.D = head_dim; a.NM = NM;
    a.NV = num_vertical; a.scale_log2 = sm_scale * kLog2e;
    return launch_sparse_prefill(a, (hipStream_t)stream);
}

}  // extern "C"
