// Internal launch interfaces of the kernels (not part of the ABI).
#pragma once

#include "common.h"

namespace pkv {

struct DecodeArgs {
    void *out;               // [B, Hq, D] (non-split)
    float *lse;              // [B, Hq] or null (non-split)
    float *part_out;         // [B, Hq, nparts, D] (split)
    float *part_lse;         // [B, Hq, nparts] (split)
    const void *q;           // [B, Hq, D]
    const void *k_cache;     // [NB, bs, Hkv, D]
    const void *v_cache;
    const int32_t *block_table;  // [B, mbps]
    const int32_t *seqlens;      // [B]
    const float *sink;           // [Hq] or null
    const float *alibi;          // [Hq] ALiBi slopes or null
    int32_t B, Hq, Hkv, G, D;
    int32_t bs_log2, mbps, window_left;
    int32_t part_size, nparts, split;
    float scale_log2;            // sm_scale * log2(e)
};

// Balanced decode schedule (decode_stream_kernel): the 16-token tiles of all
// sequences laid end to end (the same list for every head group) and cut into
// K equal contiguous ranges per head group, one per wave.  A workgroup of
// kStreamWaves waves takes consecutive (head group, range) pairs, head group
// fastest, so its waves read the columns of the same token rows together.
// Range k's partial result for sequence b goes to slot k + b (unique: a
// range moves forward through the sequences).
constexpr int kStreamWaves = 4;
// What a stream launch computes: per-range pieces for the merge kernel
// (stage), final outputs with the merge fused in (fused), the stage's pieces
// with each sequence's new token appended first (append; the merge kernel
// follows), or fixed partitions of part_size tokens written to part_out /
// part_lse, each partition wholly in one wave's range (parts).
enum { kStreamStage = 0, kStreamFused = 1, kStreamAppend = 2, kStreamParts = 3 };
constexpr int kStreamMaxB = 4096;

struct StreamArgs {
    float *part_out;             // [slots, Hq, D], slots = K + B (parts mode: see below)
    float *part_lse;             // [slots, Hq]
    int32_t *cum_out;            // [B + 2]: tile prefix sums, then the per-wave chunk
    // Fused merge (counters != null): the last wave to finish a (sequence,
    // head group) merges its pieces into out/lse.  counters [B, Hq / HU],
    // 64 bits each: the call's epoch in the high half, the pieces counted so
    // far in the low half.  A counter whose epoch is not this call's is stale
    // (left by an interrupted call, or never used) and counts as zero; the
    // wave that completes a count sets the counter back to zero.
    uint64_t *counters;
    uint32_t epoch;              // nonzero, different from the previous calls'
    void *out;                   // [B, Hq, D] bf16
    float *lse;                  // [B, Hq] or null
    const float *sink;           // [Hq] or null
    const float *alibi;          // [Hq] ALiBi slopes or null
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_table;
    const int32_t *seqlens;
    // Append (fused merge only): each sequence's new token k_new/v_new [B, Hkv,
    // D] is stored at position seqlens[b] and attended as key seqlens[b].
    const void *k_new;
    const void *v_new;
    int32_t append;              // 0 or 1
    // Append with rotary embedding (rope != null): the [positions, rope_dim]
    // table, cos then sin.  k_new is rotated by its position as it is stored,
    // and q by the same position into q_rot [B, Hq, D] (workspace), which the
    // waves then read in place of q.
    const float *rope;
    int32_t rope_dim, rope_neox;
    void *q_rot;
    int32_t mode;                // kStream*
    // parts mode: part_out [B, Hq, max_parts, D] / part_lse [B, Hq, max_parts]
    int32_t part_size, max_parts;
    int32_t B, Hq, Hkv, G, D;
    int32_t bs_log2, mbps, window_left;
    int32_t K;                   // ranges (waves) per head group
    float scale_log2;
};

// First visible key of a decode query over L keys (the window's left edge).
__device__ __forceinline__ int stream_lo(int L, int window_left) {
    return window_left >= 0 ? max(0, L - 1 - window_left) : 0;
}
// 16-token tiles covering [stream_lo & ~15, L).
__device__ __forceinline__ int stream_tiles(int L, int window_left) {
    if (L <= 0) return 0;
    return (L - (stream_lo(L, window_left) & ~15) + 15) >> 4;
}
__device__ __forceinline__ int stream_chunk(int T, int nwaves) {
    return max(1, (T + nwaves - 1) / nwaves);
}
// Block-wide (NT threads): s_cum[b] = tiles of sequences 0..b-1, b <= B.
// The key counts seqlens[b] + add are kept in s_len[b] (the lengths are read
// from global memory once; add = 1 counts an appended token).
template <int NT>
__device__ __forceinline__ void stream_prefix_tiles(const int32_t *seqlens, int add, int B,
                                                    int window_left, int *s_cum, int *s_part,
                                                    int *s_len) {
    static_assert(NT % 64 == 0 && NT <= 1024, "whole waves");
    constexpr int PL = NT / 64;       // strip sums per lane of the scanning wave
    const int tid = threadIdx.x;
    const int per = (B + NT - 1) / NT;
    const int b0 = tid * per;
    int sum = 0;
    for (int b = b0; b < min(b0 + per, B); ++b) {
        const int L = seqlens[b] + add;
        s_len[b] = L;
        sum += stream_tiles(L, window_left);
    }
    s_part[tid] = sum;
    __syncthreads();
    if (tid < 64) {   // exclusive scan of the NT strip sums by one wave
        int x[PL];
        int mine = 0;
#pragma unroll
        for (int u = 0; u < PL; ++u) {
            x[u] = s_part[PL * tid + u];
            mine += x[u];
        }
        int incl = mine;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off, 64);
            if (tid >= off) incl += y;
        }
        int run = incl - mine;
#pragma unroll
        for (int u = 0; u < PL; ++u) {
            s_part[PL * tid + u] = run;
            run += x[u];
        }
    }
    __syncthreads();
    int run = s_part[tid];
    for (int b = b0; b < min(b0 + per, B); ++b) {
        s_cum[b] = run;
        run += stream_tiles(s_len[b], window_left);
    }
    if (tid == NT - 1) s_cum[B] = run;   // the last strip ends at B (B <= NT * per)
    __syncthreads();
}

struct MergeArgs {
    void *out;
    float *lse;
    const float *part_out;
    const float *part_lse;
    const int32_t *seqlens;
    const float *sink;
    int32_t B, Hq, D, part_size, nparts;
    int32_t dtype;
};

// One query row per wave, plain fp32 VALU arithmetic: the fp32 path of decode
// and prefill.  mode 0 = paged decode, 1 = varlen prefill.
struct RowArgs {
    int32_t mode;
    void *out;
    float *lse;
    float *part_out;
    float *part_lse;
    const void *q;
    const void *k;               // prefill contiguous [sum Lk, Hkv, D] or null
    const void *v;
    const void *k_cache;         // paged [NB, bs, Hkv, D]
    const void *v_cache;
    const int32_t *block_table;
    const int32_t *seqlens;      // decode: [B]
    // decode with append: the new token k_new/v_new [B, Hkv, D] is key
    // seqlens[b] (read from k_new/v_new) and is stored into the cache there
    const void *k_new;
    const void *v_new;
    int32_t append;
    const int32_t *cu_q;         // prefill: [B+1]
    const int32_t *cu_k;
    const float *sink;
    const float *alibi;          // [Hq] ALiBi slopes or null
    const float *rope;           // prefill: q rotary table or null (as PrefillArgs)
    int32_t rope_dim, rope_neox;
    int32_t rope_k;              // prefill: contiguous K rotated too (as PrefillArgs)
    int32_t B, T, Hq, Hkv, G, D;   // prefill: T = max_seqlen_q
    int32_t bs_log2, mbps, window_left;
    // prefill: 1 = key j visible to position p only when j <= p; 0 = every
    // key of the request (a window still bounds the left side)
    int32_t causal;
    int32_t part_size, nparts, split;
    float scale_log2;
};

struct PrefillArgs {
    void *out;                   // [sum Lq, Hq, D]
    float *lse;                  // [sum Lq, Hq] or null
    const void *q;
    const void *k;               // contiguous or null
    const void *v;
    const void *k_cache;         // paged or null
    const void *v_cache;
    const int32_t *block_table;
    const int32_t *cu_q;
    const int32_t *cu_k;
    const float *sink;
    const float *alibi;          // [Hq] ALiBi slopes or null
    // rotary embedding of q by its position (table [positions, rope_dim]:
    // cos then sin) or null
    const float *rope;
    int32_t rope_dim, rope_neox;
    // 1: contiguous K is rotated by key position as it is loaded (the
    // table above; paged keys are rotated when they are cached)
    int32_t rope_k;
    int32_t B, Hq, Hkv, G, D;
    int32_t bs_log2, mbps, window_left;
    int32_t causal;              // as RowArgs::causal
    int32_t hpw;                 // query heads per workgroup: prefill_heads_per_wg(G)
    int32_t max_q_tiles;         // ceil(max_seqlen_q / prefill_block_m())
    // runs (sliding windows): each workgroup walks run_steps consecutive
    // blocks of 128 / hpw positions; runs = ceil(blocks per request /
    // run_steps).  run_steps == 0: one block per workgroup.
    int32_t runs, run_steps;
    float scale_log2;
};

// The arguments of pkv_paged_decode without its workspace.
struct DecodeCall {
    void *out;
    float *lse;
    const void *q, *k_cache, *v_cache;
    const int32_t *block_table, *cache_seqlens;
    const float *sink;
    int32_t B, Hq, Hkv, D, block_size, num_blocks, mbps, max_seqlen_k;
    float sm_scale;
    int32_t window_left;
    const float *alibi;
    int32_t partition_size;
    pkv_dtype dtype;
    void *stream;
};
// pkv_paged_decode in three steps: the host checks (PKV_OK for a valid call),
// the workspace bytes the call uses, and the launches with a workspace of at
// least that size (256-byte aligned).
pkv_status decode_check(const DecodeCall &c);
size_t decode_workspace_need(const DecodeCall &c);
pkv_status decode_launch(const DecodeCall &c, void *workspace);
// bytes of the fused merge's counters at the start of a decode workspace
size_t decode_counter_bytes(int32_t Hq);

int decode_heads_per_unit(int G);
pkv_status launch_decode_bf16(const DecodeArgs &a, hipStream_t stream);
pkv_status launch_decode_stream_bf16(const StreamArgs &a, hipStream_t stream);
pkv_status launch_merge(const MergeArgs &a, hipStream_t stream);
// Merge of the balanced schedule's pieces written by a stage launch (mode 0):
// reads part_out, part_lse, cum_out; writes out, lse; sink optional.
pkv_status launch_stream_merge(const StreamArgs &a, hipStream_t stream);
// Vertical + slash block lists (pkv_vertical_slash_blocks).
struct VerticalSlashArgs {
    int32_t *block_count;        // [B, H, NM]
    int32_t *block_offset;       // [B, H, NM, NM]
    int32_t *column_count;       // [B, H, NM]
    int32_t *column_index;       // [B, H, NM, NV]
    const int32_t *vertical;     // [B, H, NV]
    const int32_t *slash;        // [B, H, NS]
    const int32_t *cu;           // [B + 1]
    int32_t B, H, NV, NS, NM;    // NM = ceil(max_seqlen / 64)
};

// Block-sparse prefill over those lists (pkv_sparse_prefill), bf16.
struct SparseArgs {
    void *out;                   // [sum L, Hq, D]
    float *lse;                  // [sum L, Hq] or null
    const void *q, *k, *v;       // q [sum L, Hq, D], k / v [sum L, Hkv, D]
    const int32_t *cu;           // [B + 1]
    const int32_t *block_count, *block_offset, *column_count, *column_index;
    const float *sink;
    int32_t B, Hq, Hkv, G, D, NM, NV;
    float scale_log2;
};

pkv_status launch_rows(const RowArgs &a, hipStream_t stream);
// block size 8 (decode_bs8.hip)
pkv_status launch_decode_bf16_bs8(const DecodeArgs &a, hipStream_t stream);
pkv_status launch_decode_stream_bf16_bs8(const StreamArgs &a, hipStream_t stream);
pkv_status launch_prefill_bf16(const PrefillArgs &a, hipStream_t stream);
pkv_status launch_vertical_slash(const VerticalSlashArgs &a, hipStream_t stream);
pkv_status launch_sparse_prefill(const SparseArgs &a, hipStream_t stream);
int prefill_heads_per_wg(int G);
int prefill_block_m();
pkv_status launch_rope_table(float *cos_sin, int n_pos, int rd, double base, int scaling,
                             double factor, int max_position, hipStream_t stream);
pkv_status launch_rope_apply(void *x, const int32_t *positions, const float *cos_sin, int T,
                             int H, int D, long long row_stride, int rd, int neox, bool bf16,
                             hipStream_t stream);
// bf16 keys of varlen requests rotated into dst (same rows), positions 0..L-1
pkv_status launch_rope_keys(const void *k, void *dst, const int32_t *cu_k,
                            const float *cos_sin, int B, int max_len, int H, int D, int rd,
                            int neox, hipStream_t stream);
pkv_status launch_rope_cache(const void *key, const void *value, void *k_cache, void *v_cache,
                             const int32_t *slot_mapping, const int32_t *positions,
                             const float *cos_sin, int T, long long key_stride,
                             long long value_stride, int Hkv, int D, int rd, int neox, bool bf16,
                             hipStream_t stream);
pkv_status launch_reshape_and_cache(const void *key, const void *value, void *k_cache,
                                    void *v_cache, const int32_t *slot_mapping, int32_t T,
                                    int64_t key_stride, int64_t value_stride, int32_t Hkv,
                                    int32_t D, int32_t elem_bytes, hipStream_t stream);

}  // namespace pkv
