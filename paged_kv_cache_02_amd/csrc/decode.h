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
    int32_t B, Hq, Hkv, G, D;
    int32_t bs_log2, mbps, window_left;
    int32_t part_size, nparts, split;
    float scale_log2;            // sm_scale * log2(e)
};

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

// One query row per wave, plain VALU arithmetic: the fp32 path of decode and
// prefill.  mode 0 = paged decode, 1 = varlen prefill.
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
    const int32_t *cu_q;         // prefill: [B+1]
    const int32_t *cu_k;
    const float *sink;
    int32_t B, T, Hq, Hkv, G, D;   // prefill: T = max_seqlen_q
    int32_t bs_log2, mbps, window_left;
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
    int32_t B, Hq, Hkv, G, D;
    int32_t bs_log2, mbps, window_left;
    int32_t max_q_tiles;         // ceil(max_seqlen_q / BLOCK_M)
    float scale_log2;
};

int decode_heads_per_unit(int G);
pkv_status launch_decode_bf16(const DecodeArgs &a, hipStream_t stream);
pkv_status launch_merge(const MergeArgs &a, hipStream_t stream);
pkv_status launch_rows(const RowArgs &a, bool bf16, hipStream_t stream);
pkv_status launch_prefill_bf16(const PrefillArgs &a, hipStream_t stream);
int prefill_block_m();
pkv_status launch_reshape_and_cache(const void *key, const void *value, void *k_cache,
                                    void *v_cache, const int32_t *slot_mapping, int32_t T,
                                    int64_t key_stride, int64_t value_stride, int32_t Hkv,
                                    int32_t D, int32_t elem_bytes, hipStream_t stream);

}  // namespace pkv
