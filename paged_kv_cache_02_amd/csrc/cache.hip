// reshape_and_cache: store new tokens' K/V rows into paged cache slots.
//
// vLLM "attention.py" page, PagedAttention.forward: after prompt attention the
// new key/value rows are written to the cache at slot_mapping, and decode then
// reads them back through the block table.  Slot s of a cache laid out as
// [num_blocks, block_size, Hkv, D] is row s of the flat [num_blocks*block_size,
// Hkv, D] view, so one token's K (or V) is one contiguous row of Hkv*D
// elements: the copy is a 16-byte-vector memcpy per row, bit exact.
//
// HBM-bound: each token reads 2 rows and writes 2 rows.  A token's row is
// split over row_chunks / kChunks threads; each thread moves kChunks 16-byte
// chunks of K and of V, issuing all its loads before its stores so that
// kChunks loads of each are in flight, and the chunks of one load
// instruction are consecutive across the wave (whole 1 KiB spans).

#include <algorithm>

#include "common.h"

namespace pkv {

constexpr int kChunks = 2;   // 16-byte chunks per thread and row (rows are multiples of 8)

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const char *__restrict__ key, const char *__restrict__ value, char *__restrict__ k_cache,
    char *__restrict__ v_cache, const int32_t *__restrict__ slot_mapping, int32_t T,
    int64_t key_stride_bytes, int64_t value_stride_bytes, int32_t row_chunks /* 16-byte chunks per row */,
    int32_t threads_per_token, int32_t tokens_per_block)
{
    const int t = blockIdx.x * tokens_per_block + (int)threadIdx.x / threads_per_token;
    if ((int)threadIdx.x >= tokens_per_block * threads_per_token || t >= T) return;
    const int32_t s = slot_mapping[t];
    if (s < 0) return;  // padding token
    const int64_t row_bytes = (int64_t)row_chunks * 16;
    const char *kr = key + t * key_stride_bytes;
    const char *vr = value + t * value_stride_bytes;
    char *kc = k_cache + (int64_t)s * row_bytes;
    char *vc = v_cache + (int64_t)s * row_bytes;
    // chunk c0 + u * threads_per_token, u < kChunks, for each pass over the row
    for (int c0 = (int)threadIdx.x % threads_per_token; c0 < row_chunks;
         c0 += threads_per_token * kChunks) {
        u32x4 kv[kChunks], vv[kChunks];
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            const int c = c0 + u * threads_per_token;
            if (c < row_chunks) {
                kv[u] = *reinterpret_cast<const u32x4 *>(kr + c * 16);
                vv[u] = *reinterpret_cast<const u32x4 *>(vr + c * 16);
            }
        }
#pragma unroll
        for (int u = 0; u < kChunks; ++u) {
            const int c = c0 + u * threads_per_token;
            if (c < row_chunks) {
                *reinterpret_cast<u32x4 *>(kc + c * 16) = kv[u];
                *reinterpret_cast<u32x4 *>(vc + c * 16) = vv[u];
            }
        }
    }
}

pkv_status launch_reshape_and_cache(const void *key, const void *value, void *k_cache,
                                    void *v_cache, const int32_t *slot_mapping, int32_t T,
                                    int64_t key_stride, int64_t value_stride, int32_t Hkv,
                                    int32_t D, int32_t elem_bytes, hipStream_t stream)
{
    const int32_t row_bytes = Hkv * D * elem_bytes;
    const int32_t row_chunks = row_bytes / 16;
    // threads per token: a row's chunks in kChunks passes, at most one block
    const int32_t threads_per_token = std::min(256, (row_chunks + kChunks - 1) / kChunks);
    const int32_t tokens_per_block = 256 / threads_per_token;
    const int32_t blocks = (T + tokens_per_block - 1) / tokens_per_block;
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(blocks), dim3(256), 0, stream,
                       (const char *)key, (const char *)value, (char *)k_cache, (char *)v_cache,
                       slot_mapping, T, key_stride * elem_bytes, value_stride * elem_bytes,
                       row_chunks, threads_per_token, tokens_per_block);
    return launch_status();
}

}  // namespace pkv
