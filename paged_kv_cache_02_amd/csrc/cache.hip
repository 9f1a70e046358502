// reshape_and_cache: store new tokens' K/V rows into paged cache slots.
//
// vLLM "attention.py" page, PagedAttention.forward: after prompt attention the
// new key/value rows are written to the cache at slot_mapping, and decode then
// reads them back through the block table.  Slot s of a cache laid out as
// [num_blocks, block_size, Hkv, D] is row s of the flat [num_blocks*block_size,
// Hkv, D] view, so one token's K (or V) is one contiguous row of Hkv*D
// elements: the copy is a 16-byte-vector memcpy per row, bit exact.
//
// HBM-bound: each token reads 2 rows and writes 2 rows.  One thread moves 16
// bytes of K and 16 bytes of V; consecutive threads cover consecutive 16-byte
// chunks of a row, so every wave reads and writes whole 1 KiB spans.

#include "common.h"

namespace pkv {

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const char *__restrict__ key, const char *__restrict__ value, char *__restrict__ k_cache,
    char *__restrict__ v_cache, const int32_t *__restrict__ slot_mapping, int32_t T,
    int64_t key_stride_bytes, int64_t value_stride_bytes, int32_t row_chunks /* 16-byte chunks per row */,
    int32_t tokens_per_block)
{
    // tokens_per_block tokens share the block's 256 threads; a row longer
    // than 256 chunks is covered by one token per block, looping.
    const int per_token = tokens_per_block > 1 ? row_chunks : 256;
    const int t = blockIdx.x * tokens_per_block + (int)threadIdx.x / per_token;
    if ((int)threadIdx.x >= tokens_per_block * per_token || t >= T) return;
    const int32_t s = slot_mapping[t];
    if (s < 0) return;  // padding token
    const int64_t row_bytes = (int64_t)row_chunks * 16;
    for (int chunk = (int)threadIdx.x % per_token; chunk < row_chunks; chunk += per_token) {
        const u32x4 kv = *reinterpret_cast<const u32x4 *>(key + t * key_stride_bytes + chunk * 16);
        const u32x4 vv =
            *reinterpret_cast<const u32x4 *>(value + t * value_stride_bytes + chunk * 16);
        *reinterpret_cast<u32x4 *>(k_cache + (int64_t)s * row_bytes + chunk * 16) = kv;
        *reinterpret_cast<u32x4 *>(v_cache + (int64_t)s * row_bytes + chunk * 16) = vv;
    }
}

pkv_status launch_reshape_and_cache(const void *key, const void *value, void *k_cache,
                                    void *v_cache, const int32_t *slot_mapping, int32_t T,
                                    int64_t key_stride, int64_t value_stride, int32_t Hkv,
                                    int32_t D, int32_t elem_bytes, hipStream_t stream)
{
    const int32_t row_bytes = Hkv * D * elem_bytes;
    const int32_t row_chunks = row_bytes / 16;
    int32_t tokens_per_block = 256 / row_chunks;
    if (tokens_per_block < 1) tokens_per_block = 1;
    const int32_t blocks = (T + tokens_per_block - 1) / tokens_per_block;
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(blocks), dim3(256), 0, stream,
                       (const char *)key, (const char *)value, (char *)k_cache, (char *)v_cache,
                       slot_mapping, T, key_stride * elem_bytes, value_stride * elem_bytes,
                       row_chunks, tokens_per_block);
    return launch_status();
}

}  // namespace pkv
