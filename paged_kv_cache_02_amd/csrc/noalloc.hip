// pkv_paged_decode_noalloc: paged decode for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The workspace that pkv_paged_decode takes from its
// caller lives here in a static device array instead.
//
// The array's name is only a host-side stand-in for a device address: host
// code never passes it to a kernel.  Its address on each device is looked up
// once, with that device current, and every use goes through that pointer.

#include "common.h"
#include "decode.h"

#include <mutex>

namespace pkv {
namespace {

constexpr size_t kScratchBytes = (size_t)PKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void zero_words_kernel(u32x4 *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

std::mutex g_mutex;
void *g_ptr[kMaxDevices] = {};

// The scratch array's address on the current device.  On the first call on a
// device the array is cleared with a fill kernel on `stream` (not a memset, so
// that the first call may itself be captured into a graph), ahead of the work
// that call enqueues; later calls find it as the previous call left it.
pkv_status scratch_ptr(hipStream_t stream, void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_ERR_HIP;
        hipLaunchKernelGGL(zero_words_kernel, dim3(1024), dim3(256), 0, stream, (u32x4 *)p,
                           kScratchBytes / sizeof(u32x4));
        if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return PKV_OK;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" pkv_status pkv_paged_decode_noalloc(
    void *out, float *lse, const void *q, const void *k_cache, const void *v_cache,
    const int32_t *block_table, const int32_t *cache_seqlens, const float *sink, int32_t B,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_seqlen_k, float sm_scale,
    int32_t window_left, const float *alibi_slopes, int32_t partition_size, pkv_dtype dtype,
    void *stream)
{
    const DecodeCall c{out, lse, q, k_cache, v_cache, block_table, cache_seqlens, sink,
                       B, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_seqlen_k, sm_scale, window_left, alibi_slopes,
                       partition_size, dtype, stream};
    pkv_status st = decode_check(c);
    if (st != PKV_OK || B == 0) return st;
    if (decode_workspace_need(c) > kScratchBytes) return PKV_ERR_SCRATCH;
    void *ws = nullptr;
    if ((st = scratch_ptr((hipStream_t)stream, &ws)) != PKV_OK) return st;
    return decode_launch(c, ws);
}
