// Split-KV merge: combine per-partition attention results by log-sum-exp.
//
// vLLM "attention.py" page, single_query_cached_kv_attention: the partitioned
// decode keeps, per (sequence, head, partition), a partial output plus its
// softmax statistics and reduces them in a second step.  Here each partition p
// holds o_p (normalised over its own visible keys) and lse_p = ln sum_p exp(s);
// with the per-head sink s_h (FlashInfer sink-attention page: one more term of
// the denominator, no value row) added exactly once:
//     LSE = ln(sum_p exp(lse_p) + exp(s_h)),   out = sum_p exp(lse_p - LSE) o_p.
//
// One 256-thread workgroup per (sequence, head): the threads first reduce the
// partition maxima and the denominator over the lse vector, then stream the
// partial rows as float4 chunks, 256 / (D/4) partitions side by side, and
// sum those lanes of partitions through LDS.

#include "common.h"
#include "decode.h"

namespace pkv {

template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a)
{
    constexpr int CH = D / 4;            // float4 chunks per partial row
    constexpr int ROWS = 256 / CH;       // partitions streamed in parallel
    __shared__ float red[8];
    __shared__ f32x4 part[ROWS][CH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x;
    const int b = bh / a.Hq, h = bh % a.Hq;
    // partial results of (b, h): n partitions, partition p at row bh * nparts + p
    const int L = a.seqlens[b];
    const int n = (L + a.part_size - 1) / a.part_size;
    const size_t pl0 = (size_t)bh * a.nparts, pls = 1;
    const size_t po0 = pl0 * D, pos = pls * D;
    const float *pl = a.part_lse + pl0;
    const float *po_base = a.part_out + po0;
    const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;

    // lse in log2 units, rounded once (no FMA contraction) so that the same
    // value enters the maximum and the weights: the dominant partition then
    // gets a weight of exactly 1.
    auto lse2 = [&](int p) { return __fmul_rn(pl[(size_t)p * pls], kLog2e); };
    auto prow = [&](int p, int c) {
        return *reinterpret_cast<const f32x4 *>(po_base + (size_t)p * pos + 4 * c);
    };

    auto block_max = [&](float x) {
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, shfl_xor(x, m));
        if (lane == 0) red[wave] = x;
        __syncthreads();
        x = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        return x;
    };
    auto block_sum = [&](float x) {
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) x += shfl_xor(x, m);
        if (lane == 0) red[4 + wave] = x;
        __syncthreads();
        return (red[4] + red[5]) + (red[6] + red[7]);
    };

    float M = tid == 0 ? sig : -INFINITY;
    for (int p = tid; p < n; p += 256) M = fmaxf(M, lse2(p));
    M = block_max(M);

    const int c = tid % CH, row = tid / CH;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lse_out = -INFINITY;
    if (M != -INFINITY) {
        float Z = tid == 0 ? fast_exp2(sig - M) : 0.f;
        for (int p = tid; p < n; p += 256) Z += fast_exp2(lse2(p) - M);
        Z = block_sum(Z);
        const float LSE = M + fast_log2(Z);   // log2 units
        lse_out = LSE * kLn2;
        int p = row;
        for (; p + ROWS < n; p += 2 * ROWS) {
            const float l0 = lse2(p), l1 = lse2(p + ROWS);
            const f32x4 x0 = prow(p, c);
            const f32x4 x1 = prow(p + ROWS, c);
            if (l0 != -INFINITY) o += fast_exp2(l0 - LSE) * x0;
            if (l1 != -INFINITY) o += fast_exp2(l1 - LSE) * x1;
        }
        if (p < n) {
            const float l0 = lse2(p);
            if (l0 != -INFINITY) o += fast_exp2(l0 - LSE) * prow(p, c);
        }
    }
    part[row][c] = o;
    __syncthreads();
    if (tid < CH) {
        f32x4 t = part[0][tid];
#pragma unroll
        for (int r2 = 1; r2 < ROWS; ++r2) t += part[r2][tid];
        const size_t oi = (size_t)bh * D + 4 * tid;
        if (BF16) {
            u32x2 w = {pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])};
            *reinterpret_cast<u32x2 *>((uint16_t *)a.out + oi) = w;
        } else {
            *reinterpret_cast<f32x4 *>((float *)a.out + oi) = t;
        }
    }
    if (a.lse && tid == 0) a.lse[bh] = lse_out;
}

pkv_status launch_merge(const MergeArgs &a, hipStream_t stream)
{
    const long long rows = (long long)a.B * a.Hq;
    if (rows == 0) return PKV_OK;
    if (rows > 0x7fffffffLL) return PKV_ERR_SHAPE;
    const int grid = (int)rows;
    const bool bf = a.dtype == PKV_BF16;
    if (a.D == 128) {
        if (bf) hipLaunchKernelGGL((merge_kernel<128, true>), dim3(grid), dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((merge_kernel<128, false>), dim3(grid), dim3(256), 0, stream, a);
    } else {
        if (bf) hipLaunchKernelGGL((merge_kernel<64, true>), dim3(grid), dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((merge_kernel<64, false>), dim3(grid), dim3(256), 0, stream, a);
    }
    return launch_status();
}

}  // namespace pkv
