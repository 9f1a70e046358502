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
// One wave per (sequence, head): the lanes first reduce the partition
// maxima and the denominator over the (cheap) lse vector, then stream the
// partial rows, D/64 dims per lane, four partitions per loop trip.

#include "common.h"
#include "decode.h"

namespace pkv {

template <int D, bool BF16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a)
{
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (bh >= a.B * a.Hq) return;
    const int b = bh / a.Hq, h = bh % a.Hq;
    const int L = a.seqlens[b];
    const int n = (L + a.part_size - 1) / a.part_size;
    const float *pl = a.part_lse + (size_t)bh * a.nparts;
    const float *po = a.part_out + (size_t)bh * a.nparts * D;
    const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;

    // lse in log2 units, rounded once (no FMA contraction) so that the same
    // value enters the maximum and the weights: the dominant partition then
    // gets a weight of exactly 1.
    auto lse2 = [&](int p) { return __fmul_rn(pl[p], kLog2e); };
    float M = sig;
    for (int p = lane; p < n; p += 64) M = fmaxf(M, lse2(p));
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, shfl_xor(M, m));

    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = 0.f;
    float lse_out = -INFINITY;
    if (M != -INFINITY) {
        float Z = lane == 0 ? fast_exp2(sig - M) : 0.f;
        for (int p = lane; p < n; p += 64) Z += fast_exp2(lse2(p) - M);
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) Z += shfl_xor(Z, m);
        const float LSE = M + fast_log2(Z);   // log2 units
        lse_out = LSE * kLn2;
        int p = 0;
        for (; p + 4 <= n; p += 4) {
            float w[4], x[4][E];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float lp = lse2(p + u);
                w[u] = lp == -INFINITY ? 0.f : fast_exp2(lp - LSE);
#pragma unroll
                for (int e = 0; e < E; ++e) x[u][e] = po[(size_t)(p + u) * D + lane + 64 * e];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (w[u] > 0.f)
#pragma unroll
                    for (int e = 0; e < E; ++e) o[e] = fmaf(w[u], x[u][e], o[e]);
        }
        for (; p < n; ++p) {
            const float lp = lse2(p);
            if (lp == -INFINITY) continue;
            const float w = fast_exp2(lp - LSE);
#pragma unroll
            for (int e = 0; e < E; ++e) o[e] = fmaf(w, po[(size_t)p * D + lane + 64 * e], o[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const size_t oi = (size_t)bh * D + lane + 64 * e;
        if (BF16) ((uint16_t *)a.out)[oi] = f32_to_bf16(o[e]);
        else ((float *)a.out)[oi] = o[e];
    }
    if (a.lse && lane == 0) a.lse[bh] = lse_out;
}

pkv_status launch_merge(const MergeArgs &a, hipStream_t stream)
{
    const long long waves = (long long)a.B * a.Hq;
    if (waves == 0) return PKV_OK;
    const int grid = (int)((waves + 3) / 4);
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
