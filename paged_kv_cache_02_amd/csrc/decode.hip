// Paged decode: one query token per sequence over a paged KV cache.
//
// Transformers "Paged attention" doc, decode path: each sequence has one query
// token, its keys are cache_seqlens[b] cached tokens reached through the
// sequence's block_table row.  FlashInfer "sink_attention_reference.py"
// page, incremental branch: the query sits at position Lk-1; GQA head h reads
// kv head h / (Hq/Hkv); the sink logit joins the softmax denominator.  vLLM
// "attention.py" page, single_query_cached_kv_attention: a long context can
// be split into fixed-size token partitions whose partial results are merged
// afterwards (the merge is in merge.hip).
//
// gfx950 design (bf16, head_dim 64/128):
//   * one workgroup (4 waves) per (sequence, group of HU <= 4 query heads that
//     share a kv head, partition); the HU heads are packed into one MFMA so
//     every K/V tile is read from HBM once for all of them;
//   * a wave handles 16-token tiles (tile i of the partition goes to wave
//     i % 4), double-buffered in registers: the next tile's K/V 16-byte loads
//     are in flight while the current one is computed;
//   * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16: K rows are the A operand
//     straight from the 16-byte loads (lane r%16 = token, 8 consecutive dims
//     per lane), the HU query heads (replicated to 16 columns) are the B
//     operand held in registers; lane (j, r) receives the logits of tokens
//     4j..4j+3 for head r % HU;
//   * P.V on the VALU: lane (j, r) loads V rows of the same 4 tokens (16
//     lanes cover a whole row, so each row is one contiguous 256-byte read)
//     and takes the other heads' probabilities from its quad with DPP
//     broadcasts;
//   * online softmax with a wave-uniform reference maximum per head that is
//     only raised when a logit exceeds it by more than 2^8 (checked with one
//     ballot per tile), so the accumulator is almost never rescaled;
//   * the 4 waves' partial (max, sum, acc) are merged through LDS.
// The fp32 path (small correctness workloads) is a plain one-wave-per-row
// kernel in rowattn.hip.

#include "common.h"
#include "decode.h"

namespace pkv {

namespace {

constexpr int kWaves = 4;
constexpr float kTau = 8.0f;  // log2 headroom before the reference max is raised

template <int HU>
__device__ __forceinline__ float bcast_head(float x, int hh) {
    // quad lane hh holds head hh (lanes r, r%4 == hh; HU divides 4)
    switch (hh) {
        case 0: return quad_bcast<0>(x);
        case 1: return quad_bcast<1>(x);
        case 2: return quad_bcast<2>(x);
        default: return quad_bcast<3>(x);
    }
}

template <int D, int HU>
__global__ __launch_bounds__(256) void decode_bf16_kernel(DecodeArgs a)
{
    constexpr int KSTEPS = D / 32;            // MFMA k-steps over head_dim
    constexpr int VLD = D == 128 ? 4 : 2;     // V rows loaded per lane per tile
    static_assert(HU == 1 || HU == 2 || HU == 4, "heads per unit");

    __shared__ float sm_m[kWaves][HU];
    __shared__ float sm_l[kWaves][HU];
    __shared__ float sm_acc[kWaves][HU][D];

    const int lane = threadIdx.x & 63;
    const int wave = readfirstlane(threadIdx.x >> 6);
    const int j = lane >> 4, r = lane & 15;

    const int NHG = a.Hq / HU;
    int unit = blockIdx.x;
    const int pidx = unit % a.nparts;
    unit /= a.nparts;
    const int hg = unit % NHG;
    const int b = unit / NHG;
    const int h0 = hg * HU;
    const int g = h0 / a.G;
    const int L = a.seqlens[b];
    int start = pidx * a.part_size;
    const int end = min(start + a.part_size, L);
    if (a.window_left >= 0) start = max(start, L - 1 - a.window_left);

    const int tok_bytes = a.Hkv * D * 2;               // one token row, all kv heads
    const int bs_mask = (1 << a.bs_log2) - 1;

    // Q as the MFMA B operand: lane (j, r) holds dims 32c+8j..+8 of head h0 + r%HU.
    bf16x8 qf[KSTEPS];
    {
        const char *qp = (const char *)a.q +
                         (((size_t)b * a.Hq + h0 + (r % HU)) * D + 8 * j) * 2;
#pragma unroll
        for (int c = 0; c < KSTEPS; ++c) qf[c] = __builtin_bit_cast(bf16x8, ld16(qp, 64 * c));
    }

    // Per-lane byte offsets inside a tile (relative to the tile's first token row).
    const uint32_t koff = (uint32_t)(r * tok_bytes + (g * D + 8 * j) * 2);
    uint32_t voff[VLD];
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
        const int tv = D == 128 ? 4 * j + i : 4 * j + 2 * (r >> 3) + i;
        const int dv = D == 128 ? 8 * r : 8 * (r & 7);
        voff[i] = (uint32_t)(tv * tok_bytes + (g * D + dv) * 2);
    }

    float acc[HU][8];
#pragma unroll
    for (int hh = 0; hh < HU; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
    float m_lane = kNoMax;   // reference max (log2 units) of head r%HU; equal across those lanes
    float l_lane = 0.f;      // sum of p over this lane's 4 tokens, head r%HU

    const int tile0 = start & ~15;
    const int ntiles = start < end ? (end - tile0 + 15) >> 4 : 0;
    const int my_n = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;

    const int32_t *bt = a.block_table + (size_t)b * a.mbps;

    auto tile_base = [&](int t, const void *cache) -> const char * {
        const int blk = bt[t >> a.bs_log2];
        const size_t row0 = ((size_t)blk << a.bs_log2) + (t & bs_mask);
        return (const char *)cache + row0 * (size_t)tok_bytes;
    };

    auto load = [&](int t, u32x4 (&kb)[KSTEPS], u32x4 (&vb)[VLD]) {
        const char *kbase = tile_base(t, a.k_cache);
        const char *vbase = (const char *)a.v_cache + (kbase - (const char *)a.k_cache);
#pragma unroll
        for (int c = 0; c < KSTEPS; ++c) kb[c] = ld16(kbase, koff + 64 * c);
#pragma unroll
        for (int i = 0; i < VLD; ++i) vb[i] = ld16(vbase, voff[i]);
    };

    auto process = [&](int t, const u32x4 (&kb)[KSTEPS], u32x4 (&vb)[VLD]) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KSTEPS; ++c)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[c]), qf[c],
                                                        s, 0, 0, 0);
        // s[i]: token t + 4j + i, head h0 + r%HU
        const bool partial = t < start || t + 16 > end;
        bool valid[4];
        float sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pos = t + 4 * j + i;
            valid[i] = !partial || (pos >= start && pos < end);
            sv[i] = valid[i] ? s[i] * a.scale_log2 : -INFINITY;
        }
        const float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        if (__any(mx > m_lane + kTau)) {
            // raise the reference max of every head to its running maximum
            float tm = mx;
#pragma unroll
            for (int msk = HU; msk < 64; msk <<= 1) tm = fmaxf(tm, shfl_xor(tm, msk));
            const float nm = fmaxf(m_lane, tm);
            const float alpha = fast_exp2(m_lane - nm);
            l_lane *= alpha;
            m_lane = nm;
#pragma unroll
            for (int hh = 0; hh < HU; ++hh) {
                const float ah = bcast_head<HU>(alpha, hh);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[hh][e] *= ah;
            }
        }
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[i] - m_lane);
        l_lane += (p[0] + p[1]) + (p[2] + p[3]);

        if (partial) {
#pragma unroll
            for (int i = 0; i < VLD; ++i) {
                const bool vv = D == 128 ? valid[i] : ((r >> 3) ? valid[2 + i] : valid[i]);
                if (!vv) vb[i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const float pi = D == 128 ? p[i] : ((r >> 3) ? p[2 + i] : p[i]);
            float v[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                v[2 * w] = bf16_lo(vb[i][w]);
                v[2 * w + 1] = bf16_hi(vb[i][w]);
            }
#pragma unroll
            for (int hh = 0; hh < HU; ++hh) {
                const float ph = bcast_head<HU>(pi, hh);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(ph, v[e], acc[hh][e]);
            }
        }
    };

    if (my_n > 0) {
        u32x4 ka[KSTEPS], va[VLD], kb2[KSTEPS], vb2[VLD];
        int t = tile0 + 16 * wave;
        load(t, ka, va);
        for (int it = 0; it < my_n; it += 2) {
            const int t1 = t + 16 * kWaves;
            if (it + 1 < my_n) load(t1, kb2, vb2);
            process(t, ka, va);
            const int t2 = t1 + 16 * kWaves;
            if (it + 2 < my_n) load(t2, ka, va);
            if (it + 1 < my_n) process(t1, kb2, vb2);
            t = t2;
        }
    }

    // ---- reduce within the wave ----
    // l: lanes (j, r) with r < HU hold head r; sum over the 4 lane groups.
    float lsum = l_lane + shfl_xor(l_lane, 16);
    lsum += shfl_xor(lsum, 32);
    // acc: sum over lane groups j (and, for D=64, the two token halves r>>3).
#pragma unroll
    for (int hh = 0; hh < HU; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = acc[hh][e];
            if (D == 64) x += shfl_xor(x, 8);
            x += shfl_xor(x, 16);
            x += shfl_xor(x, 32);
            acc[hh][e] = x;
        }
    if (j == 0 && r < HU) {
        sm_m[wave][r] = m_lane;
        sm_l[wave][r] = lsum;
    }
    if (j == 0 && (D == 128 || r < 8)) {
        const int d0 = 8 * (D == 128 ? r : (r & 7));
#pragma unroll
        for (int hh = 0; hh < HU; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) sm_acc[wave][hh][d0 + e] = acc[hh][e];
    }
    __syncthreads();

    // ---- merge the waves and write ----
    for (int idx = threadIdx.x; idx < HU * D; idx += 256) {
        const int hh = idx / D, d = idx % D;
        const int h = h0 + hh;
        float M = sm_m[0][hh];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][hh]);
        float Ls = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = fast_exp2(sm_m[w][hh] - M);
            Ls = fmaf(sm_l[w][hh], sc, Ls);
            o = fmaf(sm_acc[w][hh][d], sc, o);
        }
        if (a.split) {
            const size_t pi = ((size_t)b * a.Hq + h) * a.nparts + pidx;
            a.part_out[pi * D + d] = Ls > 0.f ? o / Ls : 0.f;
            if (d == 0) a.part_lse[pi] = Ls > 0.f ? M * kLn2 + logf(Ls) : -INFINITY;
        } else {
            const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;
            const float Mt = fmaxf(Ls > 0.f ? M : kNoMax, sig);
            const float sc = fast_exp2(M - Mt);
            const float Lt = Ls * sc + fast_exp2(sig - Mt);
            const float res = Lt > 0.f ? o * sc / Lt : 0.f;
            const size_t oi = ((size_t)b * a.Hq + h) * D + d;
            ((uint16_t *)a.out)[oi] = f32_to_bf16(res);
            if (a.lse && d == 0)
                a.lse[(size_t)b * a.Hq + h] = Lt > 0.f ? Mt * kLn2 + logf(Lt) : -INFINITY;
        }
    }
}

template <int D, int HU>
void launch_one(const DecodeArgs &a, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((decode_bf16_kernel<D, HU>), dim3(grid), dim3(256), 0, stream, a);
}

}  // namespace

int decode_heads_per_unit(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

pkv_status launch_decode_bf16(const DecodeArgs &a, hipStream_t stream)
{
    const int HU = decode_heads_per_unit(a.G);
    const long long grid = (long long)a.B * (a.Hq / HU) * a.nparts;
    if (grid <= 0) return PKV_OK;
    if (grid > 0x7fffffffLL) return PKV_ERR_SHAPE;
    if (a.D == 128) {
        if (HU == 4) launch_one<128, 4>(a, (int)grid, stream);
        else if (HU == 2) launch_one<128, 2>(a, (int)grid, stream);
        else launch_one<128, 1>(a, (int)grid, stream);
    } else {
        if (HU == 4) launch_one<64, 4>(a, (int)grid, stream);
        else if (HU == 2) launch_one<64, 2>(a, (int)grid, stream);
        else launch_one<64, 1>(a, (int)grid, stream);
    }
    return launch_status();
}

}  // namespace pkv
