// Varlen causal prefill over contiguous or paged K/V, bf16 with fp32 accumulation.
//
// Transformers "Paged attention" doc, varlen path: packed requests indexed by
// cu_seq_lens_q/k, launch sized by max_length_q/k; FlashInfer
// "sink_attention_reference.py" page, varlen branch: request r's query row i
// sits at position p = Lk - Lq + i (queries are the last Lq positions), sees
// keys j <= p with p - window_left <= j when a window is set, GQA h -> h / G,
// and the per-head sink joins the denominator; vLLM "attention.py" page,
// multi_query_kv_attention: block-diagonal causal attention over packed
// prompts.  Paged mode reads K/V through the request's block_table row, so a
// query chunk can attend to keys already in the cache.
//
// gfx950 design:
//   * workgroup = (request, 128-row query tile, query head), 4 waves of 32
//     rows; tiles are issued longest-first (highest tile index first);
//   * K/V tiles of 64 keys are staged in LDS, double-buffered: global loads of
//     tile t+1 are in flight while tile t is computed; K is stored row-major
//     (padded), V transposed (V^T[d][key]) as it is written, so both MFMA
//     operands are read with plain ds_read_b128 / ds_read_b64;
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 with Q held in registers, so
//     each lane owns one query row: the row max/sum need one cross-lane step;
//   * O^T = V^T . P^T on the same MFMA; P goes from the S^T accumulators to
//     bf16 in place (the key order inside a k-step is the accumulator order,
//     matched by the V^T reads);
//   * online softmax with a reference max raised only when a logit exceeds it
//     by more than 2^8 (one ballot per tile), exp2 with the log2(e) scale folded
//     into the logit scale;
//   * masks are applied only on tiles that straddle the causal diagonal, the
//     window edge or the end of the keys; tiles outside a wave's visible range
//     are skipped.

#include "common.h"
#include "decode.h"

namespace pkv {

namespace {

constexpr int BM = 128;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile
constexpr float kTau = 8.0f;

template <int D>
struct Lds {
    static constexpr int KSTRIDE = D * 2 + 16;     // bytes per K row
    static constexpr int VSTRIDE = BN * 2 + 16;    // bytes per V^T row
    static constexpr int KBYTES = BN * KSTRIDE;
    static constexpr int VBYTES = D * VSTRIDE;
    static constexpr int BUF = KBYTES + VBYTES;
};

__device__ __forceinline__ uint32_t perm_lo(uint32_t a, uint32_t b) {
    // low halves: result = (a.lo) | (b.lo << 16)
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi(uint32_t a, uint32_t b) {
    // high halves: result = (a.hi) | (b.hi << 16)
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillArgs a)
{
    using L = Lds<D>;
    constexpr int QK_STEPS = D / 16;      // k-steps of 16 dims
    constexpr int DT = D / 32;            // 32-dim output tiles
    constexpr int NPAIR = (BN / 4) * (D / 8);   // (4-key group, 8-dim chunk) pairs per tile
    constexpr int PER_THREAD = (2 * NPAIR) / 256;  // K+V pairs per thread (2 or 1)
    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = readfirstlane(tid >> 6);
    const int lr = lane & 31;     // row within the wave / column of the MFMA
    const int lh = lane >> 5;     // lane half

    // ---- which (request, q tile, head) ----
    const int h = blockIdx.x % a.Hq;
    const int slot = blockIdx.x / a.Hq;
    const int r = slot % a.B;
    const int qt = a.max_q_tiles - 1 - slot / a.B;
    const int cq0 = a.cu_q[r], Lq = a.cu_q[r + 1] - cq0;
    if (qt * BM >= Lq) return;
    const int ck0 = a.cu_k[r], Lk = a.cu_k[r + 1] - ck0;
    const int g = h / a.G;
    const int row0 = qt * BM;                       // first row of the tile (within request)
    const int nrows = min(BM, Lq - row0);
    const int pos0 = Lk - Lq + row0;                // position of the tile's first row
    const int pos_last = pos0 + nrows - 1;
    int kv_lo = 0;
    if (a.window_left >= 0) kv_lo = max(0, pos0 - a.window_left);
    const int kv_hi = min(Lk, pos_last + 1);        // exclusive
    const int t_begin = kv_lo & ~(BN - 1);
    const int ntiles = kv_hi > kv_lo ? (kv_hi - t_begin + BN - 1) / BN : 0;

    // this wave's rows and visible key range
    const int wrow0 = row0 + 32 * wave;
    const int wrows = max(0, min(32, Lq - wrow0));
    const int wpos0 = Lk - Lq + wrow0;
    const int wpos1 = wpos0 + wrows - 1;
    const int w_lo = a.window_left >= 0 ? max(0, wpos0 - a.window_left) : 0;
    const int w_hi = min(Lk, wpos1 + 1);

    const size_t qstride = (size_t)a.Hq * D;     // elements between tokens of q/out
    const size_t kvstride = (size_t)a.Hkv * D;   // elements between tokens of k/v

    // ---- Q^T operand: lane holds row lr, dims 16c + 8lh .. +8 ----
    bf16x8 qf[QK_STEPS];
    {
        const bool ok = lr < wrows;
        const uint16_t *qp = (const uint16_t *)a.q + (size_t)(cq0 + wrow0 + (ok ? lr : 0)) * qstride +
                             (size_t)h * D + 8 * lh;
#pragma unroll
        for (int c = 0; c < QK_STEPS; ++c) {
            u32x4 x = u32x4{0u, 0u, 0u, 0u};
            if (ok) x = *reinterpret_cast<const u32x4 *>(qp + 16 * c);
            qf[c] = __builtin_bit_cast(bf16x8, x);
        }
    }

    f32x16 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
    float m = kNoMax, l = 0.f;

    // ---- tile loading: each thread owns PER_THREAD (4-key, 8-dim) pairs ----
    const int32_t *bt = a.block_table ? a.block_table + (size_t)r * a.mbps : nullptr;
    const int bs_mask = (1 << a.bs_log2) - 1;
    u32x4 stage[PER_THREAD][4];

    auto key_row = [&](int key) -> size_t {   // element offset of (key, kv head g, dim 0)
        size_t row;
        if (bt) row = ((size_t)bt[key >> a.bs_log2] << a.bs_log2) + (key & bs_mask);
        else row = (size_t)ck0 + key;
        return row * kvstride + (size_t)g * D;
    };

    auto issue_loads = [&](int t0) {
#pragma unroll
        for (int u = 0; u < PER_THREAD; ++u) {
            const int pidx = tid + 256 * u;
            const bool isv = pidx >= NPAIR;
            const int pp = isv ? pidx - NPAIR : pidx;
            // K: 8-dim chunk fastest (coalesced rows); V: 4-key group fastest
            const int kq = isv ? (pp % (BN / 4)) : (pp / (D / 8));
            const int dc = isv ? (pp / (BN / 4)) : (pp % (D / 8));
            const int key0 = t0 + 4 * kq;
            const uint16_t *base = (const uint16_t *)(isv ? (bt ? a.v_cache : a.v)
                                                          : (bt ? a.k_cache : a.k));
            if (key0 + 3 < Lk) {
                const size_t off = key_row(key0) + 8 * dc;   // 4 keys share a block (bs >= 16)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    stage[u][c] = *reinterpret_cast<const u32x4 *>(base + off + c * kvstride);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    stage[u][c] = u32x4{0u, 0u, 0u, 0u};
                    if (key0 + c < Lk)
                        stage[u][c] = *reinterpret_cast<const u32x4 *>(base + key_row(key0 + c) +
                                                                        8 * dc);
                }
            }
        }
    };

    auto store_lds = [&](int buf) {
        char *kl = lds + buf * L::BUF;
        char *vl = kl + L::KBYTES;
#pragma unroll
        for (int u = 0; u < PER_THREAD; ++u) {
            const int pidx = tid + 256 * u;
            const bool isv = pidx >= NPAIR;
            const int pp = isv ? pidx - NPAIR : pidx;
            const int kq = isv ? (pp % (BN / 4)) : (pp / (D / 8));
            const int dc = isv ? (pp / (BN / 4)) : (pp % (D / 8));
            if (!isv) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *reinterpret_cast<u32x4 *>(kl + (4 * kq + c) * L::KSTRIDE + 16 * dc) =
                        stage[u][c];
            } else {
                // transpose 4 keys x 8 dims into 8 rows of V^T, 4 keys (8 bytes) each
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const u32x2 lo = {perm_lo(stage[u][0][w], stage[u][1][w]),
                                      perm_lo(stage[u][2][w], stage[u][3][w])};
                    const u32x2 hi = {perm_hi(stage[u][0][w], stage[u][1][w]),
                                      perm_hi(stage[u][2][w], stage[u][3][w])};
                    *reinterpret_cast<u32x2 *>(vl + (8 * dc + 2 * w) * L::VSTRIDE + 8 * kq) = lo;
                    *reinterpret_cast<u32x2 *>(vl + (8 * dc + 2 * w + 1) * L::VSTRIDE + 8 * kq) = hi;
                }
            }
        }
    };

    auto compute = [&](int buf, int t0) {
        const char *kl = lds + buf * L::BUF;
        const char *vl = kl + L::KBYTES;
        // S^T for the two 32-key chunks
        f32x16 s[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kc][i] = 0.f;
            const char *krow = kl + (32 * kc + lr) * L::KSTRIDE + 16 * lh;
#pragma unroll
            for (int c = 0; c < QK_STEPS; ++c) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(krow + 32 * c);
                s[kc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kc], 0, 0, 0);
            }
        }
        // scale + mask.  Key of accumulator (kc, i): t0 + 32kc + 8(i/4) + 4lh + i%4.
        const int pos = wpos0 + lr;
        const bool full = (t0 + BN - 1 <= wpos0) && (t0 + BN <= Lk) &&
                          (a.window_left < 0 || t0 >= wpos1 - a.window_left);
        float mx = -INFINITY;
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float x = s[kc][i] * a.scale_log2;
                if (!full) {
                    const int key = t0 + 32 * kc + 8 * (i >> 2) + 4 * lh + (i & 3);
                    const bool vis = key <= pos && key < Lk &&
                                     (a.window_left < 0 || key >= pos - a.window_left);
                    x = vis ? x : -INFINITY;
                }
                s[kc][i] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, shfl_xor(mx, 32));
        if (__any(mx > m + kTau)) {
            const float nm = fmaxf(m, mx);
            const float alpha = fast_exp2(m - nm);
            l *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
            m = nm;
        }
        // P = exp2(S - m) -> bf16, 4 k-steps of 16 keys
        bf16x8 pf[4];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int sp = 0; sp < 2; ++sp) {
                u32x4 w;
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const float p0 = fast_exp2(s[kc][8 * sp + 2 * e2] - m);
                    const float p1 = fast_exp2(s[kc][8 * sp + 2 * e2 + 1] - m);
                    l += p0 + p1;
                    w[e2] = pack_bf16x2(p0, p1);
                }
                pf[2 * kc + sp] = __builtin_bit_cast(bf16x8, w);
            }
        // O^T += V^T . P^T
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            const char *vrow = vl + (32 * t + lr) * L::VSTRIDE;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int kb = 16 * ks + 4 * lh;   // key of element 0 (elements 4..7: kb + 8)
                const u32x2 v0 = *reinterpret_cast<const u32x2 *>(vrow + 2 * kb);
                const u32x2 v1 = *reinterpret_cast<const u32x2 *>(vrow + 2 * (kb + 8));
                const u32x4 vv = {v0[0], v0[1], v1[0], v1[1]};
                o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv),
                                                               pf[ks], o[t], 0, 0, 0);
            }
        }
    };

    if (ntiles > 0) {
        issue_loads(t_begin);
        store_lds(0);
        __syncthreads();
        for (int it = 0; it < ntiles; ++it) {
            const int t0 = t_begin + it * BN;
            if (it + 1 < ntiles) issue_loads(t0 + BN);
            if (wrows > 0 && t0 < w_hi && t0 + BN > w_lo) compute(it & 1, t0);
            if (it + 1 < ntiles) store_lds((it + 1) & 1);
            __syncthreads();
        }
    }

    // ---- epilogue: normalise with the sink, write the wave's rows ----
    l += shfl_xor(l, 32);
    const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;
    const float Mt = fmaxf(l > 0.f ? m : kNoMax, sig);
    const float sc = fast_exp2(m - Mt);
    const float Lt = l * sc + fast_exp2(sig - Mt);
    const float f = Lt > 0.f ? sc / Lt : 0.f;
    if (lr < wrows) {
        uint16_t *op = (uint16_t *)a.out + (size_t)(cq0 + wrow0 + lr) * qstride + (size_t)h * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 32 * t + 8 * q4 + 4 * lh;
                const u32x2 w = {pack_bf16x2(o[t][4 * q4] * f, o[t][4 * q4 + 1] * f),
                                 pack_bf16x2(o[t][4 * q4 + 2] * f, o[t][4 * q4 + 3] * f)};
                *reinterpret_cast<u32x2 *>(op + d) = w;
            }
        if (a.lse && lh == 0)
            a.lse[(size_t)(cq0 + wrow0 + lr) * a.Hq + h] =
                Lt > 0.f ? Mt * kLn2 + logf(Lt) : -INFINITY;
    }
}

}  // namespace

pkv_status launch_prefill_bf16(const PrefillArgs &a, hipStream_t stream)
{
    const long long grid = (long long)a.B * a.max_q_tiles * a.Hq;
    if (grid == 0) return PKV_OK;
    if (grid > 0x7fffffffLL) return PKV_ERR_SHAPE;
    // more than 64 KiB of dynamic LDS: raise the per-kernel limit once
    static const bool raised = [] {
        hipFuncSetAttribute((const void *)prefill_bf16_kernel<128>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 2 * Lds<128>::BUF);
        hipFuncSetAttribute((const void *)prefill_bf16_kernel<64>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 2 * Lds<64>::BUF);
        return true;
    }();
    (void)raised;
    if (a.D == 128) {
        const int lds = 2 * Lds<128>::BUF;
        hipLaunchKernelGGL((prefill_bf16_kernel<128>), dim3((int)grid), dim3(256), lds, stream, a);
    } else {
        const int lds = 2 * Lds<64>::BUF;
        hipLaunchKernelGGL((prefill_bf16_kernel<64>), dim3((int)grid), dim3(256), lds, stream, a);
    }
    return launch_status();
}

int prefill_block_m() { return BM; }

}  // namespace pkv
