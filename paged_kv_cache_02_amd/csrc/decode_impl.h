// Paged decode: one query token per sequence over a paged KV cache.
//
// Transformers "Paged attention" doc, decode path: each sequence has one query
// token, its keys are cache_seqlens[b] cached tokens reached through the
// sequence's block_table row.  FlashInfer "sink_attention_reference.py"
// page, incremental branch: the query sits at position Lk-1; GQA head h reads
// kv head h / (Hq/Hkv); the sink logit joins the softmax denominator.  vLLM
// "attention.py" page, single_query_cached_kv_attention: the keys can be split
// into parts whose partial results are combined by log-sum-exp afterwards
// (merge.hip).
//
// gfx950 design (bf16, head_dim 64/128).  The work is a stream of 16-token
// tiles; a tile is 16 consecutive token rows of one block (of two blocks when
// the block size is 8: rows 8..15 are read from the second one through
// per-lane addresses), read for one kv head.  Each wave runs the same tile engine (DecodeWave below):
//   * HU <= 4 query heads that share a kv head are packed into one MFMA, so
//     each K/V tile is read from HBM once for all of them;
//   * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16: K rows are the A operand
//     straight from 16-byte loads (lane r%16 = token, 8 dims per lane), the
//     HU heads (replicated to 16 columns) are the B operand in registers;
//     lane (j, r) receives the logits of tokens 4j..4j+3 for head r % HU;
//   * O^T += V^T . P on v_mfma_f32_16x16x16_bf16, one MFMA per 16 dims: lane
//     (j, r) loads V rows of the same 4 tokens (16 lanes cover a 256-byte
//     row) and leaves them in the wave's LDS buffer, token-major; the V^T
//     operand comes back by the LDS transpose read, P (the logits' lanes,
//     rounded to bf16) is the B operand as it stands, and lane (j, r) then
//     holds head r % HU at dims 16 db + 4 j .. +3 of every 16-dim block db;
//   * online softmax with a reference maximum per head that is raised only
//     when a logit exceeds it by more than 2^8 (one ballot per tile);
//   * a ring of 4 register buffers keeps 3 tiles in flight per wave; loads go
//     through buffer descriptors (an empty range for padding tiles, which then
//     cost no memory traffic) so every trip issues the same loads and the
//     in-order vmcnt waits stay exact.
//
// Two schedules use the engine:
//   * decode_part_kernel: fixed token partitions [p*P, (p+1)*P) (the API's
//     explicit partition_size, or no split): one workgroup per (sequence,
//     head group, partition), its 4 waves interleave the partition's tiles and
//     merge through LDS;
//   * decode_stream_kernel: balanced persistent schedule.  The tiles of all
//     sequences of a head group are laid end to end; each wave of a grid sized
//     to the machine takes an equal contiguous range of that list (computed on
//     the device from cache_seqlens), streams it without stopping at sequence
//     boundaries and writes one partial result per sequence it touches.  A
//     wave's pipeline is filled and drained once, not once per partition, and
//     no wave is left with a short last partition.  The pieces are merged
//     either by the merge kernel (two launches) or inside the same launch:
//     each wave counts its pieces in a per-(sequence, head group) counter
//     after its stream, and the wave whose count completes a sequence merges
//     it (a sequence held by one wave alone is written directly).
// The fp32 path (small correctness workloads) is rowattn.hip.
//
// This header holds the engine and both schedules as templates; decode.hip
// instantiates them for block sizes of 16 and more, decode_bs8.hip for block
// size 8 (a tile then spans two blocks).
#pragma once

#include "common.h"
#include "decode.h"
#include "rope.h"

namespace pkv {

namespace {

constexpr int kWaves = 4;
constexpr float kTau = 8.0f;  // log2 headroom before the reference max is raised
constexpr int kDepth = 3;     // K/V tiles in flight per wave
constexpr int kRing = kDepth + 1;
// s_waitcnt immediate for vmcnt(0) with expcnt/lgkmcnt left at their maxima
// (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
constexpr int kWaitVmcnt0 = (7 << 4) | (15 << 8);
// the same immediate for vmcnt(n), n < 64
constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int HU>
__device__ __forceinline__ float bcast_head(float x, int hh) {
    // quad lane hh holds head hh (lanes r with r % 4 == hh; HU divides 4)
    switch (hh) {
        case 0: return quad_bcast<0>(x);
        case 1: return quad_bcast<1>(x);
        case 2: return quad_bcast<2>(x);
        default: return quad_bcast<3>(x);
    }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// The per-wave LDS buffer of the P.V step: 16 token rows of V (head_dim bf16
// plus 16 bytes of padding, so that the lanes' 16-byte row writes spread over
// all banks); reduce() reuses it for the accumulators.
template <int D> constexpr int vt_row_bytes() { return D * 2 + 16; }
template <int D> constexpr int vt_bytes() { return 16 * vt_row_bytes<D>(); }

template <int D, int HU, bool ALIBI = false, bool BS8 = false>
struct DecodeWave {
    static constexpr int KSTEPS = D / 32;          // MFMA k-steps over head_dim
    static constexpr int VLD = D == 128 ? 4 : 2;   // V rows loaded per lane per tile
    static constexpr int DB = D / 16;              // 16-dim blocks of the output
    static constexpr int VROW = vt_row_bytes<D>();
    static_assert(HU == 1 || HU == 2 || HU == 4, "heads per unit");
    static_assert(HU * D * 4 <= vt_bytes<D>(), "reduce() fits in the buffer");

    int lane, j, r;
    int tok_bytes;          // one token row, all kv heads
    uint32_t koff, voff[VLD];
    // BS8: whether this lane's K row (and each V row) lies in the second
    // 8-token block of a tile
    bool khi, vhi[VLD];
    bf16x8 qf[KSTEPS];
    f32x4 oacc[DB];         // O^T: head r % HU, dims 16 db + 4 j + i
    float acc[HU][8];       // after reduce(): see there
    char *vt;               // this wave's LDS buffer
    float m_lane, l_lane;
    float scale_log2;
    // ALiBi: the slope of this lane's head (column r % HU) times log2(e), 0
    // without; the logit of key pos gets slope * (pos - qpos) added, qpos
    // being the query's position
    float slope_log2;
    int qpos;

    __device__ void setup(int g, int Hkv, float sl2, const float *alibi, int h0, char *vt_buf) {
        vt = vt_buf;
        lane = threadIdx.x & 63;
        j = lane >> 4;
        r = lane & 15;
        tok_bytes = Hkv * D * 2;
        scale_log2 = sl2;
        slope_log2 = alibi ? alibi[h0 + r % HU] * kLog2e : 0.f;
        qpos = 0;
        koff = (uint32_t)(r * tok_bytes + (g * D + 8 * j) * 2);
        khi = r >= 8;
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int tv = D == 128 ? 4 * j + i : 4 * j + 2 * (r >> 3) + i;
            const int dv = D == 128 ? 8 * r : 8 * (r & 7);
            voff[i] = (uint32_t)(tv * tok_bytes + (g * D + dv) * 2);
            vhi[i] = tv >= 8;
        }
    }

    // Q as the MFMA B operand: lane (j, r) holds dims 32c+8j..+8 of head h0 + r%HU.
    __device__ void load_q(const void *q, size_t first_head_row) { load_q_to(qf, q, first_head_row); }
    __device__ void load_q_to(bf16x8 (&dst)[KSTEPS], const void *q, size_t first_head_row) const {
        const char *qp = (const char *)q + ((first_head_row + (r % HU)) * D + 8 * j) * 2;
#pragma unroll
        for (int c = 0; c < KSTEPS; ++c) dst[c] = __builtin_bit_cast(bf16x8, ld16(qp, 64 * c));
    }

    __device__ void reset() {
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_lane = kNoMax;
        l_lane = 0.f;
    }

    // Issue the 16-byte loads of one tile whose first token row starts
    // `row_off` bytes into the caches; a dead tile gets an empty range.
    // BS8: rows 8..15 start `row_off1` bytes in (the tile's second block);
    // the loads take per-lane addresses, and a dead tile reads block 0.
    __device__ void load(const void *kc, const void *vc, size_t row_off, size_t row_off1,
                         bool live, u32x4 (&kb)[KSTEPS], u32x4 (&vb)[VLD]) const {
        if constexpr (BS8) {
            typedef __attribute__((address_space(1))) const char gchar;
            const size_t o0 = live ? row_off : 0;
            const size_t o1 = (live ? row_off1 : 0) - (size_t)8 * tok_bytes;
            gchar *kg = (gchar *)kc, *vg = (gchar *)vc;
            gchar *kb0 = kg + (khi ? o1 : o0) + koff;
#pragma unroll
            for (int c = 0; c < KSTEPS; ++c) kb[c] = *reinterpret_cast<const __attribute__((address_space(1))) u32x4 *>(kb0 + 64 * c);
#pragma unroll
            for (int i = 0; i < VLD; ++i)
                vb[i] = *reinterpret_cast<const __attribute__((address_space(1))) u32x4 *>(vg + (vhi[i] ? o1 : o0) + voff[i]);
            return;
        }
        const int span = live ? 16 * tok_bytes : 0;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const char *)kc + row_off), (short)0, span, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const char *)vc + row_off), (short)0, span, kBufferWord3);
#pragma unroll
        for (int c = 0; c < KSTEPS; ++c)
            kb[c] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(koff + 64 * c), 0, 0);
#pragma unroll
        for (int i = 0; i < VLD; ++i)
            vb[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)voff[i], 0, 0);
    }

    // Fold tile [t, t+16) into the running state; positions outside [lo, hi)
    // (or every position, for a dead tile) are masked.
    __device__ void process(int t, int lo, int hi, bool live, const u32x4 (&kb)[KSTEPS],
                            u32x4 (&vb)[VLD]) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KSTEPS; ++c)
            s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[c]), qf[c],
                                                        s, 0, 0, 0);
        const bool partial = !live || t < lo || t + 16 > hi;
        bool valid[4];
        float sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pos = t + 4 * j + i;
            valid[i] = !partial || (live && pos >= lo && pos < hi);
            const float x = ALIBI ? fmaf(s[i], scale_log2, slope_log2 * (float)(pos - qpos))
                                  : s[i] * scale_log2;
            sv[i] = valid[i] ? x : -INFINITY;
        }
        const float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        if (__any(mx > m_lane + kTau)) {
            // raise every head's reference max to its running maximum
            float tm = mx;
#pragma unroll
            for (int msk = HU; msk < 64; msk <<= 1) tm = fmaxf(tm, shfl_xor(tm, msk));
            const float nm = fmaxf(m_lane, tm);
            const float alpha = fast_exp2(m_lane - nm);
            l_lane *= alpha;
            m_lane = nm;
            // lane (j, r) holds head r % HU only: its own alpha
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        }
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[i] - m_lane);
        // P rounded to bf16 for the MFMA; the row sum takes the rounded values
        const uint32_t p01 = pack_bf16x2(p[0], p[1]), p23 = pack_bf16x2(p[2], p[3]);
        l_lane += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));

        // V rows at masked positions are zeroed: whatever those cache slots
        // hold (never written, NaN) must not reach the MFMA, even times 0
        if (partial) {
#pragma unroll
            for (int i = 0; i < VLD; ++i) {
                const bool vv = D == 128 ? valid[i] : ((r >> 3) ? valid[2 + i] : valid[i]);
                if (!vv) vb[i] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        // V token-major into the wave's buffer (lane (j, r) has rows tv of
        // dims dv .. dv + 7), then O^T += V^T . P per 16-dim block: lane
        // (j, r) reads by the transpose read the 4 dims 16 db + 4 (r % 4) of
        // token row 4 j + r / 4, and receives dim 16 db + r of tokens 4 j ..
        // 4 j + 3, the A operand; P of those tokens for head column r is the
        // B operand.  A wave's LDS accesses run in order, so the reads see
        // this tile's writes and the next tile's writes come after them.
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int tv = D == 128 ? 4 * j + i : 4 * j + 2 * (r >> 3) + i;
            const int dv = D == 128 ? 8 * r : 8 * (r & 7);
            *reinterpret_cast<u32x4 *>(vt + tv * VROW + dv * 2) = vb[i];
        }
        const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{p01, p23});
        const char *vr = vt + (4 * j + (r >> 2)) * VROW + 8 * (r & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(vr + 32 * db));
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, va), pb,
                                                                 oacc[db], 0, 0, 0);
        }
    }

    // Gather the state: afterwards lanes with j == 0 (and r < 8 for D = 64)
    // hold acc[hh] for dims d0()..d0()+7 of every head hh, and the returned
    // sum of p is complete in lanes r < HU (for head r).
    // x + x^16 and x + x^32 (lane index xor 16 / 32) with the VALU lane swaps
    // of gfx950: permlane16_swap(x, x) returns the even and the odd 16-lane
    // rows of each pair side by side, permlane32_swap(x, x) the two halves
    // of the wave, so the two results summed give the pairwise sum in every
    // lane (no LDS permute)
    static __device__ __forceinline__ float sum_xor16(float x) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                         false, false);
        return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    static __device__ __forceinline__ float sum_xor32(float x) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                         false, false);
        return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    // x + x^8 within each 16-lane row (DPP row rotate by 8)
    static __device__ __forceinline__ float sum_xor8(float x) {
        return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf,
                                                              0xf, false));
    }
    __device__ float reduce() {
        const float lsum = sum_xor32(sum_xor16(l_lane));
        // the MFMA summed over the tokens already; the lanes of head column
        // r < HU leave their dims in the buffer as [head][dim] floats, and
        // the holding lanes read their 8 dims of every head back (in order
        // within the wave, like the P.V step)
        float *sa = reinterpret_cast<float *>(vt);
        if (r < HU) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
                *reinterpret_cast<f32x4 *>(sa + r * D + 16 * db + 4 * j) = oacc[db];
        }
        if (holds_acc()) {
#pragma unroll
            for (int hh = 0; hh < HU; ++hh) {
                const f32x4 lo4 = *reinterpret_cast<const f32x4 *>(sa + hh * D + d0());
                const f32x4 hi4 = *reinterpret_cast<const f32x4 *>(sa + hh * D + d0() + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[hh][e] = lo4[e];
                    acc[hh][4 + e] = hi4[e];
                }
            }
        }
        return lsum;
    }
    __device__ bool holds_acc() const { return j == 0 && (D == 128 || r < 8); }
    __device__ int d0() const { return 8 * (D == 128 ? r : (r & 7)); }
};

// ---------------------------------------------------------------------------
// Fixed partitions: one workgroup per (sequence, head group, partition).
// ---------------------------------------------------------------------------
template <int D, int HU, bool ALIBI, bool BS8>
__global__ __launch_bounds__(256) void decode_part_kernel(DecodeArgs a)
{
    __shared__ float sm_m[kWaves][HU];
    __shared__ float sm_l[kWaves][HU];
    __shared__ float sm_acc[kWaves][HU][D];
    __shared__ __attribute__((aligned(16))) char s_vt[kWaves][vt_bytes<D>()];

    const int wave = readfirstlane(threadIdx.x >> 6);
    const int NHG = a.Hq / HU;
    // Head groups of one (sequence, partition) are adjacent in dispatch order,
    // so the workgroups that share a block's token rows run together.
    int unit = blockIdx.x;
    const int hg = unit % NHG;
    unit /= NHG;
    const int pidx = unit % a.nparts;
    const int b = unit / a.nparts;
    const int h0 = hg * HU;
    const int g = h0 / a.G;
    const int L = a.seqlens[b];
    int start = pidx * a.part_size;
    const int end = min(start + a.part_size, L);
    if (a.window_left >= 0) start = max(start, L - 1 - a.window_left);

    DecodeWave<D, HU, ALIBI, BS8> w;
    w.setup(g, a.Hkv, a.scale_log2, a.alibi, h0, s_vt[wave]);
    w.qpos = L - 1;
    w.load_q(a.q, (size_t)b * a.Hq + h0);
    w.reset();

    const int bs_mask = (1 << a.bs_log2) - 1;
    const int tile0 = start & ~15;
    const int ntiles = start < end ? (end - tile0 + 15) >> 4 : 0;
    const int my_n = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;

    // block ids through the scalar cache (constant address space)
    const __attribute__((address_space(4))) int32_t *bt =
        (const __attribute__((address_space(4))) int32_t *)(a.block_table + (size_t)b * a.mbps);
    auto tile_tok = [&](int i) { return tile0 + 16 * (wave + kWaves * i); };
    auto block_of = [&](int i) { return bt[tile_tok(i) >> a.bs_log2]; };
    auto row_off = [&](int i, int blk) {
        return (((size_t)blk << a.bs_log2) + (tile_tok(i) & bs_mask)) * (size_t)w.tok_bytes;
    };
    // BS8: the block of the tile's rows 8..15 (the tile's first block when
    // they lie past the sequence, so that no entry past its blocks is read)
    auto block_of1 = [&](int i) { return BS8 ? bt[min(tile_tok(i) + 8, L - 1) >> 3] : 0; };
    auto row_off1 = [&](int blk1) { return ((size_t)blk1 << 3) * (size_t)w.tok_bytes; };

    if (my_n > 0) {
        u32x4 kbuf[kRing][DecodeWave<D, HU>::KSTEPS], vbuf[kRing][DecodeWave<D, HU>::VLD];
        const int last = my_n - 1;
        const int n_pad = (my_n + kRing - 1) / kRing * kRing;
#pragma unroll
        for (int k = 0; k < kDepth; ++k) {
            const int i = min(k, last);
            w.load(a.k_cache, a.v_cache, row_off(i, block_of(i)), row_off1(block_of1(i)),
                   k < my_n, kbuf[k], vbuf[k]);
            __builtin_amdgcn_sched_barrier(0);
        }
        int blk_next = block_of(min(kDepth, last));
        int blk_next1 = block_of1(min(kDepth, last));
        for (int it = 0; it < n_pad; it += kRing) {
#pragma unroll
            for (int k = 0; k < kRing; ++k) {
                const int cur = it + k;
                const int nxt = cur + kDepth;
                const int ni = min(nxt, last);
                w.load(a.k_cache, a.v_cache, row_off(ni, blk_next), row_off1(blk_next1),
                       nxt < my_n, kbuf[(k + kDepth) % kRing], vbuf[(k + kDepth) % kRing]);
                blk_next = block_of(min(nxt + 1, last));
                blk_next1 = block_of1(min(nxt + 1, last));
                __builtin_amdgcn_sched_barrier(0);
                w.process(tile_tok(cur), start, end, cur < my_n, kbuf[k], vbuf[k]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    const float lsum = w.reduce();
    if (w.j == 0 && w.r < HU) {
        sm_m[wave][w.r] = w.m_lane;
        sm_l[wave][w.r] = lsum;
    }
    if (w.holds_acc()) {
#pragma unroll
        for (int hh = 0; hh < HU; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) sm_acc[wave][hh][w.d0() + e] = w.acc[hh][e];
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < HU * D; idx += 256) {
        const int hh = idx / D, d = idx % D;
        const int h = h0 + hh;
        float M = sm_m[0][hh];
#pragma unroll
        for (int v = 1; v < kWaves; ++v) M = fmaxf(M, sm_m[v][hh]);
        float Ls = 0.f, o = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            const float sc = fast_exp2(sm_m[v][hh] - M);
            Ls = fmaf(sm_l[v][hh], sc, Ls);
            o = fmaf(sm_acc[v][hh][d], sc, o);
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
            ((uint16_t *)a.out)[((size_t)b * a.Hq + h) * D + d] = f32_to_bf16(res);
            if (a.lse && d == 0)
                a.lse[(size_t)b * a.Hq + h] = Lt > 0.f ? Mt * kLn2 + logf(Lt) : -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// Balanced stream: equal contiguous tile ranges per wave.
// ---------------------------------------------------------------------------

// Pieces of the fused merge travel between waves on different XCDs, whose
// L2 caches are not coherent with each other.  They are written and read with
// device-coherent accesses (the sc1 cache policy of the buffer loads and
// stores, the form agent-scope atomic loads and stores take), so no L2
// writeback or invalidation is needed; a wait for the stores to complete
// orders them before the arrival count, and the last arriver reads them only
// after its count returned.  `base` is wave-uniform.
constexpr int kSc1 = 16;   // cache-policy operand bit of sc1 on gfx950
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const float *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, bytes,
                                             kBufferWord3);
}

// Global -> LDS copy of one 4-byte word per lane, lane L's word landing at
// LDS address dst + 4 L (dst wave-uniform), written as an instruction so that
// the compiler does not track it.  The stream's block-id batches travel this
// way: a batch kept in a VGPR whose load is still in flight made the compiler
// wait for every outstanding load (vmcnt 0, the whole K/V ring) on the path
// that joins the batch switch, which every tile takes.  The copy of batch
// n + 1 is issued at the switch to batch n and read 64 tiles later; vector
// memory operations complete in issue order, and the ring's waits on the
// tiles in between have retired it by then.  These kernels use m0 nowhere
// else.
__device__ __forceinline__ void copy4_to_lds(const int32_t *src, uint32_t dst) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :: "v"(src), "s"(dst) : "memory", "m0");
}

__device__ __forceinline__ float readfirstlane_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// bf16 image of a row of E floats.
template <int E>
__device__ __forceinline__ void store_row_bf16(uint16_t *p, const float (&x)[E]) {
    if constexpr (E == 8) {
        const u32x4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                         pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
        *reinterpret_cast<u32x4 *>(p) = w;
    } else if constexpr (E == 4) {
        const u32x2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        *reinterpret_cast<u32x2 *>(p) = w;
    } else if constexpr (E == 2) {
        *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(x[0], x[1]);
    } else {
        p[0] = f32_to_bf16(x[0]);
    }
}

// Log-sum-exp merge by one wave of the nb pieces of (sequence b, heads
// h0..h0+HU-1) in slots s0..s0+nb-1, with the sink, into out / lse.  The
// formula is the one of merge.hip (vLLM attention.py page, the reduction
// step of single_query_cached_kv_attention; FlashInfer sink page for the
// sink term), folded in slot order with a running maximum, so the result
// does not depend on which wave runs it.  COHERENT: the pieces were written
// in this launch, by waves on other XCDs (device-coherent loads); otherwise
// by an earlier launch.
template <int D, int HU, bool COHERENT = true>
__device__ void stream_merge_wave(const StreamArgs &a, int b, int h0, int s0, int nb) {
    constexpr int kPolicy = COHERENT ? kSc1 : 0;
    constexpr int E = HU * D / 64;                // floats of the head rows per lane
    const int lane = threadIdx.x & 63;
    const int hh = lane * E / D, d = lane * E % D;
    const int h = h0 + hh;
    float M = -INFINITY, Z = 0.f, o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = 0.f;
    constexpr int U = 8;                          // pieces whose loads are issued together
    for (int i0 = 0; i0 < nb; i0 += U) {
        float l[U], x[U][E];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t row0 = (size_t)(s0 + min(i0 + u, nb - 1)) * a.Hq + h0;   // uniform
            const __amdgpu_buffer_rsrc_t rl = coherent_rsrc(a.part_lse + row0, HU * 4);
            const __amdgpu_buffer_rsrc_t ro = coherent_rsrc(a.part_out + row0 * D, HU * D * 4);
            l[u] = __builtin_bit_cast(float,
                                      __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * hh, 0, kPolicy));
            const int off = 4 * (hh * D + d);
            // (whole-vector bit casts: a bit cast of one vector element
            // reads element 0 with this compiler)
            if constexpr (E >= 4) {
#pragma unroll
                for (int c = 0; c < E / 4; ++c) {
                    const f32x4 v = __builtin_bit_cast(
                        f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, off + 16 * c, 0, kPolicy));
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[u][4 * c + e] = v[e];
                }
            } else if constexpr (E == 2) {
                const f32x2 v =
                    __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(ro, off, 0, kPolicy));
                x[u][0] = v[0];
                x[u][1] = v[1];
            } else {
                x[u][0] = __builtin_bit_cast(float,
                                             __builtin_amdgcn_raw_buffer_load_b32(ro, off, 0, kPolicy));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float l2 = __fmul_rn(l[u], kLog2e);
            if (i0 + u >= nb || l2 == -INFINITY) continue;
            if (l2 > M) {
                const float sc = fast_exp2(M - l2);
                Z = fmaf(Z, sc, 1.f);
#pragma unroll
                for (int e = 0; e < E; ++e) o[e] = fmaf(o[e], sc, x[u][e]);
                M = l2;
            } else {
                const float wt = fast_exp2(l2 - M);
                Z += wt;
#pragma unroll
                for (int e = 0; e < E; ++e) o[e] = fmaf(wt, x[u][e], o[e]);
            }
        }
    }
    const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;
    const float Mt = fmaxf(M, sig);
    float lse_v = -INFINITY;
    if (Mt != -INFINITY) {
        const float sc = fast_exp2(M - Mt);
        const float Zt = fmaf(Z, sc, fast_exp2(sig - Mt));
        const float f = sc / Zt;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] *= f;
        lse_v = (Mt + fast_log2(Zt)) * kLn2;
    }
    store_row_bf16<E>((uint16_t *)a.out + ((size_t)b * a.Hq + h) * D + d, o);
    if (a.lse && d == 0) a.lse[(size_t)b * a.Hq + h] = lse_v;
}

template <int D, int HU, int MODE, bool ALIBI, bool BS8>
__global__ __launch_bounds__(64 * kStreamWaves) void decode_stream_kernel(StreamArgs a)
{
    constexpr bool FUSED = MODE == kStreamFused;
    constexpr bool APPEND = MODE == kStreamAppend;
    constexpr bool PARTS = MODE == kStreamParts;
    constexpr int NT = 64 * kStreamWaves;
    __shared__ int s_cum[kStreamMaxB + 1];   // tiles of the sequences before b
    __shared__ int s_len[kStreamMaxB];       // cache_seqlens
    __shared__ int s_part[NT];
    // partitions mode: each wave stages up to kStage partition results and
    // writes them in one burst (rows of consecutive partitions of a head are
    // contiguous), so the few writes do not trickle through the read stream
    constexpr int kStage = 8;
    __shared__ __attribute__((aligned(16))) float s_stage[PARTS ? kStreamWaves : 1]
                                                         [PARTS ? kStage * HU * D : 1];
    __shared__ float s_stage_lse[PARTS ? kStreamWaves : 1][PARTS ? kStage * HU : 1];
    __shared__ __attribute__((aligned(16))) char s_vt[kStreamWaves][vt_bytes<D>()];
    // block-id batches 1, 2, ... of each wave, alternating between two slots
    // (BS8: two more for the second block of each tile)
    __shared__ int32_t s_blk[kStreamWaves][BS8 ? 4 : 2][64];

    const int tid = threadIdx.x;
    const int wave = readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int NHG = a.Hq / HU;
    // (head group, range) of this wave: head group fastest, so the waves of a
    // workgroup stream the columns of the same token rows at the same time
    // (one compute unit reads whole token rows, whatever speed each column's
    // addresses get from the memory system)
    const int gwid = readfirstlane((int)blockIdx.x * kStreamWaves + wave);
    const int hg = gwid % NHG;
    const int k = gwid / NHG;                     // this wave's range
    const int h0 = hg * HU;
    const int g = h0 / a.G;

    // the sink logits of this wave's heads (log2 units), read once here: a
    // load at a sequence's end inside the stream waited for the whole ring
    float sig_h[HU];
#pragma unroll
    for (int hh = 0; hh < HU; ++hh)
        sig_h[hh] = FUSED && a.sink ? readfirstlane_f(a.sink[h0 + hh] * kLog2e) : -INFINITY;
    stream_prefix_tiles<NT>(a.seqlens, APPEND ? 1 : 0, a.B, a.window_left, s_cum, s_part, s_len);
    const int T = s_cum[a.B];
    const int chunk = stream_chunk(T, a.K);
    if (k >= a.K) return;                         // a padding wave of the last workgroup
    // the sequence that holds flattened tile x < T: s_cum[b] <= x < s_cum[b+1]
    auto seq_of = [&](int x) {
        int lo = 0, hi = a.B;                     // s_cum[lo] <= x < s_cum[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_cum[mid] <= x) lo = mid; else hi = mid;
        }
        return lo;
    };
    const int P = a.part_size;                    // partitions mode: tokens per partition
    if (PARTS) {
        // Partitions with no tile in the list (left of the window, past the
        // sequence, or of an empty sequence): output 0 and lse -inf, written
        // by the range-0 wave of each head group.
        if (k == 0) {
            for (int b = lane; b < a.B; b += 64) {
                const int L = s_len[b];
                // partitions [pf, pl] of b have tiles; the others are empty
                const int pf = L > 0 ? stream_lo(L, a.window_left) / P : a.max_parts;
                const int pl = L > 0 ? (L - 1) / P : a.max_parts - 1;
                for (int pp = 0; pp < a.max_parts; ++pp) {
                    if (pp == pf) pp = pl + 1;
                    if (pp >= a.max_parts) break;
                    for (int hh = 0; hh < HU; ++hh) {
                        const size_t row = ((size_t)b * a.Hq + h0 + hh) * a.max_parts + pp;
                        for (int d = 0; d < D; d += 4)
                            *reinterpret_cast<f32x4 *>(a.part_out + row * D + d) =
                                f32x4{0.f, 0.f, 0.f, 0.f};
                        a.part_lse[row] = -INFINITY;
                    }
                }
            }
        }
    } else if (FUSED) {
        // sequences without tiles: zero output, lse = sink (or -inf); the
        // range-0 wave of each head group writes them
        if (k == 0) {
            for (int idx = lane; idx < a.B * HU; idx += 64) {
                const int b = idx / HU, h = h0 + idx % HU;
                if (s_cum[b + 1] != s_cum[b]) continue;
                uint16_t *po = (uint16_t *)a.out + ((size_t)b * a.Hq + h) * D;
                for (int d = 0; d < D; d += 8)
                    *reinterpret_cast<u32x4 *>(po + d) = u32x4{0u, 0u, 0u, 0u};
                if (a.lse) a.lse[(size_t)b * a.Hq + h] = a.sink ? a.sink[h] : -INFINITY;
            }
        }
    } else if (gwid == 0) {
        for (int b = lane; b <= a.B; b += 64) a.cum_out[b] = s_cum[b];
        if (lane == 0) a.cum_out[a.B + 1] = chunk;
    }

    const int gw = k;                             // slot base of this range
    int x0 = min(T, gw * chunk);
    int n = min(T, x0 + chunk) - x0;              // tiles of this wave
    if (PARTS) {
        // whole partitions per wave: both ends of the range move up to the
        // next partition start (a sequence start, or a token multiple of P)
        auto snap = [&](int x) {
            if (x >= T) return T;
            const int b = seq_of(x);
            if (x == s_cum[b]) return x;
            const int lo_al = stream_lo(s_len[b], a.window_left) & ~15;
            const int t = lo_al + 16 * (x - s_cum[b]);
            if (t % P == 0) return x;
            return min(s_cum[b] + ((t / P + 1) * P - lo_al) / 16, s_cum[b + 1]);
        };
        const int x1 = snap(min(T, (gw + 1) * chunk));
        x0 = snap(x0);
        n = x1 - x0;
    }
    if (n <= 0) return;

    DecodeWave<D, HU, ALIBI, BS8> w;
    w.setup(g, a.Hkv, a.scale_log2, a.alibi, h0, s_vt[wave]);
    const int bs_mask = (1 << a.bs_log2) - 1;

    // the sequence that holds flattened tile x0
    int b_ld = readfirstlane(seq_of(x0));
    int L_ld = readfirstlane(s_len[b_ld]);
    int t_ld = readfirstlane((stream_lo(L_ld, a.window_left) & ~15) + 16 * (x0 - s_cum[b_ld]));
    int x_ld = x0;                                // flattened index of the cursor's tile
    // partitions mode: the cursor tile's partition and the token where the
    // next one starts, kept up to date without a division per tile
    int p_ld = PARTS ? t_ld / P : 0;
    int pb_ld = PARTS ? (p_ld + 1) * P : 0;
    // advance the load cursor by one tile, skipping sequences with no tiles
    auto advance = [&]() {
        t_ld += 16;
        ++x_ld;
        if (t_ld >= L_ld) {
            do { ++b_ld; } while (b_ld < a.B && s_cum[b_ld + 1] == s_cum[b_ld]);
            b_ld = readfirstlane(b_ld);
            if (b_ld < a.B) {
                L_ld = readfirstlane(s_len[b_ld]);
                t_ld = stream_lo(L_ld, a.window_left) & ~15;
                if (PARTS) {
                    p_ld = readfirstlane(t_ld / P);
                    pb_ld = (p_ld + 1) * P;
                }
            }
        } else if (PARTS && t_ld >= pb_ld) {
            ++p_ld;
            pb_ld += P;
        }
    };
    // Block ids of this wave's tiles, 64 at a time: lane i of a batch holds
    // the block of tile xb + i.  A tile's block id is then a lane read, not a
    // dependent memory load per tile queued behind the K/V stream (that
    // dependency, not bandwidth, limited short-context decode).  The first
    // batch is read into a VGPR before any tile load; each later one is
    // copied to LDS 64 tiles ahead (copy4_to_lds) and read from there.
    const int x_end = x0 + n;
    // Address of the block-table entry of tile xs + lane (second: BS8, the
    // block of the tile's rows 8..15, which is its first block when they lie
    // past the sequence); lanes past the range get entry 0, which exists
    // (the kernel runs only with B >= 1 and max_blocks_per_seq >= 1) and
    // whose value is never used.
    auto gather_ptr = [&](int xs, bool second = false) {
        const int x = xs + lane;
        const int32_t *p = a.block_table;
        if (x < x_end) {
            int lo = 0, hi = a.B;                 // s_cum[lo] <= x < s_cum[hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_cum[mid] <= x) lo = mid; else hi = mid;
            }
            const int t = (stream_lo(s_len[lo], a.window_left) & ~15) + 16 * (x - s_cum[lo]);
            p += (size_t)lo * a.mbps + (second ? (min(t + 8, s_len[lo] - 1) >> 3) : (t >> a.bs_log2));
        }
        return p;
    };
    auto copy_batch = [&](int xs, int slot) {
        copy4_to_lds(gather_ptr(xs),
                     (uint32_t)(uintptr_t)(const lds_void_t *)&s_blk[wave][slot][0]);
        if constexpr (BS8)
            copy4_to_lds(gather_ptr(xs, true),
                         (uint32_t)(uintptr_t)(const lds_void_t *)&s_blk[wave][2 + slot][0]);
    };
    // Append with rotary embedding: this wave's q rows (its head group, every
    // sequence its range meets) rotated by the new token's position into
    // q_rot, read back below in place of q.  Waves that share a sequence
    // write the same bytes; each reads only rows it has written itself.
    const void *qsrc = a.q;
    if constexpr (APPEND) {
        if (a.rope) {
            constexpr int LPR = D / 8;            // 16-byte chunks per head row
            const int b_last = seq_of(x_end - 1);
            const int total = (b_last - b_ld + 1) * HU * LPR;
            for (int base = 0; base < total; base += 64) {
                const int e = base + lane;
                if (e < total) {
                    const int b = b_ld + e / (HU * LPR);
                    const int hh = (e / LPR) % HU;
                    const size_t row = ((size_t)b * a.Hq + h0 + hh) * D * 2;
                    rope_chunk<true>((const char *)a.q + row, (char *)a.q_rot + row,
                                     a.rope + (size_t)(s_len[b] - 1) * a.rope_dim, a.rope_dim,
                                     a.rope_neox != 0, e % LPR);
                }
            }
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            qsrc = a.q_rot;
        }
    }
    int xb = x0, nbat = 0, blk_batch = *gather_ptr(x0);
    [[maybe_unused]] int blk_batch1 = 0;
    if constexpr (BS8) blk_batch1 = *gather_ptr(x0, true);
    if (x0 + 64 < x_end) copy_batch(x0 + 64, 1);

    // Q of the first two sequences of the range, loaded before the first
    // tiles and waited for on their own after the tiles are issued, so that
    // neither the first tile nor the change to the second sequence waits for
    // the K/V loads in flight.  A later sequence (ranges over short
    // sequences) loads its Q at the change and waits for it there.
    using DW = DecodeWave<D, HU>;
    bf16x8 q_next[DW::KSTEPS];
    int q_held = b_ld, q_nb = -1;
    if (s_cum[b_ld + 1] < x_end) {
        int lo = b_ld + 1, hi = a.B;              // s_cum[lo] <= s_cum[b_ld+1] < s_cum[hi]
        const int xs = s_cum[b_ld + 1];
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_cum[mid] <= xs) lo = mid; else hi = mid;
        }
        q_nb = readfirstlane(lo);
    }
    w.load_q(qsrc, (size_t)q_held * a.Hq + h0);
    if (q_nb >= 0) w.load_q_to(q_next, qsrc, (size_t)q_nb * a.Hq + h0);
    __builtin_amdgcn_sched_barrier(0);
    int blk1_at = 0;                              // BS8: block_at's second block
    auto block_at = [&]() {
        if (x_ld - xb >= 64) {                    // next batch (copied 64 tiles ago)
            xb += 64;
            const int sl = ++nbat & 1;
            blk_batch = s_blk[wave][sl][lane];
            if constexpr (BS8) blk_batch1 = s_blk[wave][2 + sl][lane];
            // the reads complete here, in the rare branch; then the other
            // slot (read at the previous switch) takes the batch after
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
            if (xb + 64 < x_end) copy_batch(xb + 64, sl ^ 1);
        }
        if constexpr (BS8) blk1_at = __builtin_amdgcn_readlane(blk_batch1, x_ld - xb);
        return __builtin_amdgcn_readlane(blk_batch, x_ld - xb);
    };
    auto row_off = [&](int blk, int t) {
        return (((size_t)blk << a.bs_log2) + (t & bs_mask)) * (size_t)w.tok_bytes;
    };
    auto row_off1 = [&](int blk1) { return ((size_t)blk1 << 3) * (size_t)w.tok_bytes; };

    // Pieces of sequence b: the waves whose ranges meet its tiles; their
    // slots are consecutive from first_slot(b).
    auto pieces = [&](int b) { return (s_cum[b + 1] - 1) / chunk - s_cum[b] / chunk + 1; };
    auto first_slot = [&](int b) { return s_cum[b] / chunk + b; };

    int seg_b = -1, seg_p = 0, seg_lo = 0, seg_hi = 0;
    // partitions mode: results staged in s_stage[wave], lane i of staged_row
    // holding b * max_parts + p of slot i
    int n_staged = 0, staged_row = 0;
    auto write_staged = [&]() {
        if (!PARTS || n_staged == 0) return;
        // the stage was written by other lanes of this wave: make those LDS
        // writes complete and visible before reading them back
        __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        constexpr int C4 = D / 4;                 // 16-byte chunks per row
        // rows (slot i, head hh) in order hh-major: consecutive partitions of
        // one head sit next to each other in part_out.  Every lane runs every
        // iteration (the shuffles read lanes 0 .. n_staged-1); only the
        // stores are guarded.
        const int total = HU * n_staged * C4;
        for (int base = 0; base < total; base += 64) {
            const int e = min(base + lane, total - 1);
            const int c = e % C4, i = (e / C4) % n_staged, hh = e / (C4 * n_staged);
            const int bp = __shfl(staged_row, i, 64);
            if (base + lane < total) {
                const int b = bp / a.max_parts, pp = bp % a.max_parts;
                const size_t row = ((size_t)b * a.Hq + h0 + hh) * a.max_parts + pp;
                // nontemporal: the rows are read once, by the merge kernel,
                // and need not displace anything on their way out
                __builtin_nontemporal_store(
                    *reinterpret_cast<const f32x4 *>(s_stage[wave] + (i * HU + hh) * D + 4 * c),
                    reinterpret_cast<f32x4 *>(a.part_out + row * D + 4 * c));
            }
        }
        {
            const int li = min(lane, HU * n_staged - 1);
            const int bp = __shfl(staged_row, li / HU, 64);
            if (lane < HU * n_staged) {
                const int b = bp / a.max_parts, pp = bp % a.max_parts;
                a.part_lse[((size_t)b * a.Hq + h0 + li % HU) * a.max_parts + pp] =
                    s_stage_lse[wave][li];
            }
        }
        // the next stage writes must not overtake these reads
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        n_staged = 0;
    };
    // sequences whose pieces this wave wrote but has not counted yet: only the
    // first and the last sequence of a range can be shared with other waves
    int shared_a = -1, shared_b = -1;
    auto flush = [&]() {
        const float lsum = w.reduce();
        if (PARTS) {
            // partition (seg_b, seg_p) is this wave's alone: its normalised
            // output and lse (sink left out), staged for the next burst
            float *st = s_stage[wave] + n_staged * HU * D;
#pragma unroll
            for (int hh = 0; hh < HU; ++hh) {
                const float lh = __shfl(lsum, hh, 64);
                const float inv = lh > 0.f ? 1.f / lh : 0.f;
                if (w.holds_acc()) {
                    float *ps = st + hh * D + w.d0();
                    *reinterpret_cast<f32x4 *>(ps) = f32x4{w.acc[hh][0] * inv, w.acc[hh][1] * inv,
                                                           w.acc[hh][2] * inv, w.acc[hh][3] * inv};
                    *reinterpret_cast<f32x4 *>(ps + 4) = f32x4{w.acc[hh][4] * inv,
                                                               w.acc[hh][5] * inv,
                                                               w.acc[hh][6] * inv,
                                                               w.acc[hh][7] * inv};
                }
            }
            if (w.j == 0 && w.r < HU)
                s_stage_lse[wave][n_staged * HU + w.r] =
                    lsum > 0.f ? w.m_lane * kLn2 + logf(lsum) : -INFINITY;
            // (b, p) of the staged slot, kept in lane n_staged of a VGPR
            if (lane == n_staged) staged_row = seg_b * a.max_parts + seg_p;
            if (++n_staged == kStage) write_staged();
            return;
        }
        if (FUSED && pieces(seg_b) == 1) {
            // the whole sequence was this wave's: final result with the sink
#pragma unroll
            for (int hh = 0; hh < HU; ++hh) {
                const int h = h0 + hh;
                const float lh = __shfl(lsum, hh, 64);
                const float mh = __shfl(w.m_lane, hh, 64);
                const float sig = sig_h[hh];
                const float Mt = fmaxf(lh > 0.f ? mh : kNoMax, sig);
                const float sc = fast_exp2(mh - Mt);
                const float Lt = fmaf(lh, sc, fast_exp2(sig - Mt));
                const float f = Lt > 0.f ? sc / Lt : 0.f;
                if (w.holds_acc()) {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = w.acc[hh][e] * f;
                    store_row_bf16<8>((uint16_t *)a.out + ((size_t)seg_b * a.Hq + h) * D + w.d0(),
                                      x);
                }
                if (a.lse && lane == hh)
                    a.lse[(size_t)seg_b * a.Hq + h] =
                        Lt > 0.f ? (Mt + fast_log2(Lt)) * kLn2 : -INFINITY;
            }
            return;
        }
        const size_t slot = (size_t)gw + seg_b;   // unique per (wave, sequence)
        float *po = a.part_out + (slot * a.Hq + h0) * D;
        const __amdgpu_buffer_rsrc_t rpo = coherent_rsrc(po, HU * D * 4);
#pragma unroll
        for (int hh = 0; hh < HU; ++hh) {
            const float lh = __shfl(lsum, hh, 64);
            const float inv = lh > 0.f ? 1.f / lh : 0.f;
            if (w.holds_acc()) {
                const f32x4 v0 = {w.acc[hh][0] * inv, w.acc[hh][1] * inv, w.acc[hh][2] * inv,
                                  w.acc[hh][3] * inv};
                const f32x4 v1 = {w.acc[hh][4] * inv, w.acc[hh][5] * inv, w.acc[hh][6] * inv,
                                  w.acc[hh][7] * inv};
                if (FUSED) {
                    const int off = 4 * (hh * D + w.d0());
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v0), rpo, off,
                                                           0, kSc1);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v1), rpo,
                                                           off + 16, 0, kSc1);
                } else {
                    *reinterpret_cast<f32x4 *>(po + hh * D + w.d0()) = v0;
                    *reinterpret_cast<f32x4 *>(po + hh * D + w.d0() + 4) = v1;
                }
            }
        }
        if (w.j == 0 && w.r < HU) {
            const float lse_p = lsum > 0.f ? w.m_lane * kLn2 + logf(lsum) : -INFINITY;
            if (FUSED)
                __builtin_amdgcn_raw_buffer_store_b32(
                    __builtin_bit_cast(uint32_t, lse_p),
                    coherent_rsrc(a.part_lse + slot * a.Hq + h0, HU * 4), 4 * w.r, 0, kSc1);
            else
                a.part_lse[slot * a.Hq + h0 + w.r] = lse_p;
        }
        if (FUSED) {
            if (shared_a < 0) shared_a = seg_b; else shared_b = seg_b;
        }
    };

    if constexpr (APPEND) {
        // Each sequence's new token is key L = s_len[b] - 1, in its last
        // tile.  The wave that loads that tile is the only reader of the
        // position in this head group, so it copies the row from k_new /
        // v_new into the cache slot itself and waits for its stores before
        // its first tile load.  (Head groups that share a kv head each copy
        // the same bytes.)  Sequences b_ld .. b_end-1 end inside the range.
        // With a rotary table the key row is rotated by position L as it is
        // copied.
        int b_end = b_ld;
        while (b_end < a.B && s_cum[b_end + 1] <= x_end) ++b_end;
        constexpr int LPR = D / 8;                // lanes per row, 16 bytes each
        constexpr int SPP = 64 / (2 * LPR);       // sequences per pass (K and V rows)
        for (int bb = b_ld; bb < b_end; bb += SPP) {
            const int b = bb + lane / (2 * LPR);
            const int part = lane % (2 * LPR);
            if (b < b_end) {
                const int L = s_len[b] - 1;
                const int blk = a.block_table[(size_t)b * a.mbps + (L >> a.bs_log2)];
                const bool is_v = part >= LPR;
                const int u = part % LPR;
                const char *src = (const char *)(is_v ? a.v_new : a.k_new) +
                                  ((size_t)b * a.Hkv + g) * D * 2;
                char *dst = (char *)(is_v ? a.v_cache : a.k_cache) + row_off(blk, L) +
                            (size_t)g * D * 2;
                if (!is_v && a.rope)
                    rope_chunk<true>(src, dst, a.rope + (size_t)L * a.rope_dim, a.rope_dim,
                                     a.rope_neox != 0, u);
                else
                    *reinterpret_cast<u32x4 *>(dst + 16 * u) =
                        *reinterpret_cast<const u32x4 *>(src + 16 * u);
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    u32x4 kbuf[kRing][DecodeWave<D, HU>::KSTEPS], vbuf[kRing][DecodeWave<D, HU>::VLD];
    int rb[kRing], rt[kRing];                     // (sequence, first token) of each ring slot
    int rp[kRing];                                // partitions mode: partition of each slot
    const int n_pad = (n + kRing - 1) / kRing * kRing;
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
        const bool live = k < n;
        rb[k] = b_ld;
        rt[k] = t_ld;
        if (PARTS) rp[k] = p_ld;
        const size_t off0 = live ? row_off(block_at(), t_ld) : 0;
        w.load(a.k_cache, a.v_cache, off0, live ? row_off1(blk1_at) : 0, live, kbuf[k], vbuf[k]);
        if (k + 1 < n) advance();
        __builtin_amdgcn_sched_barrier(0);
    }
    // every tile issues KSTEPS + VLD loads: this waits for the Q loads only
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(kDepth * (DW::KSTEPS + DW::VLD)));
    int blk_next = kDepth < n ? block_at() : 0;
    int blk_next1 = blk1_at;
    for (int it = 0; it < n_pad; it += kRing) {
#pragma unroll
        for (int k = 0; k < kRing; ++k) {
            const int cur = it + k;
            const int nxt = cur + kDepth;
            const int slot = (k + kDepth) % kRing;
            const bool live_n = nxt < n;
            rb[slot] = b_ld;
            rt[slot] = t_ld;
            if (PARTS) rp[slot] = p_ld;
            w.load(a.k_cache, a.v_cache, live_n ? row_off(blk_next, t_ld) : 0,
                   live_n ? row_off1(blk_next1) : 0, live_n, kbuf[slot], vbuf[slot]);
            if (nxt + 1 < n) {
                advance();
                blk_next = block_at();
                blk_next1 = blk1_at;
            }
            __builtin_amdgcn_sched_barrier(0);
            if (cur < n) {
                const int pk = PARTS ? rp[k] : 0;
                if (rb[k] != seg_b || (PARTS && pk != seg_p)) {   // a new sequence (or partition)
                    if (seg_b >= 0) flush();
                    seg_b = rb[k];
                    seg_p = pk;
                    const int L = s_len[seg_b];
                    seg_lo = stream_lo(L, a.window_left);
                    seg_hi = L;
                    if (PARTS) {
                        seg_lo = max(seg_lo, pk * P);
                        seg_hi = min(L, (pk + 1) * P);
                    }
                    w.qpos = L - 1;
                    if (seg_b != q_held) {
                        if (seg_b == q_nb) {
#pragma unroll
                            for (int c = 0; c < DW::KSTEPS; ++c) w.qf[c] = q_next[c];
                        } else {
                            w.load_q(qsrc, (size_t)seg_b * a.Hq + h0);
                            // Wait for Q here, inside the rare branch: otherwise the
                            // wait lands after the join and drains the ring every trip.
                            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                        }
                        q_held = seg_b;
                    }
                    w.reset();
                }
                w.process(rt[k], seg_lo, seg_hi, true, kbuf[k], vbuf[k]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (seg_b >= 0) flush();
    write_staged();
    if (FUSED && shared_a >= 0) {
        // Count this wave's shared pieces once its stream is over (the
        // pieces are complete first), so the stream itself never waits on a
        // count.  The wave that brings a count to pieces(b) merges b and
        // leaves its counter zero for the next call.
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        // A counter holds (epoch << 32) | count, and zero at rest.  The first
        // arrival of a call claims the counter with one compare-and-swap
        // (whatever epoch it held: a counter left by an interrupted call, or
        // never used, restarts from zero); every later arrival, seeing this
        // call's epoch, adds one.  A counter that holds this call's epoch
        // keeps it until its last arrival, so the add never lands on a stale
        // count, and no wave retries more than once (a compare-and-swap loop
        // per arrival serialised the many waves that end together on one
        // sequence when a batch is small).
        auto arrive = [&](int b) {
            int arrived = 0;
            if (lane == 0) {
                uint64_t *ctr = a.counters + (size_t)b * NHG + hg;
                const uint64_t mine = (uint64_t)a.epoch << 32;
                uint64_t v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((v >> 32) != a.epoch &&
                    __hip_atomic_compare_exchange_strong(ctr, &v, mine | 1u, __ATOMIC_RELAXED,
                                                         __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT)) {
                    arrived = 1;
                } else {
                    // v holds this call's epoch: read so, or left by the
                    // compare-and-swap that another arrival won
                    v = __hip_atomic_fetch_add(ctr, (uint64_t)1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                    arrived = (int)(uint32_t)v + 1;
                }
            }
            return __builtin_amdgcn_readlane(arrived, 0) == pieces(b);
        };
        const bool last_a = arrive(shared_a);
        const bool last_b = shared_b >= 0 && arrive(shared_b);
        if (last_a) {
            stream_merge_wave<D, HU>(a, shared_a, h0, first_slot(shared_a), pieces(shared_a));
            if (lane == 0)
                __hip_atomic_store(a.counters + (size_t)shared_a * NHG + hg, (uint64_t)0,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (last_b) {
            stream_merge_wave<D, HU>(a, shared_b, h0, first_slot(shared_b), pieces(shared_b));
            if (lane == 0)
                __hip_atomic_store(a.counters + (size_t)shared_b * NHG + hg, (uint64_t)0,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Second launch of the two-launch balanced decode: one wave per (sequence,
// HU heads) merges that sequence's pieces, which the stage launch wrote to
// the slots the tile prefix sums it left in cum_out ([B + 2]: the sums, then
// the per-wave chunk) place them in.
template <int D, int HU>
__global__ __launch_bounds__(256) void stream_merge_kernel(StreamArgs a)
{
    const int w = readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
    const int NHG = a.Hq / HU;
    if (w >= a.B * NHG) return;
    const int b = w / NHG, h0 = (w % NHG) * HU;
    const int c0 = a.cum_out[b], c1 = a.cum_out[b + 1], chunk = a.cum_out[a.B + 1];
    const int nb = c1 > c0 ? (c1 - 1) / chunk - c0 / chunk + 1 : 0;
    stream_merge_wave<D, HU, false>(a, b, h0, c0 / chunk + b, nb);
}

template <int D, int HU, bool BS8>
void launch_part(const DecodeArgs &a, int grid, hipStream_t stream) {
    if (a.alibi)
        hipLaunchKernelGGL((decode_part_kernel<D, HU, true, BS8>), dim3(grid), dim3(256), 0, stream,
                           a);
    else
        hipLaunchKernelGGL((decode_part_kernel<D, HU, false, BS8>), dim3(grid), dim3(256), 0,
                           stream, a);
}
// ALiBi is a separate instantiation, so that calls without slopes run the
// plain product for the scaled logit.
template <int D, int HU, bool ALIBI, bool BS8>
void launch_stream_al(const StreamArgs &a, int grid, hipStream_t stream) {
    const dim3 g(grid), b(64 * kStreamWaves);
    switch (a.mode) {
        case kStreamAppend:
            hipLaunchKernelGGL((decode_stream_kernel<D, HU, kStreamAppend, ALIBI, BS8>), g, b, 0, stream, a);
            break;
        case kStreamFused:
            hipLaunchKernelGGL((decode_stream_kernel<D, HU, kStreamFused, ALIBI, BS8>), g, b, 0, stream, a);
            break;
        case kStreamParts:
            hipLaunchKernelGGL((decode_stream_kernel<D, HU, kStreamParts, ALIBI, BS8>), g, b, 0, stream, a);
            break;
        default:
            hipLaunchKernelGGL((decode_stream_kernel<D, HU, kStreamStage, ALIBI, BS8>), g, b, 0, stream, a);
    }
}
template <int D, int HU, bool BS8>
void launch_stream(const StreamArgs &a, int grid, hipStream_t stream) {
    if (a.alibi) launch_stream_al<D, HU, true, BS8>(a, grid, stream);
    else launch_stream_al<D, HU, false, BS8>(a, grid, stream);
}

template <bool BS8>
pkv_status launch_part_all(const DecodeArgs &a, hipStream_t stream)
{
    const int HU = decode_heads_per_unit(a.G);
    const long long grid = (long long)a.B * (a.Hq / HU) * a.nparts;
    if (grid <= 0) return PKV_OK;
    if (grid > 0x7fffffffLL) return PKV_ERR_SHAPE;
    if (a.D == 128) {
        if (HU == 4) launch_part<128, 4, BS8>(a, (int)grid, stream);
        else if (HU == 2) launch_part<128, 2, BS8>(a, (int)grid, stream);
        else launch_part<128, 1, BS8>(a, (int)grid, stream);
    } else {
        if (HU == 4) launch_part<64, 4, BS8>(a, (int)grid, stream);
        else if (HU == 2) launch_part<64, 2, BS8>(a, (int)grid, stream);
        else launch_part<64, 1, BS8>(a, (int)grid, stream);
    }
    return launch_status();
}

template <bool BS8>
pkv_status launch_stream_all(const StreamArgs &a, hipStream_t stream)
{
    const int HU = decode_heads_per_unit(a.G);
    const long long grid = ((long long)a.K * (a.Hq / HU) + kStreamWaves - 1) / kStreamWaves;
    if (a.B == 0 || grid <= 0) return PKV_OK;
    if (a.B > kStreamMaxB || grid > 0x7fffffffLL) return PKV_ERR_SHAPE;
    if (a.D == 128) {
        if (HU == 4) launch_stream<128, 4, BS8>(a, (int)grid, stream);
        else if (HU == 2) launch_stream<128, 2, BS8>(a, (int)grid, stream);
        else launch_stream<128, 1, BS8>(a, (int)grid, stream);
    } else {
        if (HU == 4) launch_stream<64, 4, BS8>(a, (int)grid, stream);
        else if (HU == 2) launch_stream<64, 2, BS8>(a, (int)grid, stream);
        else launch_stream<64, 1, BS8>(a, (int)grid, stream);
    }
    return launch_status();
}

}  // namespace
}  // namespace pkv
