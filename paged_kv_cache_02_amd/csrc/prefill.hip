// Varlen prefill over contiguous or paged K/V, bf16 with fp32 accumulation.
//
// Transformers "Paged attention" doc, varlen path: packed requests indexed by
// cu_seq_lens_q/k, launch sized by max_length_q/k; FlashInfer
// "sink_attention_reference.py" page, varlen branch: request r's query row i
// sits at position p = Lk - Lq + i (queries are the last Lq positions), sees
// keys j <= p with p - window_left <= j when a window is set, GQA h -> h / G,
// and the per-head sink joins the denominator (its non-causal branch: every
// key of the request, a window bounding only the left side, p - window_left
// <= j); vLLM "attention.py" page,
// multi_query_kv_attention: block-diagonal causal attention over packed
// prompts.  Paged mode reads K/V through the request's block_table row, so a
// query chunk can attend to keys already in the cache.
//
// gfx950 design:
//   * workgroup = 4 waves of 32 query rows that share one kv head: the
//     query heads of a GQA group at the same 32 positions when the group
//     has 4 (or a multiple of 4) heads, else 2 heads x 64 positions or 1 head
//     x 128 positions.  Waves that read the same K/V at the same positions
//     see the same causal and window range, so no wave idles at the
//     diagonal while the others finish it.  Tiles are issued longest-first
//     (highest position tile first), and the workgroups of one kv head are
//     placed on the same XCD so that its K/V tiles are fetched into that
//     XCD's L2 once for all of them;
//   * K and V tiles of 64 keys go straight from global memory into LDS with
//     the load-to-LDS forms of buffer_load_dwordx4 / global_load_dwordx4 (no
//     register staging, no VALU work), double buffered: the next tile's loads
//     are issued before the current tile is computed and waited for only at
//     its end; each 16-byte piece is placed with an XOR swizzle chosen so
//     that the operand reads below hit distinct LDS banks;
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 with Q held in registers, so
//     each lane owns one query row: the row max/sum need one cross-lane step;
//     K operands are read with ds_read_b128;
//   * O^T = V^T . P^T on the same MFMA: P goes from the S^T accumulators to
//     bf16 in place, and the V^T operand comes from the row-major V tile via
//     the LDS transpose read ds_read_b64_tr_b16 (within each 16-lane group,
//     lane 4a+b receives element b of the rows addressed by lanes a, a+4,
//     a+8, a+12), so no transpose pass is needed;
//   * online softmax with a reference max raised only when a logit exceeds it
//     by more than 2^8 (one ballot per tile); the logit scale and log2(e) are
//     folded into one FMA per exp2;
//   * masks only on tiles that straddle the causal diagonal, the window edge
//     or the end of the keys; tiles outside a wave's visible range are skipped;
//   * ALiBi (vLLM "attention.py" page, PagedAttentionWithALiBi: slope_h times
//     key position minus query position, added to the scaled logits) is a
//     separate instantiation: each 32-key chunk is first turned into biased
//     log2-unit logits with one more FMA per score.

#include "common.h"
#include "decode.h"
#include "tile.h"

#include <type_traits>

namespace pkv {

namespace {

constexpr float kTau = 8.0f;
// Runs of position blocks keep their key tiles in a ring of 4 LDS slots and
// stage the output rows in passes of 16 (head_dim 64: 73 KB, two workgroups
// per compute unit) or 8 rows per wave (head_dim 128: 137 KB, one workgroup,
// whose registers also hold the next step's Q).
template <int D> constexpr int run_slots() { return 4; }
template <int D> constexpr int run_stage_rows() { return D == 128 ? 8 : 16; }
// LDS operand reads are issued this many MFMAs ahead of their use (K for S,
// V^T for P.V), to cover LDS latency with eight waves per CU reading (2 and 3
// ahead left 15 % of the C3 time on the table; 6 and 7 gain nothing more)
constexpr int KA = 4;
constexpr int VA = 5;

// Rotary embedding of a lane's Q registers (lane half lh holds dims
// 16c + 8lh .. +8 of register c).  tab: the row's table, cos then sin;
// lanes with rot false keep their values.
// neox, rope_dim = 32 OFF: register c < OFF pairs with register c + OFF.
template <int OFF, int QK>
__device__ __forceinline__ void rope_neox(bf16x8 (&qf)[QK], const float *tab, int lh, bool rot) {
    static_assert(2 * OFF <= QK, "rotary dims within the head");
    constexpr int half = 16 * OFF;
#pragma unroll
    for (int c = 0; c < OFF; ++c) {
        const int d0 = 16 * c + 8 * lh;
        bf16x8 x = qf[c], y = qf[c + OFF];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float co = tab[d0 + e], si = tab[half + d0 + e];
            const float x0 = (float)qf[c][e], x1 = (float)qf[c + OFF][e];
            x[e] = rot ? (__bf16)(x0 * co - x1 * si) : qf[c][e];
            y[e] = rot ? (__bf16)(x1 * co + x0 * si) : qf[c + OFF][e];
        }
        qf[c] = x;
        qf[c + OFF] = y;
    }
}
// interleaved pairs (2i, 2i + 1) sit next to each other in a register
template <int QK>
__device__ __forceinline__ void rope_pairs(bf16x8 (&qf)[QK], const float *tab, int lh, int rd,
                                           bool rot) {
    const int half = rd / 2;
#pragma unroll
    for (int c = 0; c < QK; ++c) {
        const int d0 = 16 * c + 8 * lh;
        if (d0 >= rd) continue;
        bf16x8 x = qf[c];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int i = (d0 + e) / 2;
            const float co = tab[i], si = tab[half + i];
            const float x0 = (float)qf[c][e], x1 = (float)qf[c][e + 1];
            x[e] = rot ? (__bf16)(x0 * co - x1 * si) : qf[c][e];
            x[e + 1] = rot ? (__bf16)(x1 * co + x0 * si) : qf[c][e + 1];
        }
        qf[c] = x;
    }
}

template <int D, bool PAGED, bool ALIBI, bool RUN, bool ROPEK = false>
__global__ __launch_bounds__(256, (RUN && D == 128) ? 1 : 2) void prefill_bf16_kernel(PrefillArgs a)
{
    using TL = Tile<D>;
    constexpr int U = TL::U;
    constexpr int QK_STEPS = D / 16;      // k-steps of 16 dims
    constexpr int DT = D / 32;            // 32-dim output tiles
    extern __shared__ __attribute__((aligned(16))) char lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = readfirstlane(tid >> 6);
    const int lr = lane & 31;     // row within the wave / column of the MFMA
    const int lh = lane >> 5;     // lane half

    // ---- which (request, positions, kv head, query heads) ----
    // A workgroup holds hpw query heads of one kv head (hpw = 4, 2 or 1,
    // dividing G) at bm = 128 / hpw positions; wave w takes head w % hpw of
    // them and the 32 rows from 32 (w / hpw).  The grid has Hq workgroups per
    // (request, 128-position tile): G / hpw head subgroups x hpw position
    // blocks for each kv head.  Consecutive workgroups go to the eight XCDs
    // in turn (each with its own L2), and an XCD hands its workgroups to its
    // shader engines in turn.  Position p among the Hq takes kv head p % Hkv,
    // so the workgroups that read the same K/V land on the same XCD (whenever
    // Hkv divides 8 or 8 divides Hkv, and Hq is a multiple of 8), and the
    // position blocks of one tile are consecutive in that XCD's queue, so
    // they spread over its shader engines.  The block order rotates from tile
    // to tile: the partly empty last tiles of the requests would otherwise
    // hand their work to the same engines, and an XCD stalls its queue on
    // the first full engine while the others sit idle.
    const int hpw = a.hpw;
    const int bm = 128 / hpw;                       // positions per workgroup
    const int ng = a.G / hpw;                       // head subgroups per kv head
    int g, hs, r, blk0, nsteps;                     // blk0: first block of bm positions
    if constexpr (RUN) {
        // Runs: workgroup (run u, request, head subgroup, kv head), kv head
        // fastest so that the subgroups of a kv head share an XCD's L2, and
        // the last runs of the requests first (the heaviest, when causal); it
        // walks the run_steps consecutive position blocks of run u, each
        // step's keys overlapping the last one's
        int id = blockIdx.x;
        g = id % a.Hkv;
        id /= a.Hkv;
        hs = id % ng;
        id /= ng;
        r = id % a.B;
        const int u = a.runs - 1 - id / a.B;
        blk0 = u * a.run_steps;
        nsteps = a.run_steps;
    } else {
        const int p = blockIdx.x % a.Hq;
        const int slot = blockIdx.x / a.Hq;
        g = p % a.Hkv;
        hs = (p / a.Hkv) % ng;
        const int blk = (hpw - 1 - (p / a.Hkv) / ng + slot) % hpw;   // position block
        r = slot % a.B;
        const int qt = a.max_q_tiles - 1 - slot / a.B;
        blk0 = qt * hpw + blk;
        nsteps = 1;
    }
    const int h = g * a.G + hs * hpw + wave % hpw;
    const int cq0 = a.cu_q[r], Lq = a.cu_q[r + 1] - cq0;
    if (blk0 * bm >= Lq) return;
    const int ck0 = a.cu_k[r], Lk = a.cu_k[r + 1] - ck0;
    // the sink logit is needed only at the end: fetch it now, off the tail
    const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;
    const float slope_log2 = ALIBI ? a.alibi[h] * kLog2e : 0.f;

    // Rows, positions and key range of the workgroup and of this wave at
    // position block blk0 + s (one step).
    int row0, nrows, pos0, pos_last, kv_lo, kv_hi, t_begin, ntiles;
    int wrow0, wrows, wpos0, wpos1, w_lo, w_hi;
    auto block_keys = [&](int row0_, int &lo_, int &tb_, int &nt_) {
        const int nr = min(bm, Lq - row0_);
        const int p0 = Lk - Lq + row0_;
        lo_ = a.window_left >= 0 ? max(0, p0 - a.window_left) : 0;
        const int hi_ = a.causal ? min(Lk, p0 + nr) : Lk;
        tb_ = lo_ & ~(BN - 1);
        nt_ = hi_ > lo_ ? (hi_ - tb_ + BN - 1) / BN : 0;
    };
    auto set_step = [&](int s) {
        row0 = (blk0 + s) * bm;                     // first row of the workgroup (within request)
        nrows = min(bm, Lq - row0);
        pos0 = Lk - Lq + row0;                      // position of the first row
        pos_last = pos0 + nrows - 1;
        block_keys(row0, kv_lo, t_begin, ntiles);
        kv_hi = a.causal ? min(Lk, pos_last + 1) : Lk;   // exclusive
        // this wave's rows and visible key range
        wrow0 = row0 + 32 * (wave / hpw);
        wrows = max(0, min(32, Lq - wrow0));
        wpos0 = Lk - Lq + wrow0;
        wpos1 = wpos0 + wrows - 1;
        w_lo = a.window_left >= 0 ? max(0, wpos0 - a.window_left) : 0;
        w_hi = a.causal ? min(Lk, wpos1 + 1) : Lk;
    };
    set_step(0);

    const size_t qstride = (size_t)a.Hq * D;     // elements between tokens of q/out
    const size_t kvstride = (size_t)a.Hkv * D;   // elements between tokens of k/v

    // ---- Q^T operand: lane holds row lr, dims 16c + 8lh .. +8 ----
    auto load_q = [&](bf16x8 (&dst)[QK_STEPS], int wrow0_, int wrows_) {
        const bool ok = lr < wrows_;
        const uint16_t *qp = (const uint16_t *)a.q + (size_t)(cq0 + wrow0_ + (ok ? lr : 0)) * qstride +
                             (size_t)h * D + 8 * lh;
#pragma unroll
        for (int c = 0; c < QK_STEPS; ++c) {
            u32x4 x = u32x4{0u, 0u, 0u, 0u};
            if (ok) x = *reinterpret_cast<const u32x4 *>(qp + 16 * c);
            dst[c] = __builtin_bit_cast(bf16x8, x);
        }
    };
    bf16x8 qf[QK_STEPS];
    load_q(qf, wrow0, wrows);

    // Rotary embedding of the Q rows at their positions (rope_dim a multiple
    // of 32): the neox partner of dims 16c + 8lh + e is register
    // c + rope_dim / 32 of this lane; interleaved pairs are adjacent.
    // Register indices stay compile-time constants (a runtime index would
    // move qf to scratch memory).  Rows past the request (zero q) and rows at
    // a negative position (Lq > Lk) read table row 0, so every read stays
    // inside the table, and keep q as it is: a negative position has no table
    // row (causal rows there see no key; non-causal rows see them all).
    // Called once the first K/V tile is in flight, so the table loads overlap
    // that tile's.
    auto rotate_q = [&]() {
        const int tpos = wpos0 + lr;
        const bool rot = lr < wrows && tpos >= 0;
        const float *tab = a.rope + (size_t)(rot ? tpos : 0) * a.rope_dim;
        if (a.rope_neox) {
            switch (a.rope_dim / 32) {
                case 1: rope_neox<1>(qf, tab, lh, rot); break;
                case 2: rope_neox<2>(qf, tab, lh, rot); break;
                case 3: if constexpr (QK_STEPS >= 6) rope_neox<3>(qf, tab, lh, rot); break;
                case 4: if constexpr (QK_STEPS >= 8) rope_neox<4>(qf, tab, lh, rot); break;
                default: break;
            }
        } else {
            rope_pairs(qf, tab, lh, a.rope_dim, rot);
        }
    };

    // ---- ROPEK: contiguous K rotated by key position in LDS ----
    // Once a K tile has landed, each wave rotates 16 of its rows in place
    // (row 16 wave + lane / 4; lane % 4 takes every fourth chunk pair (neox)
    // or chunk (interleaved) of the row) before any wave reads the tile.
    // Rows past the request's keys stay as they are (zeros, masked).  The
    // table rows of a tile are loaded after the tile before it has been
    // computed, in flight with that tile's last copies.
    static_assert(!(ROPEK && (PAGED || ALIBI)),
                  "paged keys are rotated when they are cached; rotary and ALiBi positions "
                  "are alternatives");
    constexpr int KR = ROPEK ? (D == 128 ? 32 : 16) : 1;    // table floats per lane
    [[maybe_unused]] float ktab[KR];
    const int kr_row = 16 * wave + (lane >> 2), kr_part = lane & 3;
    [[maybe_unused]] auto load_ktab = [&](int t0) {
        if constexpr (ROPEK) {
            const int half = a.rope_dim / 2;
            const float *tab = a.rope + (size_t)max(0, min(t0 + kr_row, Lk - 1)) * a.rope_dim;
            if (a.rope_neox) {
#pragma unroll
                for (int k = 0; k < KR / 16; ++k) {          // chunk pair p: dims 8p and half + 8p
                    const int p = kr_part + 4 * k;
                    if (8 * p < half) {
#pragma unroll
                        for (int e = 0; e < 8; e += 4) {
                            *reinterpret_cast<f32x4 *>(ktab + 16 * k + e) =
                                *reinterpret_cast<const f32x4 *>(tab + 8 * p + e);
                            *reinterpret_cast<f32x4 *>(ktab + 16 * k + 8 + e) =
                                *reinterpret_cast<const f32x4 *>(tab + half + 8 * p + e);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int k = 0; k < KR / 8; ++k) {           // chunk c: pairs 4c .. 4c + 3
                    const int c = kr_part + 4 * k;
                    if (8 * c < a.rope_dim) {
                        *reinterpret_cast<f32x4 *>(ktab + 8 * k) =
                            *reinterpret_cast<const f32x4 *>(tab + 4 * c);
                        *reinterpret_cast<f32x4 *>(ktab + 8 * k + 4) =
                            *reinterpret_cast<const f32x4 *>(tab + half + 4 * c);
                    }
                }
            }
        }
    };
    [[maybe_unused]] auto rotate_k = [&](int buf, int t0) {
        if constexpr (ROPEK) {
            if (t0 + kr_row >= Lk) return;
            char *kr = lds + buf * TL::BUF + kr_row * U * 16;
            const int sw = TL::swz_k(kr_row);
            const int half = a.rope_dim / 2;
            auto unpack = [](u32x4 w, float (&x)[8]) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[2 * j] = bf16_lo(w[j]);
                    x[2 * j + 1] = bf16_hi(w[j]);
                }
            };
            if (a.rope_neox) {
#pragma unroll
                for (int k = 0; k < KR / 16; ++k) {
                    const int p = kr_part + 4 * k;
                    if (8 * p < half) {
                        u32x4 *pu = reinterpret_cast<u32x4 *>(kr + ((p ^ sw) * 16));
                        u32x4 *pv = reinterpret_cast<u32x4 *>(kr + (((p + half / 8) ^ sw) * 16));
                        float x[8], y[8];
                        unpack(*pu, x);
                        unpack(*pv, y);
                        u32x4 wx, wy;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float c0 = ktab[16 * k + 2 * j], c1 = ktab[16 * k + 2 * j + 1];
                            const float s0 = ktab[16 * k + 8 + 2 * j], s1 = ktab[16 * k + 9 + 2 * j];
                            wx[j] = pack_bf16x2(x[2 * j] * c0 - y[2 * j] * s0,
                                                x[2 * j + 1] * c1 - y[2 * j + 1] * s1);
                            wy[j] = pack_bf16x2(y[2 * j] * c0 + x[2 * j] * s0,
                                                y[2 * j + 1] * c1 + x[2 * j + 1] * s1);
                        }
                        *pu = wx;
                        *pv = wy;
                    }
                }
            } else {
#pragma unroll
                for (int k = 0; k < KR / 8; ++k) {
                    const int c = kr_part + 4 * k;
                    if (8 * c < a.rope_dim) {
                        u32x4 *pc = reinterpret_cast<u32x4 *>(kr + ((c ^ sw) * 16));
                        float x[8];
                        unpack(*pc, x);
                        u32x4 w;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float co = ktab[8 * k + j], si = ktab[8 * k + 4 + j];
                            w[j] = pack_bf16x2(x[2 * j] * co - x[2 * j + 1] * si,
                                               x[2 * j + 1] * co + x[2 * j] * si);
                        }
                        *pc = w;
                    }
                }
            }
        }
    };

    f32x16 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
    float m = kNoMax, l = 0.f;

    // ---- direct loads.  Instruction i = wave + 4n (n < LOADS) of a tile fills
    // LDS bytes [1024i, 1024i + 1024): lane L writes unit 64i + L, i.e. row
    // RPI*i + L/U at swizzled position (L % U) ^ swz(row).  A wave's
    // instructions are 4 RPI rows apart and both swizzles repeat with a period
    // that divides 4 RPI, so a lane's swizzle is the same in every one of its
    // instructions: one K and one V lane offset.
    constexpr int RPI = 64 / U;                     // key rows per load instruction
    const uint32_t rowbytes = (uint32_t)kvstride * 2;
    const int lrow = lane / U;                      // row of this lane within an instruction
    const int lrow_w = RPI * wave + lrow;           // its row in the wave's first instruction
    const uint32_t off_k = lrow * rowbytes + 16 * ((lane % U) ^ TL::swz_k(lrow_w));
    const uint32_t off_v = lrow * rowbytes + 16 * ((lane % U) ^ TL::swz_v(lrow_w));
    constexpr uint32_t kStepRows = 4 * RPI;         // rows between a wave's instructions

    // Contiguous K/V: one buffer descriptor per tile whose range ends at the
    // request's last key, so rows past it read as zeros (finite, and masked)
    // and no load leaves the request; the row offset inside the tile goes in
    // the range-checked vector offset.
    const char *kreq = (const char *)a.k + ((size_t)ck0 * kvstride + (size_t)g * D) * 2;
    const char *vreq = (const char *)a.v + ((size_t)ck0 * kvstride + (size_t)g * D) * 2;
    // Paged K/V: the RPI <= 8 rows of one instruction form an aligned group
    // inside one cache block (block size >= 16), so its global address is a
    // wave-uniform row base (one block-table read) plus the lane offset.
    typedef __attribute__((address_space(4))) const int32_t cint32;
    cint32 *bt = PAGED ? (cint32 *)a.block_table + (size_t)r * a.mbps : nullptr;
    const int bs_mask = (1 << a.bs_log2) - 1;
    const char *kcache = (const char *)a.k_cache + (size_t)g * D * 2;
    const char *vcache = (const char *)a.v_cache + (size_t)g * D * 2;

    auto issue = [&](int t0, int buf) {
        char *kl = lds + buf * TL::BUF;
        char *vl = kl + TL::BYTES;
        if constexpr (!PAGED) {
            const uint32_t left = (uint32_t)(Lk - t0) * rowbytes;      // bytes from row t0 to the end
            const u32x4 kr = buffer_rsrc(kreq + (size_t)t0 * rowbytes, left);
            const u32x4 vr = buffer_rsrc(vreq + (size_t)t0 * rowbytes, left);
#pragma unroll
            for (int n = 0; n < TL::LOADS; ++n) {
                const int i = wave + 4 * n;
                const uint32_t rows = (uint32_t)(RPI * wave) + n * kStepRows;
                copy16_buffer(kr, off_k + rows * rowbytes, lds_addr(kl + 1024 * i));
                copy16_buffer(vr, off_v + rows * rowbytes, lds_addr(vl + 1024 * i));
            }
        } else {
            const bool tail = t0 + BN > Lk;
#pragma unroll
            for (int n = 0; n < TL::LOADS; ++n) {
                const int i = wave + 4 * n;
                // rows past the end read the last key instead (finite values
                // whose logits are masked), so no load leaves the request
                const int key0 = tail ? min(t0 + RPI * i, Lk - 1) : t0 + RPI * i;
                const size_t rb = (size_t)(((uint32_t)bt[key0 >> a.bs_log2] << a.bs_log2) |
                                           (key0 & bs_mask)) * rowbytes;
                const uint32_t back = tail ? (uint32_t)(lrow - min(lrow, Lk - 1 - key0)) * rowbytes : 0u;
                copy16_global(kcache + rb, off_k - back, lds_addr(kl + 1024 * i));
                copy16_global(vcache + rb, off_v - back, lds_addr(vl + 1024 * i));
            }
        }
    };

    // ---- LDS operand addresses (lane constants) ----
    // K: row 32kc + lr, unit 2c + lh  ->  (row * U + ((2c + lh) ^ swz_k(lr))) * 16
    const int k_lane = lr * U * 16;
    int k_unit[QK_STEPS];
#pragma unroll
    for (int c = 0; c < QK_STEPS; ++c) k_unit[c] = ((2 * c + lh) ^ TL::swz_k(lr)) * 16;
    // V (transpose read): lane k = lane%16 of group G = lane/16 addresses row
    // 16ks + 4lh + k/4 (+8), dims 32dt + 16(G%2) + 4(k%4) .. +3
    const int vk = lane & 15, vG = (lane >> 4) & 1;
    const int v_row = 4 * lh + (vk >> 2);
    const int v_swz = TL::swz_v(v_row);                 // same for rows +16ks and +8
    const int v_lane = v_row * U * 16 + ((vk & 3) & 1) * 8;
    int v_unit[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) v_unit[t] = ((4 * t + 2 * vG + ((vk & 3) >> 1)) ^ v_swz) * 16;

    // Mask chunk sx (32 keys from c0) where needed, then raise the reference
    // max when a logit exceeds it by more than 2^kTau, rescaling O and the
    // running sums.  Accumulator i holds key c0 + 8(i/4) + 4lh + i%4.
    float l1 = 0.f;                    // second running sum (two add chains)
    auto finish = [&](f32x16 &sx, int c0) {
        const int pos = wpos0 + lr;
        if constexpr (ALIBI) {
            // biased logits in log2 units: s * scale + slope * (key - pos)
            const float base = slope_log2 * (float)(c0 - pos);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float kx = (float)(8 * (i >> 2) + 4 * lh + (i & 3));
                sx[i] = fmaf(sx[i], a.scale_log2, fmaf(slope_log2, kx, base));
            }
        }
        const bool full = (!a.causal || c0 + 31 <= wpos0) && (c0 + 32 <= Lk) &&
                          (a.window_left < 0 || c0 >= wpos1 - a.window_left);
        if (!full) {
            const int hi = (a.causal ? min(pos, Lk - 1) : Lk - 1) - c0;   // keys <= hi visible
            const int lo = a.window_left >= 0 ? pos - a.window_left - c0 : -1 << 30;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kx = 8 * (i >> 2) + 4 * lh + (i & 3);
                sx[i] = ((kx <= hi) & (kx >= lo)) ? sx[i] : -INFINITY;
            }
        }
        float ma = __builtin_fmaxf(sx[0], sx[1]), mb = __builtin_fmaxf(sx[2], sx[3]);
#pragma unroll
        for (int i = 4; i < 16; i += 4) {
            ma = __builtin_fmaxf(__builtin_fmaxf(ma, sx[i]), sx[i + 1]);
            mb = __builtin_fmaxf(__builtin_fmaxf(mb, sx[i + 2]), sx[i + 3]);
        }
        const float mw = __builtin_fmaxf(ma, mb);
        // the other lane half holds the row's other keys
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mw), __float_as_uint(mw),
                                                         false, false);
        const float mx = ALIBI ? __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]))
                               : __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) *
                                     a.scale_log2;
        if (__any(mx > m + kTau)) {
            const float nm = fmaxf(m, mx);
            const float alpha = fast_exp2(m - nm);
            l *= alpha;
            l1 *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
            m = nm;
        }
    };
    // P of 16-key step sp of chunk sx: exp2(S * scale - m) rounded to bf16;
    // slot (lh, e) is key 16sp + 8(e/4) + 4lh + e%4 of the chunk.  The row
    // sums take the rounded values.
    auto make_p = [&](const f32x16 &sx, int sp) {
        u32x4 w;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            const float p0 = ALIBI ? fast_exp2(sx[8 * sp + 2 * e2] - m)
                                   : fast_exp2(fmaf(sx[8 * sp + 2 * e2], a.scale_log2, -m));
            const float p1 = ALIBI ? fast_exp2(sx[8 * sp + 2 * e2 + 1] - m)
                                   : fast_exp2(fmaf(sx[8 * sp + 2 * e2 + 1], a.scale_log2, -m));
            w[e2] = pack_bf16x2(p0, p1);
        }
        l = add_bf16_pair(w[0], l);
        l1 = add_bf16_pair(w[1], l1);
        l = add_bf16_pair(w[2], l);
        l1 = add_bf16_pair(w[3], l1);
        return __builtin_bit_cast(bf16x8, w);
    };

    // One 64-key tile as two 32-key chunks.  MFMA issue order: S of chunk 0,
    // S of chunk 1, then P.V by 16-key steps.  The softmax work of chunk 0
    // runs while the S MFMAs of chunk 1 execute, and that of chunk 1 while the
    // first P.V step executes, so the matrix pipe is rarely left idle.
    auto compute = [&](int buf, int t0) {
        const char *kl = lds + buf * TL::BUF;
        const char *vl = kl + TL::BYTES;
        // A 32-key chunk that no row of the wave sees (left of the window of
        // its first row, or right of the diagonal of its last) skips the
        // softmax: its logits would all be masked, its P all zero.  The
        // MFMAs still run, which keeps the instruction schedule one shape.
        const bool dead0 = t0 + 32 <= w_lo || t0 >= w_hi;
        const bool dead1 = t0 + BN <= w_lo || t0 + 32 >= w_hi;
        auto p_of = [&](const f32x16 &sx, int sp, bool dead) {
            return dead ? bf16x8{} : make_p(sx, sp);
        };
        auto kread = [&](int n) {      // K operand of S MFMA n: chunk n / QK, k-step n % QK
            return *reinterpret_cast<const bf16x8 *>(kl + k_lane + 32 * (n / QK_STEPS) * U * 16 +
                                                     k_unit[n % QK_STEPS]);
        };
        f32x16 s0, s1;
#pragma unroll
        for (int i = 0; i < 16; ++i) s0[i] = s1[i] = 0.f;
        constexpr int NS = 2 * QK_STEPS;
        bf16x8 kk[KA + 1];
#pragma unroll
        for (int n = 0; n < KA; ++n) kk[n] = kread(n);
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            if (n + KA < NS) kk[(n + KA) % (KA + 1)] = kread(n + KA);
            __builtin_amdgcn_sched_barrier(0);
            if (n < QK_STEPS) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[n % (KA + 1)], qf[n], s0, 0, 0, 0);
            else s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[n % (KA + 1)], qf[n - QK_STEPS], s1, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (n == QK_STEPS + 1 && !dead0) finish(s0, t0);
        }
        // O^T += V^T . P^T, one 16-key step at a time (ks 0, 1 from chunk 0,
        // ks 2, 3 from chunk 1); V^T operands (transpose reads) VA ahead
        auto vread = [&](int ks, int t) {
            const char *p0 = vl + v_lane + 16 * ks * U * 16 + v_unit[t];
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
            const bf16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p0 + 8 * U * 16));
            return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        constexpr int NPV = 4 * DT;
        bf16x8 vv[VA + 1];
#pragma unroll
        for (int n = 0; n < VA; ++n) vv[n] = vread(n / DT, n % DT);
        bf16x8 pf = p_of(s0, 0, dead0);
#pragma unroll
        for (int n = 0; n < NPV; ++n) {
            const int ks = n / DT, t = n % DT;
            if (n + VA < NPV) vv[(n + VA) % (VA + 1)] = vread((n + VA) / DT, (n + VA) % DT);
            __builtin_amdgcn_sched_barrier(0);
            o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv[n % (VA + 1)], pf, o[t], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (t == DT - 1) {
                // a rescale may only fall between whole k-steps of P.V
                if (ks == 0 && !dead1) finish(s1, t0 + 32);
                if (ks + 1 < 4)
                    pf = ks + 1 < 2 ? p_of(s0, (ks + 1) & 1, dead0) : p_of(s1, (ks + 1) & 1, dead1);
            }
        }
    };

    // ---- epilogue: normalise with the sink, write the wave's rows ----
    // The accumulators hold 4 dims of a row per lane, so a direct store would
    // write 32 separate 16-byte pieces per instruction.  Instead each wave
    // stages its rows in LDS and writes whole rows, 16 bytes per lane: all 32
    // at once in the K/V buffers, which are free after the last barrier, or,
    // with RUN, 16 at a time in a region of their own (the ring still holds
    // tiles of the next step).  Staged rows are padded by 16 bytes so that
    // consecutive rows start on different banks.
    constexpr int kRowPad = D * 2 + 16;
    constexpr int SR = RUN ? run_stage_rows<D>() : 32;   // rows staged per pass
    auto epilogue = [&]() {
        float lt = l + l1;
        lt += shfl_xor(lt, 32);
        const float Mt = fmaxf(lt > 0.f ? m : kNoMax, sig);
        const float sc = fast_exp2(m - Mt);
        const float Lt = lt * sc + fast_exp2(sig - Mt);
        const float f = Lt > 0.f ? sc / Lt : 0.f;
        static_assert(4 * 32 * kRowPad <= 2 * TL::BUF, "staging fits in the K/V buffers");
        char *stage = lds + (RUN ? run_slots<D>() * TL::BUF : 0) + wave * SR * kRowPad;
        constexpr int LPR = D / 8;      // lanes per row, 16 bytes each
        constexpr int RPS = 64 / LPR;   // rows per store instruction
        const int srow = lane / LPR, sunit = lane % LPR;
        uint16_t *ob = (uint16_t *)a.out + (size_t)(cq0 + wrow0) * qstride + (size_t)h * D;
#pragma unroll
        for (int ps = 0; ps < 32 / SR; ++ps) {
            // a wave's LDS accesses run in order: the reads of one pass are
            // done before the next pass writes the same rows
            if (lr >= SR * ps && lr < SR * (ps + 1)) {
#pragma unroll
                for (int t = 0; t < DT; ++t)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int d = 32 * t + 8 * q4 + 4 * lh;
                        const u32x2 w = {pack_bf16x2(o[t][4 * q4] * f, o[t][4 * q4 + 1] * f),
                                         pack_bf16x2(o[t][4 * q4 + 2] * f, o[t][4 * q4 + 3] * f)};
                        *reinterpret_cast<u32x2 *>(stage + (lr - SR * ps) * kRowPad + d * 2) = w;
                    }
            }
#pragma unroll
            for (int k = 0; k < SR / RPS; ++k) {
                const int row = srow + RPS * k;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + row * kRowPad + sunit * 16);
                if (SR * ps + row < wrows)
                    *reinterpret_cast<u32x4 *>(ob + (size_t)(SR * ps + row) * qstride + sunit * 8) = v;
            }
        }
        if (a.lse && lh == 0 && lr < wrows)
            a.lse[(size_t)(cq0 + wrow0 + lr) * a.Hq + h] = Lt > 0.f ? Mt * kLn2 + logf(Lt) : -INFINITY;
    };

    if constexpr (!RUN) {
        // one block of positions: its tiles streamed through two buffers
        int buf = 0;
        if (ntiles > 0) {
            issue(t_begin, buf);
            if (a.rope) rotate_q();
            if constexpr (ROPEK) load_ktab(t_begin);
        }
        // Q (and the first tile) landed, on both paths: the compiler then
        // knows Q's registers are complete inside the loop.  With the wait on
        // one path only it waited for Q again before each tile's first
        // MFMAs, with a count that ignores the copies it does not track, so
        // each tile waited for the next tile's copies.
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        if (ntiles > 0) __syncthreads();
        for (int it = 0; it < ntiles; ++it) {
            const int t0 = t_begin + it * BN;
            if constexpr (ROPEK) {
                // the landed tile rotated before any wave reads it, and before
                // the next tile's copies are issued (nothing is in flight at
                // this barrier)
                rotate_k(buf, t0);
                __syncthreads();
            }
            if (it + 1 < ntiles) issue(t0 + BN, buf ^ 1);
            if (wrows > 0 && t0 < w_hi && t0 + BN > w_lo) compute(buf, t0);
            // the next tile's table rows, in flight with its copies (loaded
            // after the tile's compute, so that they take no registers there)
            if constexpr (ROPEK) {
                if (it + 1 < ntiles) load_ktab(t0 + BN);
            }
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            buf ^= 1;
        }
        epilogue();
    } else {
        // Runs: the tiles live in a ring of R slots, tile n (keys [BN n,
        // BN n + BN)) in slot n % R.  The key ranges of consecutive steps
        // overlap, so a tile that is still resident is not loaded again.  A
        // step's tiles are taken in chunks: all of them at once when they fit
        // in the ring, else R / 2 at a time.  A chunk's missing tiles are
        // issued together (one wait for all of them), and while it is
        // computed the next chunk's tiles (the rest of the step, or the next
        // step's first ones) are copied into the slots it does not read, with
        // the next step's Q.  Tiles [res_lo, res_hi) are resident (or in
        // flight); they only move forward, so a tile is evicted only once no
        // later chunk needs it.
        constexpr int R = run_slots<D>();
        auto chunk_of = [&](int nt) { return nt <= R ? R : max(1, R / 2); };
        bf16x8 qn[QK_STEPS];
        int res_lo = 0, res_hi = 0;
        [[maybe_unused]] int rot_hi = 0;        // ROPEK: resident tiles below it are rotated
        auto load_tile = [&](int tn) { issue(tn * BN, tn % R); };
        for (int s = 0; s < nsteps; ++s) {
            if (s > 0) {
                set_step(s);
                if (row0 >= Lq) break;
#pragma unroll
                for (int c = 0; c < QK_STEPS; ++c) qf[c] = qn[c];
#pragma unroll
                for (int t = 0; t < DT; ++t)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
                m = kNoMax;
                l = 0.f;
                l1 = 0.f;
            }
            // the next step, if this workgroup has one
            int nx_lo = 0, nx_tb = 0, nx_nt = 0;
            const int nx_row0 = row0 + bm;
            const bool has_next = s + 1 < nsteps && nx_row0 < Lq;
            if (has_next) block_keys(nx_row0, nx_lo, nx_tb, nx_nt);
            const int nx_w0 = nx_row0 + 32 * (wave / hpw);
            const int tb0 = t_begin / BN, tb1 = tb0 + ntiles;
            const int ch = chunk_of(ntiles);
            for (int c0 = tb0; c0 < tb1; c0 += ch) {
                const int c1 = min(tb1, c0 + ch);
                // the chunk's missing tiles; the slots they refill may still
                // be read by slower waves, so all waves meet first
                if (c0 < res_lo || c0 > res_hi) {
                    res_lo = res_hi = c0;
                    if constexpr (ROPEK) rot_hi = c0;
                }
                if (res_hi < c1) {
                    __syncthreads();
                    while (res_hi < c1) load_tile(res_hi++);
                    res_lo = max(res_lo, res_hi - R);
                }
                if (c0 == tb0 && a.rope) rotate_q();
                __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                __syncthreads();
                if constexpr (ROPEK) {
                    // landed tiles rotated once, before any wave reads them
                    if (rot_hi < c1) {
                        for (int tn = max(rot_hi, c0); tn < c1; ++tn) {
                            load_ktab(tn * BN);
                            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                            rotate_k(tn % R, tn * BN);
                        }
                        rot_hi = c1;
                        __syncthreads();
                    }
                }
                // the next chunk: the rest of this step, or the next step's first
                int n0 = 0, n1 = 0;
                if (c1 < tb1) {
                    n0 = c1;
                    n1 = min(tb1, c1 + ch);
                } else if (has_next && nx_nt > 0) {
                    n0 = nx_tb / BN;
                    n1 = n0 + min(nx_nt, chunk_of(nx_nt));
                }
                // its tiles that continue the resident range, into slots this
                // chunk does not read (tile n evicts tile n - R < c0); every
                // wave has passed the barrier above, so no wave still reads
                // an earlier chunk
                if (n1 > n0 && n0 <= res_hi && n0 >= res_lo) {
                    while (res_hi < n1 && res_hi < c0 + R) load_tile(res_hi++);
                    res_lo = max(res_lo, res_hi - R);
                }
                if (c1 == tb1 && has_next) load_q(qn, nx_w0, max(0, min(32, Lq - nx_w0)));
                for (int tn = c0; tn < c1; ++tn) {
                    const int t0 = tn * BN;
                    if (wrows > 0 && t0 < w_hi && t0 + BN > w_lo) compute(tn % R, t0);
                }
            }
            // no tile in this step: the next step's Q still has to arrive
            if (ntiles == 0 && has_next) load_q(qn, nx_w0, max(0, min(32, Lq - nx_w0)));
            epilogue();
        }
    }
}

}  // namespace

template <int D>
constexpr int prefill_lds_bytes(bool run) {
    // runs: the tile ring and the staged rows of the four waves
    return run ? run_slots<D>() * Tile<D>::BUF + 4 * run_stage_rows<D>() * (D * 2 + 16)
               : 2 * Tile<D>::BUF;
}

pkv_status launch_prefill_bf16(const PrefillArgs &a, hipStream_t stream)
{
    if (a.hpw != prefill_heads_per_wg(a.G) || a.Hq % a.hpw) return PKV_ERR_SHAPE;
    const bool run = a.run_steps > 0;
    long long grid;
    if (run) {
        if (a.runs <= 0) return PKV_ERR_SHAPE;
        grid = (long long)a.B * a.runs * (a.G / a.hpw) * a.Hkv;
    } else {
        grid = (long long)a.B * a.max_q_tiles * a.Hq;
    }
    if (grid == 0) return PKV_OK;
    if (grid > 0x7fffffffLL) return PKV_ERR_SHAPE;
    // more dynamic LDS than the default limit: raise the per-kernel limit
    // once; a failure there is reported by every call rather than by a
    // faulting launch
    static const hipError_t raised = [] {
        hipError_t first = hipSuccess;
        auto set = [&](const void *fn, int bytes) {
            const hipError_t e =
                hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
            if (first == hipSuccess) first = e;
        };
#define PKV_SET(DD, PG, AL, RN) \
        set((const void *)prefill_bf16_kernel<DD, PG, AL, RN>, prefill_lds_bytes<DD>(RN))
#define PKV_SET_RK(DD, AL, RN) \
        set((const void *)prefill_bf16_kernel<DD, false, AL, RN, true>, prefill_lds_bytes<DD>(RN))
        PKV_SET(128, false, false, false); PKV_SET(128, true, false, false);
        PKV_SET(64, false, false, false); PKV_SET(64, true, false, false);
        PKV_SET(128, false, true, false); PKV_SET(128, true, true, false);
        PKV_SET(64, false, true, false); PKV_SET(64, true, true, false);
        PKV_SET(128, false, false, true); PKV_SET(128, true, false, true);
        PKV_SET(64, false, false, true); PKV_SET(64, true, false, true);
        PKV_SET(128, false, true, true); PKV_SET(128, true, true, true);
        PKV_SET(64, false, true, true); PKV_SET(64, true, true, true);
        PKV_SET_RK(128, false, false); PKV_SET_RK(64, false, false);
        PKV_SET_RK(128, false, true); PKV_SET_RK(64, false, true);
#undef PKV_SET_RK
#undef PKV_SET
        return first;
    }();
    if (raised != hipSuccess) return PKV_ERR_HIP;
    const bool paged = a.block_table != nullptr;
    if (a.rope_k && (paged || !a.rope || a.alibi)) return PKV_ERR_UNSUPPORTED;
    const dim3 g((unsigned)grid), b(256);
    auto go = [&](auto kernel, int lds) { hipLaunchKernelGGL(kernel, g, b, lds, stream, a); };
    auto pick = [&](auto dtag) {
        constexpr int DD = decltype(dtag)::value;
        const int lds = prefill_lds_bytes<DD>(run);
        if (a.rope_k) {
            if (run) go(prefill_bf16_kernel<DD, false, false, true, true>, lds);
            else go(prefill_bf16_kernel<DD, false, false, false, true>, lds);
            return;
        }
        if (a.alibi) {
            if (run) {
                if (paged) go(prefill_bf16_kernel<DD, true, true, true>, lds);
                else go(prefill_bf16_kernel<DD, false, true, true>, lds);
            } else {
                if (paged) go(prefill_bf16_kernel<DD, true, true, false>, lds);
                else go(prefill_bf16_kernel<DD, false, true, false>, lds);
            }
        } else {
            if (run) {
                if (paged) go(prefill_bf16_kernel<DD, true, false, true>, lds);
                else go(prefill_bf16_kernel<DD, false, false, true>, lds);
            } else {
                if (paged) go(prefill_bf16_kernel<DD, true, false, false>, lds);
                else go(prefill_bf16_kernel<DD, false, false, false>, lds);
            }
        }
    };
    if (a.D == 128) pick(std::integral_constant<int, 128>{});
    else pick(std::integral_constant<int, 64>{});
    return launch_status();
}

int prefill_heads_per_wg(int G) { return G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1; }
int prefill_block_m() { return 128; }

}  // namespace pkv
