// Vertical + slash block-sparse prefill, bf16 with fp32 accumulation.
//
// nano-vllm "minference.py" page, MInferencePolicy: estimate_pattern gives,
// per query head, vertical key positions and slash diagonal offsets (a query
// at position i and a key at j lie on diagonal i - j), and
// sparse_prefill_attention converts them into a block form with 64-row and
// 64-key blocks before attending.  The page does not print the conversion;
// the block form here: row block m holds rows [64m, 64m + 64) of a request,
// key block n keys [64n, 64n + 64).  Key block n is a slash block of m when a
// diagonal of the head meets it within m's rows; vertical columns outside
// m's slash blocks, up to m's last row, are listed one by one.  Row i of m
// attends the keys j <= i of its slash blocks and of its columns; the sink,
// when given, joins the denominator as everywhere in the library.
//
// gfx950 design:
//   * vertical_slash_kernel: one wave per (request, head, row block) marks
//     the slash blocks in an LDS bit set (a diagonal meets one or two key
//     blocks), then writes the offsets in ascending order (a wave prefix sum
//     over the set's words) and the surviving columns in the order given
//     (ballot and bit count);
//   * sparse_prefill_kernel: one workgroup of four waves per (request, head,
//     row block), row blocks issued longest first; wave w takes query rows
//     32 (w % 2) .. +32 (Q in registers) against keys 32 (w / 2) .. +32 of
//     every tile, so that a 64-row block still keeps eight waves on a compute
//     unit, and the two key halves of a row are merged through LDS at the
//     end.  It walks its slash blocks, then its columns 64 at a time, with
//     the dense prefill's tile layout: K and V rows go
//     straight from global memory into a swizzled LDS tile (a 64-key block
//     through a range-checked buffer descriptor, 64 columns as gathered
//     rows), double buffered; S^T = K . Q^T and O^T += V^T . P^T on
//     v_mfma_f32_32x32x16_bf16 with the V^T operand read by the LDS
//     transpose read; keys are masked by position, a gathered tile keeping
//     its 64 positions in LDS.  HBM-light and MFMA-bound like the dense
//     prefill, on the selected blocks only.

#include "common.h"
#include "decode.h"
#include "tile.h"

namespace pkv {

namespace {

constexpr int kSparseWaves = 4;
constexpr int kNoKey = 0x7fffffff;       // position of a padding row: never visible

__global__ __launch_bounds__(64) void vertical_slash_kernel(VerticalSlashArgs a)
{
    extern __shared__ uint32_t sel[];    // bit n: key block n is a slash block of this row block
    const int lane = threadIdx.x;
    const int NMW = (a.NM + 31) / 32;
    int id = blockIdx.x;
    const int m = id % a.NM;
    id /= a.NM;
    const int h = id % a.H;
    const int b = id / a.H;
    const size_t bhm = ((size_t)b * a.H + h) * a.NM + m;
    // a request longer than max_seqlen breaks the contract; its rows past
    // 64 NM are left alone so that no index leaves the arrays
    const int L = min(a.cu[b + 1] - a.cu[b], 64 * a.NM);
    const int r0 = 64 * m;
    if (r0 >= L) {
        if (lane == 0) {
            a.block_count[bhm] = 0;
            a.column_count[bhm] = 0;
        }
        return;
    }
    const int r1 = min(L, r0 + 64);              // rows [r0, r1)
    for (int w = lane; w < NMW; w += 64) sel[w] = 0u;
    __syncthreads();
    const int32_t *S = a.slash + ((size_t)b * a.H + h) * a.NS;
    for (int t = lane; t < a.NS; t += 64) {
        const int s = S[t];
        if (s < 0 || s >= L) continue;
        const int hi = r1 - 1 - s;               // keys i - s of the rows, clipped at 0
        if (hi < 0) continue;
        const int lo = max(0, r0 - s);
        const int n0 = lo >> 6, n1 = hi >> 6;
        atomicOr(&sel[n0 >> 5], 1u << (n0 & 31));
        if (n1 != n0) atomicOr(&sel[n1 >> 5], 1u << (n1 & 31));
    }
    __syncthreads();
    // offsets of the slash blocks, ascending: word w holds blocks 32w .. 32w + 31
    int32_t *bo = a.block_offset + bhm * a.NM;
    int nb = 0;
    for (int w0 = 0; w0 < NMW; w0 += 64) {
        const int w = w0 + lane;
        uint32_t bits = w < NMW ? sel[w] : 0u;
        const int cnt = __popc(bits);
        int incl = cnt;                          // inclusive prefix sum over the wave
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d, 64);
            if (lane >= d) incl += y;
        }
        int pos = nb + incl - cnt;
        while (bits) {
            const int n = __ffs(bits) - 1;
            bits &= bits - 1;
            bo[pos++] = 64 * (32 * w + n);
        }
        nb += __shfl(incl, 63, 64);
    }
    // the vertical columns of the rows that no slash block covers, in order
    const int32_t *V = a.vertical + ((size_t)b * a.H + h) * a.NV;
    int32_t *ci = a.column_index + bhm * a.NV;
    int nc = 0;
    for (int t0 = 0; t0 < a.NV; t0 += 64) {
        const int t = t0 + lane;
        const int v = t < a.NV ? V[t] : -1;
        bool keep = v >= 0 && v < r1;
        if (keep) keep = !((sel[v >> 11] >> ((v >> 6) & 31)) & 1u);
        const uint64_t ball = __ballot(keep);
        if (keep) ci[nc + __popcll(ball & ((1ull << lane) - 1ull))] = v;
        nc += __popcll(ball);
    }
    if (lane == 0) {
        a.block_count[bhm] = nb;
        a.column_count[bhm] = nc;
    }
}

template <int D>
constexpr int sparse_lds_bytes() { return 2 * Tile<D>::BUF + 2 * BN * (int)sizeof(int); }

template <int D>
__global__ __launch_bounds__(64 * kSparseWaves, 2) void sparse_prefill_kernel(SparseArgs a)
{
    using TL = Tile<D>;
    constexpr int U = TL::U;
    constexpr int QK_STEPS = D / 16;             // k-steps of 16 dims
    constexpr int DT = D / 32;                   // 32-dim output tiles
    constexpr int RPI = 64 / U;                  // key rows per load instruction
    constexpr int NLOAD = U / kSparseWaves;      // load instructions per wave per K (or V) tile
    extern __shared__ __attribute__((aligned(16))) char lds[];
    int *s_pos = reinterpret_cast<int *>(lds + 2 * TL::BUF);   // [2][BN]: gathered positions

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = readfirstlane(tid >> 6);
    const int lr = lane & 31;                    // row within the wave / column of the MFMA
    const int lh = lane >> 5;                    // lane half

    // Consecutive workgroups go to the eight XCDs in turn.  Position p among
    // the Hq workgroups of one (request, row block) takes kv head p % Hkv
    // and its query head p / Hkv within the group, so the query heads of a
    // kv head, and its successive row blocks, land on the same XCD and share
    // that XCD's L2 (whenever Hkv divides 8 or 8 divides Hkv, and Hq is a
    // multiple of 8).
    int id = blockIdx.x;
    const int p = id % a.Hq;
    const int h = (p % a.Hkv) * a.G + p / a.Hkv;
    id /= a.Hq;
    const int m = a.NM - 1 - id % a.NM;          // the longest row blocks first
    const int b = id / a.NM;
    // values every lane agrees on, held in scalar registers (the load
    // descriptors and LDS destinations below must be)
    const int cq0 = readfirstlane(a.cu[b]);
    const int L = readfirstlane(min(a.cu[b + 1] - cq0, 64 * a.NM));
    const int r0 = 64 * m;
    if (r0 >= L) return;
    const int g = h / a.G;
    const size_t bhm = ((size_t)b * a.Hq + h) * a.NM + m;
    const int nb = readfirstlane(a.block_count[bhm]);
    const int nc = readfirstlane(a.column_count[bhm]);
    const int ntiles = nb + (nc + BN - 1) / BN;
    const int32_t *boff = a.block_offset + bhm * a.NM;
    const int32_t *cidx = a.column_index + bhm * a.NV;
    const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;

    const int kh = wave >> 1;                    // this wave's 32 keys of each tile
    const int wrow0 = r0 + 32 * (wave & 1);      // this wave's first row
    const int wrows = max(0, min(32, L - wrow0));
    const int qpos = wrow0 + lr;                 // this lane's query position

    const size_t qstride = (size_t)a.Hq * D;
    const size_t kvstride = (size_t)a.Hkv * D;
    bf16x8 qf[QK_STEPS];
    {
        const bool ok = lr < wrows;
        const uint16_t *qp = (const uint16_t *)a.q +
                             (size_t)(cq0 + wrow0 + (ok ? lr : 0)) * qstride + (size_t)h * D + 8 * lh;
#pragma unroll
        for (int c = 0; c < QK_STEPS; ++c) {
            u32x4 x = u32x4{0u, 0u, 0u, 0u};
            if (ok) x = *reinterpret_cast<const u32x4 *>(qp + 16 * c);
            qf[c] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // ---- direct loads: instruction i = wave + 4n of a tile fills LDS bytes
    // [1024i, 1024i + 1024), lane L writing row RPI*i + L/U at swizzled unit
    // position (L % U) ^ swz(row) ----
    const uint32_t rowbytes = (uint32_t)kvstride * 2;
    const char *kreq = (const char *)a.k + ((size_t)cq0 * kvstride + (size_t)g * D) * 2;
    const char *vreq = (const char *)a.v + ((size_t)cq0 * kvstride + (size_t)g * D) * 2;
    const int lrow = lane / U;
    auto issue = [&](int it, int buf) {
        char *kl = lds + buf * TL::BUF;
        char *vl = kl + TL::BYTES;
        if (it < nb) {
            // a 64-key block: one descriptor whose range ends at the request's
            // last key, so rows past it read as zeros (and are masked)
            const int t0 = readfirstlane(boff[it]);
            const uint32_t left = (uint32_t)(L - t0) * rowbytes;
            const u32x4 kr = buffer_rsrc(kreq + (size_t)t0 * rowbytes, left);
            const u32x4 vr = buffer_rsrc(vreq + (size_t)t0 * rowbytes, left);
#pragma unroll
            for (int n = 0; n < NLOAD; ++n) {
                const int i = wave + kSparseWaves * n;
                const int row = RPI * i + lrow;
                copy16_buffer(kr, row * rowbytes + 16 * ((lane % U) ^ TL::swz_k(row)),
                              lds_addr(kl + 1024 * i));
                copy16_buffer(vr, row * rowbytes + 16 * ((lane % U) ^ TL::swz_v(row)),
                              lds_addr(vl + 1024 * i));
            }
        } else {
            // 64 columns gathered row by row (a padding row repeats the
            // tile's first column; its position marks it invisible)
            // (all index loads first: a copy issued between them would be
            // waited for with the next index, the counter being in order)
            const int c0 = (it - nb) * BN;
            uint32_t col[NLOAD];
#pragma unroll
            for (int n = 0; n < NLOAD; ++n) {
                const int e = c0 + RPI * (wave + kSparseWaves * n) + lrow;
                col[n] = (uint32_t)cidx[e < nc ? e : c0];
            }
            const int p = c0 + lane < nc ? cidx[c0 + lane] : kNoKey;
            if (wave == 0) s_pos[buf * BN + lane] = p;
#pragma unroll
            for (int n = 0; n < NLOAD; ++n) {
                const int i = wave + kSparseWaves * n;
                const int row = RPI * i + lrow;
                copy16_global(kreq, col[n] * rowbytes + 16 * ((lane % U) ^ TL::swz_k(row)),
                              lds_addr(kl + 1024 * i));
                copy16_global(vreq, col[n] * rowbytes + 16 * ((lane % U) ^ TL::swz_v(row)),
                              lds_addr(vl + 1024 * i));
            }
        }
    };

    // ---- LDS operand addresses (the dense prefill's layout) ----
    // K: row 32kc + lr, unit 2c + lh
    const int k_lane = lr * U * 16;
    int k_unit[QK_STEPS];
#pragma unroll
    for (int c = 0; c < QK_STEPS; ++c) k_unit[c] = ((2 * c + lh) ^ TL::swz_k(lr)) * 16;
    // V (transpose read): lane k = lane%16 of group G = lane/16 addresses row
    // 16ks + 4lh + k/4 (+8), dims 32dt + 16(G%2) + 4(k%4) .. +3
    const int vk = lane & 15, vG = (lane >> 4) & 1;
    const int v_row = 4 * lh + (vk >> 2);
    const int v_swz = TL::swz_v(v_row);
    const int v_lane = v_row * U * 16 + ((vk & 3) & 1) * 8;
    int v_unit[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) v_unit[t] = ((4 * t + 2 * vG + ((vk & 3) >> 1)) ^ v_swz) * 16;

    f32x16 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
    float m_run = kNoMax, l = 0.f, l1 = 0.f;

    // One tile, this wave's 32 keys: S^T, the mask by position, one online
    // softmax update, then P.V by 16-key steps.  Accumulator i holds key
    // 32kh + 8(i/4) + 4lh + i%4 of query row lr.  LDS operand reads run
    // ahead of the MFMAs that use them (K reads KA ahead; the V^T reads of
    // P.V are issued before the softmax work and consumed VA behind), and
    // the reference max is raised only when a logit exceeds it by more than
    // 2^kTau (a wave-uniform branch), as in the dense prefill.
    constexpr int KA = 4;
    constexpr int NPV = 2 * DT;                  // P.V MFMAs per tile
    constexpr int VA = NPV < 5 ? NPV : 5;
    constexpr float kTau = 8.0f;
    auto compute = [&](int buf, int it) {
        const char *kl = lds + buf * TL::BUF;
        const char *vl = kl + TL::BYTES;
        const bool gathered = it >= nb;
        const int t0 = gathered ? 0 : readfirstlane(boff[it]);
        auto kread = [&](int c) {
            return *reinterpret_cast<const bf16x8 *>(kl + k_lane + 32 * kh * U * 16 + k_unit[c]);
        };
        // V^T operand of P.V MFMA n: 16-key step 2kh + n / DT, dims tile n % DT
        auto vread = [&](int n) {
            const char *p0 = vl + v_lane + 16 * (2 * kh + n / DT) * U * 16 + v_unit[n % DT];
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
            const bf16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p0 + 8 * U * 16));
            return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        f32x16 sx;
#pragma unroll
        for (int i = 0; i < 16; ++i) sx[i] = 0.f;
        bf16x8 kk[KA + 1];
#pragma unroll
        for (int n = 0; n < KA; ++n) kk[n] = kread(n);
#pragma unroll
        for (int n = 0; n < QK_STEPS; ++n) {
            if (n + KA < QK_STEPS) kk[(n + KA) % (KA + 1)] = kread(n + KA);
            __builtin_amdgcn_sched_barrier(0);
            sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[n % (KA + 1)], qf[n], sx, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 vv[VA + 1];
#pragma unroll
        for (int n = 0; n < VA; ++n) vv[n] = vread(n);
        float mx = -INFINITY;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int k0 = 32 * kh + 8 * q4 + 4 * lh;
            int pos[4];
            if (gathered) {
                const u32x4 p4 = *reinterpret_cast<const u32x4 *>(s_pos + buf * BN + k0);
#pragma unroll
                for (int e = 0; e < 4; ++e) pos[e] = (int)p4[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) pos[e] = t0 + k0 + e;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool vis = pos[e] <= qpos && pos[e] < L;
                const float x = vis ? sx[4 * q4 + e] * a.scale_log2 : -INFINITY;
                sx[4 * q4 + e] = x;
                mx = __builtin_fmaxf(mx, x);
            }
        }
        // the other lane half holds the row's other keys
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        if (__any(mx > m_run + kTau)) {
            const float nm = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - nm);
            l *= alpha;
            l1 *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[t][i] *= alpha;
            m_run = nm;
        }
        // O^T += V^T . P^T: P slot (lh, e) of 16-key step sp is key
        // 16sp + 8(e/4) + 4lh + e%4 of this wave's 32
        auto make_p = [&](int sp) {
            u32x4 w;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2)
                w[e2] = pack_bf16x2(fast_exp2(sx[8 * sp + 2 * e2] - m_run),
                                    fast_exp2(sx[8 * sp + 2 * e2 + 1] - m_run));
            l = add_bf16_pair(w[0], l);
            l1 = add_bf16_pair(w[1], l1);
            l = add_bf16_pair(w[2], l);
            l1 = add_bf16_pair(w[3], l1);
            return __builtin_bit_cast(bf16x8, w);
        };
        bf16x8 pf = make_p(0);
#pragma unroll
        for (int n = 0; n < NPV; ++n) {
            if (n + VA < NPV) vv[(n + VA) % (VA + 1)] = vread(n + VA);
            __builtin_amdgcn_sched_barrier(0);
            o[n % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv[n % (VA + 1)], pf, o[n % DT], 0,
                                                               0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (n == DT - 1) pf = make_p(1);
        }
    };

    if (ntiles > 0) issue(0, 0);
    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        // this wave's copies of tile it have landed; after the barrier every
        // wave's have (and the tile's positions), and no wave reads buf ^ 1
        // (tile it - 1) any more
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (it + 1 < ntiles) issue(it + 1, buf ^ 1);
        if (wrows > 0) compute(buf, it);
    }

    // ---- the two key halves of each row: the kh = 1 waves leave their
    // running max, sums and accumulators in LDS (the tile buffers are free
    // once every wave is past its last tile); the kh = 0 waves rescale both
    // to the larger max and add ----
    float lsum = l + l1;
    __syncthreads();
    constexpr int OW = DT * 16;                  // accumulator floats per lane
    float *xch = reinterpret_cast<float *>(lds) + (wave & 1) * 64 * (OW + 2);
    static_assert(2 * 64 * (OW + 2) * 4 <= 2 * TL::BUF, "the exchange fits in the tile buffers");
    if (kh == 1) {
        xch[lane] = m_run;
        xch[64 + lane] = lsum;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int i = 0; i < 16; i += 4)
                *reinterpret_cast<f32x4 *>(xch + 128 + lane * OW + 16 * t + i) =
                    f32x4{o[t][i], o[t][i + 1], o[t][i + 2], o[t][i + 3]};
    }
    __syncthreads();
    if (kh == 1 || wrows == 0) return;
    {
        const float m1 = xch[lane], l1s = xch[64 + lane];
        const float M = fmaxf(m_run, m1);
        const float a0 = fast_exp2(m_run - M), a1 = fast_exp2(m1 - M);
        lsum = lsum * a0 + l1s * a1;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                const f32x4 y = *reinterpret_cast<const f32x4 *>(xch + 128 + lane * OW + 16 * t + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) o[t][i + e] = o[t][i + e] * a0 + y[e] * a1;
            }
        m_run = M;
    }

    // ---- epilogue: the sink joins the denominator; each lane stores 4 dims
    // of its row per accumulator quad ----
    float lt = lsum;
    lt += shfl_xor(lt, 32);
    const float Mt = fmaxf(lt > 0.f ? m_run : kNoMax, sig);
    const float sc = fast_exp2(m_run - Mt);
    const float Lt = lt * sc + fast_exp2(sig - Mt);
    const float f = Lt > 0.f ? sc / Lt : 0.f;
    if (lr < wrows) {
        uint16_t *orow = (uint16_t *)a.out + (size_t)(cq0 + wrow0 + lr) * qstride + (size_t)h * D;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 32 * t + 8 * q4 + 4 * lh;
                *reinterpret_cast<u32x2 *>(orow + d) =
                    u32x2{pack_bf16x2(o[t][4 * q4] * f, o[t][4 * q4 + 1] * f),
                          pack_bf16x2(o[t][4 * q4 + 2] * f, o[t][4 * q4 + 3] * f)};
            }
        if (a.lse && lh == 0)
            a.lse[(size_t)(cq0 + wrow0 + lr) * a.Hq + h] =
                Lt > 0.f ? Mt * kLn2 + logf(Lt) : -INFINITY;
    }
}

}  // namespace

pkv_status launch_vertical_slash(const VerticalSlashArgs &a, hipStream_t stream)
{
    const long long grid = (long long)a.B * a.H * a.NM;
    if (grid == 0) return PKV_OK;
    if (grid > 0x7fffffffLL) return PKV_ERR_SHAPE;
    const int lds = (a.NM + 31) / 32 * (int)sizeof(uint32_t);
    hipLaunchKernelGGL(vertical_slash_kernel, dim3((unsigned)grid), dim3(64), lds, stream, a);
    return launch_status();
}

pkv_status launch_sparse_prefill(const SparseArgs &a, hipStream_t stream)
{
    const long long grid = (long long)a.B * a.NM * a.Hq;
    if (grid == 0) return PKV_OK;
    if (grid > 0x7fffffffLL) return PKV_ERR_SHAPE;
    static const hipError_t raised = [] {
        hipError_t e = hipFuncSetAttribute((const void *)sparse_prefill_kernel<128>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           sparse_lds_bytes<128>());
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void *)sparse_prefill_kernel<64>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    sparse_lds_bytes<64>());
        return e;
    }();
    if (raised != hipSuccess) return PKV_ERR_HIP;
    const dim3 g((unsigned)grid), blk(64 * kSparseWaves);
    if (a.D == 128)
        hipLaunchKernelGGL(sparse_prefill_kernel<128>, g, blk, sparse_lds_bytes<128>(), stream, a);
    else
        hipLaunchKernelGGL(sparse_prefill_kernel<64>, g, blk, sparse_lds_bytes<64>(), stream, a);
    return launch_status();
}

}  // namespace pkv
