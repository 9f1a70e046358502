// Rotation of one 16-byte chunk of a row by the rotary embedding, shared by
// the rotary kernels and the decode-with-append kernels.
//
// vLLM "attention.py" page, PagedAttentionWithRoPE: query and key are rotated
// by their positions before attention; the neox pairing rotates dimension d
// with d + rotary_dim / 2, the other pairing 2i with 2i + 1, and dimensions
// from rotary_dim on pass through.  tab is the position's row of the
// [positions, rotary_dim] table (cos of the angles, then sin).  Rotation runs
// in float32; bf16 results are rounded to nearest even.
#pragma once

#include "common.h"

namespace pkv {

// 16-byte chunk of a row as floats (8 bf16 or 4 float32), and back.
template <bool BF16> struct Chunk {
    static constexpr int N = BF16 ? 8 : 4;
    float x[N];
    __device__ void load(const char *p) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (BF16) {
                x[2 * w] = bf16_lo(v[w]);
                x[2 * w + 1] = bf16_hi(v[w]);
            } else {
                x[w] = __uint_as_float(v[w]);
            }
        }
    }
    __device__ void store(char *p) const {
        u32x4 v;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            v[w] = BF16 ? pack_bf16x2(x[2 * w], x[2 * w + 1]) : __float_as_uint(x[w]);
        *reinterpret_cast<u32x4 *>(p) = v;
    }
};

// Rotate (and move) one head row of D elements whose chunk u this thread
// owns.  src/dst point at the row; tab at the position's table row.
//   neox: chunk u < rd/2 / N rotates with chunk u + rd/2 / N (both written
//         here); chunks of the second half are written by their partner;
//   interleaved: chunk u < rd / N rotates its own pairs;
//   chunks from rd / N on are copied when src != dst.
template <bool BF16>
__device__ __forceinline__ void rope_chunk(const char *src, char *dst, const float *tab, int rd,
                                           bool neox, int u)
{
    using C = Chunk<BF16>;
    constexpr int N = C::N;
    const int half = rd / 2;
    if (u * N >= rd) {
        if (src != dst) *reinterpret_cast<u32x4 *>(dst + 16 * u) =
            *reinterpret_cast<const u32x4 *>(src + 16 * u);
        return;
    }
    if (neox) {
        if (u * N >= half) return;                 // written with its partner
        const int v = u + half / N;
        C a, b;
        a.load(src + 16 * u);
        b.load(src + 16 * v);
#pragma unroll
        for (int e = 0; e < N; ++e) {
            const float c = tab[u * N + e], s = tab[half + u * N + e];
            const float x0 = a.x[e], x1 = b.x[e];
            a.x[e] = x0 * c - x1 * s;
            b.x[e] = x1 * c + x0 * s;
        }
        a.store(dst + 16 * u);
        b.store(dst + 16 * v);
    } else {
        C a;
        a.load(src + 16 * u);
#pragma unroll
        for (int e = 0; e < N; e += 2) {
            const int i = (u * N + e) / 2;
            const float c = tab[i], s = tab[half + i];
            const float x0 = a.x[e], x1 = a.x[e + 1];
            a.x[e] = x0 * c - x1 * s;
            a.x[e + 1] = x1 * c + x0 * s;
        }
        a.store(dst + 16 * u);
    }
}

}  // namespace pkv
