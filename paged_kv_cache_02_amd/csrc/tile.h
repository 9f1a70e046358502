// Shared pieces of the tiled bf16 attention kernels (dense and block-sparse
// prefill): the 64-key K/V tile layout in LDS, direct global -> LDS copies,
// buffer descriptors and a packed-pair add.
#pragma once

#include "common.h"

namespace pkv {

constexpr int BN = 64;    // keys per tile
constexpr int kWaitVmcnt0 = (7 << 4) | (15 << 8);   // s_waitcnt vmcnt(0)

template <int D>
struct Tile {
    static constexpr int U = D / 8;             // 16-byte units per key row
    static constexpr int BYTES = BN * D * 2;    // one K (or V) tile
    static constexpr int BUF = 2 * BYTES;       // K + V
    static constexpr int LOADS = U / 4;         // direct loads per wave per K (or V) tile
    // Swizzled unit position inside a row: LDS unit u ^ swz(row) holds the
    // row's 16-byte unit u.  LDS has 64 banks of 4 bytes, and a 256-byte row
    // (D = 128) starts on bank 0, a 128-byte row (D = 64) on bank 0 or 32.
    // K is read 16 bytes per lane, 16 rows at a time, each row at its own
    // unit: swz_k gives the rows that start on the same bank distinct units.
    // V is read 8 bytes per lane by the transpose read, 4 rows x 4 units per
    // half wave: swz_v moves each row's 4 units to their own 64 bytes.  Both
    // depend on row bits 0-4 only, so rows 32 apart share a swizzle.
    __device__ static int swz_k(int row) { return U == 16 ? (row & 15) : ((row >> 1) & 7); }
    __device__ static int swz_v(int row) { return U == 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
    static_assert(U == 16 || U == 8, "head_dim 128 or 64");
};

// acc + lo(a) + hi(a) for a packed bf16 pair, in one v_dot2_f32_bf16 against
// (1, 1).  Written as an instruction rather than the dot2 builtin: this
// compiler's rewrite of that builtin into the accumulator-tied VOP2 form read
// operand registers after they had been reused.
__device__ __forceinline__ float add_bf16_pair(uint32_t a, float acc) {
    float d;
    asm("v_dot2_f32_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(0x3f803f80u), "v"(acc));
    return d;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ uint32_t lds_addr(const char *p) {
    return (uint32_t)(uintptr_t)(const lds_void *)p;
}

// Global -> LDS copies, 16 bytes per lane, lane L's bytes landing at LDS
// address dst + 16 L.  They are written as instructions: the compiler tracks
// an LDS read issued after a copy it knows of as possibly depending on it and
// waits for every outstanding copy first, which here would stall each tile on
// the copies just issued for the next one.  The kernel orders them itself:
// each tile's copies are waited for (vmcnt 0) and published with a barrier
// before any wave reads them, and each buffer is refilled only after the
// barrier that follows the last read of its previous contents.
//   buffer form: rsrc = raw buffer descriptor, voff = byte offset checked
//   against its range (lanes past it read zeros and touch no memory);
__device__ __forceinline__ void copy16_buffer(u32x4 rsrc, uint32_t voff, uint32_t dst) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(dst) : "memory", "m0");
}
//   global form: base (wave-uniform) + voff.
__device__ __forceinline__ void copy16_global(const void *base, uint32_t voff, uint32_t dst) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "s"(dst) : "memory", "m0");
}

// Raw buffer descriptor of `bytes` bytes from base (stride 0).
__device__ __forceinline__ u32x4 buffer_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, (uint32_t)kBufferWord3};
}

}  // namespace pkv
