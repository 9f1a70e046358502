// Internal helpers shared by the gfx950 kernels of libpkv (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer descriptor on gfx9-family GPUs (32-bit data, no
// swizzle, offsets checked against num_records).
constexpr int kBufferWord3 = 0x00020000;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Reference maximum of a row that has seen no visible key yet: finite, so
// exp2(-inf - kNoMax) is 0 rather than NaN.
constexpr float kNoMax = -1.0e30f;

// bf16 <-> f32.  A bf16 value is the upper half of an f32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// f32 -> bf16, round to nearest even (NaN stays a quiet NaN): the language
// conversion, which gfx950 executes as v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Pack two f32 into bf16x2 (round to nearest even), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of lane (quad_base + k) broadcast to the 4 lanes of every quad (DPP).
template <int K>
__device__ __forceinline__ float quad_bcast(float x) {
    constexpr int ctrl = K | (K << 2) | (K << 4) | (K << 6);
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xf, 0xf, false));
}

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// 16-byte global load through a uniform base plus a 32-bit byte offset.
__device__ __forceinline__ u32x4 ld16(const void *base, uint32_t byte_off) {
    return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(base) + byte_off);
}

__device__ __forceinline__ int readfirstlane(int x) { return __builtin_amdgcn_readfirstlane(x); }

inline pkv_status launch_status() {
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv
