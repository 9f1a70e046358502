// Rotary position embedding: the cos/sin table, in-place rotation of rows,
// and reshape_and_cache with the key rotated as it is stored.
//
// vLLM "attention.py" page, PagedAttentionWithRoPE: query and key are rotated
// by their positions before attention, with rotary_dim, base, is_neox_style
// and an optional linear or dynamic rope_scaling; the rotation is the
// standard rotary embedding (the page names it, it does not print it):
// frequency i < rotary_dim / 2 turns by base^(-2i / rotary_dim) per
// position; the neox pairing rotates dimension d with d + rotary_dim / 2,
// the other pairing 2i with 2i + 1; dimensions from rotary_dim on pass
// through.  Linear scaling divides positions by the factor; dynamic scaling
// raises the base when the table is longer than max_position.
//
// The table [positions, rotary_dim] holds cos of the angles, then sin, in
// float32 (computed in double).  Rows are rotated in float32 and rounded to
// the storage type.  HBM-bound: one read and one write of each rotated row.

#include <algorithm>

#include "common.h"
#include "decode.h"
#include "rope.h"

namespace pkv {

namespace {

__global__ __launch_bounds__(256) void rope_table_kernel(float *cos_sin, int n_pos, int rd,
                                                         double base, int linear, double factor)
{
    const int half = rd / 2;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)n_pos * half) return;
    const int pos = (int)(idx / half), i = (int)(idx % half);
    const double inv_freq = pow(base, -2.0 * i / rd);
    const double t = linear ? pos / factor : (double)pos;
    double s, c;
    sincos(t * inv_freq, &s, &c);
    cos_sin[(size_t)pos * rd + i] = (float)c;
    cos_sin[(size_t)pos * rd + half + i] = (float)s;
}

// In place: x [T, H, D] with rows row_stride elements apart; one thread per
// 16-byte chunk of one (token, head) row.
template <bool BF16>
__global__ __launch_bounds__(256) void rope_apply_kernel(char *x, const int32_t *positions,
                                                         const float *cos_sin, int T, int H,
                                                         int D, long long row_stride_bytes,
                                                         int rd, int neox)
{
    constexpr int N = Chunk<BF16>::N;
    const int cpr = D / N;                         // chunks per head row
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)T * H * cpr) return;
    const int u = (int)(idx % cpr);
    const long long th = idx / cpr;
    const int h = (int)(th % H), t = (int)(th / H);
    char *row = x + t * row_stride_bytes + (size_t)h * D * (BF16 ? 2 : 4);
    rope_chunk<BF16>(row, row, cos_sin + (size_t)positions[t] * rd, rd, neox != 0, u);
}

// The contiguous keys of varlen requests rotated by their positions into a
// copy: row cu_k[r] + j of k (position j of request r) goes to the same row
// of dst.  One thread per 16-byte chunk of one (request, position, kv head)
// row, positions up to max_len; rows past a request's keys do nothing.
__global__ __launch_bounds__(256) void rope_keys_kernel(const char *k, char *dst,
                                                        const int32_t *cu_k,
                                                        const float *cos_sin, int B, int max_len,
                                                        int H, int D, int rd, int neox)
{
    const int cpr = D / 8;                         // chunks per head row
    long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const int u = (int)(idx % cpr);
    idx /= cpr;
    const int h = (int)(idx % H);
    idx /= H;
    const int j = (int)(idx % max_len);
    const long long r = idx / max_len;
    if (r >= B) return;
    const int c0 = cu_k[r];
    if (j >= cu_k[r + 1] - c0) return;
    const size_t row = ((size_t)(c0 + j) * H + h) * D * 2;
    rope_chunk<true>(k + row, dst + row, cos_sin + (size_t)j * rd, rd, neox != 0, u);
}

// reshape_and_cache with the key rotated: one thread per 16-byte chunk of a
// token's K row (all kv heads) and of its V row.
template <bool BF16>
__global__ __launch_bounds__(256) void rope_cache_kernel(
    const char *key, const char *value, char *k_cache, char *v_cache,
    const int32_t *slot_mapping, const int32_t *positions, const float *cos_sin, int T,
    long long key_stride_bytes, long long value_stride_bytes, int Hkv, int D, int rd, int neox)
{
    constexpr int N = Chunk<BF16>::N;
    const int cpr = D / N;
    const int row_chunks = Hkv * cpr;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)T * row_chunks) return;
    const int t = (int)(idx / row_chunks), c = (int)(idx % row_chunks);
    const int s = slot_mapping[t];
    if (s < 0) return;                             // padding token
    const size_t row_bytes = (size_t)Hkv * D * (BF16 ? 2 : 4);
    const size_t head_bytes = (size_t)D * (BF16 ? 2 : 4);
    const int g = c / cpr, u = c % cpr;
    const char *kr = key + t * key_stride_bytes + g * head_bytes;
    char *kc = k_cache + (size_t)s * row_bytes + g * head_bytes;
    rope_chunk<BF16>(kr, kc, cos_sin + (size_t)positions[t] * rd, rd, neox != 0, u);
    *reinterpret_cast<u32x4 *>(v_cache + (size_t)s * row_bytes + 16 * (size_t)c) =
        *reinterpret_cast<const u32x4 *>(value + t * value_stride_bytes + 16 * (size_t)c);
}

}  // namespace

pkv_status launch_rope_table(float *cos_sin, int n_pos, int rd, double base, int scaling,
                             double factor, int max_position, hipStream_t stream)
{
    double b = base;
    if (scaling == 2 && n_pos > max_position)      // dynamic (NTK-aware) base
        b = base * std::pow(factor * n_pos / max_position - (factor - 1.0),
                            (double)rd / (rd - 2));
    const long long n = (long long)n_pos * (rd / 2);
    if (n == 0) return PKV_OK;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       cos_sin, n_pos, rd, b, scaling == 1 ? 1 : 0, factor);
    return launch_status();
}

pkv_status launch_rope_apply(void *x, const int32_t *positions, const float *cos_sin, int T,
                             int H, int D, long long row_stride, int rd, int neox, bool bf16,
                             hipStream_t stream)
{
    const long long n = (long long)T * H * (D / (bf16 ? 8 : 4));
    if (n == 0) return PKV_OK;
    const unsigned grid = (unsigned)((n + 255) / 256);
    const long long stride_bytes = row_stride * (bf16 ? 2 : 4);
    if (bf16)
        hipLaunchKernelGGL(rope_apply_kernel<true>, dim3(grid), dim3(256), 0, stream, (char *)x,
                           positions, cos_sin, T, H, D, stride_bytes, rd, neox);
    else
        hipLaunchKernelGGL(rope_apply_kernel<false>, dim3(grid), dim3(256), 0, stream, (char *)x,
                           positions, cos_sin, T, H, D, stride_bytes, rd, neox);
    return launch_status();
}

pkv_status launch_rope_keys(const void *k, void *dst, const int32_t *cu_k,
                            const float *cos_sin, int B, int max_len, int H, int D, int rd,
                            int neox, hipStream_t stream)
{
    const long long n = (long long)B * max_len * H * (D / 8);
    if (n == 0) return PKV_OK;
    const long long grid = (n + 255) / 256;
    if (grid > 0x7fffffffLL) return PKV_ERR_SHAPE;
    hipLaunchKernelGGL(rope_keys_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       (const char *)k, (char *)dst, cu_k, cos_sin, B, max_len, H, D, rd, neox);
    return launch_status();
}

pkv_status launch_rope_cache(const void *key, const void *value, void *k_cache, void *v_cache,
                             const int32_t *slot_mapping, const int32_t *positions,
                             const float *cos_sin, int T, long long key_stride,
                             long long value_stride, int Hkv, int D, int rd, int neox, bool bf16,
                             hipStream_t stream)
{
    const long long n = (long long)T * Hkv * (D / (bf16 ? 8 : 4));
    if (n == 0) return PKV_OK;
    const unsigned grid = (unsigned)((n + 255) / 256);
    const int eb = bf16 ? 2 : 4;
    if (bf16)
        hipLaunchKernelGGL(rope_cache_kernel<true>, dim3(grid), dim3(256), 0, stream,
                           (const char *)key, (const char *)value, (char *)k_cache,
                           (char *)v_cache, slot_mapping, positions, cos_sin, T, key_stride * eb,
                           value_stride * eb, Hkv, D, rd, neox);
    else
        hipLaunchKernelGGL(rope_cache_kernel<false>, dim3(grid), dim3(256), 0, stream,
                           (const char *)key, (const char *)value, (char *)k_cache,
                           (char *)v_cache, slot_mapping, positions, cos_sin, T, key_stride * eb,
                           value_stride * eb, Hkv, D, rd, neox);
    return launch_status();
}

}  // namespace pkv
