// Attention with one wave per (query row, head): the float32 path of paged
// decode and varlen prefill.
//
// Same definition as the bf16 kernels (FlashInfer sink-attention page:
// logits sm_scale*q.k, bottom-right causal position p = Lk - Lq + i, window
// p - window_left <= j <= p, GQA h -> h / G, sink in the denominator only;
// its non-causal branch drops j <= p and keeps the window's left bound;
// Transformers paged-attention doc: keys through block_table / cu_seqlens),
// computed with plain fp32 FMAs: the 64 lanes split head_dim, each key's dot
// product is a wave reduction, and the softmax is updated online one key at
// a time.  It serves the small float32 workloads, where accuracy (1e-4), not
// speed, is asked for.

#include "common.h"
#include "decode.h"

namespace pkv {

__device__ __forceinline__ float ld_elem(const void *p, size_t i) {
    return ((const float *)p)[i];
}

template <int D>
__global__ __launch_bounds__(256) void rows_kernel(RowArgs a)
{
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const long long wid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);

    int h, Lq, Lk, i, pidx = 0, req;
    size_t qrow;
    if (a.mode == 0) {  // decode: unit = (b*Hq + h)*nparts + p
        if (wid >= (long long)a.B * a.Hq * a.nparts) return;
        pidx = (int)(wid % a.nparts);
        const int bh = (int)(wid / a.nparts);
        req = bh / a.Hq;
        h = bh % a.Hq;
        Lk = a.seqlens[req] + a.append;
        Lq = 1;
        i = 0;
        qrow = (size_t)bh;
    } else {            // prefill: unit = (r * max_seqlen_q + i) * Hq + h
        if (wid >= (long long)a.B * a.T * a.Hq) return;
        h = (int)(wid % a.Hq);
        const long long ri = wid / a.Hq;
        req = (int)(ri / a.T);
        i = (int)(ri % a.T);
        Lq = a.cu_q[req + 1] - a.cu_q[req];
        if (i >= Lq) return;
        Lk = a.cu_k[req + 1] - a.cu_k[req];
        qrow = ((size_t)a.cu_q[req] + i) * a.Hq + h;
    }
    const int g = h / a.G;
    const int pos = Lk - Lq + i;
    int jlo = 0, jhi = (a.mode == 1 && !a.causal) ? Lk : min(Lk, pos + 1);
    if (a.window_left >= 0) jlo = max(jlo, pos - a.window_left);
    if (a.split) {
        jlo = max(jlo, pidx * a.part_size);
        jhi = min(jhi, (pidx + 1) * a.part_size);
    }

    float qv[E], acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        qv[e] = ld_elem(a.q, qrow * D + lane + 64 * e);
        acc[e] = 0.f;
    }
    // Rotary embedding of row x (elements row0 .. row0 + D) at position p,
    // this lane's elements xv: the partner element is read from memory
    // (neox: d +- rope_dim / 2; interleaved: d ^ 1).
    auto rotate = [&](float (&xv)[E], const void *x, size_t row0, int p) {
        const int rd = a.rope_dim, half = rd / 2;
        const float *tab = a.rope + (size_t)p * rd;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int d = lane + 64 * e;
            if (d >= rd) continue;
            const bool hi = a.rope_neox ? d >= half : (d & 1);
            const int pd = a.rope_neox ? (hi ? d - half : d + half) : (d ^ 1);
            const int i = a.rope_neox ? (hi ? d - half : d) : d / 2;
            const float xp = ld_elem(x, row0 + pd);
            const float co = tab[i], si = tab[half + i];
            xv[e] = hi ? fmaf(xv[e], co, xp * si) : fmaf(xv[e], co, -xp * si);
        }
    };
    // q at its position (prefill: Lk - Lq + i; decode with append: the new
    // token's).  A prefill row at a negative position (Lq > Lk) has no table
    // row and is not rotated.
    if ((a.mode == 1 || a.append) && a.rope && pos >= 0) rotate(qv, a.q, qrow * D, pos);
#pragma unroll
    for (int e = 0; e < E; ++e) qv[e] *= a.scale_log2;
    float m = kNoMax, l = 0.f;
    // ALiBi: slope * (key position - query position), in log2 units like qv
    const float slope_log2 = a.alibi ? a.alibi[h] * kLog2e : 0.f;
    const int32_t *bt = a.block_table ? a.block_table + (size_t)req * a.mbps : nullptr;
    const int bs_mask = (1 << a.bs_log2) - 1;
    // decode with append: the new token's key (rotated by its position with
    // a rotary table), which every wave of this call reads from here
    float kn[E] = {};
    if (a.mode == 0 && a.append) {
        const size_t src = ((size_t)req * a.Hkv + g) * D;
#pragma unroll
        for (int e = 0; e < E; ++e) kn[e] = ld_elem(a.k_new, src + lane + 64 * e);
        if (a.rope) rotate(kn, a.k_new, src, Lk - 1);
    }
    if (a.mode == 0 && a.append && h % a.G == 0 && pidx == 0) {
        // store the new token at position Lk - 1; every wave of this call reads
        // that key from kn / v_new, so no reader waits for this store
        const int L = Lk - 1;
        const size_t slot = ((size_t)bt[L >> a.bs_log2] << a.bs_log2) + (L & bs_mask);
        const size_t src = ((size_t)req * a.Hkv + g) * D, dst = (slot * a.Hkv + g) * D;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int d = lane + 64 * e;
            ((float *)a.k_cache)[dst + d] = kn[e];
            ((float *)a.v_cache)[dst + d] = ((const float *)a.v_new)[src + d];
        }
    }
    for (int jj = jlo; jj < jhi; ++jj) {
        size_t row;
        const void *kb, *vb;
        if (a.mode == 0 && a.append && jj == Lk - 1) {   // the new token
            row = req;
            kb = a.k_new;
            vb = a.v_new;
        } else if (a.k) {
            row = (size_t)a.cu_k[req] + jj;
            kb = a.k;
            vb = a.v;
        } else {
            row = ((size_t)bt[jj >> a.bs_log2] << a.bs_log2) + (jj & bs_mask);
            kb = a.k_cache;
            vb = a.v_cache;
        }
        const size_t off = (row * a.Hkv + g) * D;
        const bool is_new = a.mode == 0 && a.append && jj == Lk - 1;
        float kv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) kv[e] = is_new ? kn[e] : ld_elem(kb, off + lane + 64 * e);
        // prefill over contiguous K with rope_k: the key rotated by its position
        if (a.mode == 1 && a.rope_k && a.k) rotate(kv, kb, off, jj);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) s = fmaf(qv[e], kv[e], s);
#pragma unroll
        for (int msk = 1; msk < 64; msk <<= 1) s += shfl_xor(s, msk);
        s = fmaf(slope_log2, (float)(jj - pos), s);
        const float nm = fmaxf(m, s);
        const float c = fast_exp2(m - nm);
        const float p = fast_exp2(s - nm);
        l = fmaf(l, c, p);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(acc[e], c, p * ld_elem(vb, off + lane + 64 * e));
        m = nm;
    }

    if (a.split) {
        const size_t pi = ((size_t)req * a.Hq + h) * a.nparts + pidx;
#pragma unroll
        for (int e = 0; e < E; ++e) a.part_out[pi * D + lane + 64 * e] = l > 0.f ? acc[e] / l : 0.f;
        if (lane == 0) a.part_lse[pi] = l > 0.f ? m * kLn2 + logf(l) : -INFINITY;
        return;
    }
    const float sig = a.sink ? a.sink[h] * kLog2e : -INFINITY;
    const float Mt = fmaxf(l > 0.f ? m : kNoMax, sig);
    const float sc = fast_exp2(m - Mt);
    const float Lt = l * sc + fast_exp2(sig - Mt);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float res = Lt > 0.f ? acc[e] * sc / Lt : 0.f;
        ((float *)a.out)[qrow * D + lane + 64 * e] = res;
    }
    if (a.lse && lane == 0) a.lse[qrow] = Lt > 0.f ? Mt * kLn2 + logf(Lt) : -INFINITY;
}

pkv_status launch_rows(const RowArgs &a, hipStream_t stream)
{
    const long long waves =
        a.mode == 0 ? (long long)a.B * a.Hq * a.nparts : (long long)a.B * a.T * a.Hq;
    if (waves == 0) return PKV_OK;
    if ((waves + 3) / 4 > 0x7fffffffLL) return PKV_ERR_SHAPE;
    const int grid = (int)((waves + 3) / 4);
    if (a.D == 128) hipLaunchKernelGGL((rows_kernel<128>), dim3(grid), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((rows_kernel<64>), dim3(grid), dim3(256), 0, stream, a);
    return launch_status();
}

}  // namespace pkv
