/*
 * oracle.c -- plain, slow fp64 CPU oracle for attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes (per request r, query head h, query row i), following the
 * FlashInfer sink-attention test reference (page "sink_attention_reference.py":
 * functions sink_softmax and sink_attention_unified, varlen and incremental
 * branches) and the argument conventions of the Transformers "paged attention"
 * doc page (varlen path: cu_seq_lens_q/k; decode path: block_table and
 * cache_seqlens):
 *
 *   G = Hq / Hkv, kv head g = h / G               (repeat_interleave grouping)
 *   p = Lk - Lq + i                               (queries are the last Lq positions)
 *   visible j: 0 <= j < Lk, j <= p (causal; no upper bound otherwise),
 *              and (w < 0 or j >= p - w)
 *   s_j   = sm_scale * sum_d q[d] * K(j)[d]       (fp64)
 *           + slope[h] * (j - p)                   (ALiBi, when slopes are given:
 *             vLLM page "attention.py", PagedAttentionWithALiBi.set_attn_bias --
 *             the per-head slope times key position minus query position,
 *             added to the scaled logits under the causal mask; computed from
 *             the exact integer distance)
 *   sigma = sink[h], a logit in scaled units, never multiplied by sm_scale;
 *           -inf when no sink is given
 *   M = max({s_j} U {sigma}),  Z = sum_j exp(s_j - M) + exp(sigma - M)
 *   o = sum_j exp(s_j - M) V(j) / Z,  lse = M + ln Z
 *   a row with no visible key and no sink: o = 0, lse = -inf
 *
 * Two explicit passes (max, then sums) over an explicit visible-key list; no
 * tiling, no online rescaling.  Stored values are read exactly (fp32 or bf16
 * bit patterns) and widened to double before any arithmetic.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1 };

static double load_elem(const void *base, size_t idx, int dtype)
{
    if (dtype == ORC_F32)
        return (double)((const float *)base)[idx];
    /* bf16: the 16 stored bits are the upper half of an fp32 pattern */
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Physical token row of logical position j through one block-table row
 * (decode path of the paged-attention doc: row b lists the request's blocks
 * in logical order). */
long long oracle_slot_of(const int32_t *block_table_row, int pos, int block_size)
{
    return (long long)block_table_row[pos / block_size] * block_size + pos % block_size;
}

/* Request that owns packed token t given cumulative lengths cu[0..B]:
 * the r with cu[r] <= t < cu[r+1] (varlen path of the paged-attention doc).
 * Empty requests own no token.  Writes -1 for t outside [cu[0], cu[B]). */
void oracle_token_request(const int32_t *cu, int B, int T, int32_t *out)
{
    for (int t = 0; t < T; ++t) {
        out[t] = -1;
        for (int r = 0; r < B; ++r)
            if (cu[r] <= t && t < cu[r + 1]) { out[t] = r; break; }
    }
}

/* One query row against an explicit list of visible key rows.
 * krow[n] is the element offset of key row n (the same offset addresses V).
 * Writes o[0..D) and *lse. */
static void attend_row(double *o, double *lse, const void *qbase, size_t qoff,
                       const void *kbase, const void *vbase, const size_t *krow,
                       const int *js, int nvis, int p, double slope, int D, int dtype,
                       double sm_scale, double sigma, double *s)
{
    /* pass 1: logits and their maximum, sink included */
    double M = sigma;
    for (int n = 0; n < nvis; ++n) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += load_elem(qbase, qoff + d, dtype) * load_elem(kbase, krow[n] + d, dtype);
        s[n] = sm_scale * acc + slope * (double)(js[n] - p);
        if (s[n] > M) M = s[n];
    }
    if (M == -INFINITY) {          /* nothing visible and no sink */
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        *lse = -INFINITY;
        return;
    }
    /* pass 2: denominator (the sink joins it, with no value row) and output */
    double Z = exp(sigma - M);
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int n = 0; n < nvis; ++n) {
        double e = exp(s[n] - M);
        Z += e;
        for (int d = 0; d < D; ++d)
            o[d] += e * load_elem(vbase, krow[n] + d, dtype);
    }
    for (int d = 0; d < D; ++d) o[d] /= Z;
    *lse = M + log(Z);
}

/* Visible logical keys of a query at absolute position p among Lk keys.
 * causal: keys after the query are hidden (j <= p).  Non-causal (FlashInfer
 * page, sink_attention_unified, the non-causal branches): every key is a
 * candidate and a window only bounds the left side, p - window_left <= j. */
static int visible_keys(int Lk, int p, int causal, int window_left, int lo, int hi, int *js)
{
    int n = 0;
    for (int j = 0; j < Lk; ++j) {
        if (causal && j > p) continue;
        if (window_left >= 0 && j < p - window_left) continue;
        if (j < lo || j >= hi) continue;      /* partition restriction */
        js[n++] = j;
    }
    return n;
}

/* ------------------------------------------------------------------------ */
/* A tiny thread pool: units [0, nunits) split round-robin over threads.    */

typedef void (*unit_fn)(void *ctx, int unit, double *s, size_t *krow, int *js);

typedef struct {
    unit_fn fn; void *ctx; int nunits, tid, nthreads, maxk;
} worker_arg;

static void *worker(void *p)
{
    worker_arg *a = (worker_arg *)p;
    int mk = a->maxk > 0 ? a->maxk : 1;
    double *s = (double *)malloc(sizeof(double) * mk);
    size_t *krow = (size_t *)malloc(sizeof(size_t) * mk);
    int *js = (int *)malloc(sizeof(int) * mk);
    for (int u = a->tid; u < a->nunits; u += a->nthreads)
        a->fn(a->ctx, u, s, krow, js);
    free(s); free(krow); free(js);
    return NULL;
}

static void run_units(unit_fn fn, void *ctx, int nunits, int nthreads, int maxk)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nunits) nthreads = nunits > 0 ? nunits : 1;
    pthread_t th[256];
    worker_arg args[256];
    if (nthreads > 256) nthreads = 256;
    for (int t = 0; t < nthreads; ++t) {
        args[t] = (worker_arg){fn, ctx, nunits, t, nthreads, maxk};
        if (t == 0) continue;
        pthread_create(&th[t], NULL, worker, &args[t]);
    }
    worker(&args[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------ */
/* Paged decode: one query per sequence, Lq = 1, Lk = cache_seqlens[b],     */
/* the query at position Lk - 1.  With partition_size > 0 the visible set   */
/* is restricted to [p*P, (p+1)*P) and the sink is left out (a partition    */
/* result); the caller merges partitions with oracle_merge.                 */

typedef struct {
    double *out, *lse;
    const void *q, *kc, *vc;
    const int32_t *bt, *seqlens;
    const float *sink, *alibi;
    int B, Hq, Hkv, D, bs, mbps, window, dtype, part, nparts;
    double scale;
    const int32_t *units;
} decode_ctx;

static void decode_unit(void *vctx, int u, double *s, size_t *krow, int *js)
{
    decode_ctx *c = (decode_ctx *)vctx;
    int id = c->units ? c->units[u] : u;          /* (b*Hq + h) * nparts + p */
    int p = id % c->nparts;
    int bh = id / c->nparts;
    int b = bh / c->Hq, h = bh % c->Hq;
    int G = c->Hq / c->Hkv, g = h / G;
    int Lk = c->seqlens[b];
    int lo = 0, hi = Lk;
    if (c->part > 0) { lo = p * c->part; hi = lo + c->part; }
    int n = visible_keys(Lk, Lk - 1, 1, c->window, lo, hi, js);
    for (int t = 0; t < n; ++t) {
        long long row = oracle_slot_of(c->bt + (size_t)b * c->mbps, js[t], c->bs);
        krow[t] = ((size_t)row * c->Hkv + g) * c->D;
    }
    double sigma = (c->part > 0 || !c->sink) ? -INFINITY : (double)c->sink[h];
    double slope = c->alibi ? (double)c->alibi[h] : 0.0;
    attend_row(c->out + (size_t)id * c->D, c->lse + id, c->q, (size_t)bh * c->D,
               c->kc, c->vc, krow, js, n, Lk - 1, slope, c->D, c->dtype, c->scale, sigma, s);
}

/* out [B,Hq,D] / lse [B,Hq] (partition_size == 0) or
 * out [B,Hq,nparts,D] / lse [B,Hq,nparts] (partition_size > 0).
 * units: NULL for all, else a list of flat unit ids to compute. */
int oracle_paged_decode(double *out, double *lse, const void *q, const void *k_cache,
                        const void *v_cache, const int32_t *block_table,
                        const int32_t *cache_seqlens, const float *sink, const float *alibi,
                        int B, int Hq, int Hkv, int D, int block_size, int max_blocks_per_seq,
                        double sm_scale, int window_left, int partition_size, int nparts,
                        int dtype, const int32_t *units, int nunits, int nthreads)
{
    if (Hkv <= 0 || Hq % Hkv || block_size <= 0 || D <= 0) return 1;
    if (partition_size <= 0) nparts = 1;
    decode_ctx c = {out, lse, q, k_cache, v_cache, block_table, cache_seqlens, sink, alibi,
                    B, Hq, Hkv, D, block_size, max_blocks_per_seq, window_left, dtype,
                    partition_size > 0 ? partition_size : 0, nparts, sm_scale, units};
    int maxk = 1;
    for (int b = 0; b < B; ++b) if (cache_seqlens[b] > maxk) maxk = cache_seqlens[b];
    int total = units ? nunits : B * Hq * nparts;
    run_units(decode_unit, &c, total, nthreads, maxk);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Varlen causal prefill.  Request r has Lq = cu_q[r+1]-cu_q[r] queries and */
/* Lk = cu_k[r+1]-cu_k[r] keys.  K/V are contiguous (k,v non-NULL: row      */
/* cu_k[r]+j) or paged (k_cache/v_cache through block_table row r).        */

typedef struct {
    double *out, *lse;
    const void *q, *k, *v, *kc, *vc;
    const int32_t *bt, *cu_q, *cu_k, *tok_req;
    const float *sink, *alibi;
    int B, Hq, Hkv, D, bs, mbps, window, causal, dtype;
    double scale;
    const int32_t *units;
} prefill_ctx;

static void prefill_unit(void *vctx, int u, double *s, size_t *krow, int *js)
{
    prefill_ctx *c = (prefill_ctx *)vctx;
    int id = c->units ? c->units[u] : u;          /* t*Hq + h */
    int t = id / c->Hq, h = id % c->Hq;
    int r = c->tok_req[t];
    int G = c->Hq / c->Hkv, g = h / G;
    int Lq = c->cu_q[r + 1] - c->cu_q[r], Lk = c->cu_k[r + 1] - c->cu_k[r];
    int i = t - c->cu_q[r];
    int p = Lk - Lq + i;
    int n = visible_keys(Lk, p, c->causal, c->window, 0, Lk, js);
    const void *kb = c->k ? c->k : c->kc, *vb = c->k ? c->v : c->vc;
    for (int m = 0; m < n; ++m) {
        long long row = c->k ? (long long)c->cu_k[r] + js[m]
                             : oracle_slot_of(c->bt + (size_t)r * c->mbps, js[m], c->bs);
        krow[m] = ((size_t)row * c->Hkv + g) * c->D;
    }
    double sigma = c->sink ? (double)c->sink[h] : -INFINITY;
    double slope = c->alibi ? (double)c->alibi[h] : 0.0;
    attend_row(c->out + (size_t)id * c->D, c->lse + id, c->q, (size_t)id * c->D, kb, vb,
               krow, js, n, p, slope, c->D, c->dtype, c->scale, sigma, s);
}

/* out [sumLq,Hq,D], lse [sumLq,Hq]; causal 1 or 0 (no upper bound on the
 * visible keys). */
int oracle_varlen_prefill(double *out, double *lse, const void *q, const void *k, const void *v,
                          const void *k_cache, const void *v_cache, const int32_t *block_table,
                          int block_size, int max_blocks_per_seq, const int32_t *cu_q,
                          const int32_t *cu_k, int B, int Hq, int Hkv, int D, double sm_scale,
                          int causal, int window_left, const float *sink, const float *alibi,
                          int dtype, const int32_t *units, int nunits, int nthreads)
{
    if (Hkv <= 0 || Hq % Hkv || D <= 0 || B < 0) return 1;
    int T = cu_q[B] - cu_q[0];
    int32_t *tok_req = (int32_t *)malloc(sizeof(int32_t) * (T > 0 ? T : 1));
    oracle_token_request(cu_q, B, T, tok_req);
    int maxk = 1;
    for (int r = 0; r < B; ++r) if (cu_k[r + 1] - cu_k[r] > maxk) maxk = cu_k[r + 1] - cu_k[r];
    prefill_ctx c = {out, lse, q, k, v, k_cache, v_cache, block_table, cu_q, cu_k, tok_req, sink,
                     alibi,
                     B, Hq, Hkv, D, block_size, max_blocks_per_seq, window_left, causal ? 1 : 0,
                     dtype, sm_scale, units};
    run_units(prefill_unit, &c, units ? nunits : T * Hq, nthreads, maxk);
    free(tok_req);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Split-KV merge: combine partition results (each normalised over its own  */
/* visible keys, sink excluded) and the sink once:                          */
/*   LSE = log( sum_p exp(part_lse_p) + exp(sigma) )                        */
/*   out = sum_p exp(part_lse_p - LSE) * part_out_p                         */
/* Partitions p < nparts_b take part; -inf partitions contribute nothing.   */
int oracle_merge(double *out, double *lse, const double *part_out, const double *part_lse,
                 const int32_t *nparts_per_seq, const float *sink, int B, int Hq, int D,
                 int max_parts)
{
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hq; ++h) {
            const double *pl = part_lse + ((size_t)b * Hq + h) * max_parts;
            const double *po = part_out + ((size_t)b * Hq + h) * max_parts * D;
            double *o = out + ((size_t)b * Hq + h) * D;
            double sigma = sink ? (double)sink[h] : -INFINITY;
            int np = nparts_per_seq[b];
            double M = sigma;
            for (int p = 0; p < np; ++p) if (pl[p] > M) M = pl[p];
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            if (M == -INFINITY) { lse[(size_t)b * Hq + h] = -INFINITY; continue; }
            double Z = exp(sigma - M);
            for (int p = 0; p < np; ++p) Z += exp(pl[p] - M);
            double L = M + log(Z);
            for (int p = 0; p < np; ++p) {
                if (pl[p] == -INFINITY) continue;
                double wgt = exp(pl[p] - L);
                for (int d = 0; d < D; ++d) o[d] += wgt * po[(size_t)p * D + d];
            }
            lse[(size_t)b * Hq + h] = L;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* reshape_and_cache: for each token t with slot s = slot_mapping[t] >= 0,  */
/* copy the [Hkv, D] rows of key[t] / value[t] byte for byte into row s of  */
/* the paged caches ([num_blocks*block_size, Hkv, D] viewed flat).  A       */
/* negative slot is skipped (a padding token).                              */
int oracle_reshape_and_cache(const void *key, const void *value, void *k_cache, void *v_cache,
                             const int32_t *slot_mapping, int T, int Hkv, int D, int block_size,
                             int num_blocks, int elem_bytes)
{
    size_t row = (size_t)Hkv * D * elem_bytes;
    for (int t = 0; t < T; ++t) {
        int s = slot_mapping[t];
        if (s < 0) continue;
        if ((long long)s >= (long long)num_blocks * block_size) return 2;
        int blk = s / block_size, off = s % block_size;
        size_t dst = ((size_t)blk * block_size + off) * row;
        memcpy((char *)k_cache + dst, (const char *)key + (size_t)t * row, row);
        memcpy((char *)v_cache + dst, (const char *)value + (size_t)t * row, row);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Vertical + slash sparse prefill (nano-vllm "minference.py" page,          */
/* MInferencePolicy: estimate_pattern returns per head a set of key          */
/* positions, vertical_indices, and a set of diagonal offsets,               */
/* slash_indices, where a query at position i and a key at position j lie    */
/* on diagonal i - j; sparse_prefill_attention converts them into a block    */
/* form with block_size_M = block_size_N = 64 before attending).  The page   */
/* does not print the conversion.  Reading taken here: row block m holds     */
/* rows [64m, min(64m + 64, L)); key block n holds keys [64n, 64n + 64).     */
/* Key block n is a slash block of row block m when some diagonal s of the   */
/* head meets it within m's rows: i - s lies in block n for a row i of m,    */
/* with 0 <= i - s.  A vertical column v (v < L, v <= m's last row) is       */
/* listed for m when its key block is not a slash block of m.  Attention     */
/* for row i of m then covers the keys j <= i of m's slash blocks and the    */
/* listed columns j <= i.                                                    */
/*                                                                           */
/* Per request b (L = cu[b+1] - cu[b]), head h, row block m < NM:            */
/*   block_count[b,h,m], block_offset[b,h,m, 0..count) = 64n ascending;     */
/*   column_count[b,h,m], column_index[b,h,m, 0..count) in the order the     */
/*   vertical indices are given.  Row blocks at or past L have no entries.  */
/* vertical [B,H,NV], slash [B,H,NS]; entries outside [0, L) are ignored.   */
int oracle_vertical_slash_blocks(int32_t *block_count, int32_t *block_offset,
                                 int32_t *column_count, int32_t *column_index,
                                 const int32_t *vertical, const int32_t *slash,
                                 const int32_t *cu, int B, int H, int NV, int NS, int NM)
{
    char *sel = (char *)malloc(NM > 0 ? (size_t)NM : 1);
    for (int b = 0; b < B; ++b) {
        int L = cu[b + 1] - cu[b];
        for (int h = 0; h < H; ++h) {
            const int32_t *S = slash + ((size_t)b * H + h) * NS;
            const int32_t *V = vertical + ((size_t)b * H + h) * NV;
            for (int m = 0; m < NM; ++m) {
                size_t bhm = ((size_t)b * H + h) * NM + m;
                int r0 = 64 * m, r1 = 64 * m + 64 < L ? 64 * m + 64 : L;   /* rows [r0, r1) */
                memset(sel, 0, (size_t)NM);
                int nb = 0, nc = 0;
                if (r0 < L) {
                    for (int t = 0; t < NS; ++t) {
                        int s = S[t];
                        if (s < 0 || s >= L) continue;
                        int lo = r0 - s, hi = r1 - 1 - s;     /* keys of diagonal s */
                        if (hi < 0) continue;
                        if (lo < 0) lo = 0;
                        for (int n = lo / 64; n <= hi / 64; ++n) sel[n] = 1;
                    }
                    for (int n = 0; n < NM; ++n)
                        if (sel[n]) block_offset[bhm * NM + nb++] = 64 * n;
                    for (int t = 0; t < NV; ++t) {
                        int v = V[t];
                        if (v < 0 || v >= L || v > r1 - 1) continue;
                        if (sel[v / 64]) continue;
                        column_index[bhm * NV + nc++] = v;
                    }
                }
                block_count[bhm] = nb;
                column_count[bhm] = nc;
            }
        }
    }
    free(sel);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention under an explicit mask (self-attention prefill, Lq = Lk = L    */
/* per request, packed by cu): query row t (request r, row i = t - cu[r])   */
/* of head h sees exactly the keys j < L whose bit is set in its mask row,  */
/* mask[(u * W) + j / 64] bit j % 64, u = the unit's index in `units` (or   */
/* t * Hq + h without units).  Logits, sink and normalisation as above;      */
/* nothing is implied by position (no causal bound of its own).             */

typedef struct {
    double *out, *lse;
    const void *q, *k, *v;
    const int32_t *cu, *tok_req;
    const uint64_t *mask;
    const float *sink;
    int Hq, Hkv, D, W, dtype;
    double scale;
    const int32_t *units;
} masked_ctx;

static void masked_unit(void *vctx, int u, double *s, size_t *krow, int *js)
{
    masked_ctx *c = (masked_ctx *)vctx;
    int id = c->units ? c->units[u] : u;          /* t*Hq + h */
    int t = id / c->Hq, h = id % c->Hq;
    int r = c->tok_req[t];
    int G = c->Hq / c->Hkv, g = h / G;
    int L = c->cu[r + 1] - c->cu[r];
    const uint64_t *row = c->mask + (size_t)u * c->W;
    int n = 0;
    for (int j = 0; j < L && j < 64 * c->W; ++j) {
        if (!((row[j / 64] >> (j % 64)) & 1u)) continue;
        js[n] = j;
        krow[n] = ((size_t)(c->cu[r] + j) * c->Hkv + g) * c->D;
        ++n;
    }
    double sigma = c->sink ? (double)c->sink[h] : -INFINITY;
    attend_row(c->out + (size_t)id * c->D, c->lse + id, c->q, (size_t)id * c->D, c->k, c->v,
               krow, js, n, t - c->cu[r], 0.0, c->D, c->dtype, c->scale, sigma, s);
}

/* out [T,Hq,D], lse [T,Hq] for the rows computed (all, or `units`). */
int oracle_masked_prefill(double *out, double *lse, const void *q, const void *k, const void *v,
                          const int32_t *cu, int B, int Hq, int Hkv, int D, double sm_scale,
                          const uint64_t *mask, int W, const float *sink, int dtype,
                          const int32_t *units, int nunits, int nthreads)
{
    if (Hkv <= 0 || Hq % Hkv || D <= 0 || B < 0 || W < 0) return 1;
    int T = cu[B] - cu[0];
    int32_t *tok_req = (int32_t *)malloc(sizeof(int32_t) * (T > 0 ? T : 1));
    oracle_token_request(cu, B, T, tok_req);
    int maxk = 1;
    for (int r = 0; r < B; ++r) if (cu[r + 1] - cu[r] > maxk) maxk = cu[r + 1] - cu[r];
    masked_ctx c = {out, lse, q, k, v, cu, tok_req, mask, sink, Hq, Hkv, D, W, dtype, sm_scale,
                    units};
    run_units(masked_unit, &c, units ? nunits : T * Hq, nthreads, maxk);
    free(tok_req);
    return 0;
}
