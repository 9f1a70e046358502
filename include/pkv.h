/*
 * pkv.h -- C ABI of libpkv.so: attention over a paged KV cache on AMD
 * Instinct MI355X (gfx950).
 *
 * Four operations, named after the pages that state the problem:
 *
 *   pkv_reshape_and_cache   store new K/V rows into cache slots
 *                           (vLLM "attention.py" page, PagedAttention.forward:
 *                           the cache_ops.reshape_and_cache call and its
 *                           slot_mapping argument)
 *   pkv_rope_cos_sin,       rotary position embedding: the cos/sin table,
 *   pkv_rope_apply,         in-place rotation of rows by their positions, and
 *   pkv_reshape_and_cache_rope  the cache store with the key rotated as it
 *                           is written (vLLM page, PagedAttentionWithRoPE)
 *   pkv_paged_decode        one query token per sequence over a paged cache
 *                           (Transformers "Paged attention" doc, decode path:
 *                           block_table and cache_seqlens; vLLM page,
 *                           single_query_cached_kv_attention)
 *   pkv_paged_decode_append store each sequence's new K/V token into the cache
 *                           and attend to it in the same call (Transformers
 *                           doc, flash_attn_with_kvcache: the cache is
 *                           "updated in place" at cache_seqlens)
 *   pkv_merge_partitions    log-sum-exp merge of split-KV partition results
 *                           (vLLM page, single_query_cached_kv_attention: the
 *                           partitioned "v2" path with exp_sums / max_logits /
 *                           tmp_output)
 *   pkv_vertical_slash_blocks / pkv_sparse_prefill
 *                           vertical + slash block-sparse prefill (nano-vllm
 *                           minference.py page, MInferencePolicy)
 *   pkv_varlen_prefill      causal or non-causal attention for packed variable-length
 *                           requests (Transformers doc, varlen path:
 *                           cu_seq_lens_q/k and max_length_q/k), over
 *                           contiguous K/V or over the paged cache
 *
 * What every attention call computes (FlashInfer "sink_attention_reference.py"
 * page, sink_softmax and sink_attention_unified): for request r with Lq
 * queries and Lk keys, query row i sits at absolute position p = Lk - Lq + i
 * and sees key j iff 0 <= j <= p and (window_left < 0 or j >= p - window_left);
 * a non-causal prefill (same page, the non-causal branches) drops j <= p, so
 * row i sees every key j < Lk with (window_left < 0 or j >= p - window_left).
 * Query head h reads kv head h / (Hq / Hkv).  Logits are sm_scale * q.k;
 * the optional per-query-head sink is one more logit, NOT multiplied by
 * sm_scale, that joins the softmax denominator and has no value row.  A row
 * with no visible key gets output 0 (its lse is the sink, or -inf without one).
 * lse, when requested, is the natural-log log-sum-exp of the row's logits
 * including the sink.
 *
 * ALiBi (vLLM page "attention.py", PagedAttentionWithALiBi: a per-head slope
 * times key position minus query position, added to the scaled logits):
 * every call that computes logits takes alibi_slopes, float32 [num_q_heads]
 * or NULL for none; with slopes, the logit of key j for a query at position
 * p is sm_scale * q.k_j + alibi_slopes[h] * (j - p).  The sink is not biased.
 *
 * Conventions for every entry point:
 *   - Array arguments are DEVICE pointers owned by the caller; the library
 *     allocates nothing and never prints.  Its only host state is a cached
 *     compute-unit count per device, a once-per-process kernel attribute and
 *     a per-process call counter that tags the fused merge's counters.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the legacy
 *     default stream) and the call returns without waiting; results are
 *     valid in stream order.
 *   - q, k, v, the caches and out share one dtype (pkv_dtype); sink, lse and
 *     split-KV partials are always float32; index arrays are int32.
 *   - Output dtype is the input dtype; bf16 results are rounded to nearest
 *     even from float32 accumulators.
 *   - Arguments are checked on the host before anything is launched; a bad
 *     argument returns an error status and launches nothing.  sm_scale must
 *     be positive and finite (PKV_ERR_SHAPE otherwise).  Device-resident
 *     index data (block_table entries, cache_seqlens, cu_seqlens, slots) is
 *     NOT checked, since that would need a device-to-host copy: it is a
 *     caller contract (see each function), and violating it is undefined.
 *   - out/lse/workspace must not alias any input.
 *
 * Cache layout (both caches): [num_blocks, block_size, num_kv_heads,
 * head_dim], contiguous, token-major like the packed [tokens, heads, dim]
 * activations.  Logical token j of sequence b lives in physical block
 * block_table[b * max_blocks_per_seq + j / block_size] at offset
 * j % block_size.  Entries of block_table past the ones a sequence needs are
 * never read (they may hold -1).
 *
 * Supported: head_dim in {64, 128}; block_size a power of two in [8, 512];
 * num_q_heads a multiple of num_kv_heads; dtype PKV_F32 or PKV_BF16.  The
 * bf16 decode kernels read keys in tiles of 16 tokens: with block_size 8 a
 * tile spans two blocks (read through per-lane addresses instead of one
 * range-checked descriptor), and bf16 partitions must be multiples of 16.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_ERR_NULL = 1,        /* a required pointer is NULL                    */
    PKV_ERR_SHAPE = 2,       /* sizes inconsistent or out of range            */
    PKV_ERR_UNSUPPORTED = 3, /* valid request this library does not implement */
    PKV_ERR_WORKSPACE = 4,   /* workspace missing or too small                */
    PKV_ERR_HIP = 5,         /* a HIP launch failed (hipGetLastError)         */
    PKV_ERR_SCRATCH = 6      /* the call needs more than the static scratch of
                                pkv_paged_decode_noalloc                      */
} pkv_status;

typedef enum pkv_dtype { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Human-readable name of a status code (static storage; never NULL). */
const char *pkv_status_string(pkv_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int pkv_version(void);

/*
 * pkv_reshape_and_cache -- store T new tokens' K and V rows into the paged
 * caches (vLLM page, PagedAttention.forward, cache_ops.reshape_and_cache).
 *
 *   key, value      [T, num_kv_heads, head_dim]; token t starts at element
 *                   t * key_stride (value_stride); a stride of 0 means dense
 *                   (num_kv_heads * head_dim), which allows K and V sliced out
 *                   of a fused QKV buffer.  Strides must be multiples of 8
 *                   elements and the pointers 16-byte aligned.
 *   k_cache,v_cache [num_blocks, block_size, num_kv_heads, head_dim], written
 *                   in place.
 *   slot_mapping    [T] int32: slot s = block * block_size + offset receives
 *                   token t; s < 0 marks a padding token, which is skipped.
 *                   Contract: 0 <= s < num_blocks * block_size and no two
 *                   tokens share a slot.
 * Bytes are copied exactly; no slot other than the listed ones is touched.
 * T == 0 is a no-op.
 */
pkv_status pkv_reshape_and_cache(const void *key, const void *value, void *k_cache,
                                 void *v_cache, const int32_t *slot_mapping, int32_t T,
                                 int64_t key_stride, int64_t value_stride, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                 pkv_dtype dtype, void *stream);

/*
 * Rotary position embedding (vLLM "attention.py" page, PagedAttentionWithRoPE:
 * query and key are rotated by their positions before attention, with
 * rotary_dim, base, is_neox_style and an optional rope_scaling of type
 * "linear" or "dynamic" with a factor).  The pages name the rotation but do
 * not print it; it is the standard rotary embedding: frequency i <
 * rotary_dim / 2 turns by base^(-2i / rotary_dim) per position; neox style
 * (neox != 0) rotates dimension d with d + rotary_dim / 2, the other style
 * 2i with 2i + 1:  x'_a = x_a cos - x_b sin,  x'_b = x_b cos + x_a sin.
 * Dimensions from rotary_dim on are unchanged.
 *
 * pkv_rope_cos_sin -- the table cos_sin [num_positions, rotary_dim] float32:
 * columns [0, rotary_dim/2) hold cos(angle(p, i)), the rest sin(angle(p, i)),
 * computed in double.  scaling 0: angle = p * f_i; 1 (linear): (p / factor) *
 * f_i; 2 (dynamic, NTK-aware): the base becomes base * (factor *
 * num_positions / max_position - (factor - 1))^(rotary_dim / (rotary_dim -
 * 2)) when num_positions > max_position.  rotary_dim even >= 2.
 *
 * pkv_rope_apply -- rotate x [T, num_heads, head_dim] in place, row t by
 * positions[t] (int32, contract: < the table's num_positions); row_stride
 * elements between tokens (0: dense; a multiple of 8).  rotary_dim a
 * multiple of 16 in [16, head_dim]; head_dim 64 or 128.
 *
 * pkv_reshape_and_cache_rope -- pkv_reshape_and_cache with each key row
 * rotated by positions[t] as it is stored (values stored unchanged); the
 * same arguments as pkv_reshape_and_cache plus positions, cos_sin, rotary_dim
 * (as for pkv_rope_apply) and neox.  Rotation runs in float32; bf16 results
 * are rounded to nearest even.
 */
pkv_status pkv_rope_cos_sin(float *cos_sin, int32_t num_positions, int32_t rotary_dim,
                           float base, int32_t scaling, float factor, int32_t max_position,
                           void *stream);
pkv_status pkv_rope_apply(void *x, const int32_t *positions, const float *cos_sin, int32_t T,
                          int32_t num_heads, int32_t head_dim, int64_t row_stride,
                          int32_t rotary_dim, int32_t neox, pkv_dtype dtype, void *stream);
pkv_status pkv_reshape_and_cache_rope(const void *key, const void *value, void *k_cache,
                                      void *v_cache, const int32_t *slot_mapping,
                                      const int32_t *positions, const float *cos_sin, int32_t T,
                                      int64_t key_stride, int64_t value_stride,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int32_t num_blocks, int32_t rotary_dim, int32_t neox,
                                      pkv_dtype dtype, void *stream);

/*
 * pkv_paged_decode_workspace_bytes -- bytes of device workspace a decode call
 * may need, so that the caller can allocate it (vLLM "attention.py" page,
 * single_query_cached_kv_attention: the caller allocates the split-KV
 * buffers tmp_output [num_seqs, num_heads, max_num_partitions, head_size],
 * exp_sums and max_logits before the partitioned kernel runs).  The
 * arguments are those of that allocation: batch, query heads, head_dim, the
 * longest sequence and the partition size (0 or -1: the balanced schedule, in
 * two launches or one).  The result
 * covers every kv-head count that divides num_q_heads, both dtypes and
 * every block size, and does not depend on the sequence lengths (device
 * data).  It is 0 for B == 0 and (size_t)-1 for invalid sizes.  Layout
 * (private to the library; stated so that reuse is safe):
 *   - the first kStreamMaxB * num_q_heads * 8 bytes (256-byte aligned) hold
 *     the balanced schedule's arrival counters; no other mode writes them;
 *   - partition_size 0 or -1 (bf16, B <= 4096): the balanced schedule's
 *     partial results after them, (4 * W + B) * Hq * (head_dim + 1) floats
 *     plus B + 2 ints, W = ceil(compute units / head groups), then room for
 *     q rotated by pkv_paged_decode_append (B * Hq * head_dim bf16);
 *   - partition_size > 0 and max_seqlen_k > partition_size: float32
 *     part_out [B, Hq, P, head_dim] and part_lse [B, Hq, P],
 *     P = ceil(max_seqlen_k / partition_size), after them.
 * pkv_paged_decode_append needs pkv_paged_decode_workspace_bytes(B,
 * num_q_heads, head_dim, max_seqlen_k + 1, 0).
 */
size_t pkv_paged_decode_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t head_dim,
                                        int32_t max_seqlen_k, int32_t partition_size);

/*
 * pkv_paged_decode -- one query token per sequence attending to its
 * cache_seqlens[b] cached keys (Transformers doc, decode path; vLLM page,
 * single_query_cached_kv_attention).  The query sits at position
 * cache_seqlens[b] - 1: a token that is being generated must already have
 * been stored with pkv_reshape_and_cache (write the cache, then attend, the
 * order of PagedAttention.forward).
 *
 *   out             [B, num_q_heads, head_dim]
 *   lse             [B, num_q_heads] float32, or NULL
 *   q               [B, num_q_heads, head_dim]
 *   block_table     [B, max_blocks_per_seq] int32
 *   cache_seqlens   [B] int32.  Contract: 0 <= cache_seqlens[b] <=
 *                   max_seqlen_k <= max_blocks_per_seq * block_size, and the
 *                   first ceil(cache_seqlens[b] / block_size) entries of row b
 *                   are valid block ids < num_blocks.
 *   sink            [num_q_heads] float32, or NULL for none
 *   max_seqlen_k    host upper bound on cache_seqlens (sizes the launch)
 *   window_left     -1 for none, else >= 0
 *   partition_size  > 0: split the keys into [p*P, (p+1)*P) partitions (a
 *                   multiple of block_size, and of 16 in bf16; otherwise
 *                   PKV_ERR_SHAPE), each reduced on its own, then
 *                   merged by log-sum-exp.  0: automatic -- bf16 uses a balanced
 *                   schedule that gives every wave of the device an equal share
 *                   of all sequences' key tiles and merges the pieces the same
 *                   way (B <= 4096), in two launches: the stage launch writes
 *                   each wave's partial result per sequence to the workspace,
 *                   the merge launch combines them (the two calls
 *                   pkv_paged_decode_stage + pkv_paged_decode_finish); fp32
 *                   (and larger B) does not split.  -1: the same schedule in
 *                   one launch, the last wave to finish a (sequence, head
 *                   group) merging its pieces (the same result, bit for bit;
 *                   one launch fewer, a longer tail).  Results are bitwise
 *                   reproducible for fixed arguments on a given device.
 *                   Below -1: PKV_ERR_SHAPE.
 *   workspace       device buffer of at least
 *                   pkv_paged_decode_workspace_bytes(...) bytes (may be NULL
 *                   when that is 0), 256-byte aligned, reused across calls.
 *                   The one-launch balanced schedule (-1) counts the pieces of
 *                   each (sequence, head group) in 64-bit counters at its start,
 *                   tagged with a per-call epoch: a counter left by an
 *                   interrupted call or holding bytes from another use reads
 *                   as zero, and every completed call leaves its counters
 *                   zero.  Zero-fill a new workspace once (so that it holds
 *                   no stale epoch by chance); the fixed-partition modes
 *                   never write the counters.  Calls that share a workspace
 *                   must not overlap in time.
 */
pkv_status pkv_paged_decode(void *out, float *lse, const void *q, const void *k_cache,
                            const void *v_cache, const int32_t *block_table,
                            const int32_t *cache_seqlens, const float *sink, int32_t B,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_seqlen_k, float sm_scale, int32_t window_left,
                            const float *alibi_slopes, int32_t partition_size, void *workspace,
                            size_t workspace_bytes, pkv_dtype dtype, void *stream);

/*
 * pkv_paged_decode_noalloc -- pkv_paged_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The arguments and the result are those of
 * pkv_paged_decode without workspace / workspace_bytes: the workspace is a
 * static device array of PKV_NOALLOC_SCRATCH_BYTES (32 MiB) inside the
 * library, which each device it runs on holds until the process ends.  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library call);
 * the caller still owns every input and output.
 *   - PKV_ERR_SCRATCH (nothing launched) when the call would need more than
 *     PKV_NOALLOC_SCRATCH_BYTES, i.e. when
 *     pkv_paged_decode_workspace_bytes for its arguments exceeds it (for
 *     example very large batches, or a split into many fixed partitions).
 *   - The first call on a device looks up the array's address there and
 *     clears it with a fill kernel on `stream`, ahead of its own work.
 *   - Every call on one device shares that device's array and leaves it as the
 *     last call left it (the merge counters at zero): calls that overlap in
 *     time on one device race and must be serialised, e.g. on one stream.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)
pkv_status pkv_paged_decode_noalloc(void *out, float *lse, const void *q, const void *k_cache,
                                    const void *v_cache, const int32_t *block_table,
                                    const int32_t *cache_seqlens, const float *sink, int32_t B,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks,
                                    int32_t max_blocks_per_seq, int32_t max_seqlen_k,
                                    float sm_scale, int32_t window_left,
                                    const float *alibi_slopes, int32_t partition_size,
                                    pkv_dtype dtype, void *stream);

/*
 * pkv_paged_decode_append -- decode with the new token appended in the same
 * call (Transformers doc, flash_attn_with_kvcache: k and v are written into
 * the cache at index cache_seqlens[b], the cache is updated in place, and the
 * query attends to the cache including the new token; the doc's example puts
 * the new tokens of lengths 30 / 32 / 70 at slots 94 / 32 / 198 with
 * block_size 32).  For each sequence b with L = cache_seqlens[b] tokens
 * already cached: k_new[b] / v_new[b] are stored at position L (slot
 * block_table[b][L / block_size] * block_size + L % block_size), and the
 * query, at position L, attends to keys 0..L (window: L - window_left <= j)
 * with the sink -- exactly pkv_reshape_and_cache of the new rows followed by
 * pkv_paged_decode over cache_seqlens[b] + 1 keys, in one call.
 *
 *   k_new, v_new    [B, num_kv_heads, head_dim], same dtype as the caches
 *   k_cache,        written at the new tokens' slots and nowhere else
 *   v_cache
 *   cache_seqlens   [B] int32, NOT modified (the caller advances it).
 *                   Contract: 0 <= cache_seqlens[b] <= max_seqlen_k, the
 *                   first cache_seqlens[b] / block_size + 1 entries of row b
 *                   are valid block ids < num_blocks, and no other sequence
 *                   of the call reads the slot of position cache_seqlens[b].
 *   max_seqlen_k    host upper bound on cache_seqlens; max_seqlen_k + 1 <=
 *                   max_blocks_per_seq * block_size
 *   rope_cos_sin    NULL, or a pkv_rope_cos_sin table of rope_positions rows
 *                   (>= max_seqlen_k + 1) with rotary_dim (a multiple of 32
 *                   in [32, head_dim]) and rope_neox as for pkv_rope_apply:
 *                   q and k_new are then rotated by the new token's position
 *                   cache_seqlens[b] inside the call (vLLM page,
 *                   PagedAttentionWithRoPE.forward: query and key rotated
 *                   before attention), the rotated key is what the cache
 *                   receives, and q itself is not modified.  The cached keys
 *                   must already be rotated (pkv_reshape_and_cache_rope).
 *                   Equal to pkv_rope_apply on q and k_new followed by this
 *                   call without a table.
 *   workspace       bf16: at least pkv_paged_decode_workspace_bytes(B,
 *                   num_q_heads, head_dim, max_seqlen_k + 1, 0) bytes,
 *                   reused under the same rules as pkv_paged_decode's
 *                   balanced schedule (B <= 4096); fp32: none (may be NULL).
 * Other arguments as for pkv_paged_decode.  bf16 runs the balanced schedule
 * as two launches, like pkv_paged_decode's default: the stage launch (the
 * wave that reads a sequence's last tile stores its new row first) and the
 * merge launch; fp32 runs one wave per (sequence, head).  Returns
 * PKV_ERR_SHAPE for B > 4096 in bf16 or when the new token does not fit.
 */
pkv_status pkv_paged_decode_append(void *out, float *lse, const void *q, const void *k_new,
                                   const void *v_new, void *k_cache, void *v_cache,
                                   const int32_t *block_table, const int32_t *cache_seqlens,
                                   const float *sink, int32_t B, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t num_blocks, int32_t max_blocks_per_seq,
                                   int32_t max_seqlen_k, float sm_scale, int32_t window_left,
                                   const float *alibi_slopes, const float *rope_cos_sin,
                                   int32_t rope_positions, int32_t rotary_dim, int32_t rope_neox,
                                   void *workspace, size_t workspace_bytes, pkv_dtype dtype,
                                   void *stream);

/*
 * The two launches of pkv_paged_decode with partition_size == 0 in bf16 (the
 * balanced schedule), as separate calls for callers that want to time or
 * overlap them; pkv_paged_decode(partition_size = 0) is exactly these two:
 *   pkv_paged_decode_stage   every wave of the device takes an equal share of
 *                            all sequences' key tiles and writes one partial
 *                            result (normalised output + lse, sink left out)
 *                            per sequence it touches into `workspace`;
 *   pkv_paged_decode_finish  log-sum-exp merge of those pieces with the sink
 *                            into out / lse (same formula as
 *                            pkv_merge_partitions).
 * Arguments mean what they mean for pkv_paged_decode; `workspace` must hold
 * pkv_paged_decode_workspace_bytes(B, num_q_heads, head_dim, max_seqlen_k, 0) bytes,
 * and finish must run after stage (stream order) with the same B,
 * num_q_heads, num_kv_heads, head_dim and workspace.  The workspace layout is
 * private to the library.  dtype must be PKV_BF16 and B <= 4096.
 */
pkv_status pkv_paged_decode_stage(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_table, const int32_t *cache_seqlens,
                                  int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_seqlen_k, float sm_scale,
                                  int32_t window_left, const float *alibi_slopes, void *workspace,
                                  size_t workspace_bytes, pkv_dtype dtype, void *stream);
pkv_status pkv_paged_decode_finish(void *out, float *lse, const float *sink, int32_t B,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   const void *workspace, size_t workspace_bytes,
                                   pkv_dtype dtype, void *stream);

/*
 * pkv_paged_decode_partitions -- the first stage of split-KV decode (vLLM
 * page, the paged_attention_v2 path that fills tmp_output / exp_sums /
 * max_logits): for every sequence b, query head h and partition
 * p < max_partitions, attention restricted to the visible keys in
 * [p * partition_size, (p + 1) * partition_size), WITHOUT the sink:
 *     part_out[b,h,p,:] = that partition's normalised output (0 if no key)
 *     part_lse[b,h,p]   = ln of its softmax denominator (-inf if no key)
 * pkv_merge_partitions then adds the sink once and combines them.
 * pkv_paged_decode with partition_size > 0 is exactly these two calls.
 *
 *   part_out        [B, num_q_heads, max_partitions, head_dim] float32
 *   part_lse        [B, num_q_heads, max_partitions] float32
 *   max_partitions  >= ceil(max_seqlen_k / partition_size)
 *   other arguments as for pkv_paged_decode (partition_size > 0, a multiple
 *   of block_size).
 */
pkv_status pkv_paged_decode_partitions(float *part_out, float *part_lse, const void *q,
                                       const void *k_cache, const void *v_cache,
                                       const int32_t *block_table, const int32_t *cache_seqlens,
                                       int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t max_blocks_per_seq, int32_t max_seqlen_k,
                                       float sm_scale, int32_t window_left,
                                       const float *alibi_slopes, int32_t partition_size,
                                       int32_t max_partitions, pkv_dtype dtype, void *stream);

/*
 * pkv_merge_partitions -- combine split-KV partition results (vLLM page, the
 * paged_attention_v2 path): for (b, h), with n_b = ceil(cache_seqlens[b] /
 * partition_size) partitions and sink s (or -inf),
 *     LSE = log(sum_{p < n_b} exp(part_lse[b,h,p]) + exp(s))
 *     out = sum_{p < n_b} exp(part_lse[b,h,p] - LSE) * part_out[b,h,p,:]
 * A partition with part_lse = -inf (no visible key) contributes nothing;
 * entries p >= n_b are never read.  If every term is -inf, out = 0 and
 * lse = -inf.
 *
 *   part_out        [B, num_q_heads, max_partitions, head_dim] float32, each
 *                   row normalised over its own partition
 *   part_lse        [B, num_q_heads, max_partitions] float32, natural log,
 *                   sink excluded
 *   cache_seqlens   [B] int32.  Contract: ceil(cache_seqlens[b] /
 *                   partition_size) <= max_partitions.
 *   out             [B, num_q_heads, head_dim] in dtype; lse [B, Hq] or NULL
 */
pkv_status pkv_merge_partitions(void *out, float *lse, const float *part_out,
                                const float *part_lse, const int32_t *cache_seqlens,
                                int32_t partition_size, const float *sink, int32_t B,
                                int32_t num_q_heads, int32_t head_dim, int32_t max_partitions,
                                pkv_dtype dtype, void *stream);

/*
 * pkv_varlen_prefill -- attention over packed variable-length requests
 * (Transformers doc, varlen path; FlashInfer page, varlen branch).
 *
 *   out             [sum Lq, num_q_heads, head_dim]
 *   lse             [sum Lq, num_q_heads] float32, or NULL
 *   q               [sum Lq, num_q_heads, head_dim]
 *   K/V, one of:
 *     contiguous    k, v [sum Lk, num_kv_heads, head_dim]; request r's key j
 *                   is row cu_seqlens_k[r] + j.  k_cache/v_cache/block_table
 *                   must be NULL.
 *     paged         k = v = NULL; k_cache, v_cache and block_table
 *                   [B, max_blocks_per_seq] as for pkv_paged_decode; request
 *                   r's key j is at block_table[r][j / block_size], offset
 *                   j % block_size; cu_seqlens_k still gives Lk per request.
 *   cu_seqlens_q/k  [B + 1] int32 exclusive prefix sums starting at 0.
 *                   Contract: nondecreasing; every Lq <= max_seqlen_q and
 *                   Lk <= max_seqlen_k (host upper bounds that size the
 *                   launch); paged: Lk <= max_blocks_per_seq * block_size.
 *   causal          1: row i at position p = Lk - Lq + i (queries are the
 *                   last Lq positions of the request's keys) sees keys j <= p;
 *                   0: it sees every key of the request.  A window (window_left
 *                   >= 0) bounds the left side in both, j >= p - window_left.
 *                   Other values: PKV_ERR_SHAPE.
 *   rope_cos_sin    NULL, or a pkv_rope_cos_sin table of rope_positions rows
 *                   (>= max_seqlen_k): q is then rotated by its position p =
 *                   Lk - Lq + i as it is loaded, with rotary_dim (a multiple
 *                   of 32 in [32, head_dim]) and rope_neox as for
 *                   pkv_rope_apply.  Rows at a negative position (Lq > Lk)
 *                   are not rotated.
 *   rope_k          0: the keys are already rotated (for example stored with
 *                   pkv_reshape_and_cache_rope; always so for paged keys).
 *                   1 (contiguous K and a table only): key j is rotated by
 *                   its position j before attention (vLLM page,
 *                   PagedAttentionWithRoPE.forward rotates query and key
 *                   before attention); k itself is not modified.  The
 *                   rotated keys are rounded to bf16 as pkv_rope_apply
 *                   would store them.  bfloat16 with a workspace: the keys
 *                   are rotated once into it by a first launch and attended
 *                   from there; without one, each workgroup of the attention
 *                   kernel rotates the key tiles it loads, in LDS (no
 *                   workspace, but every tile is rotated once per workgroup
 *                   that reads it, which costs more on long requests).
 *                   Other values: PKV_ERR_SHAPE; 1 with paged keys or
 *                   without a table: PKV_ERR_UNSUPPORTED; 1 with ALiBi
 *                   slopes is supported only through the workspace (else
 *                   PKV_ERR_UNSUPPORTED).
 *   workspace,      NULL / 0, or device memory (16-byte aligned) of at least
 *   workspace_bytes pkv_varlen_prefill_workspace_bytes(B, max_seqlen_k,
 *                   num_kv_heads, head_dim, rope_k, dtype) bytes, owned by
 *                   the caller, used only for bfloat16 with rope_k = 1 (the
 *                   rotated keys, [sum Lk, num_kv_heads, head_dim]); its
 *                   contents need no initialisation and are scratch after
 *                   the call.  Too small: PKV_ERR_WORKSPACE.
 *
 * Errors besides the common ones: PKV_ERR_UNSUPPORTED for bfloat16 with
 * contiguous K/V when max_seqlen_k * num_kv_heads * head_dim * 2 bytes (one
 * request's K rows) reaches 4 GiB; use the paged form for such requests.
 */
pkv_status pkv_varlen_prefill(void *out, float *lse, const void *q, const void *k, const void *v,
                              const void *k_cache, const void *v_cache, const int32_t *block_table,
                              int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                              const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t B,
                              int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                              int32_t causal, int32_t window_left, const float *alibi_slopes,
                              const float *rope_cos_sin, int32_t rope_positions,
                              int32_t rotary_dim, int32_t rope_neox, int32_t rope_k,
                              const float *sink, void *workspace, size_t workspace_bytes,
                              pkv_dtype dtype, void *stream);

/*
 * pkv_varlen_prefill_workspace_bytes -- the workspace pkv_varlen_prefill
 * needs to rotate contiguous keys once (bfloat16, rope_k = 1): room for
 * B * max_seqlen_k key rows, rounded up to 256 bytes; 0 for any other call.
 * (size_t)-1 for a negative B or max_seqlen_k, or no heads.
 */
size_t pkv_varlen_prefill_workspace_bytes(int32_t B, int32_t max_seqlen_k, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t rope_k, pkv_dtype dtype);

/*
 * Vertical + slash sparse prefill (nano-vllm "minference.py" page,
 * MInferencePolicy: estimate_pattern returns, per head, vertical_indices --
 * key positions to keep -- and slash_indices -- diagonal offsets i - j of a
 * query at position i and a key at j -- and sparse_prefill_attention turns
 * them into a block form with block_size_M = block_size_N = 64 before
 * attending).  The page does not print that conversion; this library's block
 * form: row block m of a request holds rows [64m, 64m + 64), key block n
 * keys [64n, 64n + 64).  Key block n is a SLASH BLOCK of m when some diagonal
 * s of the head meets it within m's rows (a key i - s >= 0 in block n for a
 * row i of m); m's COLUMNS are its vertical indices v < L, v <= m's last row,
 * whose key block is not a slash block of m.  Row i of m attends keys j <= i
 * of m's slash blocks and columns (self-attention prefill: Lq = Lk = L per
 * request, queries at positions 0 .. L - 1), with the optional sink in the
 * denominator.  Estimating the pattern is not part of the library.
 *
 * pkv_vertical_slash_blocks -- the block form of every (request, head, row
 * block):
 *   vertical_indices [B, num_heads, num_vertical] int32; the entries of a
 *                    row that lie in [0, L) must be distinct (the page's are
 *                    sorted top-k indices); entries outside [0, L) are
 *                    ignored (padding)
 *   slash_indices    [B, num_heads, num_slash] int32, any order, repeats
 *                    allowed; entries outside [0, L) are ignored
 *   cu_seqlens       [B + 1] int32 prefix sums of the request lengths L,
 *                    each L <= max_seqlen
 *   block_count      [B, num_heads, NM] out, NM = ceil(max_seqlen / 64)
 *   block_offset     [B, num_heads, NM, NM] out: the first key (64n) of each
 *                    slash block, ascending, block_count entries per row
 *   column_count     [B, num_heads, NM] out
 *   column_index     [B, num_heads, NM, num_vertical] out: the columns in the
 *                    order given, column_count entries per row
 * Entries past a count are not written.  Row blocks at or past a request's
 * end get counts 0.  Device pointers, caller-owned; all integers exact.
 *
 * pkv_sparse_prefill -- attention over that block form, bf16 only:
 *   q [sum L, num_q_heads, head_dim], k / v [sum L, num_kv_heads, head_dim]
 *   packed by cu_seqlens; out like q; lse [sum L, num_q_heads] float32 or
 *   NULL; the block form as written by pkv_vertical_slash_blocks for
 *   num_heads = num_q_heads (query head h reads kv head h / (Hq / Hkv)) and
 *   the same max_seqlen / num_vertical.
 * Errors besides the common ones: PKV_ERR_UNSUPPORTED for float32, and when
 * max_seqlen * num_kv_heads * head_dim * 2 bytes (one request's K rows)
 * reaches 4 GiB.
 */
pkv_status pkv_vertical_slash_blocks(int32_t *block_count, int32_t *block_offset,
                                     int32_t *column_count, int32_t *column_index,
                                     const int32_t *vertical_indices,
                                     const int32_t *slash_indices, const int32_t *cu_seqlens,
                                     int32_t B, int32_t num_heads, int32_t num_vertical,
                                     int32_t num_slash, int32_t max_seqlen, void *stream);
pkv_status pkv_sparse_prefill(void *out, float *lse, const void *q, const void *k, const void *v,
                              const int32_t *cu_seqlens, const int32_t *block_count,
                              const int32_t *block_offset, const int32_t *column_count,
                              const int32_t *column_index, int32_t B, int32_t max_seqlen,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t num_vertical, float sm_scale, const float *sink,
                              pkv_dtype dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
