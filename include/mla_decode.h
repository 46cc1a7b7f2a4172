/*
 * mla_decode.h: C ABI of the MI355X (gfx950) MLA decode library.
 *
 * The operation: one absorbed query token per request attends over that
 * request's rows of a paged latent KV cache.  A query is cat[ql_nope, q_pe]
 * of width kv_lora_rank + qk_rope_head_dim = 512 + 64 = 576; a cache row is
 * cat[kv_c, k_pe] of the same width; the value of a row is its kv_c part
 * (its first 512 columns).  This is the data-movement-friendly path of
 * multi-head latent attention:
 *   - vLLM API docs, vllm.model_executor.layers.attention.mla_attention,
 *     module docstring, "Data-Movement Friendly Approach (i.e. forward_mqa)":
 *     SDPA(cat[ql_nope, q_pe], cat[kv_c, k_pe], kv_c), a multi-query
 *     attention with QK width Lkv + R and value width Lkv.
 *   - Model-Optimizer docs, modelopt.torch.kernels.quantization.attention.mla,
 *     mla_attention_decode: arguments q, latent_cache, block_table,
 *     b_seq_len, softmax_scale, num_kv_splits, return_lse; result
 *     (out [batch, num_heads, 512], lse [batch, num_heads] | None).
 *
 * For request b with L = seq_lens[b] and head n:
 *     s_t   = softmax_scale * <q[b,n,:], K_t>            t = 0 .. L-1
 *     lse   = ln sum_t exp(s_t)
 *     out_l = sum_t exp(s_t - lse) * K_t[l]                l = 0 .. 511
 * where K_t is row (t mod page_size) of block block_table[b][t / page_size].
 * L == 0 gives out = 0 and lse = -inf, the state that carries no weight in a
 * merge (vLLM API docs, neutralize_empty_context_partials).
 *
 * Work is split over the KV axis into num_kv_splits contiguous chunks per
 * request; each chunk yields a partial (normalised output, LSE) and the
 * partials are combined with the LSE merge.  The split count is a fixed
 * argument, so the reduction order depends only on (seq_len, num_kv_splits,
 * num_heads), never on the batch or the device: the decode API fixes the
 * split count rather than choosing it per batch, so that results repeat
 * whatever the batch shape or the device (Model-Optimizer docs,
 * mla_attention_decode, "Parameters", num_kv_splits).
 * Chunk s of a request of length L covers tokens
 *     [s*C, min((s+1)*C, L)),
 *     C = max(32 * ceil(ceil(L / num_kv_splits) / 32), 2048);
 * trailing chunks may be empty (a request shorter than 2048 * S fills only
 * its first ceil(L / C) chunks, so no chunk is dominated by fixed costs and
 * the fp32 partials stay few).
 *
 * Memory and threading contract, for every entry point:
 *   - Pointers marked "device" point to device memory allocated by the
 *     caller; the library allocates nothing, keeps no pointer after it
 *     returns, and holds no state: calls are reentrant.  The one exception
 *     is mla_decode_noalloc, whose partials live in a static device array
 *     (see its declaration).
 *   - Every call only enqueues kernels on `stream` and returns.  It performs
 *     no host<->device copy and never reads device data on the host, so the
 *     launch configuration depends only on the shape arguments and the calls
 *     can be captured into a HIP graph.
 *   - Arguments the host can check are checked before anything is launched;
 *     a failed check returns an error status and launches nothing.
 *   - Device-side data is not validated on the host.  Preconditions the caller
 *     owns: 0 <= seq_lens[b] <= max_blocks_per_seq * page_size, and the first
 *     ceil(seq_lens[b] / page_size) entries of block_table row b are in
 *     [0, num_blocks).  The kernels clamp both into range before addressing
 *     memory, so a violation gives wrong numbers for that request, never an
 *     out-of-bounds access.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_OK = 0,
    MLA_ERR_NULL_POINTER = 1,   /* a required pointer is NULL */
    MLA_ERR_BAD_SHAPE = 2,      /* a dimension is negative or inconsistent */
    MLA_ERR_UNSUPPORTED = 3,    /* a shape or dtype this build does not handle */
    MLA_ERR_BAD_SPLITS = 4,     /* num_kv_splits outside [1, MLA_MAX_KV_SPLITS] */
    MLA_ERR_WORKSPACE = 5,      /* workspace missing or smaller than required */
    MLA_ERR_HIP = 6,            /* the HIP runtime rejected a launch */
    MLA_ERR_SCRATCH_LIMIT = 7   /* mla_decode_noalloc: the partials exceed
                                   its static scratch */
} mla_status_t;

/* Cache element type.  It is explicit because the bytes alone are ambiguous:
 * a uint8 cache must be read as E4M3, not as a packed 4-bit format, which
 * would double the apparent row width (raon-1-mini mla_attention.py,
 * _attn_read_kv_cache). */
typedef enum {
    MLA_CACHE_BF16 = 0,         /* bfloat16 rows, 1152 bytes each */
    MLA_CACHE_FP8_E4M3FN = 1    /* OCP E4M3 ("FN": no inf, max 448) rows,
                                   576 bytes each, times a per-tensor scale */
} mla_cache_dtype_t;

#define MLA_KV_LORA_RANK 512
#define MLA_QK_ROPE_HEAD_DIM 64
#define MLA_MAX_KV_SPLITS 256
#define MLA_MAX_QUERY_LEN 16

typedef struct {
    int32_t batch;              /* B >= 0 requests, one query token each */
    int32_t num_heads;          /* N > 0, a multiple of 16 */
    int32_t kv_lora_rank;       /* must be 512 */
    int32_t qk_rope_head_dim;   /* must be 64 */
    int32_t num_blocks;         /* physical pages in the cache, > 0 */
    int32_t page_size;          /* rows per page: a power of two, 16 .. 1024 */
    int32_t max_blocks_per_seq; /* columns of block_table, > 0 */
    mla_cache_dtype_t cache_dtype;
} mla_decode_shape_t;

/* Human-readable name of a status; never NULL. */
const char *mla_status_string(mla_status_t status);

/* Bytes of device workspace mla_decode needs for this shape and split
 * count: B * N * S * (512 + 1) * 4 (fp32 partial outputs and LSEs), or 0
 * when num_kv_splits == 1 (the single chunk is written to `out` directly).
 * Returns 0 for a NULL shape or an invalid split count. */
size_t mla_decode_workspace_size(const mla_decode_shape_t *shape,
                                 int32_t num_kv_splits);

/*
 * Decode attention, split over KV and merged.
 *
 *   q             device, bf16 [B, N, 576], contiguous: cat[ql_nope, q_pe].
 *   latent_cache  device, [num_blocks, page_size, 576] contiguous rows
 *                 cat[kv_c, k_pe]; bf16, or E4M3 bytes per cache_dtype.
 *   cache_scale   device, one float: the per-tensor dequantisation scale of
 *                 an fp8 cache (the cache stores latent / scale; readers
 *                 multiply it back into both kv_c and k_pe, raon-1-mini
 *                 mla_attention.py, dequantize_context_latent).  Must be
 *                 NULL for a bf16 cache, non-NULL for fp8.
 *   block_table   device, int32 [B, max_blocks_per_seq]: logical page i of
 *                 request b lives in physical block block_table[b][i].
 *   seq_lens      device, int32 [B]: KV length of each request, the current
 *                 token included.  0 is allowed (padding rows).
 *   softmax_scale the scale applied to the full 576-wide dot product
 *                 (required; an MLA layer folds its mscale into it).
 *   num_kv_splits S in [1, 256], fixed by the caller.
 *   workspace     device, at least mla_decode_workspace_size() bytes; may
 *                 be NULL when that size is 0.  Overwritten.
 *   out           device, bf16 [B, N, 512], written in full (the pages' default
 *                 output dtype is the model compute dtype, which is bf16 for
 *                 both cache types).  Rounded to nearest even.
 *   lse           device, float [B, N] natural-log LSE, or NULL to skip it.
 *   stream        HIP stream the kernels are enqueued on (0 = null stream).
 *
 * Returns MLA_OK after enqueuing, or an error status with nothing enqueued
 * (MLA_ERR_HIP if a launch itself failed).  B == 0 is a no-op.
 */
mla_status_t mla_decode(const mla_decode_shape_t *shape, const void *q,
                        const void *latent_cache, const float *cache_scale,
                        const int32_t *block_table, const int32_t *seq_lens,
                        float softmax_scale, int32_t num_kv_splits,
                        void *workspace, size_t workspace_bytes, void *out,
                        float *lse, hipStream_t stream);

/* Size of the static device scratch of mla_decode_noalloc: 160 MiB. */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)160 << 20)

/*
 * mla_decode without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc.  The call allocates nothing (no hipMalloc, hipFree
 * or allocating library routine): the split partials go to a static device
 * array of MLA_NOALLOC_SCRATCH_BYTES that the library holds on each device it
 * runs on until the process ends.  Its device address is looked up once per
 * device, on that device's first call, with the device current.
 *
 * Arguments, checks, kernels and results are those of mla_decode (bitwise
 * the same outputs), minus workspace and workspace_bytes.  The caller still
 * supplies out and lse.  The stream must belong to the current device.
 * Returns MLA_ERR_SCRATCH_LIMIT, with nothing enqueued, when
 * mla_decode_workspace_size(shape, num_kv_splits) exceeds the scratch:
 * B * N * S * 513 * 4 bytes must be at most 160 MiB (e.g. B = 64, N = 128
 * up to S = 9; B = 256, N = 128 up to S = 2).  S == 1 needs no scratch.
 *
 * Every call on a device shares that device's one scratch array and leaves
 * its partials there; nothing in it needs clearing between calls (every
 * state the merge reads is written by the same call).  Calls that overlap
 * on one device (on different streams, or from different host threads
 * without ordering) race on the scratch and give wrong results: order them.
 */
mla_status_t mla_decode_noalloc(const mla_decode_shape_t *shape,
                                const void *q, const void *latent_cache,
                                const float *cache_scale,
                                const int32_t *block_table,
                                const int32_t *seq_lens, float softmax_scale,
                                int32_t num_kv_splits, void *out, float *lse,
                                hipStream_t stream);

/*
 * The split stage of mla_decode alone: writes the per-chunk partial states
 *   part_out  = workspace as float [B, N, S, 512] (normalised chunk outputs)
 *   part_lse  = workspace + B*N*S*512 floats, float [B, N, S] (natural log)
 * with lse = -inf for an empty chunk, whose part_out rows are left
 * unwritten (the merge never reads a state of weight zero).  Same arguments
 * and checks as
 * mla_decode; requires num_kv_splits >= 1 and a workspace of
 * B * N * S * 513 * 4 bytes (for S == 1 too).  mla_decode is exactly this
 * followed by mla_merge_states on the same workspace.
 */
mla_status_t mla_decode_partials(const mla_decode_shape_t *shape, const void *q,
                                 const void *latent_cache,
                                 const float *cache_scale,
                                 const int32_t *block_table,
                                 const int32_t *seq_lens, float softmax_scale,
                                 int32_t num_kv_splits, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * S-way LSE merge of partial attention states (the combination performed by
 * merge_attn_states for two states in the vLLM API docs, "Chunked Prefill",
 * here for S states with the decode layout):
 *     lse[r]    = ln sum_s exp(part_lse[r, s])
 *     out[r, l] = sum_s exp(part_lse[r, s] - lse[r]) * part_out[r, s, l]
 * A state with lse = -inf carries no weight and its part_out row is not
 * read (it may hold anything, NaN included); a row whose states are all
 * -inf gives out = 0 and lse = -inf.
 *
 *   batch     B >= 0 requests.
 *   num_heads N >= 0 heads per request; B * N must fit an int32.
 *   S         states per row, in [1, 256].
 *   dv        row width; must be 512.
 *   part_out  device, float [B, N, S, dv], contiguous.
 *   part_lse  device, float [B, N, S], contiguous.
 *   out       device, bf16 [B, N, dv] (round to nearest even).
 *   lse       device, float [B, N], or NULL.
 * Each (b, n) row is merged on its own: its bits depend only on its S
 * states, not on B or N (the launch shape follows B * N, the arithmetic of
 * an element does not).
 * Errors: MLA_ERR_BAD_SHAPE for a negative B or N, MLA_ERR_BAD_SPLITS for S
 * outside [1, 256], MLA_ERR_UNSUPPORTED for dv != 512 or B * N beyond int32,
 * MLA_ERR_NULL_POINTER for a missing part_out, part_lse or out when
 * B * N > 0.
 */
mla_status_t mla_merge_states(int32_t batch, int32_t num_heads, int32_t S,
                              int32_t dv, const float *part_out,
                              const float *part_lse, void *out, float *lse,
                              hipStream_t stream);

/*
 * Device-side check of the data preconditions above, for debugging a caller:
 * the decode entry points never read these on the host and only clamp them
 * on the device, so a violation gives wrong numbers for that request.  This
 * call checks them on the device, asynchronously, and reports into a status
 * word that the caller reads when it chooses.
 *   shape        as for mla_decode; batch, max_blocks_per_seq, page_size and
 *                num_blocks are used (the shape must pass mla_decode's checks).
 *   block_table  device, int32 [batch, max_blocks_per_seq].
 *   seq_lens     device, int32 [batch].
 *   status       device, int32 [3], overwritten (not accumulated):
 *                status[0]  number of requests that break a precondition;
 *                status[1]  the lowest such request, or -1;
 *                status[2]  bit 0: some seq_len lies outside
 *                           [0, max_blocks_per_seq * page_size];
 *                           bit 1: some block id among a request's first
 *                           ceil(seq_len / page_size) entries lies outside
 *                           [0, num_blocks).
 * One workgroup; it reads each seq_len and at most max_blocks_per_seq table
 * entries of each request (none past the row).  Errors: missing pointers
 * MLA_ERR_NULL_POINTER; a shape mla_decode rejects, the same status.
 */
mla_status_t mla_check_inputs(const mla_decode_shape_t *shape, const int32_t *block_table,
                              const int32_t *seq_lens, int32_t *status, hipStream_t stream);

/*
 * The per-head matmuls on either side of the attention (vLLM API docs,
 * mla_attention, "Data-Movement Friendly Approach (i.e. forward_mqa)":
 * ql_nope = q_nope . W_UK contracting P, then the latent output times W_UV;
 * the decode path runs them as batched matmuls over the heads with the
 * weights prepared once as W_UK_T = W_UK permuted to [N, P, Lkv] and W_UV
 * transposed to [N, Lkv, V], as the MLA common page's weight processing
 * does).  fp32 accumulation, bf16 results rounded to nearest even.
 *
 * mla_absorb_query:  ql_nope[b, n, l] = sum_p q_nope[b, n, p] * w_uk_t[n, p, l]
 *   q_nope   device, bf16, element (b, n, p) at b * q_token_stride +
 *            n * q_head_stride + p (P = 128; a slice of a wider query row is
 *            fine: contiguous is q_token_stride = N * 128, q_head_stride = 128).
 *   w_uk_t   device, bf16 [N, 128, 512], contiguous.
 *   ql_nope  device, bf16 [batch, N, 512], contiguous.
 * mla_up_project:    out[b, n, v] = sum_l latent_out[b, n, l] * w_uv[n, l, v]
 *   latent_out  device, bf16, element (b, n, l) at b * x_token_stride +
 *               n * x_head_stride + l (Lkv = 512).
 *   w_uv        device, bf16 [N, 512, 128], contiguous.
 *   out         device, bf16 [batch, N, 128], contiguous.
 * Strides are in elements and must be multiples of 8, the input and weight
 * pointers and the output 16-byte aligned, else
 * MLA_ERR_UNSUPPORTED.  Negative sizes or strides: MLA_ERR_BAD_SHAPE.
 * Missing pointers: MLA_ERR_NULL_POINTER.
 */
mla_status_t mla_absorb_query(int32_t batch, int32_t num_heads, const void *q_nope,
                              int64_t q_token_stride, int64_t q_head_stride,
                              const void *w_uk_t, void *ql_nope, hipStream_t stream);
mla_status_t mla_up_project(int32_t batch, int32_t num_heads, const void *latent_out,
                            int64_t x_token_stride, int64_t x_head_stride, const void *w_uv,
                            void *out, hipStream_t stream);

/*
 * Multi-token decode (speculative decoding with a uniform query length; vLLM
 * API docs, mla_attention, QueryLenSupport "UNIFORM": every request of the
 * batch has the same q_len > 1 new tokens; the metadata builder's causal /
 * non-causal multi-token decode).  Request b has seq_lens[b] = L tokens in
 * the cache, its q_len new ones included (their rows are inserted before the
 * attention).  Query row j (0 <= j < q_len) of request b is the absorbed query
 * of its new token j and attends over
 *     causal != 0:  tokens [0, L - q_len + 1 + j)   (itself and what precedes)
 *     causal == 0:  tokens [0, L)
 * with the same definition and merge as mla_decode.  The request's q_len
 * rows share one split: the chunks of mla_decode for length L, each cut at a
 * causal row's own end (its last chunks may be empty).  A row whose range is
 * empty gives out = 0, lse = -inf.
 *
 *   q_len        1 .. MLA_MAX_QUERY_LEN query rows per request.
 *   q            device, bf16 [batch, q_len, num_heads, 576].
 *   out          device, bf16 [batch, q_len, num_heads, 512].
 *   lse          device, float [batch, q_len, num_heads], or NULL.
 *   workspace    mla_decode_multi_workspace_size(shape, q_len, S) bytes
 *                (0 when S == 1).
 * Other arguments and errors as for mla_decode; q_len outside the range
 * gives MLA_ERR_BAD_SHAPE.  The q_len * num_heads query heads of a request
 * form the M dimension of its workgroups' contractions, so each KV tile is
 * read once for as many of them as a workgroup holds.
 */
size_t mla_decode_multi_workspace_size(const mla_decode_shape_t *shape, int32_t q_len,
                                       int32_t num_kv_splits);
mla_status_t mla_decode_multi(const mla_decode_shape_t *shape, int32_t q_len, int32_t causal,
                              const void *q, const void *latent_cache,
                              const float *cache_scale, const int32_t *block_table,
                              const int32_t *seq_lens, float softmax_scale,
                              int32_t num_kv_splits, void *workspace, size_t workspace_bytes,
                              void *out, float *lse, hipStream_t stream);

/*
 * Chunked-context gather (vLLM API docs, mla_attention, _compute_prefill_context,
 * section "Chunked Prefill" of the module docstring): copies a chunk of the
 * requests' cached context rows out of the paged cache into a contiguous
 * workspace, dequantizing an fp8 cache on the way (the gather_and_maybe_
 * dequant_cache step).  Workspace row i belongs to request b = token_to_seq[i]
 * and holds that request's token
 *     seq_starts[b] + (i - cu_seq_lens[b])          (seq_starts NULL: 0)
 * found through block_table like the decode path.  A bf16 cache is copied
 * bit for bit; an fp8 element becomes bf16(code_value * cache_scale), the
 * product in fp32, rounded to nearest even.  The pages' gather needs chunk
 * starts aligned to page_size; this one takes any start.
 *
 *   num_tokens        rows to write (>= 0).
 *   latent_cache      device, [num_blocks, page_size, 576] bf16 or E4M3FN.
 *   cache_scale       device, one float (fp8 only).
 *   block_table       device, int32 [batch, max_blocks_per_seq].
 *   cu_seq_lens       device, int32 [batch + 1]: request b's rows start at
 *                     cu_seq_lens[b].
 *   token_to_seq      device, int32 [num_tokens].
 *   seq_starts        device, int32 [batch], or NULL.
 *   dst               device, bf16 [num_tokens, 576].
 * Device-data preconditions (not checked): the indices are consistent and
 * name valid pages; out-of-range values are clamped so that every read stays
 * in bounds, and the row is then unspecified.  Errors as for the other entry
 * points; nothing is launched on an error.
 */
mla_status_t mla_gather_cache(int32_t num_tokens, const void *latent_cache, int32_t num_blocks,
                              int32_t page_size, mla_cache_dtype_t cache_dtype,
                              const float *cache_scale, const int32_t *block_table,
                              int32_t batch, int32_t max_blocks_per_seq,
                              const int32_t *cu_seq_lens, const int32_t *token_to_seq,
                              const int32_t *seq_starts, void *dst, hipStream_t stream);

/*
 * Two-state LSE merge with the prefill layout (vLLM API docs, merge_attn_states
 * as called by accumulate_mla_context_chunk, and the chunked-prefill listing
 * of the mla_attention module docstring): for every token t and head n
 *     M   = max(prefix_lse[n, t], suffix_lse[n, t])
 *     wp  = exp(prefix_lse - M),  ws = exp(suffix_lse - M)
 *     out = (wp * prefix_out[t, n, :] + ws * suffix_out[t, n, :]) / (wp + ws)
 *     out_lse[n, t] = M + ln(wp + ws)
 * A state with lse = -inf carries no weight and its output is not read; two
 * such states give out = 0, lse = -inf.
 *
 *   prefix_out, suffix_out, out   device, bf16 [T, N, head_dim]; out may be
 *                                 the same buffer as either input.
 *   prefix_lse, suffix_lse        device, float [N, T] (natural log).
 *   out_lse                       device, float [N, T], or NULL; may be the
 *                                 same buffer as either input lse.
 *   head_dim                      a power of two in [8, 2048], else
 *                                 MLA_ERR_UNSUPPORTED.
 */
mla_status_t mla_merge_attn_states(int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                                   const void *prefix_out, const float *prefix_lse,
                                   const void *suffix_out, const float *suffix_lse,
                                   void *out, float *out_lse, hipStream_t stream);

/*
 * The step before the attention of a decode step: form the absorbed query and
 * insert the step's new latent row into the paged cache, in one launch
 * (raon-1-mini mla_attention.py, the model-layer page, decode path of forward
 * and _decode_concat_cache; vLLM API docs, mla_attention, forward with a
 * direct call and unified_mla_kv_cache_update: the insert precedes the
 * attention of the same step, at the slot given by slot_mapping).
 *     q_out[t, n, :]          = cat[ql_nope[t, n, :], q_pe[t, n, :]]   (512 + 64)
 *     cache row slot_mapping[t] = cat[kv_c[t, :], k_pe[t, :]]
 * For an fp8 cache each element is stored as the E4M3FN code nearest to the
 * fp32 product x * cache_scale_inv (round to nearest even, saturating at
 * +-448): the pre-inverted per-tensor scale of the model-layer page, so that
 * a reader multiplying by cache_scale (= 1 / cache_scale_inv) gets x back.
 *
 *   num_tokens       T >= 0 new tokens (one per decoding request).
 *   num_heads        N >= 0; N == 0 inserts without forming a query.
 *   ql_nope          device, bf16 [T, N, 512] (the absorbed no-rope query).
 *   q_pe             device, bf16 [T, N, 64].
 *   kv_c, k_pe       device, bf16 [T, 512] and [T, 64] (the new latent row).
 *   slot_mapping     device, int64 [T]: flat row block * page_size + row of
 *                    the [num_blocks, page_size, 576] cache.  A negative
 *                    slot (a padding token) and a slot >= num_blocks *
 *                    page_size write nothing.  Slots must be distinct.
 *   num_blocks, page_size   the cache's shape (page_size >= 1).
 *   cache_dtype      MLA_CACHE_BF16 or MLA_CACHE_FP8_E4M3FN.
 *   cache_scale_inv  device, one float (fp8 only; ignored and may be NULL
 *                    for bf16).
 *   latent_cache     device, updated in place.
 *   q_out            device, bf16 [T, N, 576]; may be NULL when N == 0.
 * Errors: MLA_ERR_BAD_SHAPE for a negative count or page_size < 1,
 * MLA_ERR_UNSUPPORTED for another cache dtype, MLA_ERR_NULL_POINTER for a
 * missing required pointer (nothing is launched then).  Asynchronous on
 * `stream`; the library allocates nothing.
 */
mla_status_t mla_concat_q_insert_cache(int32_t num_tokens, int32_t num_heads,
                                       const void *ql_nope, const void *q_pe,
                                       const void *kv_c, const void *k_pe,
                                       const int64_t *slot_mapping, int32_t num_blocks,
                                       int32_t page_size, mla_cache_dtype_t cache_dtype,
                                       const float *cache_scale_inv, void *latent_cache,
                                       void *q_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
