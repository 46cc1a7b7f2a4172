/*
 * Plain, slow, fp64 CPU reference for absorbed-query MLA decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this file:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load it.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (one query token per request, all heads share one latent
 * KV head):
 *
 *   vLLM API docs, vllm.model_executor.layers.attention.mla_attention, module
 *   docstring, section "Data-Movement Friendly Approach (i.e. forward_mqa)":
 *   attention whose query is cat[ql_nope, q_pe] (width Lkv + R = 576), whose
 *   keys are the cached rows cat[kv_c, k_pe] (width 576) and whose values are
 *   kv_c itself (the first Lkv = 512 columns of the same rows).
 *
 *   Model-Optimizer docs, modelopt.torch.kernels.quantization.attention.mla,
 *   mla_attention_decode, "Parameters" and "Returns": q [batch, num_heads,
 *   576]; latent_cache [num_blocks, page_size, 576]; block_table
 *   [batch, max_blocks_per_seq]; b_seq_len [batch]; softmax_scale is a
 *   required argument; the result is out [batch, num_heads, 512] and the
 *   natural-log LSE [batch, num_heads].
 *
 *   vllm-cpu 0.8.5.post2, vllm/v1/attention/backends/mla/common.py,
 *   get_kv_cache_shape: the cache is (num_blocks, block_size, head_size) with
 *   a single KV head.
 *
 * For one (request b, head n) with L = seq_lens[b] > 0 and
 * K[t] = row t of the request, found through the page table:
 *
 *   s_t   = softmax_scale * sum_d q[b,n,d] * K[t,d]          (d < Dqk)
 *   lse   = log(sum_t exp(s_t))              (natural log, computed stably)
 *   out_l = sum_t exp(s_t - lse) * K[t,l]                    (l < Dv)
 *
 * L == 0 gives out = 0 and lse = -inf: a zero output with an -inf LSE is the
 * state that carries no weight in an LSE merge (vLLM API docs,
 * neutralize_empty_context_partials).
 *
 * Cache element decoding:
 *   - bf16: the value is the binary32 number whose upper 16 bits are the
 *     stored bits (bfloat16 is defined as truncated binary32).
 *   - fp8: OCP 8-bit floating point, E4M3 "FN" variant (exponent bias 7, no
 *     infinities, S.1111.111 is NaN, max normal 448), multiplied by the
 *     per-tensor cache scale: the cache stores latent / scale and readers
 *     multiply the scale back into both the latent and k_pe (raon-1-mini
 *     mla_attention.py, the fp8 insert and the dequantize_context_latent
 *     comments).
 *
 * Every accumulation is a plain left-to-right fp64 loop; nothing is split,
 * blocked or fused.  Requests are processed one (b, n) row at a time; rows are
 * handed to worker threads, which changes nothing in the arithmetic of a row.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- element decoding -------------------------------------------------- */

double oracle_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP E4M3 (FN): sign 1 bit, exponent 4 bits (bias 7), mantissa 3 bits.
 * exponent 0: subnormal, value = (m / 8) * 2^-6.
 * otherwise:  value = (1 + m / 8) * 2^(e - 7); e = 15, m = 7 is NaN. */
double oracle_e4m3fn_to_double(uint8_t bits)
{
    int sign = bits >> 7;
    int e = (bits >> 3) & 0xF;
    int m = bits & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* ---- problem description ----------------------------------------------- */

typedef struct {
    int B, N, Dqk, Dv, page_size, max_blocks, num_blocks;
    int cache_is_fp8;
    const double *q;          /* [B, N, Dqk], already exact doubles        */
    const void *cache;        /* [num_blocks, page_size, Dqk] bf16 or fp8  */
    double cache_scale;       /* fp8 only; 1 for bf16                       */
    const int32_t *block_table; /* [B, max_blocks]                          */
    const int32_t *seq_lens;  /* [B]                                        */
    double softmax_scale;
} oracle_problem;

/* Value of every E4M3FN code, filled once from oracle_e4m3fn_to_double (the
 * decoder above, pinned on the full code table), so that the inner loops
 * look a code up instead of calling ldexp per element. */
static double e4m3_value[256];
static pthread_once_t e4m3_once = PTHREAD_ONCE_INIT;

static void fill_e4m3_values(void)
{
    for (int c = 0; c < 256; ++c)
        e4m3_value[c] = oracle_e4m3fn_to_double((uint8_t)c);
}

/* Start of token t's row of request b in the cache: logical page t / P of
 * the request lives in physical block block_table[b][t / P], at row t mod P.
 * The caller has already rejected tables that address rows outside the
 * cache. */
static const void *token_row(const oracle_problem *p, int b, int64_t t)
{
    int64_t page = t / p->page_size;
    int64_t row = t % p->page_size;
    int32_t blk = p->block_table[(int64_t)b * p->max_blocks + page];
    int64_t idx = ((int64_t)blk * p->page_size + row) * p->Dqk;
    if (p->cache_is_fp8)
        return (const uint8_t *)p->cache + idx;
    return (const uint16_t *)p->cache + idx;
}

/* Element d of a row: bf16 widened exactly, or an E4M3FN code's value times
 * the cache scale. */
static double row_elem(const oracle_problem *p, const void *row, int d)
{
    if (p->cache_is_fp8)
        return e4m3_value[((const uint8_t *)row)[d]] * p->cache_scale;
    return oracle_bf16_to_double(((const uint16_t *)row)[d]);
}

/* Attention of query row (b, n) over tokens [t0, t1) of request b.
 * Writes Dv outputs and the natural-log LSE.  An empty span gives the
 * neutral state (0, -inf).  `scores` must hold t1 - t0 doubles. */
static void attend_span(const oracle_problem *p, int b, int n, int64_t t0,
                        int64_t t1, double *scores, double *out, double *lse)
{
    const double *qv = p->q + ((int64_t)b * p->N + n) * p->Dqk;
    int64_t L = t1 - t0;
    for (int l = 0; l < p->Dv; ++l)
        out[l] = 0.0;
    if (L <= 0) {
        *lse = -INFINITY;
        return;
    }
    /* scores s_t = scale * <q, K[t]> over all Dqk columns */
    double mx = -INFINITY;
    for (int64_t t = 0; t < L; ++t) {
        const void *krow = token_row(p, b, t0 + t);
        double dot = 0.0;
        for (int d = 0; d < p->Dqk; ++d)
            dot += qv[d] * row_elem(p, krow, d);
        scores[t] = p->softmax_scale * dot;
        if (scores[t] > mx)
            mx = scores[t];
    }
    /* Z = sum_t exp(s_t - max);  lse = max + log Z */
    double Z = 0.0;
    for (int64_t t = 0; t < L; ++t)
        Z += exp(scores[t] - mx);
    *lse = mx + log(Z);
    /* out = sum_t softmax_t * V[t], V = first Dv columns of the row */
    for (int64_t t = 0; t < L; ++t) {
        double w = exp(scores[t] - mx) / Z;
        const void *vrow = token_row(p, b, t0 + t);
        for (int l = 0; l < p->Dv; ++l)
            out[l] += w * row_elem(p, vrow, l);
    }
}

/* ---- input validation --------------------------------------------------- */

/* Returns 0 when every row the oracle would touch is addressable. */
static int check_problem(const oracle_problem *p)
{
    if (p->B < 0 || p->N <= 0 || p->Dqk <= 0 || p->Dv <= 0 || p->Dv > p->Dqk ||
        p->page_size <= 0 || p->max_blocks < 0 || p->num_blocks <= 0)
        return 1;
    for (int b = 0; b < p->B; ++b) {
        int64_t L = p->seq_lens[b];
        if (L < 0 || L > (int64_t)p->max_blocks * p->page_size)
            return 2;
        int64_t pages = (L + p->page_size - 1) / p->page_size;
        for (int64_t i = 0; i < pages; ++i) {
            int32_t blk = p->block_table[(int64_t)b * p->max_blocks + i];
            if (blk < 0 || blk >= p->num_blocks)
                return 3;
        }
    }
    return 0;
}

/* ---- threaded driver over (b, n) rows ----------------------------------- */

typedef struct {
    const oracle_problem *p;
    int n_rows;
    const int32_t *row_b, *row_n;
    const int64_t *span_t0, *span_t1; /* NULL: the whole sequence */
    double *out, *lse;
    int next;                          /* shared work counter */
    pthread_mutex_t lock;
} oracle_job;

static void *worker(void *arg)
{
    oracle_job *job = (oracle_job *)arg;
    const oracle_problem *p = job->p;
    double *scores = NULL;
    int64_t cap = 0;
    for (;;) {
        pthread_mutex_lock(&job->lock);
        int r = job->next++;
        pthread_mutex_unlock(&job->lock);
        if (r >= job->n_rows)
            break;
        int b = job->row_b[r], n = job->row_n[r];
        int64_t t0 = job->span_t0 ? job->span_t0[r] : 0;
        int64_t t1 = job->span_t1 ? job->span_t1[r] : p->seq_lens[b];
        if (t1 - t0 > cap) {
            free(scores);
            cap = t1 - t0;
            scores = (double *)malloc((size_t)cap * sizeof(double));
            if (!scores) {
                cap = 0;
                job->lse[r] = NAN; /* out of memory: poison the row */
                continue;
            }
        }
        attend_span(p, b, n, t0, t1, scores, job->out + (int64_t)r * p->Dv,
                    job->lse + r);
    }
    free(scores);
    return NULL;
}

static int run_rows(const oracle_problem *p, int n_rows, const int32_t *row_b,
                    const int32_t *row_n, const int64_t *t0, const int64_t *t1,
                    double *out, double *lse, int nthreads)
{
    oracle_job job;
    job.p = p;
    job.n_rows = n_rows;
    job.row_b = row_b;
    job.row_n = row_n;
    job.span_t0 = t0;
    job.span_t1 = t1;
    job.out = out;
    job.lse = lse;
    job.next = 0;
    pthread_mutex_init(&job.lock, NULL);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, worker, &job) == 0)
            ++started;
    worker(&job);
    for (int i = 0; i < started; ++i)
        pthread_join(th[i], NULL);
    pthread_mutex_destroy(&job.lock);
    return 0;
}

/* ---- exported entry points ---------------------------------------------- */

/* Full decode, or a chosen list of (b, n) rows.
 * n_rows < 0: every row, in (b, n) order, out is [B, N, Dv] and lse [B, N].
 * n_rows >= 0: rows (row_b[i], row_n[i]); out is [n_rows, Dv], lse [n_rows].
 * Returns 0, or a nonzero code when the inputs address rows outside the
 * cache (the oracle refuses them rather than guessing). */
int oracle_mla_decode(int B, int N, int Dqk, int Dv, int page_size,
                      int max_blocks, int num_blocks, int cache_is_fp8,
                      const double *q, const void *cache, float cache_scale,
                      const int32_t *block_table, const int32_t *seq_lens,
                      float softmax_scale, int n_rows, const int32_t *row_b,
                      const int32_t *row_n, double *out, double *lse,
                      int nthreads)
{
    oracle_problem p = {B, N, Dqk, Dv, page_size, max_blocks, num_blocks,
                        cache_is_fp8, q, cache,
                        cache_is_fp8 ? (double)cache_scale : 1.0,
                        block_table, seq_lens, (double)softmax_scale};
    pthread_once(&e4m3_once, fill_e4m3_values);
    int rc = check_problem(&p);
    if (rc)
        return rc;
    if (n_rows < 0) {
        int total = B * N;
        int32_t *rb = (int32_t *)malloc(sizeof(int32_t) * (size_t)(total ? total : 1));
        int32_t *rn = (int32_t *)malloc(sizeof(int32_t) * (size_t)(total ? total : 1));
        if (!rb || !rn) {
            free(rb);
            free(rn);
            return 10;
        }
        for (int b = 0; b < B; ++b)
            for (int n = 0; n < N; ++n) {
                rb[b * N + n] = b;
                rn[b * N + n] = n;
            }
        run_rows(&p, total, rb, rn, NULL, NULL, out, lse, nthreads);
        free(rb);
        free(rn);
        return 0;
    }
    for (int i = 0; i < n_rows; ++i)
        if (row_b[i] < 0 || row_b[i] >= B || row_n[i] < 0 || row_n[i] >= N)
            return 4;
    run_rows(&p, n_rows, row_b, row_n, NULL, NULL, out, lse, nthreads);
    return 0;
}

/* Attention of rows (row_b[i], row_n[i]) over token spans [t0[i], t1[i]) of
 * their requests: the partial state (normalised output, natural-log LSE) of
 * one KV split.  An empty span gives (0, -inf). */
int oracle_mla_attend_spans(int B, int N, int Dqk, int Dv, int page_size,
                            int max_blocks, int num_blocks, int cache_is_fp8,
                            const double *q, const void *cache,
                            float cache_scale, const int32_t *block_table,
                            const int32_t *seq_lens, float softmax_scale,
                            int n_rows, const int32_t *row_b,
                            const int32_t *row_n, const int64_t *t0,
                            const int64_t *t1, double *out, double *lse,
                            int nthreads)
{
    oracle_problem p = {B, N, Dqk, Dv, page_size, max_blocks, num_blocks,
                        cache_is_fp8, q, cache,
                        cache_is_fp8 ? (double)cache_scale : 1.0,
                        block_table, seq_lens, (double)softmax_scale};
    pthread_once(&e4m3_once, fill_e4m3_values);
    int rc = check_problem(&p);
    if (rc)
        return rc;
    for (int i = 0; i < n_rows; ++i) {
        if (row_b[i] < 0 || row_b[i] >= B || row_n[i] < 0 || row_n[i] >= N)
            return 4;
        if (t0[i] < 0 || t1[i] > seq_lens[row_b[i]])
            return 5;
    }
    run_rows(&p, n_rows, row_b, row_n, t0, t1, out, lse, nthreads);
    return 0;
}

/* LSE merge of S partial states per row (the combination that
 * merge_attn_states performs for two states in the vLLM docs, written for S):
 *   lse   = log(sum_s exp(lse_s))          (stably, about max_s lse_s)
 *   out_l = sum_s exp(lse_s - lse) * out_s,l
 * When every lse_s is -inf the row carries no weight: out = 0, lse = -inf.
 * part_out is [R, S, Dv], part_lse [R, S]; out [R, Dv], lse [R]. */
void oracle_merge_states(int R, int S, int Dv, const double *part_out,
                         const double *part_lse, double *out, double *lse)
{
    for (int r = 0; r < R; ++r) {
        const double *ls = part_lse + (int64_t)r * S;
        double *o = out + (int64_t)r * Dv;
        double mx = -INFINITY;
        for (int s = 0; s < S; ++s)
            if (ls[s] > mx)
                mx = ls[s];
        for (int l = 0; l < Dv; ++l)
            o[l] = 0.0;
        if (mx == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double Z = 0.0;
        for (int s = 0; s < S; ++s)
            Z += exp(ls[s] - mx);
        double total = mx + log(Z);
        lse[r] = total;
        for (int s = 0; s < S; ++s) {
            double w = exp(ls[s] - total);
            const double *os = part_out + ((int64_t)r * S + s) * Dv;
            for (int l = 0; l < Dv; ++l)
                o[l] += w * os[l];
        }
    }
}

/* ---- decode-step cache insert and query concat ---------------------------
 *
 * raon-1-mini mla_attention.py (the model-layer page), the decode path of
 * forward and _decode_concat_cache: before the attention of a decode step,
 * one launch forms the absorbed query as the concatenation [ql_nope, q_pe]
 * (width 512 + 64) and writes the step's new latent row [kv_c, k_pe] into the
 * paged cache at its slot.  vLLM API docs, mla_attention (forward with a
 * direct call, and unified_mla_kv_cache_update): the slot comes from the
 * forward context's slot_mapping, and the insert happens before the
 * attention of the same step.  The vLLM MLA common page's
 * concat_and_cache_mla call writes the same row layout.  For an fp8 cache
 * the row is stored as value * cache_scale_inv, the pre-inverted scale (the
 * model-layer page's _k_scale_inv buffer): the stored value times the scale
 * gives the latent back, as the readers assume.
 *
 * Readings (the pages do not spell these out):
 *   - a slot is block * page_size + row, i.e. the flat row index of the
 *     [num_blocks, page_size, 576] cache;
 *   - a negative slot marks a padding token that writes nothing; a slot at or
 *     beyond num_blocks * page_size is likewise skipped;
 *   - the fp8 product value * scale_inv is formed in fp32 (where a float
 *     decides a code, both sides decide in the kernel's precision), then
 *     rounded to the nearest E4M3FN value with ties to the even code,
 *     magnitudes beyond 448 saturating to +-448.
 */

/* Nearest E4M3FN code to a float: magnitudes of 448 and beyond saturate to
 * the largest finite code; otherwise every finite non-negative code is tried
 * through the decoder above (pinned on the full code table), ties to the even
 * code, the sign applied last.  NaN gives the NaN code 0x7F. */
uint8_t oracle_e4m3fn_from_float(float v)
{
    if (isnan(v))
        return 0x7F;
    const double a = fabs((double)v);
    if (a >= 448.0)                 /* saturation: the largest finite code */
        return (uint8_t)(signbit(v) ? 0xFE : 0x7E);
    int best = 0;
    double best_err = INFINITY;
    for (int k = 0; k <= 0x7E; ++k) {
        const double err = fabs(oracle_e4m3fn_to_double((uint8_t)k) - a);
        if (err < best_err || (err == best_err && (k & 1) == 0 && (best & 1) == 1)) {
            best = k;
            best_err = err;
        }
    }
    return (uint8_t)(signbit(v) ? (best | 0x80) : best);
}

/* ql_nope [T, N, Dn], q_pe [T, N, Dr], kv_c [T, Dn], k_pe [T, Dr]: bf16 bits.
 * q_out [T, N, Dn + Dr] bf16 bits.  cache [num_blocks * page_size, Dn + Dr]:
 * bf16 bits (fp8 == 0) or E4M3FN codes (fp8 == 1). */
void oracle_concat_insert(int T, int N, int Dn, int Dr, const uint16_t *ql_nope,
                          const uint16_t *q_pe, const uint16_t *kv_c, const uint16_t *k_pe,
                          const int64_t *slot_mapping, int num_blocks, int page_size, int fp8,
                          float scale_inv, void *cache, uint16_t *q_out)
{
    const int D = Dn + Dr;
    for (int t = 0; t < T; ++t)
        for (int n = 0; n < N; ++n)
            for (int d = 0; d < D; ++d)
                q_out[((int64_t)t * N + n) * D + d] =
                    d < Dn ? ql_nope[((int64_t)t * N + n) * Dn + d]
                           : q_pe[((int64_t)t * N + n) * Dr + (d - Dn)];
    const int64_t rows = (int64_t)num_blocks * page_size;
    for (int t = 0; t < T; ++t) {
        const int64_t s = slot_mapping[t];
        if (s < 0 || s >= rows)
            continue;
        for (int d = 0; d < D; ++d) {
            const uint16_t bits = d < Dn ? kv_c[(int64_t)t * Dn + d] : k_pe[(int64_t)t * Dr + (d - Dn)];
            if (!fp8) {
                ((uint16_t *)cache)[s * D + d] = bits;
            } else {
                const float x = (float)oracle_bf16_to_double(bits);
                const float v = x * scale_inv;
                ((uint8_t *)cache)[s * D + d] = oracle_e4m3fn_from_float(v);
            }
        }
    }
}

/* ---- chunked-context gather and the two-state merge ----------------------
 *
 * vLLM API docs, mla_attention, _compute_prefill_context ("Chunked Prefill"):
 * the context of the requests being prefilled is processed in chunks; each
 * chunk's rows are first copied out of the paged cache into a contiguous
 * workspace (gather_and_maybe_dequant_cache, with the chunk's per-request
 * start seq_starts, the workspace offsets cu_seq_lens and the owner of each
 * workspace row token_to_seq; an fp8 cache is dequantized on the way with
 * its scale), then attended, and the chunk's partial (output, lse) is folded
 * into the running one with merge_attn_states (accumulate_mla_context_chunk),
 * whose LSE layout is [heads, tokens].  The module docstring's chunked
 * prefill listing merges the same way: the state with the larger lse
 * dominates, and the merged lse is the log of the summed exponentials.
 *
 * Readings:
 *   - workspace row i belongs to request b = token_to_seq[i] and holds token
 *     seq_starts[b] + (i - cu_seq_lens[b]) of that request, found through the
 *     page table.  A row whose owner, position, logical page or block id
 *     falls outside the table or the cache has no defined value, so the
 *     whole call is refused (nonzero return, nothing written), as the decode
 *     oracle refuses such tables;
 *   - an fp8 element is dequantized as the fp32 product code_value * scale,
 *     rounded to bf16 (nearest even): where a float decides the stored bits
 *     both sides decide in fp32;
 *   - the merge of two states of weight zero (both lse = -inf) is out = 0,
 *     lse = -inf, as for the S-way merge.
 */

/* bf16 bits of a float, round to nearest even (finite inputs and NaN). */
static uint16_t bf16_from_float(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu))
        return (uint16_t)((u >> 16) | 0x40);
    const uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* Physical row of workspace row i, or -1 when the indices that lead to it
 * leave the table or the cache. */
static int64_t gather_row(int i, int num_blocks, int page_size, const int32_t *block_table,
                          int B, int max_blocks, const int32_t *cu_seq_lens,
                          const int32_t *token_to_seq, const int32_t *seq_starts)
{
    const int b = token_to_seq[i];
    if (b < 0 || b >= B)
        return -1;
    const int64_t pos = (int64_t)(seq_starts ? seq_starts[b] : 0) + (i - cu_seq_lens[b]);
    if (pos < 0)
        return -1;
    const int64_t pg = pos / page_size;
    if (pg >= max_blocks)
        return -1;
    const int blk = block_table[(int64_t)b * max_blocks + pg];
    if (blk < 0 || blk >= num_blocks)
        return -1;
    return (int64_t)blk * page_size + pos % page_size;
}

/* dst [num_tokens, D] bf16 bits; cache [num_blocks, page_size, D] bf16 bits
 * or E4M3FN codes; block_table [B, max_blocks].  Returns 0, or 1 (and writes
 * nothing) when some row's indices leave the table or the cache. */
int oracle_gather(int num_tokens, int D, const void *cache, int num_blocks, int page_size,
                  int fp8, float scale, const int32_t *block_table, int B, int max_blocks,
                  const int32_t *cu_seq_lens, const int32_t *token_to_seq,
                  const int32_t *seq_starts, uint16_t *dst)
{
    for (int i = 0; i < num_tokens; ++i)
        if (gather_row(i, num_blocks, page_size, block_table, B, max_blocks, cu_seq_lens,
                       token_to_seq, seq_starts) < 0)
            return 1;
    for (int i = 0; i < num_tokens; ++i) {
        const int64_t row = gather_row(i, num_blocks, page_size, block_table, B, max_blocks,
                                       cu_seq_lens, token_to_seq, seq_starts);
        for (int d = 0; d < D; ++d) {
            if (!fp8) {
                dst[(int64_t)i * D + d] = ((const uint16_t *)cache)[row * D + d];
            } else {
                const float v = (float)oracle_e4m3fn_to_double(((const uint8_t *)cache)[row * D + d]);
                dst[(int64_t)i * D + d] = bf16_from_float(v * scale);
            }
        }
    }
    return 0;
}

/* Two states per (token, head): outputs [T, N, D] as doubles, lse [N, T]. */
void oracle_merge_two(int T, int N, int D, const double *prefix_out, const double *prefix_lse,
                      const double *suffix_out, const double *suffix_lse, double *out,
                      double *out_lse)
{
    for (int t = 0; t < T; ++t)
        for (int n = 0; n < N; ++n) {
            const double lp = prefix_lse[(int64_t)n * T + t], ls = suffix_lse[(int64_t)n * T + t];
            const double m = lp > ls ? lp : ls;
            double *o = out + ((int64_t)t * N + n) * D;
            const double *po = prefix_out + ((int64_t)t * N + n) * D;
            const double *so = suffix_out + ((int64_t)t * N + n) * D;
            if (m == -INFINITY) {
                for (int d = 0; d < D; ++d)
                    o[d] = 0.0;
                out_lse[(int64_t)n * T + t] = -INFINITY;
                continue;
            }
            const double wp = exp(lp - m), ws = exp(ls - m);
            for (int d = 0; d < D; ++d)
                o[d] = (wp * po[d] + ws * so[d]) / (wp + ws);
            out_lse[(int64_t)n * T + t] = m + log(wp + ws);
        }
}
