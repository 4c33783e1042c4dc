/*
 * CPU oracle for grouped-query attention with a learned per-head sink logit.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * kernels.
 *
 * What it computes (the plain definition, fp64 throughout):
 *
 *   "GPT-OSS on day 0" (Perplexity blog), section "Attention: GQA with
 *   attention sinks": every attention head owns one trained sink parameter
 *   that takes part in that head's softmax.  Section "Kernels for GPT-OSS /
 *   Sink-Attention": the sink is an extra bias term that enters the softmax
 *   next to the Q.K products; the formula itself did not survive extraction.
 *   The reading used here is the only one consistent with the rest of that
 *   section: the sink is one extra logit in the softmax denominator that has
 *   no value row, and it is not multiplied by the softmax scale (the running
 *   maximum, which lives in scaled-logit space, is seeded with the raw sink).
 *
 *   For a query row q of head h (GQA group g = h / (Hq/Hkv)) and a visible key
 *   set J:
 *       x_j = scale * sum_d q[d] * k_j[d]                 (j in J)
 *       M   = max(s_h, max_j x_j)
 *       Z   = exp(s_h - M) + sum_j exp(x_j - M)
 *       o   = sum_j exp(x_j - M) / Z * v_j
 *       lse = M + ln Z,   sink share = exp(s_h - M) / Z
 *   Prefill, causal: J = {j : j <= i} within the row's own sequence.
 *   Prefill, non-causal: J = the whole sequence.  Decode: J = the cached
 *   tokens 0 .. len_b - 1 of the request.  Multi-token decode (q_len new
 *   tokens at the end of the cache): J = tokens 0 .. len_b - q_len + t for
 *   new token t.  Chunked prefill (a chunk of len_q queries at the end of a
 *   sequence of len_k tokens): J = tokens 0 .. len_k - len_q + i for query i
 *   of the chunk, causal.
 *
 *   Same section, on the online form: the running maximum m and the running
 *   scale d start from the head's sink (d = 1 is exactly exp(s_h - m) when
 *   m = s_h), and when the key range is cut into chunks only the first chunk
 *   carries the sink.  oracle_chunk_states() writes the per-chunk state that
 *   definition implies, and oracle_merge_states() combines chunk states by
 *   their log-sum-exp weights (the merge formula is not printed on the pages;
 *   the plain reading is used).  The oracle never uses the online form for
 *   its own outputs: it evaluates the definition above in two passes.
 *
 *   "Hosting Qwen on Blackwell" (Perplexity blog), section "Deployment on
 *   GB200 NVL72": KV caches are kept in HND order (heads leading, tokens of a
 *   head contiguous).  The oracle takes explicit strides, so it reads that
 *   layout and any other with unit stride along d.
 *
 * Inputs are bfloat16 bit patterns (uint16) widened exactly to double; sinks
 * are float widened to double.  Build with -O2 -fopenmp, never -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bfloat16 is the upper half of an IEEE-754 binary32; widening is exact. */
static double bf16_to_f64(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * One output row of sink attention over n visible keys, two passes.
 * k_j starts at k + j*k_st, v_j at v + j*v_st, each with unit stride in d.
 * x is caller-provided scratch of n doubles.  with_sink = 0 drops the sink.
 */
static void attend_row(const uint16_t *q, const uint16_t *k, int64_t k_st,
                       const uint16_t *v, int64_t v_st, int64_t n, int D,
                       double scale, double sink, int with_sink, double *x,
                       double *o, double *lse, double *share)
{
    /* pass 1: logits and their maximum, the sink included */
    double M = with_sink ? sink : -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        const uint16_t *kj = k + j * k_st;
        for (int d = 0; d < D; ++d)
            dot += bf16_to_f64(q[d]) * bf16_to_f64(kj[d]);
        x[j] = scale * dot;
        if (x[j] > M) M = x[j];
    }
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (M == -INFINITY) {
        /* no visible key and a -inf sink: an empty softmax, defined as o = 0 */
        if (lse) *lse = -INFINITY;
        if (share) *share = 0.0;
        return;
    }
    /* pass 2: exponentials, denominator (sink term included), weighted sum */
    double es = with_sink ? exp(sink - M) : 0.0;
    double Z = es;
    for (int64_t j = 0; j < n; ++j) {
        x[j] = exp(x[j] - M);
        Z += x[j];
    }
    for (int64_t j = 0; j < n; ++j) {
        const uint16_t *vj = v + j * v_st;
        for (int d = 0; d < D; ++d) o[d] += x[j] * bf16_to_f64(vj[d]);
    }
    for (int d = 0; d < D; ++d) o[d] /= Z;
    if (lse) *lse = M + log(Z);
    if (share) *share = es / Z;
}

/*
 * Prefill over packed variable-length sequences.
 *   q: [T, Hq, D] with strides (q_st, q_sh) in elements, d unit-stride.
 *   k, v: token stride k_st / v_st and head stride k_sh / v_sh; token t of
 *         the packed batch (sequence s owns tokens cu_seqlens[s] ..
 *         cu_seqlens[s+1]-1) of KV head g is at k + t*k_st + g*k_sh.
 *   rows: nrows pairs (global token t, query head h); NULL with nrows = T*Hq
 *         means every (t, h) in token-major order.
 *   out_o: [nrows, D]; out_lse, out_share: [nrows] (either may be NULL).
 * Returns 0, or -1 on a malformed request (bad token or head index).
 */
int oracle_prefill(const uint16_t *q, int64_t q_st, int64_t q_sh,
                   const uint16_t *k, int64_t k_st, int64_t k_sh,
                   const uint16_t *v, int64_t v_st, int64_t v_sh,
                   const float *sinks, const int32_t *cu_seqlens, int num_seqs,
                   int Hq, int Hkv, int D, double scale, int causal,
                   const int64_t *rows, int64_t nrows, int num_threads,
                   double *out_o, double *out_lse, double *out_share)
{
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || num_seqs < 0) return -1;
    const int r = Hq / Hkv;
    const int64_t T = cu_seqlens[num_seqs];
    int64_t maxlen = 0;
    for (int s = 0; s < num_seqs; ++s) {
        int64_t len = (int64_t)cu_seqlens[s + 1] - cu_seqlens[s];
        if (len < 0) return -1;
        if (len > maxlen) maxlen = len;
    }
    int bad = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel reduction(| : bad)
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t t = rows ? rows[2 * i] : i / Hq;
            int h = rows ? (int)rows[2 * i + 1] : (int)(i % Hq);
            if (t < 0 || t >= T || h < 0 || h >= Hq || !x) { bad = 1; continue; }
            int s = 0;
            while (cu_seqlens[s + 1] <= t) ++s;       /* the row's sequence */
            int64_t start = cu_seqlens[s];
            int64_t len = (int64_t)cu_seqlens[s + 1] - start;
            int64_t pos = t - start;                   /* position inside it */
            int64_t n = causal ? pos + 1 : len;        /* visible keys 0..n-1 */
            int g = h / r;
            attend_row(q + t * q_st + h * q_sh,
                       k + start * k_st + g * k_sh, k_st,
                       v + start * v_st + g * v_sh, v_st, n, D, scale,
                       (double)sinks[h], 1, x, out_o + i * D,
                       out_lse ? out_lse + i : NULL, out_share ? out_share + i : NULL);
        }
        free(x);
    }
    return bad ? -1 : 0;
}

/*
 * Chunked prefill: per sequence a chunk of new query tokens against a key
 * range that holds the sequence's earlier tokens followed by the chunk's
 * own.  "Hosting Qwen on Blackwell" (section "Prefillers") processes long
 * inputs on dedicated prefill nodes; the split of one input into chunks is
 * the plain reading of extending that prefill to a cached prefix: query
 * token i of the chunk (0 <= i < len_q) sits at position len_k - len_q + i
 * of the sequence and, causal, sees keys 0 .. len_k - len_q + i (all len_k
 * keys when non-causal).  cu_seqlens_q == cu_seqlens_k is oracle_prefill().
 *   q: [Tq, Hq, D] packed by cu_seqlens_q; k, v packed by cu_seqlens_k with
 *   the strides of oracle_prefill().  Requires len_k >= len_q for every
 *   sequence.  rows: nrows pairs (global query token t, head h); NULL with
 *   nrows = Tq*Hq means all, token-major.
 */
int oracle_prefill_chunked(const uint16_t *q, int64_t q_st, int64_t q_sh,
                           const uint16_t *k, int64_t k_st, int64_t k_sh,
                           const uint16_t *v, int64_t v_st, int64_t v_sh,
                           const float *sinks, const int32_t *cu_seqlens_q,
                           const int32_t *cu_seqlens_k, int num_seqs,
                           int Hq, int Hkv, int D, double scale, int causal,
                           const int64_t *rows, int64_t nrows, int num_threads,
                           double *out_o, double *out_lse, double *out_share)
{
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || num_seqs < 0) return -1;
    const int r = Hq / Hkv;
    const int64_t Tq = cu_seqlens_q[num_seqs];
    int64_t maxlen = 0;
    for (int s = 0; s < num_seqs; ++s) {
        int64_t len_q = (int64_t)cu_seqlens_q[s + 1] - cu_seqlens_q[s];
        int64_t len_k = (int64_t)cu_seqlens_k[s + 1] - cu_seqlens_k[s];
        if (len_q < 0 || len_k < len_q) return -1;
        if (len_k > maxlen) maxlen = len_k;
    }
    int bad = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel reduction(| : bad)
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t t = rows ? rows[2 * i] : i / Hq;
            int h = rows ? (int)rows[2 * i + 1] : (int)(i % Hq);
            if (t < 0 || t >= Tq || h < 0 || h >= Hq || !x) { bad = 1; continue; }
            int s = 0;
            while (cu_seqlens_q[s + 1] <= t) ++s;     /* the row's sequence */
            int64_t len_q = (int64_t)cu_seqlens_q[s + 1] - cu_seqlens_q[s];
            int64_t start_k = cu_seqlens_k[s];
            int64_t len_k = (int64_t)cu_seqlens_k[s + 1] - start_k;
            int64_t pos = (len_k - len_q) + (t - cu_seqlens_q[s]);   /* position in the sequence */
            int64_t n = causal ? pos + 1 : len_k;      /* visible keys 0..n-1 */
            int g = h / r;
            attend_row(q + t * q_st + h * q_sh,
                       k + start_k * k_st + g * k_sh, k_st,
                       v + start_k * v_st + g * v_sh, v_st, n, D, scale,
                       (double)sinks[h], 1, x, out_o + i * D,
                       out_lse ? out_lse + i : NULL, out_share ? out_share + i : NULL);
        }
        free(x);
    }
    return bad ? -1 : 0;
}

/*
 * Decode: one query token per request against its cached keys.
 *   q: [B, Hq, D] with strides (q_sb, q_sh).
 *   k_cache, v_cache: element (b, g, token j, d) at b*kv_sb + g*kv_sh +
 *     j*kv_st + d (HND per request when kv_sh > kv_st).
 *   seq_lens[b] tokens of request b are visible.
 *   rows: nrows pairs (b, h); NULL with nrows = B*Hq means all, b-major.
 */
int oracle_decode(const uint16_t *q, int64_t q_sb, int64_t q_sh,
                  const uint16_t *k_cache, const uint16_t *v_cache,
                  int64_t kv_sb, int64_t kv_sh, int64_t kv_st,
                  const int32_t *seq_lens, int B, const float *sinks,
                  int Hq, int Hkv, int D, double scale,
                  const int64_t *rows, int64_t nrows, int num_threads,
                  double *out_o, double *out_lse, double *out_share)
{
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || B < 0) return -1;
    const int r = Hq / Hkv;
    int64_t maxlen = 0;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < 0) return -1;
        if (seq_lens[b] > maxlen) maxlen = seq_lens[b];
    }
    int bad = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel reduction(| : bad)
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < nrows; ++i) {
            int b = rows ? (int)rows[2 * i] : (int)(i / Hq);
            int h = rows ? (int)rows[2 * i + 1] : (int)(i % Hq);
            if (b < 0 || b >= B || h < 0 || h >= Hq || !x) { bad = 1; continue; }
            int g = h / r;
            attend_row(q + b * q_sb + h * q_sh,
                       k_cache + b * kv_sb + g * kv_sh, kv_st,
                       v_cache + b * kv_sb + g * kv_sh, kv_st, seq_lens[b], D, scale,
                       (double)sinks[h], 1, x, out_o + i * D,
                       out_lse ? out_lse + i : NULL, out_share ? out_share + i : NULL);
        }
        free(x);
    }
    return bad ? -1 : 0;
}

/*
 * Multi-token decode, as the speculative and MTP decoders of "GPT-OSS on day
 * 0" (section "Internal inference engine") and "Hosting Qwen on Blackwell"
 * (section "Decoders") need it: q_len new tokens per request, already
 * appended to the request's cache, verified in one pass.  The pages give no
 * formula; the reading used is plain causal attention of each new token over
 * the cache up to and including its own position:
 *   query t of request b (0 <= t < q_len) sees cached tokens
 *   0 .. len_b - q_len + t.
 * q_len = 1 is oracle_decode(); a row that sees no cached token sees only
 * the sink.
 *   q: [B, q_len, Hq, D] with strides (q_sb, q_st, q_sh), d unit-stride.
 *   caches and seq_lens as in oracle_decode().
 *   rows: nrows triples (b, t, h); NULL with nrows = B*q_len*Hq means all,
 *   in (b, t, h) order.
 */
int oracle_decode_multi(const uint16_t *q, int64_t q_sb, int64_t q_st, int64_t q_sh,
                        const uint16_t *k_cache, const uint16_t *v_cache,
                        int64_t kv_sb, int64_t kv_sh, int64_t kv_st,
                        const int32_t *seq_lens, int B, int q_len, const float *sinks,
                        int Hq, int Hkv, int D, double scale,
                        const int64_t *rows, int64_t nrows, int num_threads,
                        double *out_o, double *out_lse, double *out_share)
{
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || B < 0 || q_len <= 0) return -1;
    const int r = Hq / Hkv;
    int64_t maxlen = 0;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < 0) return -1;
        if (seq_lens[b] > maxlen) maxlen = seq_lens[b];
    }
    int bad = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel reduction(| : bad)
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < nrows; ++i) {
            int b, t, h;
            if (rows) {
                b = (int)rows[3 * i];
                t = (int)rows[3 * i + 1];
                h = (int)rows[3 * i + 2];
            } else {
                b = (int)(i / ((int64_t)q_len * Hq));
                t = (int)((i / Hq) % q_len);
                h = (int)(i % Hq);
            }
            if (b < 0 || b >= B || t < 0 || t >= q_len || h < 0 || h >= Hq || !x) {
                bad = 1;
                continue;
            }
            int64_t n = (int64_t)seq_lens[b] - q_len + t + 1;   /* visible tokens */
            if (n < 0) n = 0;
            int g = h / r;
            attend_row(q + b * q_sb + t * q_st + h * q_sh,
                       k_cache + b * kv_sb + g * kv_sh, kv_st,
                       v_cache + b * kv_sb + g * kv_sh, kv_st, n, D, scale,
                       (double)sinks[h], 1, x, out_o + i * D,
                       out_lse ? out_lse + i : NULL, out_share ? out_share + i : NULL);
        }
        free(x);
    }
    return bad ? -1 : 0;
}

/*
 * Per-chunk states of a decode row when the key range is cut into chunks of
 * split_size tokens: chunk c covers [c*S, min((c+1)*S, len)).  Only the chunk
 * numbered sink_chunk seeds its maximum with the sink (sink_chunk = -1 puts
 * the sink in every chunk; this is wrong and exists as a negative control).
 *   m_c = max(seed_c, max_j x_j),  d_c = [sink here] exp(s - m_c) +
 *   sum_j exp(x_j - m_c),  o_c = sum_j exp(x_j - m_c) v_j / d_c.
 * An empty chunk without the sink is (m, d, o) = (-inf, 0, 0).
 * m is in natural-log units.  out_o: [nrows, num_splits, D];
 * out_m, out_d: [nrows, num_splits].
 */
int oracle_chunk_states(const uint16_t *q, int64_t q_sb, int64_t q_sh,
                        const uint16_t *k_cache, const uint16_t *v_cache,
                        int64_t kv_sb, int64_t kv_sh, int64_t kv_st,
                        const int32_t *seq_lens, int B, const float *sinks,
                        int Hq, int Hkv, int D, double scale,
                        int split_size, int num_splits, int sink_chunk,
                        const int64_t *rows, int64_t nrows, int num_threads,
                        double *out_o, double *out_m, double *out_d)
{
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || B < 0 ||
        split_size <= 0 || num_splits <= 0)
        return -1;
    const int r = Hq / Hkv;
    int bad = 0;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
#pragma omp parallel reduction(| : bad)
    {
        double *x = (double *)malloc(sizeof(double) * (size_t)split_size);
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < nrows; ++i) {
            int b = rows ? (int)rows[2 * i] : (int)(i / Hq);
            int h = rows ? (int)rows[2 * i + 1] : (int)(i % Hq);
            if (b < 0 || b >= B || h < 0 || h >= Hq || !x) { bad = 1; continue; }
            int g = h / r;
            const uint16_t *qr = q + b * q_sb + h * q_sh;
            const uint16_t *kb = k_cache + b * kv_sb + g * kv_sh;
            const uint16_t *vb = v_cache + b * kv_sb + g * kv_sh;
            int64_t len = seq_lens[b];
            double s = (double)sinks[h];
            for (int c = 0; c < num_splits; ++c) {
                int64_t lo = (int64_t)c * split_size;
                int64_t hi = lo + split_size < len ? lo + split_size : len;
                int64_t n = hi > lo ? hi - lo : 0;
                int with_sink = (sink_chunk < 0 || sink_chunk == c) && s != -INFINITY;
                double *oc = out_o + (i * num_splits + c) * D;
                double *mc = out_m + i * num_splits + c;
                double *dc = out_d + i * num_splits + c;
                double M = with_sink ? s : -INFINITY;
                for (int64_t j = 0; j < n; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += bf16_to_f64(qr[d]) * bf16_to_f64(kb[(lo + j) * kv_st + d]);
                    x[j] = scale * dot;
                    if (x[j] > M) M = x[j];
                }
                for (int d = 0; d < D; ++d) oc[d] = 0.0;
                if (M == -INFINITY) { *mc = -INFINITY; *dc = 0.0; continue; }
                double Z = with_sink ? exp(s - M) : 0.0;
                for (int64_t j = 0; j < n; ++j) {
                    x[j] = exp(x[j] - M);
                    Z += x[j];
                }
                for (int64_t j = 0; j < n; ++j)
                    for (int d = 0; d < D; ++d)
                        oc[d] += x[j] * bf16_to_f64(vb[(lo + j) * kv_st + d]);
                for (int d = 0; d < D; ++d) oc[d] /= Z;
                *mc = M;
                *dc = Z;
            }
        }
        free(x);
    }
    return bad ? -1 : 0;
}

/*
 * Merge chunk states of each row into the final row:
 *   M = max_c m_c,  w_c = d_c * exp(m_c - M)  (0 for m_c = -inf),
 *   o = sum_c w_c o_c / sum_c w_c,  lse = M + ln sum_c w_c.
 * A row whose states are all empty gives o = 0, lse = -inf.
 */
int oracle_merge_states(const double *o_parts, const double *m_parts,
                        const double *d_parts, int64_t nrows, int num_splits,
                        int D, double *out_o, double *out_lse)
{
    if (num_splits <= 0 || D <= 0) return -1;
    for (int64_t i = 0; i < nrows; ++i) {
        const double *m = m_parts + i * num_splits;
        const double *dd = d_parts + i * num_splits;
        double M = -INFINITY;
        for (int c = 0; c < num_splits; ++c)
            if (m[c] > M) M = m[c];
        double *o = out_o + i * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (M == -INFINITY) {
            if (out_lse) out_lse[i] = -INFINITY;
            continue;
        }
        double W = 0.0;
        for (int c = 0; c < num_splits; ++c) {
            double w = m[c] == -INFINITY ? 0.0 : dd[c] * exp(m[c] - M);
            W += w;
            const double *oc = o_parts + (i * num_splits + c) * D;
            for (int d = 0; d < D; ++d) o[d] += w * oc[d];
        }
        for (int d = 0; d < D; ++d) o[d] = W > 0.0 ? o[d] / W : 0.0;
        if (out_lse) out_lse[i] = W > 0.0 ? M + log(W) : -INFINITY;
    }
    return 0;
}
