/*
 * oracle.c -- plain, slow, single-threaded fp64 CPU oracle for split-KV
 * ("flash-decoding") grouped-query decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. The test-suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only callers. The product path (the
 * HIP library and its Python binding) never loads, links or calls this file,
 * and this file shares no code, header, table or helper with it.
 *
 * Pages this follows (cited by title and section):
 *   [R4]  "10 · R4 — decode split-attention dim-parallel rewrite"
 *         (yusiwen.cn, minfer CUDA optimisation steps), sections 2.1, 2.2,
 *         3.2 and 4.
 *   [#199] dotLLM issue #199 "perf(cuda): tensor-core (mma.sync FP16) decode
 *         attention kernel", comment 1 sections 0 and 1.
 *   [RL35] "Red Lite dev35 — long-context decode: grouped split-K attention",
 *         sections Finding, Change and Parity.
 *
 * Readings of points the pages leave open (each is restated where it is used):
 *   - query head h reads KV head h / G with G = n_head / n_kv_head (contiguous
 *     groups; [R4] 3.2 uses an undefined `hk`, and [RL35] Finding describes
 *     groups of consecutive query heads served by one KV head);
 *   - the cache row of position p, KV head g starts at element
 *     ((b*max_ctx + p)*n_kv_head + g)*head_dim ([R4] 3.2 addresses rows as
 *     `pos*stride_kv + hk*hd`; stride_kv is read as n_kv_head*head_dim);
 *   - the live length is clamp(positions[b] + 1, 0, max_ctx) ([R4] 2.2 reads
 *     positions[0] + 1; the clamp and the per-sequence index are ours);
 *   - an empty context (nkv = 0) gives o = 0 ([R4] 3.2 combine writes 0 when
 *     the weight sum is not positive);
 *   - scale is an explicit fp32 argument, widened to double ([R4] 3.2 uses it
 *     without defining it).
 *
 * Every function is a plain definition written out, not a fast algorithm:
 * where the method reaches the same value by a faster route (online softmax,
 * split and merge), this file states the value's definition.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 -> double, decoded from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   e == 0      : subnormal, value = (-1)^s * 2^-14 * (f / 1024)
 *   e == 31     : f == 0 -> infinity, else NaN
 *   otherwise   : value = (-1)^s * 2^(e-15) * (1 + f / 1024)
 * [#199] section 1 states that the KV cache is stored in FP16; the oracle reads
 * those stored bits directly, so it sees exactly the values the GPU sees. */
double oracle_f16_to_f64(uint16_t bits)
{
    const int sign = (bits >> 15) & 1;
    const int e = (bits >> 10) & 0x1f;
    const int f = bits & 0x3ff;
    double mag;
    if (e == 0) {
        mag = ldexp((double)f, -24); /* 2^-14 * f / 2^10 */
    } else if (e == 31) {
        mag = (f == 0) ? INFINITY : NAN;
    } else {
        mag = ldexp(1024.0 + (double)f, e - 25); /* 2^(e-15) * (1024+f)/2^10 */
    }
    return sign ? -mag : mag;
}

/* ------------------------------------------------------------------------ */
/* Live context length of one sequence. [R4] 2.2: the kernel reads
 * positions[0] + 1 from device memory at run time. Reading: the value is taken
 * per sequence (positions[b]) and clamped to [0, max_ctx]; the sum is formed
 * in 64 bits so that positions[b] = INT32_MAX does not wrap. */
int oracle_live_length(int32_t position, int32_t max_ctx)
{
    long long n = (long long)position + 1;
    if (n < 0) n = 0;
    if (n > max_ctx) n = max_ctx;
    return (int)n;
}

/* ------------------------------------------------------------------------ */
/* Row range of every split. [R4] 2.2 / 3.2: chunk = ceil(nkv / n_splits),
 * lo = sp * chunk, hi = min(nkv, lo + chunk). [RL35] Change: with a fixed
 * block length the chunk is that length instead (block_len > 0). A split is
 * idle when lo >= hi. Integers only; the GPU must match these bit for bit. */
void oracle_split_bounds(int32_t nkv, int32_t n_splits, int32_t block_len,
                         int32_t *lo, int32_t *hi)
{
    long long chunk;
    if (block_len > 0)
        chunk = block_len;
    else
        chunk = ((long long)nkv + n_splits - 1) / n_splits;
    for (int sp = 0; sp < n_splits; ++sp) {
        long long l = (long long)sp * chunk;
        long long h = l + chunk;
        if (h > nkv) h = nkv;
        lo[sp] = (int32_t)l;
        hi[sp] = (int32_t)h;
    }
}

/* Score of query head h against cache row p: scale * sum_d q[d] * K[p][g][d]
 * in double, with g = h / G. [R4] 2.1 defines o = softmax(q·Kᵀ·scale)·V. */
static double score(const float *qrow, const uint16_t *krow, int head_dim,
                    double scale)
{
    double dot = 0.0;
    for (int d = 0; d < head_dim; ++d)
        dot += (double)qrow[d] * oracle_f16_to_f64(krow[d]);
    return scale * dot;
}

static size_t cache_row(int b, int p, int g, int max_ctx, int n_kv_head,
                        int head_dim)
{
    return (((size_t)b * (size_t)max_ctx + (size_t)p) * (size_t)n_kv_head +
            (size_t)g) * (size_t)head_dim;
}

/* ------------------------------------------------------------------------ */
/* The whole operation, unsplit: for each sequence b and query head h,
 *   s_j = scale * q_h · K_j   for j < nkv_b
 *   m   = max_j s_j
 *   o   = sum_j exp(s_j - m) V_j / sum_j exp(s_j - m)
 * ([R4] 2.1; subtracting m changes nothing mathematically and keeps exp in
 * range). nkv_b = 0 gives o = 0. Output: out[b][h][d] in double. */
void oracle_decode_attn(const float *q, const uint16_t *k_cache,
                        const uint16_t *v_cache, const int32_t *positions,
                        double *out, int batch, int n_head, int n_kv_head,
                        int head_dim, int max_ctx, float scale,
                        double *work /* >= max_ctx doubles */)
{
    const int G = n_head / n_kv_head;
    const double sc = (double)scale;
    for (int b = 0; b < batch; ++b) {
        const int nkv = oracle_live_length(positions[b], max_ctx);
        for (int h = 0; h < n_head; ++h) {
            const int g = h / G;
            const float *qrow = q + ((size_t)b * n_head + h) * head_dim;
            double *o = out + ((size_t)b * n_head + h) * head_dim;
            for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
            if (nkv == 0) continue;
            double m = -INFINITY;
            for (int j = 0; j < nkv; ++j) {
                work[j] = score(qrow, k_cache + cache_row(b, j, g, max_ctx,
                                n_kv_head, head_dim), head_dim, sc);
                if (work[j] > m) m = work[j];
            }
            double denom = 0.0;
            for (int j = 0; j < nkv; ++j) {
                const double w = exp(work[j] - m);
                const uint16_t *vrow = v_cache + cache_row(b, j, g, max_ctx,
                                                           n_kv_head, head_dim);
                denom += w;
                for (int d = 0; d < head_dim; ++d)
                    o[d] += w * oracle_f16_to_f64(vrow[d]);
            }
            for (int d = 0; d < head_dim; ++d) o[d] /= denom;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* What one split contributes, by definition. [R4] 2.1: a split keeps the
 * triple (mx, S, oc): mx the largest score over its rows, S the sum of the
 * exp weights, oc the weighted V sum; the online recurrence of [R4] 2.1
 * reaches exactly
 *   mx = max_{lo<=j<hi} s_j,  S = sum exp(s_j - mx),  oc = sum exp(s_j - mx) V_j
 * and an idle split holds (mx, S, oc) = (-inf, 0, 0) ([R4] 2.2).
 * Record layout (one per sequence, split and query head), doubles:
 *   [0] mx  [1] S  [2] lo  [3] hi  [4 .. 4+head_dim) oc
 * Slots [2], [3] are padding on the page ([R4] 3.2 writes only [0], [1] and
 * [4..]); here they carry the split's row range for the bit-exact check.
 * records: [batch][n_splits][n_head][4 + head_dim]. */
void oracle_split_partials(const float *q, const uint16_t *k_cache,
                           const uint16_t *v_cache, const int32_t *positions,
                           double *records, int batch, int n_head,
                           int n_kv_head, int head_dim, int max_ctx,
                           int n_splits, int block_len, float scale,
                           double *work /* >= max_ctx doubles */,
                           int32_t *lohi /* >= 2 * n_splits ints */)
{
    const int G = n_head / n_kv_head;
    const double sc = (double)scale;
    const size_t pstr = 4 + (size_t)head_dim;
    int32_t *lo = lohi;
    int32_t *hi = lohi + n_splits;
    for (int b = 0; b < batch; ++b) {
        const int nkv = oracle_live_length(positions[b], max_ctx);
        oracle_split_bounds(nkv, n_splits, block_len, lo, hi);
        for (int sp = 0; sp < n_splits; ++sp) {
            for (int h = 0; h < n_head; ++h) {
                double *r = records +
                    (((size_t)b * n_splits + sp) * n_head + h) * pstr;
                const int g = h / G;
                const float *qrow = q + ((size_t)b * n_head + h) * head_dim;
                r[0] = -INFINITY;
                r[1] = 0.0;
                r[2] = (double)lo[sp];
                r[3] = (double)hi[sp];
                for (int d = 0; d < head_dim; ++d) r[4 + d] = 0.0;
                if (lo[sp] >= hi[sp]) continue;
                double m = -INFINITY;
                for (int j = lo[sp]; j < hi[sp]; ++j) {
                    work[j] = score(qrow, k_cache + cache_row(b, j, g, max_ctx,
                                    n_kv_head, head_dim), head_dim, sc);
                    if (work[j] > m) m = work[j];
                }
                double S = 0.0;
                for (int j = lo[sp]; j < hi[sp]; ++j) {
                    const double w = exp(work[j] - m);
                    const uint16_t *vrow = v_cache + cache_row(b, j, g,
                                           max_ctx, n_kv_head, head_dim);
                    S += w;
                    for (int d = 0; d < head_dim; ++d)
                        r[4 + d] += w * oracle_f16_to_f64(vrow[d]);
                }
                r[0] = m;
                r[1] = S;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Merge of the split records, [R4] 2.1 (combine) and 3.2:
 *   gmx = max_sp mx_sp,  w_sp = exp(mx_sp - gmx),
 *   S = sum_sp w_sp S_sp,  acc = sum_sp w_sp oc_sp,  o = acc / S  (0 if S <= 0).
 * Reading: a record with mx = -inf has weight exactly 0, also when every
 * record is idle (gmx = -inf, where exp(-inf - -inf) would be NaN).
 * records: [batch][n_splits][n_head][4 + head_dim]; out: [batch][n_head][hd]. */
void oracle_combine(const double *records, double *out, int batch,
                    int n_splits, int n_head, int head_dim)
{
    const size_t pstr = 4 + (size_t)head_dim;
    for (int b = 0; b < batch; ++b) {
        for (int h = 0; h < n_head; ++h) {
            double gmx = -INFINITY;
            for (int sp = 0; sp < n_splits; ++sp) {
                const double *r = records +
                    (((size_t)b * n_splits + sp) * n_head + h) * pstr;
                if (r[0] > gmx) gmx = r[0];
            }
            double *o = out + ((size_t)b * n_head + h) * head_dim;
            for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
            double S = 0.0;
            for (int sp = 0; sp < n_splits; ++sp) {
                const double *r = records +
                    (((size_t)b * n_splits + sp) * n_head + h) * pstr;
                const double w = (r[0] == -INFINITY) ? 0.0 : exp(r[0] - gmx);
                S += w * r[1];
                for (int d = 0; d < head_dim; ++d) o[d] += w * r[4 + d];
            }
            for (int d = 0; d < head_dim; ++d)
                o[d] = (S > 0.0) ? o[d] / S : 0.0;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary32 -> binary16 with round-to-nearest, ties to even, from the
 * formats' definitions. [#199] section 1 (the half-precision cache update
 * ahead of attention in a decode step) names no rounding rule, so the
 * conversion is the standard one.
 *   - NaN stays NaN (returned as the quiet NaN 0x7E00 with the input's sign;
 *     the payload is not part of the definition);
 *   - the magnitude is rounded to a multiple of the binary16 quantum at its
 *     exponent: 2^(e-10) for a normal result with 2^e <= |x| < 2^(e+1),
 *     e >= -14, and 2^-24 below 2^-14 (the subnormal range);
 *   - a rounded magnitude of 2^16 or more is infinity (65504 is the largest
 *     finite value; 65520, half a quantum above it, rounds to even, i.e. up).
 * Every step is exact in double: x has 24 significant bits and the quanta are
 * powers of two, so |x| / quantum is exact and rint() does the one rounding
 * (in the default round-to-nearest-even mode). */
uint16_t oracle_f32_to_f16(float x)
{
    const double v = (double)x;
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    const double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
    int e2;
    frexp(a, &e2);             /* a = m * 2^e2, 0.5 <= m < 1, so 2^(e2-1) <= a */
    int e = e2 - 1;
    if (a == 0.0 || e < -14) e = -14;  /* subnormal range: quantum 2^-24 */
    const double quantum = ldexp(1.0, e - 10);
    const double r = rint(a / quantum) * quantum;   /* the one rounding */
    if (r >= 65536.0) return (uint16_t)(sign | 0x7C00u);
    if (r < ldexp(1.0, -14))                        /* subnormal or zero */
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
    int re2;
    frexp(r, &re2);            /* rounding may have carried into 2^(e+1) */
    const int E = re2 - 1;
    const unsigned frac = (unsigned)(r / ldexp(1.0, E - 10)) - 1024u;
    return (uint16_t)(sign | (unsigned)((E + 15) << 10) | frac);
}

void oracle_f32_to_f16_array(const float *x, uint16_t *out, size_t n)
{
    for (size_t i = 0; i < n; ++i) out[i] = oracle_f32_to_f16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Cache append, [#199] section 1 (the step before attention): the n_rows new
 * K and V rows of sequence b, fp32 [batch][n_rows][n_kv_head][head_dim], are
 * converted to FP16 and stored at cache positions
 *   p_t = positions[b] - (n_rows - 1) + t,   t = 0 .. n_rows-1,
 * so that the last new row sits at positions[b] and the live length after the
 * append is positions[b] + 1 (the same positions[] array then drives
 * attention). Reading: rows whose p_t falls outside [0, max_ctx) are not
 * written (the pages never write past the cache). Nothing else changes. */
void oracle_append_kv(const float *k_new, const float *v_new,
                      uint16_t *k_cache, uint16_t *v_cache,
                      const int32_t *positions, int batch, int n_rows,
                      int n_kv_head, int head_dim, int max_ctx)
{
    const size_t row = (size_t)n_kv_head * (size_t)head_dim;
    for (int b = 0; b < batch; ++b) {
        for (int t = 0; t < n_rows; ++t) {
            const long long p = (long long)positions[b] - (n_rows - 1) + t;
            if (p < 0 || p >= max_ctx) continue;
            const size_t src = ((size_t)b * n_rows + t) * row;
            const size_t dst = ((size_t)b * max_ctx + (size_t)p) * row;
            for (size_t i = 0; i < row; ++i) {
                k_cache[dst + i] = oracle_f32_to_f16(k_new[src + i]);
                v_cache[dst + i] = oracle_f32_to_f16(v_new[src + i]);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Several query rows per sequence, [#199] section 2: with seqQ > 1 new rows
 * (speculative verification, chunked prefill) the mask inside the online
 * softmax becomes causal, with the first new row at positionOffset. Reading:
 * the n_q rows of sequence b sit at positions
 *   positions[b] - (n_q - 1) + t,   t = 0 .. n_q-1
 * (the last row at positions[b], so positionOffset = positions[b] - n_q + 1),
 * and row t attends to cache rows j <= its own position: it is exactly a
 * one-row decode with live length clamp(positions[b] - (n_q - 1 - t) + 1,
 * 0, max_ctx). q and out: [batch][n_q][n_head][head_dim]. */
void oracle_decode_attn_rows(const float *q, const uint16_t *k_cache,
                             const uint16_t *v_cache, const int32_t *positions,
                             double *out, int batch, int n_q, int n_head,
                             int n_kv_head, int head_dim, int max_ctx,
                             float scale, double *work /* >= max_ctx */)
{
    const size_t cache_seq = (size_t)max_ctx * n_kv_head * head_dim;
    const size_t qrows = (size_t)n_head * head_dim;
    for (int b = 0; b < batch; ++b) {
        for (int t = 0; t < n_q; ++t) {
            long long p = (long long)positions[b] - (n_q - 1 - t);
            if (p < -1) p = -1;             /* live length 0 */
            if (p > max_ctx) p = max_ctx;   /* live length max_ctx */
            const int32_t pos = (int32_t)p;
            const size_t qi = ((size_t)b * n_q + t) * qrows;
            oracle_decode_attn(q + qi, k_cache + (size_t)b * cache_seq,
                               v_cache + (size_t)b * cache_seq, &pos, out + qi,
                               1, n_head, n_kv_head, head_dim, max_ctx, scale,
                               work);
        }
    }
}
