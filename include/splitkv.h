/*
 * splitkv.h -- C ABI of the MI355X (gfx950) split-KV grouped-query decode
 * attention library (libsplitkv.so).
 *
 * The operation ("10 · R4 — decode split-attention dim-parallel rewrite",
 * section 2.1): for every sequence b and query head h, with one query row per
 * head,
 *     o[b][h] = softmax(scale * q[b][h] · K[b][0:nkv_b][h/G]ᵀ) · V[b][0:nkv_b][h/G]
 * over an fp16 KV cache, computed in two stages: a partial kernel runs an
 * online softmax over each split's row range and writes one (mx, S, oc)
 * record per (sequence, split, query head); a combine kernel merges the
 * records ("10 · R4", sections 2.1 and 3.2). One workgroup of the partial
 * kernel serves one (split, KV head, sequence) and computes all G query heads
 * of that KV head, so every K/V row is read from HBM once per group ("Red Lite
 * dev35 — long-context decode: grouped split-K attention", Change).
 *
 * Common conventions for every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller. The library
 *    allocates nothing, never synchronises, and only enqueues work on
 *    `stream` (a hipStream_t passed as void*; NULL is the null stream), so the
 *    calls may be captured into a hipGraph.
 *  - The live length of sequence b is read on the device at run time:
 *    nkv_b = clamp(positions[b] + 1, 0, max_ctx) ("10 · R4", section 2.2).
 *    Launch geometry never depends on it, so one captured graph stays valid as
 *    positions[] advances. positions[] is only read.
 *  - Query head h reads KV head h / G, G = n_head / n_kv_head (contiguous
 *    groups).
 *  - Every argument is validated on the host before any HIP call; on error
 *    nothing is enqueued and a negative status is returned. Nothing throws.
 *  - The functions are reentrant and keep no state. Calls that share a
 *    `partials` buffer must be ordered on one stream.
 *
 * Layouts (row-major, innermost last):
 *   q         float32  [batch][n_head][head_dim]            16-byte aligned
 *   k_cache   fp16     [batch][max_ctx][n_kv_head][head_dim] 16-byte aligned
 *   v_cache   fp16     same as k_cache                       16-byte aligned
 *             (row of position p, KV head g starts at element
 *              ((b*max_ctx + p)*n_kv_head + g)*head_dim; "10 · R4", section 3.2
 *              addresses it as pos*stride_kv + hk*hd, read here as
 *              stride_kv = n_kv_head*head_dim); fp16 values are passed as their
 *              IEEE binary16 bit patterns (uint16_t).
 *   positions int32    [batch]                               4-byte aligned
 *   partials  float32, splitkv_partials_bytes(...) bytes, 16-byte aligned:
 *             one record per (sequence, split, query head) = { mx, S, lo, hi,
 *             oc[0..head_dim) }: mx is the largest score of the split
 *             (natural-log units, -inf when the split is idle), S the sum of
 *             exp(score - mx), oc the exp-weighted V sum (not normalised),
 *             lo/hi the split's row range as int32 bit patterns ("10 · R4",
 *             sections 2.1 and 3.2; slots 2 and 3 are unused padding on the
 *             page). The buffer holds every record's oc first, then every
 *             record's 4-float header { mx, S, lo, hi }:
 *               oc      at float [((b*n_splits + sp)*n_head + h)*head_dim]
 *               header  at float batch*n_splits*n_head*head_dim
 *                                + ((b*n_head + h)*n_splits + sp)*4
 *             (the page stores each record's fields together; apart, a
 *             32-dim slice of oc is one aligned 128-byte line and a head's
 *             headers are contiguous for the combine).
 *   out       float32  [batch][n_head][head_dim]             16-byte aligned
 *
 * Split rule ("10 · R4", section 2.2; "Red Lite dev35", Change): with
 * block_len == 0, chunk = ceil(nkv_b / n_splits); with block_len > 0, chunk =
 * block_len (requires block_len * n_splits >= max_ctx). Split sp covers rows
 * [sp*chunk, min(nkv_b, sp*chunk + chunk)); a split with no rows writes
 * (-inf, 0, lo, hi, 0...) and contributes exactly zero to the merge.
 *
 * Precision and the query range. K and V are used exactly as stored (fp16).
 * For head_dim 8/16/32 the scores and the output are computed in fp32 vector
 * arithmetic from the fp32 q. For head_dim 64/128/256 both products run on
 * the fp16 matrix cores with fp32 accumulation: each element of
 * q' = q * scale * log2(e) enters as an fp16 pair hi = fp16(q'), lo =
 * fp16(q' - hi), so it is carried to about max(2^-22 |q'|, 2^-24), and the
 * softmax weights p likewise as hi + lo pairs. This requires every |q'| to
 * stay below 65504 (the fp16 range of the hi part: larger values become
 * infinite and the output is undefined) and q to be finite; q is device
 * memory, so the host does not check it. Within that range the output meets
 * |err| <= 5e-5 or |err| <= 1e-3 |exact| per element against an exact
 * evaluation of the definition (tested with q up to 4000 x N(0, 1)).
 *
 * Supported shapes: head_dim in {8, 16, 32, 64, 128, 256}; G = n_head /
 * n_kv_head in 1..8; n_splits in 1..65535; n_kv_head and batch <= 65535;
 * max_ctx + n_splits < 2^31; (max_ctx + 64) * n_kv_head * head_dim * 2 bytes
 * (a sequence's K or V cache plus one tile) below 4 GiB; n_splits * n_head *
 * (4 + head_dim) * 4 bytes (a sequence's split records) below 2 GiB.
 */
#ifndef SPLITKV_H
#define SPLITKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SPLITKV_OK 0
#define SPLITKV_EINVAL (-1)       /* null pointer, bad size, bad split rule   */
#define SPLITKV_EUNSUPPORTED (-2) /* head_dim or group size not compiled      */
#define SPLITKV_EALIGN (-3)       /* a pointer breaks its alignment rule      */
#define SPLITKV_ELAUNCH (-4)      /* the HIP runtime refused a launch         */
#define SPLITKV_ESCRATCH (-5)     /* records exceed the no-alloc scratch      */

#define SPLITKV_ABI_VERSION 3

/* Capacity of the device-resident scratch of splitkv_decode_attn_noalloc. */
#define SPLITKV_NOALLOC_SCRATCH_BYTES (16u << 20)

/* ABI version of the loaded library (SPLITKV_ABI_VERSION at build time). */
int splitkv_abi_version(void);

/* Human-readable text for a status code; never NULL, static storage. */
const char *splitkv_strerror(int status);

/* Bytes the caller must provide for `partials`:
 * batch * n_splits * n_head * (4 + head_dim) * 4. Returns 0 for any
 * non-positive argument. */
size_t splitkv_partials_bytes(int batch, int n_head, int head_dim,
                              int n_splits);

/* Partial-kernel workgroups that can be resident on one compute unit at
 * once for (head_dim, group = n_head / n_kv_head), as the compiler's
 * register and LDS allocation of that kernel instantiation allows (a
 * workgroup is 4 waves, one per SIMD; 8 waves at head_dim 256). Used by the
 * split heuristic to size one full round of workgroups. Returns 0 for an
 * unsupported pair. */
int splitkv_workgroups_per_cu(int head_dim, int group);

/* Split heuristic: chooses n_splits (and block_len, 0 = ceil rule) for a
 * shape, from the sequence capacity max_ctx and the GPU's compute-unit count.
 * The aim, from the pages: enough workgroups to fill the GPU ("10 · R4",
 * sections 1 and 3.1; dotLLM issue #199, comment 2, recommendation 1) while
 * each split keeps enough rows that its fixed costs (query load, record
 * write, merge) stay small ("10 · R4", section 3.3; "Red Lite dev35", the
 * block-length table). The rule:
 *   fill = floor(wpc * cu_count / (batch * n_kv_head)), wpc from
 *          splitkv_workgroups_per_cu, capped at 256 / head_dim for head_dim
 *          >= 64 (the matrix-core kernel: more resident workgroups only add
 *          per-split fixed costs there, measured): one full round of
 *          resident workgroups, never a partial second round;
 *   bal  = min(ceil(16 * cu_count / (batch * n_kv_head)), max_ctx / 1024)
 *          when batch > 1, else 0: with several sequences (lengths unknown
 *          to the host) about 16 workgroups per compute unit balance uneven
 *          lengths;
 *   n_splits = min(max(fill, bal, 1), max(max_ctx / 32, 1), 65535): a
 *          full-length split keeps at least 32 rows (one wave's tile).
 * Host only; returns SPLITKV_OK or a negative status. */
int splitkv_pick_splits(int batch, int n_head, int n_kv_head, int head_dim,
                        int max_ctx, int cu_count, int *n_splits,
                        int *block_len);

/* The same rule for n_q query rows per sequence (splitkv_partial_rows /
 * splitkv_decode_attn_rows): counted over the workgroups those launch, where
 * rows that share a workgroup's MFMA columns count once. n_q = 1 is
 * splitkv_pick_splits; SPLITKV_EINVAL also for n_q < 1. */
int splitkv_pick_splits_rows(int batch, int n_q, int n_head, int n_kv_head,
                             int head_dim, int max_ctx, int cu_count,
                             int *n_splits, int *block_len);

/* Partial kernel only: writes every record of `partials`. */
int splitkv_partial(const float *q, const uint16_t *k_cache,
                    const uint16_t *v_cache, const int32_t *positions,
                    float *partials, int batch, int n_head, int n_kv_head,
                    int head_dim, int max_ctx, int n_splits, int block_len,
                    float scale, void *stream);

/* Several query rows per sequence (dotLLM issue #199, comment 1, section 2:
 * seqQ > 1 for speculative verification or chunked prefill, with the causal
 * mask taken from positionOffset). Row t = 0..n_q-1 of sequence b sits at
 * position positions[b] - (n_q - 1) + t, the last row at positions[b]
 * (positionOffset = positions[b] - n_q + 1); row t attends
 * to the cache rows 0 .. its own position (clamped to [0, max_ctx)), so each
 * row is exactly a one-row decode at its position, and a row before position
 * 0 gives 0. The new rows' K/V must already be in the cache
 * (splitkv_append_kv with n_rows = n_q does that).
 *   q         device fp32 [batch][n_q][n_head][head_dim], 16-byte aligned.
 *   partials  splitkv_partials_bytes(batch, n_q * n_head, head_dim,
 *             n_splits) bytes; the records of splitkv_partial with n_head
 *             -> n_q * n_head (record head index t * n_head + h), lo and hi
 *             the split's bounds (those of the last row's live length).
 *   out       device fp32 [batch][n_q][n_head][head_dim].
 * The splits are cut from the last row's live length positions[b] + 1, as
 * for one row; row t's rows end at min(hi, its live length). One partial
 * workgroup per (split, KV head, sequence, block of rows): a block holds the
 * R rows whose (row, head) pairs fit the workgroup's MFMA columns (G * R <= 8
 * in one 16-column block; at head_dim 64 and 128 up to 16 pairs in two
 * blocks: two rows at G = 5..8, four at G = 3 and 4, eight at G = 2; one row
 * otherwise and at head_dim 8/16/32). Each K/V row is read once per block,
 * and when n_splits is a multiple of 8 the blocks of one split run side by
 * side so that the later reads hit the cache. Other arguments and errors as for
 * splitkv_partial / splitkv_decode_attn, plus SPLITKV_EINVAL when n_q < 1,
 * batch * n_q > 65535 or n_q * n_head > 65535. n_q = 1 is exactly
 * splitkv_partial / splitkv_decode_attn. The combine of these records is
 * splitkv_combine with n_head -> n_q * n_head.
 * Non-finite cache values: a cache row that a query row cannot see yet does
 * not reach that row's output, whatever it holds (rows that share a
 * workgroup check the newest rows, which only some of them see, and take
 * any that hold an inf or NaN through a separate per-column step). A V row that a query row does see and that
 * holds inf or NaN (e.g. an fp16 overflow in appended values) makes that
 * row's output non-finite in the same places as the definition, possibly NaN
 * where the definition gives +-inf: the weight p enters the matrix product
 * as two fp16 parts, and inf times the low part can be 0 * inf or have the
 * opposite sign. */
int splitkv_partial_rows(const float *q, const uint16_t *k_cache,
                         const uint16_t *v_cache, const int32_t *positions,
                         float *partials, int batch, int n_q, int n_head,
                         int n_kv_head, int head_dim, int max_ctx, int n_splits,
                         int block_len, float scale, void *stream);
int splitkv_decode_attn_rows(const float *q, const uint16_t *k_cache,
                             const uint16_t *v_cache, const int32_t *positions,
                             float *partials, float *out, int batch, int n_q,
                             int n_head, int n_kv_head, int head_dim,
                             int max_ctx, int n_splits, int block_len,
                             float scale, void *stream);

/* Partial kernel in the per-query-head form: one workgroup per (split, query
 * head, sequence) on grid dim3(n_splits, n_head, batch), each reading its KV
 * head's rows on its own ("10 · R4", section 3.2 launches dim3(S, nh);
 * "Red Lite dev35", Finding: the earlier kernel with one threadgroup per
 * block and query head read each K/V row once per query head of the group).
 * Kept as an A/B baseline against splitkv_partial, which reads every row once
 * per group. Same arguments, records and errors as splitkv_partial; the
 * records are the same values (each query head's arithmetic is identical).
 * head_dim 64, 128 and 256 only (else SPLITKV_EUNSUPPORTED). */
int splitkv_partial_per_head(const float *q, const uint16_t *k_cache,
                             const uint16_t *v_cache, const int32_t *positions,
                             float *partials, int batch, int n_head,
                             int n_kv_head, int head_dim, int max_ctx,
                             int n_splits, int block_len, float scale,
                             void *stream);

/* Combine kernel only: merges the records into `out` ("10 · R4", section 2.1:
 * gmx = max mx, w = exp(mx - gmx), o = sum w*oc / sum w*S, 0 when the weight
 * sum is not positive; a record with mx = -inf has weight 0). */
int splitkv_combine(const float *partials, float *out, int batch, int n_head,
                    int head_dim, int n_splits, void *stream);

/* The whole operation: splitkv_partial then splitkv_combine on `stream`. */
int splitkv_decode_attn(const float *q, const uint16_t *k_cache,
                        const uint16_t *v_cache, const int32_t *positions,
                        float *partials, float *out, int batch, int n_head,
                        int n_kv_head, int head_dim, int max_ctx, int n_splits,
                        int block_len, float scale, void *stream);

/* splitkv_decode_attn for callers that cannot allocate device memory (code
 * under hipGraph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same partial and combine kernels, with the split records
 * kept in a scratch array that the library holds in device memory instead of
 * a caller `partials` buffer. The caller passes q, the caches, positions and
 * out as for splitkv_decode_attn; nothing is allocated and no allocating
 * routine is called.
 *   Limit: the records, splitkv_partials_bytes(batch, n_head, head_dim,
 *   n_splits), must fit SPLITKV_NOALLOC_SCRATCH_BYTES (16 MiB: e.g. up to
 *   1,134 splits for one 28q hd128 sequence, 31 splits for 32 sequences of
 *   32q hd128); larger requests return SPLITKV_ESCRATCH and enqueue nothing.
 *   Sharing: each GPU holds one copy of the scratch (allocated when the
 *   library's device code is loaded on it, kept until the process ends), and
 *   every call on that GPU uses it, so calls that overlap on one GPU (several
 *   streams, or several host threads) race and must be serialised by the
 *   caller. Calls enqueued on one stream are ordered and safe. The scratch
 *   keeps the last call's records; nothing in it needs clearing, because the
 *   partial kernel writes every record of a call before the combine reads it.
 *   The first call on each device resolves the scratch's device address once
 *   (hipGetSymbolAddress with that device current); make that first call
 *   outside graph capture.
 * Other arguments, layouts and errors as for splitkv_decode_attn. */
int splitkv_decode_attn_noalloc(const float *q, const uint16_t *k_cache,
                                const uint16_t *v_cache,
                                const int32_t *positions, float *out, int batch,
                                int n_head, int n_kv_head, int head_dim,
                                int max_ctx, int n_splits, int block_len,
                                float scale, void *stream);

/* KV-cache append, the step before attention in a decode step (dotLLM issue
 * #199, comment 1, section 1: the cache update that precedes attention).
 *   k_new, v_new      device, fp32 [batch][n_rows][n_kv_head][head_dim],
 *                     16-byte aligned; read only.
 *   k_cache, v_cache  device, fp16 bits [batch][max_ctx][n_kv_head][head_dim],
 *                     16-byte aligned; row t of sequence b is written at
 *                     position positions[b] - (n_rows - 1) + t (the last new
 *                     row at positions[b], so the live length afterwards is
 *                     positions[b] + 1); rows whose position falls outside
 *                     [0, max_ctx) are skipped; nothing else is written.
 *   positions         device int32 [batch], read on the device (a captured
 *                     graph appends at the current length on every replay).
 * Conversion: fp32 -> fp16 round to nearest even, overflow to infinity, NaN
 * stays NaN. k_new/v_new must not overlap the caches. Enqueued on `stream`;
 * errors as for splitkv_partial. */
int splitkv_append_kv(const float *k_new, const float *v_new,
                      uint16_t *k_cache, uint16_t *v_cache,
                      const int32_t *positions, int batch, int n_rows,
                      int n_kv_head, int head_dim, int max_ctx, void *stream);

/* One decode step of one layer: splitkv_append_kv with n_rows = 1, then
 * splitkv_decode_attn (dotLLM issue #199, comment 1, section 1: the cache
 * update, then attention over the updated cache). For
 * head_dim 64/128/256 the append is folded into the partial kernel: the
 * workgroup whose split holds position positions[b] converts sequence b's
 * new row, writes it into the caches and uses the converted values for that
 * row, so the step takes two launches instead of three. For head_dim
 * 8/16/32 the append kernel runs first. Either way the caches afterwards and
 * `out` are bit for bit those of the two separate calls.
 *   k_new, v_new      device, fp32 [batch][1][n_kv_head][head_dim], 16-byte
 *                     aligned; read only; must not overlap the caches.
 *   k_cache, v_cache  device, fp16 bits [batch][max_ctx][n_kv_head][head_dim],
 *                     16-byte aligned; row positions[b] is written for every
 *                     b with 0 <= positions[b] < max_ctx (nothing else is
 *                     written), then rows [0, nkv_b) are read.
 *   the other arguments as for splitkv_decode_attn.
 * Errors: as splitkv_decode_attn, plus SPLITKV_EINVAL for a null k_new or
 * v_new and SPLITKV_EALIGN when either is not 16-byte aligned. */
int splitkv_decode_step(const float *q, const float *k_new, const float *v_new,
                        uint16_t *k_cache, uint16_t *v_cache,
                        const int32_t *positions, float *partials, float *out,
                        int batch, int n_head, int n_kv_head, int head_dim,
                        int max_ctx, int n_splits, int block_len, float scale,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPLITKV_H */
