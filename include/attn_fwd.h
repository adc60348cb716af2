/*
 * attn_fwd.h -- C ABI of the MI355X (gfx950) fused attention forward library
 * (libattn_fwd.so).
 *
 * The operation is exact scaled-dot-product attention, forward only, with a
 * per-row log-sum-exp output:
 *
 *   for every batch b, query head h and query row i (kv head hk = h / G,
 *   G = Hq / Hkv):
 *     s_j    = scale * sum_c q[b,h,i,c] * k[b,hk,j,c]     for visible j
 *     o[b,h,i,:] = sum_j softmax(s)_j * v[b,hk,j,:]
 *     lse[b,h,i] = ln sum_j exp(s_j)
 *
 * Sources: "Lab 02 - Forward de flash attention en Triton", sections "La
 * estructura del kernel" (pointers, scale, log-sum-exp per row, one program per
 * batch x head x query tile), "Bloque A" (the wrapper over (B, H, N, d) 16-bit
 * tensors), "Bloque B" (the tiled online-softmax body, fp32 running max, sum
 * and accumulator, causal mask that keeps key <= query), "Bloque C" (the naive
 * definition) and "Errores tipicos" (contiguous inputs; a row attends to
 * itself).  Sliding window and GQA/MQA: "00 - Por que la atencion domina la
 * inferencia", section "Otras tres variantes de attention en esta fase".
 * The tiling and online softmax are from "Optimizaciones de Atencion",
 * section "FlashAttention: Nunca materializar la matriz de atencion": the
 * N x N score matrix is never written to memory.
 *
 * Visibility: key j is visible from query row i iff
 *   causal == 0 : always (window must then be 0);
 *   causal != 0 : j <= i, and when window > 0 also i - j < window (the row
 *                 sees at most `window` keys, itself included).
 * Query head h reads K/V head floor(h / (Hq / Hkv)) (contiguous groups; MQA is
 * Hkv = 1).
 *
 * Layout: all tensors row-major and contiguous.
 *   q, o : (B, Hq,  N, d) elements of `dtype` (16-bit)
 *   k, v : (B, Hkv, N, d) elements of `dtype`
 *   lse  : (B, Hq,  N) float32, natural logarithm; may be NULL (not written)
 * All pointers are device pointers (HIP device memory of the current device).
 *
 * Precision: scores, softmax statistics and the output accumulator are fp32;
 * o is rounded to `dtype` to nearest-even once, at the end.
 *
 * Ownership: the caller allocates, owns and frees every buffer and keeps it
 * alive until the work enqueued on `stream` has finished.  attn_fwd allocates
 * nothing and keeps no mutable global state, so concurrent calls on distinct
 * streams are safe; calls whose outputs overlap race.
 *
 * Errors: every check below happens on the host before anything is enqueued;
 * on any error nothing is launched and o/lse are untouched.  Device faults
 * surface at the caller's next synchronisation.  The library never
 * synchronises.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
typedef enum {
    ATTN_F16 = 0,   /* IEEE binary16 */
    ATTN_BF16 = 1   /* bfloat16 */
} attn_dtype_t;

/* Return codes. */
typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* q, k, v or o is NULL while N > 0 (N == 0 reads nothing) */
    ATTN_ERR_SHAPE = 2,       /* B, Hq, Hkv < 1, N < 0, Hq % Hkv != 0, or sizes overflow */
    ATTN_ERR_UNSUPPORTED = 3, /* d not in {64, 128}, unknown dtype, window < 0, window without causal */
    ATTN_ERR_ARG = 4,         /* scale is not finite */
    ATTN_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned */
    ATTN_ERR_ALIAS = 6,       /* o or lse overlaps q, k, v or each other */
    ATTN_ERR_LAUNCH = 7,      /* the kernel launch itself failed */
    ATTN_ERR_DEVICE = 8,      /* no usable gfx950 device is current */
    ATTN_ERR_WORKSPACE = 9,   /* split-KV workspace smaller than attn_fwd_splitkv_workspace_size */
    ATTN_ERR_SCRATCH = 10     /* attn_fwd_splitkv_noalloc: partials exceed ATTN_NOALLOC_SCRATCH_BYTES */
} attn_status_t;

/*
 * Fused attention forward.  Enqueues the work on `stream` (a hipStream_t;
 * NULL is the null stream) and returns without waiting.  N == 0 is a valid
 * no-op.  scale is any finite float (the usual value is 1/sqrt(d)); it may
 * be zero or negative.  The scaled scores scale * q.k are formed in fp32 and
 * must be finite there; results are undefined when they overflow, and for
 * inputs holding Inf or NaN.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
             int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
             int causal, int64_t window, float scale, int dtype, void *stream);

/*
 * The host-side argument checks of attn_fwd, alone: makes no HIP call,
 * touches no memory behind the pointers, and returns the status attn_fwd
 * would return before launching.
 */
int attn_fwd_validate(const void *q, const void *k, const void *v, const void *o,
                      const float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                      int64_t d, int causal, int64_t window, float scale, int dtype);

/* Static, human-readable name of a status code (never NULL). */
const char *attn_status_str(int status);

/*
 * Describes the kernel configuration attn_fwd would launch for these sizes:
 * writes up to 6 integers to cfg (may be NULL) -- query rows per workgroup,
 * keys per tile, waves per workgroup, workgroups in the grid, query tiles
 * computed with the exact two-term P, and the mask mode (0 none, 1 causal,
 * 2 causal + window) -- and returns the status of the argument checks for a
 * call with non-NULL, aligned, disjoint pointers.
 */
int attn_fwd_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                  int64_t window, int dtype, int64_t *cfg);

/*
 * Tile configurations compiled into the library, for measurement: the count,
 * and for id in [0, count) and head dim d (64 or 128) the description
 * desc[0..5] = {32-row query blocks per wave, waves per workgroup, keys per
 * K/V tile, query rows per workgroup, key groups per workgroup, depth of the
 * LDS tile ring}.  attn_fwd_config_desc returns ATTN_ERR_ARG for a bad id, a
 * bad d or a NULL desc.  Every id is built for d = 64 and d = 128: 0 = 128
 * query rows in 8 waves (two key groups), 1 = 256 rows in 8 waves, 2 = 64
 * rows in 4 waves (two key groups), 3 = 32 rows in one wave, 4 = 32 rows in 4
 * waves (four key groups).
 */
int attn_fwd_num_configs(void);
int attn_fwd_config_desc(int id, int64_t d, int64_t *desc);

/*
 * attn_fwd_plan for a given configuration id (-1 = the automatic choice);
 * writes 7 integers: the 6 of attn_fwd_plan followed by the id used.
 */
int attn_fwd_plan_ex(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                     int64_t window, int dtype, int config_id, int64_t *cfg);

/*
 * attn_fwd with an explicit tile configuration (config_id in
 * [0, attn_fwd_num_configs()), or -1 for the automatic choice that attn_fwd
 * makes).  Same semantics, layout, ownership and errors as attn_fwd, plus
 * ATTN_ERR_ARG for a bad config_id.  Every configuration computes the same
 * function; they differ only in speed.
 */
int attn_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
                int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                int causal, int64_t window, float scale, int dtype, int config_id,
                void *stream);

/*
 * Tile-configuration tuning.  "Lab 02 - Forward de flash attention en Triton",
 * section "Restricciones", fixes the tile sizes on the first pass and leaves
 * autotuning as the polishing step; this is that step for these kernels.
 * Runs attn_fwd_ex on the caller's buffers with every configuration built
 * for d: one untimed call, then `reps` (1 .. 10000) calls between two HIP
 * events on `stream`.  Writes the fastest id to *best_config (the automatic
 * choice when N == 0) and, when ms is not NULL, the mean milliseconds per call
 * of each configuration to ms[0 .. attn_fwd_num_configs()-1] (-1 for ids
 * not built for d).  o and lse are overwritten (every configuration computes
 * the same function).  Unlike every other entry point it waits for the
 * stream (an event synchronisation per configuration) and creates two HIP
 * events; it allocates no device memory.  Errors: those of attn_fwd_validate,
 * ATTN_ERR_NULL for a NULL best_config, ATTN_ERR_ARG for reps out of range,
 * ATTN_ERR_LAUNCH when a launch or an event call fails.
 */
int attn_fwd_autotune(const void *q, const void *k, const void *v, void *o, float *lse,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                      int64_t window, float scale, int dtype, int reps, int *best_config, float *ms,
                      void *stream);

/*
 * ---- Split-KV forward ("FlashDecoding") ----------------------------------
 *
 * The same operation for Nq query rows against Nk keys, with the key range cut
 * into chunks that separate workgroups process in parallel, as in
 * "Optimizaciones de Atencion", section "FlashDecoding": (1) the keys are
 * divided into P chunks of about Nk / P tokens (here whole K/V tiles), (2) each
 * chunk yields, per query row, its local row max m_p, local sum l_p and the
 * partial output normalised within the chunk, and (3) a second kernel merges
 * them: global max m = max_p m_p, each partial output weighted by
 * exp(m_p - m) * l_p, divided by the sum of those weights; the row's
 * log-sum-exp is m + ln of that sum.  The result is the exact attention of
 * attn_fwd (it differs only in rounding).  It fills the GPU when B * Hq * Nq
 * is small: decoding (Nq = 1 or a few new tokens against a long cached
 * sequence) and short prefill grids.
 *
 * Visibility with Nq != Nk: the queries are the last Nq positions of the
 * sequence (bottom-right alignment; the pages do not fix this): query row i
 * sits at position p = Nk - Nq + i, and key j is visible iff
 *   causal == 0 : always (window must then be 0);
 *   causal != 0 : j <= p, and when window > 0 also p - j < window.
 * causal != 0 requires Nq <= Nk (else the first rows would see no key).  With
 * Nq == Nk this is exactly attn_fwd.
 *
 * Layout: q, o (B, Hq, Nq, d); k, v (B, Hkv, Nk, d); lse (B, Hq, Nq) float32,
 * may be NULL; all row-major, contiguous, device memory, 16-bit `dtype`.
 *
 * Workspace: the library allocates nothing.  When the call uses more than one
 * chunk it needs a caller-owned device buffer `workspace` of at least
 * attn_fwd_splitkv_workspace_size(...) bytes, 16-byte aligned, disjoint from
 * every input and output, alive until the stream passes the call; it holds
 * the fp32 partial outputs (chunks x B*Hq*Nq x d) and partial log-sum-exps
 * (chunks x B*Hq*Nq).  Nothing in it needs clearing before the call, and its
 * contents afterwards are unspecified.  Calls that share a workspace must be
 * ordered on one stream.  With one chunk the workspace is not touched and may
 * be NULL.
 *
 * num_splits: the number of chunks wanted, 1 .. 1024, or 0 for the automatic
 * choice (enough workgroups to fill the GPU, at least four K/V tiles per
 * chunk).  The count used is ceil(key tiles / tiles per chunk) with tiles per
 * chunk = ceil(key tiles / num_splits), so it never exceeds num_splits nor the
 * number of key tiles.
 *
 * Errors (checked on the host before anything is enqueued; on error nothing
 * is launched and o, lse and the workspace are untouched): those of attn_fwd
 * with N read as Nq, plus ATTN_ERR_SHAPE for Nk < 0, Nk == 0 < Nq or causal
 * with Nq > Nk; ATTN_ERR_ARG for num_splits outside [0, 1024] or a bad
 * config_id; ATTN_ERR_NULL for a NULL workspace
 * when more than one chunk is used; ATTN_ERR_WORKSPACE when workspace_bytes
 * is too small; ATTN_ERR_ALIGN for a misaligned workspace; ATTN_ERR_ALIAS when
 * it overlaps an input or output.  Enqueues two kernels (attention, then the
 * merge) on `stream`, or one when a single chunk is used.
 */
int attn_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                     int causal, int64_t window, float scale, int dtype, int64_t num_splits,
                     void *workspace, int64_t workspace_bytes, void *stream);

/* attn_fwd_splitkv with an explicit tile configuration (-1 = automatic: with
 * R query rows per head as launched -- G * Nq when the heads are stacked, see
 * attn_fwd_splitkv_plan -- configuration 3, one-wave 32-row workgroups, for
 * R < 32; configuration 0 for 32 <= R <= 128; else the choice attn_fwd
 * makes, with configuration 2 in place of 4). */
int attn_fwd_splitkv_ex(const void *q, const void *k, const void *v, void *o, float *lse,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                        int causal, int64_t window, float scale, int dtype, int64_t num_splits,
                        int config_id, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * attn_fwd_splitkv_ex for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The chunk partials go to a fixed array of
 * ATTN_NOALLOC_SCRATCH_BYTES inside the library (one per device, alive until
 * the process ends) instead of a caller workspace; the caller still owns q, k,
 * v, o and lse.  The call allocates and frees nothing.  The first call on a
 * device looks the array's address up once (hipGetSymbolAddress, with that
 * device current).  Every call on a device shares its array, so calls on one
 * device that may overlap in time (distinct streams without ordering) race
 * and give wrong results; nothing in the array needs clearing between calls.
 * Arguments, layout, results and errors: those of attn_fwd_splitkv_ex, plus
 * ATTN_ERR_SCRATCH (nothing launched) when the partials of the chosen split,
 * attn_fwd_splitkv_workspace_size(...) bytes, exceed the array; a smaller
 * num_splits then fits.  That check is made on the host before any HIP call.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
int attn_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                             int causal, int64_t window, float scale, int dtype, int64_t num_splits,
                             int config_id, void *stream);

/* Bytes of workspace a split-KV call with these arguments needs (0 when it
 * uses one chunk), or minus the status code when the sizes are invalid.  Pure
 * host computation. */
int64_t attn_fwd_splitkv_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                                        int64_t d, int causal, int64_t window, int dtype,
                                        int64_t num_splits, int config_id);

/* The host-side checks of attn_fwd_splitkv_ex alone (no HIP call, no memory
 * behind the pointers touched). */
int attn_fwd_splitkv_validate(const void *q, const void *k, const void *v, const void *o,
                              const float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                              int64_t Nk, int64_t d, int causal, int64_t window, float scale, int dtype,
                              int64_t num_splits, int config_id, const void *workspace,
                              int64_t workspace_bytes);

/* What a split-KV call would launch: writes 9 integers to plan (may be NULL)
 * -- query rows per workgroup, keys per K/V tile, waves per workgroup,
 * workgroups of the attention kernel, chunks used, K/V tiles per chunk,
 * configuration id, workspace bytes, and 1 when the G query heads of each K/V
 * head are stacked into one tile (G > 1 and Nq <= 16: each K/V tile is then
 * read once for all G heads), else 0 -- and returns the status of the size
 * checks. */
int attn_fwd_splitkv_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                          int causal, int64_t window, int dtype, int64_t num_splits, int config_id,
                          int64_t *plan);

/*
 * ---- Paged K/V forward ----------------------------------------------------
 *
 * The split-KV forward reading K and V through a page table, as
 * PagedAttention does ("00 - Por que la atencion domina la inferencia",
 * section "PagedAttention es un problema distinto": the KV cache is kept in
 * small fixed-size blocks, e.g. 16 tokens, with one table of blocks per
 * request, and the attention kernel follows that table instead of reading a
 * flat K and V).  Each batch entry (request) has its own key count.
 *
 * Layout (row-major, contiguous, device memory):
 *   q, o         : (B, Hq, Nq, d) elements of `dtype`
 *   k_pool, v_pool: (num_pages, Hkv, page_size, d) elements of `dtype`
 *   block_table  : (B, max_pages) int32; entry [b][p] is the pool page that
 *                  holds keys p*page_size .. p*page_size + page_size - 1 of
 *                  request b (the same page index in k_pool and v_pool)
 *   seq_lens     : (B,) int32, keys of request b (its cached tokens, the Nq
 *                  new ones included)
 *   lse          : (B, Hq, Nq) float32, may be NULL
 * Key j of request b, K/V head hk, is k_pool[block_table[b][j / page_size]]
 * [hk][j % page_size][:].  Query row i of request b sits at position
 * seq_lens[b] - Nq + i (bottom-right alignment, as for attn_fwd_splitkv);
 * visibility follows the split-KV rules with Nk = seq_lens[b].
 *
 * The device data is not checked on the host: the kernel clamps seq_lens[b]
 * into [0, max_seq_len] and every page index into [0, num_pages), so a bad
 * table reads wrong pages but never leaves the pools.  Block-table entries
 * past ceil(seq_lens[b] / page_size) are not read.  A query row whose
 * position is negative (seq_lens[b] < Nq with causal) sees no key: its output
 * is 0 and its log-sum-exp -inf.  Slots of a page past seq_lens[b] are never
 * read.
 *
 * page_size: a power of two, 8 .. 256.  max_seq_len: an upper bound of every
 * seq_lens[b], at most max_pages * page_size; the work is split over
 * [0, max_seq_len).  Workspace, num_splits and the rest: as attn_fwd_splitkv
 * (num_splits = 0 is automatic).  Errors: those of attn_fwd_splitkv, plus
 * ATTN_ERR_NULL for a NULL k_pool, v_pool, block_table or seq_lens,
 * ATTN_ERR_UNSUPPORTED for a page_size that is not a power of two in
 * [8, 256], ATTN_ERR_SHAPE for num_pages or max_pages < 1 or max_seq_len
 * outside [1, max_pages * page_size], ATTN_ERR_ALIGN for a block_table or
 * seq_lens not 4-byte aligned, ATTN_ERR_ALIAS when o, lse or the workspace
 * overlaps the pools, the table or the lengths.
 */
int attn_fwd_paged(const void *q, const void *k_pool, const void *v_pool, const int32_t *block_table,
                   const int32_t *seq_lens, void *o, float *lse, int64_t B, int64_t Hq, int64_t Hkv,
                   int64_t Nq, int64_t d, int64_t page_size, int64_t num_pages, int64_t max_pages,
                   int64_t max_seq_len, int causal, int64_t window, float scale, int dtype,
                   int64_t num_splits, void *workspace, int64_t workspace_bytes, void *stream);

/* attn_fwd_paged with an explicit tile configuration (-1 = automatic). */
int attn_fwd_paged_ex(const void *q, const void *k_pool, const void *v_pool, const int32_t *block_table,
                      const int32_t *seq_lens, void *o, float *lse, int64_t B, int64_t Hq, int64_t Hkv,
                      int64_t Nq, int64_t d, int64_t page_size, int64_t num_pages, int64_t max_pages,
                      int64_t max_seq_len, int causal, int64_t window, float scale, int dtype,
                      int64_t num_splits, int config_id, void *workspace, int64_t workspace_bytes,
                      void *stream);

/* The host-side checks of attn_fwd_paged_ex alone. */
int attn_fwd_paged_validate(const void *q, const void *k_pool, const void *v_pool, const int32_t *block_table,
                            const int32_t *seq_lens, const void *o, const float *lse, int64_t B, int64_t Hq,
                            int64_t Hkv, int64_t Nq, int64_t d, int64_t page_size, int64_t num_pages,
                            int64_t max_pages, int64_t max_seq_len, int causal, int64_t window, float scale,
                            int dtype, int64_t num_splits, int config_id, const void *workspace,
                            int64_t workspace_bytes);

/* The plan of a paged call, the 9 integers of attn_fwd_splitkv_plan. */
int attn_fwd_paged_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t d, int64_t page_size,
                        int64_t num_pages, int64_t max_pages, int64_t max_seq_len, int causal, int64_t window,
                        int dtype, int64_t num_splits, int config_id, int64_t *plan);

/* Workspace bytes of a paged call (0 with one chunk), or minus the status. */
int64_t attn_fwd_paged_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t d,
                                      int64_t page_size, int64_t num_pages, int64_t max_pages,
                                      int64_t max_seq_len, int causal, int64_t window, int dtype,
                                      int64_t num_splits, int config_id);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
