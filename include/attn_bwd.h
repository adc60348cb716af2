/*
 * attn_bwd.h -- C ABI of the backward pass of the fused attention forward
 * (same library, libattn_fwd.so; status codes and dtypes of attn_fwd.h).
 *
 * The operation: for the forward O = softmax(scale * Q K^T + M) V of
 * attn_fwd.h (same visibility rules M, same GQA/MQA head map), and an
 * upstream gradient dO, compute
 *
 *   dq = d(sum dO * O)/dq,  dk = d(sum dO * O)/dk,  dv = d(sum dO * O)/dv,
 *
 * i.e. with P = softmax(scale * Q K^T + M) per (b, h):
 *   dP = dO V^T,  D_i = sum_c dO[i,c] O[i,c],  dS = P * (dP - D)
 *   dv = P^T dO,  dk = scale * dS^T Q,  dq = scale * dS K,
 * where dk and dv of a K/V head sum the contributions of its G query heads.
 *
 * Sources: the pages leave the backward out of scope; "Optimizaciones de
 * Atencion", section "FlashAttention: Nunca materializar la matriz de
 * atencion", says the backward recomputes the scores from Q and K rather
 * than storing them, and that the per-row log-sum-exp of the forward is
 * kept for it ("Lab 02", "La estructura del kernel", stores it for the same
 * reason).  attn_bwd follows that: P is recomputed tile by tile as
 * exp(scale * q.k - lse) from the forward's lse, never stored.
 *
 * Layout (row-major, contiguous, device pointers):
 *   q, o, dout, dq : (B, Hq,  N, d) elements of `dtype` (16-bit)
 *   k, v, dk, dv   : (B, Hkv, N, d) elements of `dtype`
 *   lse            : (B, Hq,  N) float32, natural log, as written by attn_fwd
 *   o and lse must be the forward's outputs for the same q, k, v and mask.
 * Nq = Nk = N only (no split-KV or paged backward).
 *
 * Precision: P and dS are rounded to `dtype` as MFMA operands (as the
 * forward rounds P); every sum is fp32; dq, dk, dv are rounded to `dtype`
 * once.  Results are bitwise reproducible (no atomics).
 *
 * Workspace: the caller passes a device buffer of at least
 * attn_bwd_workspace_size(...) bytes, 16-byte aligned, that nothing else
 * uses while the call runs; the library allocates nothing and keeps no
 * state, so calls on distinct streams with distinct workspaces are safe.
 * Its contents are scratch and are overwritten: per query row D and the
 * lse in base 2, and, for shapes with few K/V heads (MQA), where the query
 * heads of a group are split over several workgroups, their fp32 partial
 * dk and dv (summed by a fourth kernel).
 *
 * Errors (host-side, before anything is enqueued; outputs untouched):
 *   the shape, d, dtype, mask and scale rules of attn_fwd_validate;
 *   ATTN_ERR_NULL for any NULL pointer when N > 0 (lse is required);
 *   ATTN_ERR_WORKSPACE when workspace_bytes is too small;
 *   ATTN_ERR_ALIGN for a 16-bit tensor or the workspace not 16-byte aligned,
 *   or lse not 4-byte aligned;
 *   ATTN_ERR_ALIAS when dq, dk, dv or the workspace overlap an input or each
 *   other.
 * N == 0 is a no-op returning ATTN_OK.  attn_bwd enqueues three (or four) kernels on
 * `stream` (NULL = default) and never synchronises; device faults surface at
 * the caller's next synchronisation.
 */
#ifndef ATTN_BWD_H
#define ATTN_BWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of workspace attn_bwd needs: 8 bytes per query row, rows padded to
 * a multiple of 64 per head (rounded up to 256 bytes), plus 2 * S * B * Hkv
 * * N * d * 4 bytes when the query heads of a K/V group are split S > 1
 * ways (S divides Hq / Hkv and is chosen from the shape: S > 1 only when
 * B * Hkv * ceil(N / 128) < 2048).  -1 for shapes attn_bwd would reject. */
int64_t attn_bwd_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d);

/* Host-side checks only (no HIP call); the status attn_bwd would return
 * before launching. */
int attn_bwd_validate(const void *q, const void *k, const void *v, const void *o, const void *dout,
                      const float *lse, const void *dq, const void *dk, const void *dv, int64_t B,
                      int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal, int64_t window,
                      float scale, int dtype, const void *workspace, int64_t workspace_bytes);

/* The backward pass.  `stream` is a hipStream_t (NULL: default stream). */
int attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
             const float *lse, void *dq, void *dk, void *dv, int64_t B, int64_t Hq, int64_t Hkv,
             int64_t N, int64_t d, int causal, int64_t window, float scale, int dtype,
             void *workspace, int64_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_BWD_H */
