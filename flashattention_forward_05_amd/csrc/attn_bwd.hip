// attn_bwd.hip -- backward of the fused attention forward for gfx950 (MI355X),
// and its C ABI (declared in include/attn_bwd.h).
//
// The pages stop at the forward; they say only that a backward recomputes the
// scores from Q and K instead of storing them, and that the per-row
// log-sum-exp the forward writes is kept for it ("Optimizaciones de Atencion",
// section "FlashAttention: Nunca materializar la matriz de atencion").  This
// file does exactly that: with L = the forward's log-sum-exp, every tile of
//   P  = exp(scale * Q K^T - L)            (recomputed, never stored)
//   dP = dO V^T,   D = rowsum(dO * O),   dS = P * (dP - D)
// feeds the gradients
//   dV = P^T dO,   dK = scale * dS^T Q,   dQ = scale * dS K,
// the plain chain rule through softmax(scale * Q K^T) V.  dK and dV of a K/V
// head sum the contributions of all G query heads that share it.
//
// Three kernels, all on one stream:
//  * attn_bwd_pre_kernel: D and L * log2(e) per query row into the caller's
//    workspace (rows padded to a multiple of 64 with D = 0, L = +inf, which
//    makes every weight of a padding row exactly 0).
//  * attn_bwd_dkdv_kernel: one workgroup per (batch, K/V head, 32*NW keys),
//    each wave owning 32 keys whose K and V rows stay in registers as MFMA
//    operands.  It walks every visible 64-row query tile of every query head
//    of the group; Q and dO tiles (and their D, L rows) arrive in LDS by
//    direct global->LDS loads, double buffered.  S = Q K^T and dP = dO V^T
//    are formed with the query rows in the MFMA A operand, permuted (bits 2
//    and 3 of the row index exchanged) so that the accumulator registers of
//    one lane hold 8 consecutive query rows of one key: exactly the
//    B-operand layout of dV^T += dO^T . P and dK^T += Q^T . dS, whose dO^T
//    and Q^T operands come from transposing LDS reads (ds_read_b64_tr_b16).
//  * attn_bwd_dq_kernel: one workgroup per (batch, query head, 32*NW rows),
//    each wave owning 32 query rows (Q and dO in registers); it walks the
//    visible 64-key K/V tiles, forms S^T = K Q^T and dP^T = V dO^T, and
//    accumulates dQ^T += K^T . dS^T, the same operand scheme as the forward.
// No atomics: each output element is written once by one lane, so results
// are bitwise reproducible.  P and dS are rounded to the 16-bit type for the
// MFMAs (as the forward rounds P), every sum is fp32, outputs are rounded
// once.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdint>

#include "attn_bwd.h"
#include "attn_fwd.h"
#include "attn_fwd_common.hpp"

namespace attnbwd {

using namespace attnfwd;

struct BwdParams {
    const uint16_t *q, *k, *v, *o, *dout;
    const float *lse;
    uint16_t *dq, *dk, *dv;
    float2 *dl;          // workspace: per query row {D, L * log2 e}, (B * Hq, Npad)
    int N;
    int Npad;            // N rounded up to a multiple of 64
    int Hq, Hkv, group;
    int window;          // > 0 only with MASK_WINDOW
    int n_bh;            // B * Hq
    int n_bhk;           // B * Hkv
    int hsplit;          // dK/dV: query heads of a group split over this many workgroups
    float *ws_dkv;       // hsplit > 1: fp32 partial dk (scaled) and dv, 2 x (hsplit, B * Hkv, N, D)
    int n_qtiles;        // dq kernel: query tiles per head
    float c2;            // scale * log2(e)
    float scale;
};

constexpr float kLog2e = 1.4426950408889634f;

// Transposing A-operand fragment from a row-major (rows x D) LDS tile with
// the chunk swizzle swz<D>: lane l receives column (channel) 32*cb + l%32 of
// rows 16*ks + 8*(l/32) .. +7, i.e. the operand X^T of a product whose k
// index runs over the tile's rows.
template <int D>
__device__ __forceinline__ u32x4 tr_frag(const char *tile, int ks, int cb, int lane) {
    constexpr int ROWB = D * 2;
    const int hgrp = lane >> 4;
    const int tt = lane & 15;
    const int row0 = ks * 16 + 8 * (hgrp >> 1) + (tt >> 2);
    const int colb = cb * 64 + 32 * (hgrp & 1) + 8 * (tt & 3);
    const int ch = colb >> 4, within = colb & 15;
    const ATTN_LDS char *a0 = (const ATTN_LDS char *)tile + row0 * ROWB + ((ch ^ swz<D>(row0)) << 4) + within;
    const ATTN_LDS char *a1 =
        (const ATTN_LDS char *)tile + (row0 + 4) * ROWB + ((ch ^ swz<D>(row0 + 4)) << 4) + within;
    const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)a0);
    const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)a1);
    const u32x2 b0 = __builtin_bit_cast(u32x2, t0);
    const u32x2 b1 = __builtin_bit_cast(u32x2, t1);
    return u32x4{b0[0], b0[1], b1[0], b1[1]};
}

// Row-operand fragment: lane l receives channels 16*kk + 8*(l/32) .. +7 of
// tile row `row` (the MFMA A operand with rows along M).
template <int D>
__device__ __forceinline__ u32x4 row_frag(const char *tile, int row, int kk, int g) {
    const int ch = (2 * kk + g) ^ swz<D>(row);
    return *(const ATTN_LDS u32x4 *)((const ATTN_LDS char *)tile + row * (D * 2) + ch * 16);
}

// Direct loads of ROWS rows (from row0, clamped to nvalid - 1) of a
// row-major (*, D) 16-bit tensor into a swizzled LDS tile, spread over the NW
// waves of the workgroup.  Completion is tracked by the caller's vmcnt wait.
template <int D, int NW, int ROWS>
__device__ __forceinline__ void load_rows(const uint16_t *src, int row0, int nvalid, char *tile, int wave,
                                          int lane) {
    constexpr int CPR = D / 8;
    constexpr int LOADS = ROWS * CPR / (64 * NW);
    static_assert(ROWS * CPR % (64 * NW) == 0, "tile must split evenly over the waves");
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(tile + wave * 1024));
    static_for<LOADS>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int slot = (i * NW + wave) * 64 + lane;
        const int row = slot / CPR;
        const int ch = (slot % CPR) ^ swz<D>(row);
        const int64_t grow = min(row0 + row, nvalid - 1);
        lds_dma16_at<i * NW * 1024>(src + grow * D + ch * 8, base);
    });
}

// ---------------------------------------------------------------------------
// D = sum_c dO * O and L * log2(e) per query row; D / 8 lanes per row.
template <int D, int DT>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(BwdParams p) {
    constexpr int LPR = D / 8;
    constexpr int RPB = 256 / LPR;
    const int tid = threadIdx.x;
    const int sub = tid % LPR;
    const int64_t prow = (int64_t)blockIdx.x * RPB + tid / LPR;   // over (B * Hq, Npad)
    const int64_t total = (int64_t)p.n_bh * p.Npad;
    const int64_t bh = prow / p.Npad;
    const int i = (int)(prow - bh * p.Npad);
    const bool valid = prow < total && i < p.N;
    float acc = 0.0f;
    if (valid) {
        const int64_t off = (bh * p.N + i) * D + sub * 8;
        const u32x4 a = *(const u32x4 *)(p.dout + off);
        const u32x4 b = *(const u32x4 *)(p.o + off);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            acc += lo_half<DT>(a[t]) * lo_half<DT>(b[t]) + hi_half<DT>(a[t]) * hi_half<DT>(b[t]);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
    if (sub == 0 && prow < total) {
        float l2 = __builtin_inff();
        if (valid) {
            const float l = p.lse[bh * p.N + i];
            // a row that saw no key has L = -inf: give it zero weights
            l2 = (l == -__builtin_inff()) ? __builtin_inff() : l * kLog2e;
        }
        p.dl[prow] = make_float2(valid ? acc : 0.0f, l2);
    }
}

// ---------------------------------------------------------------------------
// dK and dV: one workgroup per (batch, K/V head, BN = 32 * NW keys).  With
// QG = 2 a second set of NW waves owns the same keys and takes the second
// half of the (head, query tile) steps with its own Q/dO ring; the two
// partial dK, dV are summed in LDS at the end.  At d = 64 the register budget
// of two waves per SIMD is enough; asking for it lets two workgroups share a
// compute unit.
template <int D, int DT, int MASK, int NW, int QG>
__global__ __launch_bounds__(NW * QG * 64) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1)))
void attn_bwd_dkdv_kernel(BwdParams p) {
    constexpr int BN = 32 * NW;
    constexpr int BM = 64;                  // query rows per step
    constexpr int KT = D / 16;
    constexpr int CB = D / 32;
    constexpr int TILEB = BM * D * 2;
    static_assert(QG == 1 || QG == 2, "one or two query groups");
    static_assert(QG == 1 || NW * CB * 16 * 64 * 4 <= 2 * QG * TILEB, "Q ring too small for the dK/dV merge");
    __shared__ __attribute__((aligned(1024))) char qs[2][QG * TILEB];
    __shared__ __attribute__((aligned(1024))) char dos[2][QG * TILEB];
    __shared__ __attribute__((aligned(16))) float2 dls[2][QG * BM];

    const int lane = threadIdx.x & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave = wave_all % NW;         // keys of the wave
    const int qg = wave_all / NW;           // its query group
    const int g = lane >> 5, l32 = lane & 31;
    const int N = p.N;
    const int bid = blockIdx.x;
    const int bhk = bid % p.n_bhk;
    const int rest = bid / p.n_bhk;
    const int hs = rest % p.hsplit;         // which share of the group's query heads
    const int kt = rest / p.hsplit;         // key tiles in ascending order: most visible queries first
    const int gper = p.group / p.hsplit;
    const int b = bhk / p.Hkv;
    const int hk = bhk - b * p.Hkv;
    const int j0 = kt * BN;
    const int jw = j0 + 32 * wave;          // the wave's first key
    const int mykey = jw + l32;

    // K and V rows of the wave's keys: B operands of S = Q K^T and dP = dO V^T
    // (lane: key jw + l32, channels 16 kk + 8 g .. +7)
    u32x4 kf[KT], vf[KT];
    {
        const int key = min(mykey, N - 1);
        const uint16_t *kr = p.k + ((int64_t)bhk * N + key) * D + g * 8;
        const uint16_t *vr = p.v + ((int64_t)bhk * N + key) * D + g * 8;
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
            kf[kk] = *(const u32x4 *)(kr + kk * 16);
            vf[kk] = *(const u32x4 *)(vr + kk * 16);
        }
    }
    f32x16 dka[CB], dva[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        dka[cb] = f32x16{};
        dva[cb] = f32x16{};
    }

    // query tiles that can see any key of [j0, j0 + BN)
    int qt_begin = 0, qt_end = (N + BM - 1) / BM;
    if constexpr (MASK != MASK_NONE) qt_begin = j0 / BM;
    if constexpr (MASK == MASK_WINDOW) qt_end = min(qt_end, (j0 + BN - 1 + p.window - 1) / BM + 1);
    const int nq = max(qt_end - qt_begin, 0);
    const int nsteps = nq * gper;
    // this query group's steps: [my_begin, my_begin + my_count); every wave
    // runs `half` steps so that the workgroup barriers match
    const int half = (nsteps + QG - 1) / QG;
    const int my_begin = qg * half;
    const int my_count = max(0, min(half, nsteps - qg * half));

    auto issue = [&](int s) {
        const int st = my_begin + s;
        const int h = hk * p.group + hs * gper + st / nq;
        const int i0 = (qt_begin + st % nq) * BM;
        const int64_t bh = (int64_t)b * p.Hq + h;
        load_rows<D, NW, BM>(p.q + bh * N * D, i0, N, qs[s & 1] + qg * TILEB, wave, lane);
        load_rows<D, NW, BM>(p.dout + bh * N * D, i0, N, dos[s & 1] + qg * TILEB, wave, lane);
        // D and L rows: 64 x 8 bytes by the 32 low lanes of the group's wave 0
        // (rows padded to a multiple of 64, so always in bounds)
        if (wave == 0 && lane < BM / 2)
            lds_dma16(p.dl + bh * p.Npad + i0 + 2 * lane,
                      __builtin_amdgcn_readfirstlane(lds_addr(&dls[s & 1][qg * BM])));
    };

    if (my_count > 0) issue(0);
    for (int s = 0; s < half; ++s) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        block_sync();
        if (s + 1 < my_count) issue(s + 1);
        if (s >= my_count) continue;
        const int i0 = (qt_begin + (my_begin + s) % nq) * BM;
        const char *qt_l = qs[s & 1] + qg * TILEB;
        const char *dot_l = dos[s & 1] + qg * TILEB;
        const float2 *dl_l = &dls[s & 1][qg * BM];
#pragma unroll
        for (int qb = 0; qb < BM / 32; ++qb) {
            const int qa = i0 + 32 * qb;    // first query row of the block
            bool any = true, edge = false;
            if constexpr (MASK != MASK_NONE) {
                any = qa + 31 >= jw;
                edge = jw + 31 > qa;
            }
            if constexpr (MASK == MASK_WINDOW) {
                any = any && (qa - (jw + 31) < p.window);
                edge = edge || (qa + 31 - jw >= p.window);
            }
            if (!any) continue;

            // S = Q K^T and dP = dO V^T, query rows permuted in the A operand
            f32x16 sacc = f32x16{}, pacc = f32x16{};
            const int arow = qb * 32 + key_perm(l32);
#pragma unroll
            for (int kk = 0; kk < KT; ++kk) {
                sacc = mfma32<DT>(row_frag<D>(qt_l, arow, kk, g), kf[kk], sacc);
                pacc = mfma32<DT>(row_frag<D>(dot_l, arow, kk, g), vf[kk], pacc);
            }

            // register r holds query row qa + 16 (r / 8) + 8 g + r % 8 of key mykey
            float pr[16], dsr[16];
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    // {D, L log2 e} of rows qa + 16 half + 8 g + 2t and + 1
                    const float4 dd = ((const float4 *)(dl_l + 32 * qb + 16 * half + 8 * g))[t];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int r = 8 * half + 2 * t + u;
                        const float dv = u ? dd.z : dd.x;
                        const float l2 = u ? dd.w : dd.y;
                        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], p.c2, -l2));
                        if (edge) {
                            const int qrow = qa + 16 * half + 8 * g + 2 * t + u;
                            bool vis = mykey <= qrow;
                            if constexpr (MASK == MASK_WINDOW) vis = vis && (qrow - mykey < p.window);
                            pv = vis ? pv : 0.0f;
                        }
                        pr[r] = pv;
                        dsr[r] = pv * (pacc[r] - dv);
                    }
                }
            u32x4 pb[2], dsb[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    pb[ks][t] = pack2<DT>(pr[8 * ks + 2 * t], pr[8 * ks + 2 * t + 1]);
                    dsb[ks][t] = pack2<DT>(dsr[8 * ks + 2 * t], dsr[8 * ks + 2 * t + 1]);
                }

            // dV^T += dO^T . P and dK^T += Q^T . dS over the block's 32 rows
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    dva[cb] = mfma32<DT>(tr_frag<D>(dot_l, 2 * qb + ks, cb, lane), pb[ks], dva[cb]);
                    dka[cb] = mfma32<DT>(tr_frag<D>(qt_l, 2 * qb + ks, cb, lane), dsb[ks], dka[cb]);
                }
        }
    }

    // query group 1 hands its partial dK^T and dV^T to group 0 through the
    // idle Q and dO rings
    if constexpr (QG == 2) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        float *bk = (float *)&qs[0][0];
        float *bv = (float *)&dos[0][0];
        if (qg == 1) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    bk[((wave * CB + cb) * 16 + r) * 64 + lane] = dka[cb][r];
                    bv[((wave * CB + cb) * 16 + r) * 64 + lane] = dva[cb][r];
                }
        }
        __syncthreads();
        if (qg == 1) return;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dka[cb][r] += bk[((wave * CB + cb) * 16 + r) * 64 + lane];
                dva[cb][r] += bv[((wave * CB + cb) * 16 + r) * 64 + lane];
            }
    }

    // lane: key mykey, register r: channel 32 cb + 8 (r / 4) + 4 g + r % 4
    if (mykey < N && p.hsplit > 1) {
        // partial sums over this share of the heads, reduced by attn_bwd_dkv_reduce_kernel
        const int64_t part = (int64_t)p.hsplit * p.n_bhk * N * D;
        float *dkr = p.ws_dkv + (((int64_t)hs * p.n_bhk + bhk) * N + mykey) * D;
        float *dvr = dkr + part;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int ch = 32 * cb + 8 * rq + 4 * g;
                *(float4 *)(dkr + ch) = make_float4(p.scale * dka[cb][4 * rq], p.scale * dka[cb][4 * rq + 1],
                                                    p.scale * dka[cb][4 * rq + 2], p.scale * dka[cb][4 * rq + 3]);
                *(float4 *)(dvr + ch) =
                    make_float4(dva[cb][4 * rq], dva[cb][4 * rq + 1], dva[cb][4 * rq + 2], dva[cb][4 * rq + 3]);
            }
    } else if (mykey < N) {
        uint16_t *dkr = p.dk + ((int64_t)bhk * N + mykey) * D;
        uint16_t *dvr = p.dv + ((int64_t)bhk * N + mykey) * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int ch = 32 * cb + 8 * rq + 4 * g;
                const u32x2 wk = {pack2<DT>(p.scale * dka[cb][4 * rq], p.scale * dka[cb][4 * rq + 1]),
                                  pack2<DT>(p.scale * dka[cb][4 * rq + 2], p.scale * dka[cb][4 * rq + 3])};
                const u32x2 wv = {pack2<DT>(dva[cb][4 * rq], dva[cb][4 * rq + 1]),
                                  pack2<DT>(dva[cb][4 * rq + 2], dva[cb][4 * rq + 3])};
                *(u32x2 *)(dkr + ch) = wk;
                *(u32x2 *)(dvr + ch) = wv;
            }
    }
}

// ---------------------------------------------------------------------------
// With split heads: dk / dv = sum of the hsplit fp32 partials, rounded once.
// Four channels per thread; blockIdx.y selects dk (0) or dv (1).
template <int DT>
__global__ __launch_bounds__(256) void attn_bwd_dkv_reduce_kernel(BwdParams p, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // float4 index over (B * Hkv, N, D)
    if (i >= n4) return;
    const int64_t part4 = (int64_t)p.hsplit * n4;                // float4s of one tensor's partials
    const float4 *src = (const float4 *)p.ws_dkv + blockIdx.y * part4 + i;
    float4 acc = src[0];
    for (int h = 1; h < p.hsplit; ++h) {
        const float4 t = src[h * n4];
        acc.x += t.x;
        acc.y += t.y;
        acc.z += t.z;
        acc.w += t.w;
    }
    uint16_t *dst = (blockIdx.y == 0 ? p.dk : p.dv) + 4 * i;
    *(u32x2 *)dst = u32x2{pack2<DT>(acc.x, acc.y), pack2<DT>(acc.z, acc.w)};
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (batch, query head, 32 * NW query rows).  With KG = 2
// a second set of NW waves owns the same rows and takes the second half of
// the key tiles (its own K/V ring); the two partial dQ are summed in LDS at
// the end.  That doubles the waves of a small grid.  The kernel fits two
// waves per SIMD without spilling at both head dims, and asks for them (at
// d = 128 the compiler otherwise settles on one: GQA backward 547 -> 647
// TFLOP/s with two).
template <int D, int DT, int MASK, int NW, int KG>
__global__ __launch_bounds__(NW * KG * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bwd_dq_kernel(BwdParams p) {
    constexpr int BMQ = 32 * NW;
    constexpr int BN = 64;                  // keys per tile
    constexpr int KT = D / 16;
    constexpr int CB = D / 32;
    constexpr int TILEB = BN * D * 2;
    static_assert(KG == 1 || KG == 2, "one or two key groups");
    static_assert(KG == 1 || NW * CB * 16 * 64 * 4 <= 2 * KG * TILEB, "K ring too small for the dQ merge");
    __shared__ __attribute__((aligned(1024))) char ks_[2][KG * TILEB];
    __shared__ __attribute__((aligned(1024))) char vs_[2][KG * TILEB];

    const int lane = threadIdx.x & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave = wave_all % NW;         // query rows of the wave
    const int kg = wave_all / NW;           // its key group
    const int g = lane >> 5, l32 = lane & 31;
    const int N = p.N;
    const int bid = blockIdx.x;
    const int bh = bid % p.n_bh;
    const int rank = bid / p.n_bh;
    const int qt = (MASK == MASK_NONE) ? rank : p.n_qtiles - 1 - rank;   // heaviest query tiles first
    const int b = bh / p.Hq;
    const int h = bh - b * p.Hq;
    const int64_t bhk = (int64_t)b * p.Hkv + h / p.group;
    const int i0 = qt * BMQ;
    const int iw = i0 + 32 * wave;          // the wave's first query row
    const int myq = iw + l32;

    // Q and dO rows: B operands of S^T = K Q^T and dP^T = V dO^T
    u32x4 qf[KT], dof[KT];
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
        qf[kk] = u32x4{0u, 0u, 0u, 0u};
        dof[kk] = u32x4{0u, 0u, 0u, 0u};
    }
    float dv = 0.0f, l2 = __builtin_inff();
    if (myq < N) {
        const uint16_t *qr = p.q + ((int64_t)bh * N + myq) * D + g * 8;
        const uint16_t *dr = p.dout + ((int64_t)bh * N + myq) * D + g * 8;
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
            qf[kk] = *(const u32x4 *)(qr + kk * 16);
            dof[kk] = *(const u32x4 *)(dr + kk * 16);
        }
        const float2 dl = p.dl[(int64_t)bh * p.Npad + myq];
        dv = dl.x;
        l2 = dl.y;
    }
    f32x16 dqa[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) dqa[cb] = f32x16{};

    // key tiles that some row of the workgroup can see
    const int qlast = min(i0 + BMQ, N) - 1;
    int kt_begin = 0, kt_end = (N + BN - 1) / BN;
    if constexpr (MASK != MASK_NONE) kt_end = min(kt_end, qlast / BN + 1);
    if constexpr (MASK == MASK_WINDOW) kt_begin = max(0, i0 - p.window + 1) / BN;
    const int nt = max(kt_end - kt_begin, 0);
    const uint16_t *kh = p.k + bhk * N * D;
    const uint16_t *vh = p.v + bhk * N * D;
    const int wlast = min(iw + 31, N - 1);   // the wave's last valid row
    // this key group's tiles: [my_begin, my_begin + my_count); every wave runs
    // `half` steps so that the workgroup barriers match
    const int half = (nt + KG - 1) / KG;
    const int my_begin = kt_begin + kg * half;
    const int my_count = max(0, min(half, nt - kg * half));

    auto issue = [&](int s) {
        const int jt = (my_begin + s) * BN;
        load_rows<D, NW, BN>(kh, jt, N, ks_[s & 1] + kg * TILEB, wave, lane);
        load_rows<D, NW, BN>(vh, jt, N, vs_[s & 1] + kg * TILEB, wave, lane);
    };

    if (my_count > 0) issue(0);
    for (int s = 0; s < half; ++s) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        block_sync();
        if (s + 1 < my_count) issue(s + 1);
        if (s >= my_count) continue;
        const int j0 = (my_begin + s) * BN;
        bool any = iw < N;
        bool edge = j0 + BN > N;
        if constexpr (MASK != MASK_NONE) {
            any = any && (j0 <= wlast);
            edge = edge || (j0 + BN - 1 > iw);
        }
        if constexpr (MASK == MASK_WINDOW) {
            any = any && (j0 + BN - 1 > iw - p.window);
            edge = edge || (j0 <= wlast - p.window);
        }
        if (!any) continue;
        const char *kl = ks_[s & 1] + kg * TILEB;
        const char *vl = vs_[s & 1] + kg * TILEB;

        u32x4 dsb[BN / 16];
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            f32x16 sacc = f32x16{}, pacc = f32x16{};
            const int arow = kb * 32 + key_perm(l32);
#pragma unroll
            for (int kk = 0; kk < KT; ++kk) {
                sacc = mfma32<DT>(row_frag<D>(kl, arow, kk, g), qf[kk], sacc);
                pacc = mfma32<DT>(row_frag<D>(vl, arow, kk, g), dof[kk], pacc);
            }
            // register r holds key j0 + 32 kb + 16 (r / 8) + 8 g + r % 8 of row myq
            float dsr[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], p.c2, -l2));
                if (edge) {
                    const int key = j0 + 32 * kb + 16 * (r / 8) + 8 * g + (r % 8);
                    bool vis = key < N;
                    if constexpr (MASK != MASK_NONE) vis = vis && key <= myq;
                    if constexpr (MASK == MASK_WINDOW) vis = vis && (myq - key < p.window);
                    pv = vis ? pv : 0.0f;
                }
                dsr[r] = pv * (pacc[r] - dv);
            }
#pragma unroll
            for (int hs = 0; hs < 2; ++hs)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    dsb[2 * kb + hs][t] = pack2<DT>(dsr[8 * hs + 2 * t], dsr[8 * hs + 2 * t + 1]);
        }
        // dQ^T += K^T . dS^T
#pragma unroll
        for (int kstep = 0; kstep < BN / 16; ++kstep)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) dqa[cb] = mfma32<DT>(tr_frag<D>(kl, kstep, cb, lane), dsb[kstep], dqa[cb]);
    }

    // key group 1 hands its partial dQ^T to group 0 through the idle K ring
    if constexpr (KG == 2) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __syncthreads();
        float *buf = (float *)&ks_[0][0];
        if (kg == 1) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) buf[((wave * CB + cb) * 16 + r) * 64 + lane] = dqa[cb][r];
        }
        __syncthreads();
        if (kg == 1) return;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) dqa[cb][r] += buf[((wave * CB + cb) * 16 + r) * 64 + lane];
    }

    // lane: row myq, register r: channel 32 cb + 8 (r / 4) + 4 g + r % 4
    if (myq < N) {
        uint16_t *dqr = p.dq + ((int64_t)bh * N + myq) * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int ch = 32 * cb + 8 * rq + 4 * g;
                const u32x2 w = {pack2<DT>(p.scale * dqa[cb][4 * rq], p.scale * dqa[cb][4 * rq + 1]),
                                 pack2<DT>(p.scale * dqa[cb][4 * rq + 2], p.scale * dqa[cb][4 * rq + 3])};
                *(u32x2 *)(dqr + ch) = w;
            }
    }
}

}  // namespace attnbwd

// ---------------------------------------------------------------------------
// Host side.
namespace {

using attnbwd::BwdParams;

constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxHeads = int64_t(1) << 24;

int64_t padded_rows(int64_t N) { return (N + 63) / 64 * 64; }

// Query heads of a K/V group split over this many dK/dV workgroups: with few
// K/V heads (MQA) the group's heads would otherwise run one after another in
// few, long workgroups.  Aim for 2048 workgroups of 128 keys; the split
// divides G.  Depends on the shape only, so the workspace size does too.
int64_t head_split(int64_t B, int64_t Hq, int64_t Hkv, int64_t N) {
    const int64_t G = Hq / Hkv;
    const int64_t grid4 = B * Hkv * ((N + 127) / 128);
    if (grid4 <= 0) return 1;
    int64_t want = grid4 >= 2048 ? 1 : (2048 + grid4 - 1) / grid4;
    want = std::min(want, G);
    while (want > 1 && G % want != 0) --want;
    return std::max<int64_t>(want, 1);
}

// Workspace: per-row {D, lse log2 e} (B * Hq * Npad float2), then from a
// 256-byte boundary the fp32 partial dk and dv of split heads.
int64_t dl_bytes(int64_t B, int64_t Hq, int64_t N) { return (B * Hq * padded_rows(N) * 8 + 255) / 256 * 256; }
int64_t workspace_bytes_for(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d) {
    const int64_t hs = head_split(B, Hq, Hkv, N);
    return dl_bytes(B, Hq, N) + (hs > 1 ? 2 * hs * B * Hkv * N * d * 4 : 0);
}

bool overlap(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

int check_bwd_sizes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal, int64_t window,
                    float scale, int dtype) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 0 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
    if (N > kMaxN || B > kMaxHeads || Hq > kMaxHeads || B * Hq > kMaxHeads) return ATTN_ERR_SHAPE;
    if (B * Hq * padded_rows(N) > (int64_t)INT_MAX * 64) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (window < 0 || (window > 0 && !causal)) return ATTN_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return ATTN_ERR_ARG;
    return ATTN_OK;
}

// Waves per workgroup of the two main kernels, chosen per call (measured):
// 4 (128 keys or query rows per workgroup), except for masked runs whose
// 128-wide grid has fewer than two workgroups per compute unit: there 2
// (64 wide) halves the longest workgroup, which sets the time of a causal
// run on a small grid (lab N = 4096 causal: 0.257 -> 0.217 ms).  Unmasked
// small grids stay at 4 (lab N = 4096: 0.232 ms at 4, 0.271 ms at 2).
struct Plan {
    int nw_kv, nw_q, kg_q, qg_kv, hsplit;
    int64_t grid_kv, grid_q, grid_pre;
};

template <int D, int DT, int MASK, int NW, int QG>
hipError_t launch_dkdv(const BwdParams &p, int64_t grid, hipStream_t st) {
    hipLaunchKernelGGL((attnbwd::attn_bwd_dkdv_kernel<D, DT, MASK, NW, QG>), dim3((unsigned)grid), dim3(NW * QG * 64),
                       0, st, p);
    return hipGetLastError();
}

template <int D, int DT, int MASK, int NW, int KG>
hipError_t launch_dq(const BwdParams &p, int64_t grid, hipStream_t st) {
    hipLaunchKernelGGL((attnbwd::attn_bwd_dq_kernel<D, DT, MASK, NW, KG>), dim3((unsigned)grid), dim3(NW * KG * 64), 0,
                       st, p);
    return hipGetLastError();
}

template <int D, int DT, int MASK>
hipError_t launch_main(const BwdParams &p, const Plan &pl, hipStream_t st) {
    hipLaunchKernelGGL((attnbwd::attn_bwd_pre_kernel<D, DT>), dim3((unsigned)pl.grid_pre), dim3(256), 0, st, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    bool done = false;
    if constexpr (D == 64) {
        if (pl.qg_kv == 2) {
            err = pl.nw_kv == 4 ? launch_dkdv<D, DT, MASK, 4, 2>(p, pl.grid_kv, st)
                                : launch_dkdv<D, DT, MASK, 2, 2>(p, pl.grid_kv, st);
            done = true;
        }
    }
    if (!done)
        err = pl.nw_kv == 4 ? launch_dkdv<D, DT, MASK, 4, 1>(p, pl.grid_kv, st)
                            : launch_dkdv<D, DT, MASK, 2, 1>(p, pl.grid_kv, st);
    if (err != hipSuccess) return err;
    if (pl.hsplit > 1) {
        const int64_t n4 = (int64_t)p.n_bhk * p.N * D / 4;
        hipLaunchKernelGGL((attnbwd::attn_bwd_dkv_reduce_kernel<DT>), dim3((unsigned)((n4 + 255) / 256), 2), dim3(256),
                           0, st, p, n4);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if constexpr (D == 64) {
        if (pl.kg_q == 2)
            return pl.nw_q == 4 ? launch_dq<D, DT, MASK, 4, 2>(p, pl.grid_q, st)
                                : launch_dq<D, DT, MASK, 2, 2>(p, pl.grid_q, st);
    }
    return pl.nw_q == 4 ? launch_dq<D, DT, MASK, 4, 1>(p, pl.grid_q, st) : launch_dq<D, DT, MASK, 2, 1>(p, pl.grid_q, st);
}

template <int D, int DT>
hipError_t launch_mask(int mask, const BwdParams &p, const Plan &pl, hipStream_t st) {
    if (mask == attnfwd::MASK_NONE) return launch_main<D, DT, attnfwd::MASK_NONE>(p, pl, st);
    if (mask == attnfwd::MASK_CAUSAL) return launch_main<D, DT, attnfwd::MASK_CAUSAL>(p, pl, st);
    return launch_main<D, DT, attnfwd::MASK_WINDOW>(p, pl, st);
}

constexpr int64_t kMinWorkgroups = 512;   // two per compute unit

Plan make_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int mask) {
    Plan pl;
    pl.hsplit = (int)head_split(B, Hq, Hkv, N);
    const int64_t kv4 = B * Hkv * ((N + 127) / 128) * pl.hsplit, q4 = B * Hq * ((N + 127) / 128);
    const bool masked = mask != attnfwd::MASK_NONE;
    pl.nw_kv = (masked && kv4 < kMinWorkgroups) ? 2 : 4;
    pl.nw_q = (masked && q4 < kMinWorkgroups) ? 2 : 4;
    // d = 64 dQ on a grid of fewer than two 128-row workgroups per compute
    // unit: two key groups per workgroup (twice the waves)
    pl.kg_q = (d == 64 && q4 < kMinWorkgroups) ? 2 : 1;
    // and two query groups per dK/dV workgroup likewise
    pl.qg_kv = (d == 64 && kv4 < kMinWorkgroups) ? 2 : 1;
    pl.grid_kv = B * Hkv * ((N + 32 * pl.nw_kv - 1) / (32 * pl.nw_kv)) * pl.hsplit;
    pl.grid_q = B * Hq * ((N + 32 * pl.nw_q - 1) / (32 * pl.nw_q));
    const int64_t rows_per_block = 256 / (d / 8);
    pl.grid_pre = (B * Hq * padded_rows(N) + rows_per_block - 1) / rows_per_block;
    return pl;
}

int bwd_status(hipError_t err) {
    if (err == hipErrorNoBinaryForGpu || err == hipErrorInvalidDeviceFunction || err == hipErrorNoDevice ||
        err == hipErrorInvalidDevice)
        return ATTN_ERR_DEVICE;
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int64_t attn_bwd_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d) {
    if (check_bwd_sizes(B, Hq, Hkv, N, d, 0, 0, 1.0f, ATTN_F16) != ATTN_OK) return -1;
    return workspace_bytes_for(B, Hq, Hkv, N, d);
}

int attn_bwd_validate(const void *q, const void *k, const void *v, const void *o, const void *dout,
                      const float *lse, const void *dq, const void *dk, const void *dv, int64_t B, int64_t Hq,
                      int64_t Hkv, int64_t N, int64_t d, int causal, int64_t window, float scale, int dtype,
                      const void *workspace, int64_t workspace_bytes) {
    const int rc = check_bwd_sizes(B, Hq, Hkv, N, d, causal, window, scale, dtype);
    if (rc != ATTN_OK) return rc;
    if (N == 0) return ATTN_OK;
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return ATTN_ERR_NULL;
    if (workspace_bytes < workspace_bytes_for(B, Hq, Hkv, N, d)) return ATTN_ERR_WORKSPACE;
    const uintptr_t mis = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
                          (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)workspace;
    if ((mis & 15) != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_ALIGN;
    const int64_t qb = B * Hq * N * d * 2, kvb = B * Hkv * N * d * 2, lb = B * Hq * N * 4;
    const void *outs[4] = {dq, dk, dv, workspace};
    const int64_t osz[4] = {qb, kvb, kvb, workspace_bytes};
    const void *ins[6] = {q, k, v, o, dout, lse};
    const int64_t isz[6] = {qb, kvb, kvb, qb, qb, lb};
    for (int a = 0; a < 4; ++a) {
        for (int i = 0; i < 6; ++i)
            if (overlap(outs[a], osz[a], ins[i], isz[i])) return ATTN_ERR_ALIAS;
        for (int c = a + 1; c < 4; ++c)
            if (overlap(outs[a], osz[a], outs[c], osz[c])) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

int attn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout, const float *lse,
             void *dq, void *dk, void *dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
             int64_t window, float scale, int dtype, void *workspace, int64_t workspace_bytes, void *stream) {
    const int rc = attn_bwd_validate(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, window, scale,
                                     dtype, workspace, workspace_bytes);
    if (rc != ATTN_OK || N == 0) return rc;
    const int mask = !causal ? attnfwd::MASK_NONE : (window > 0 ? attnfwd::MASK_WINDOW : attnfwd::MASK_CAUSAL);
    BwdParams p;
    p.q = (const uint16_t *)q;
    p.k = (const uint16_t *)k;
    p.v = (const uint16_t *)v;
    p.o = (const uint16_t *)o;
    p.dout = (const uint16_t *)dout;
    p.lse = lse;
    p.dq = (uint16_t *)dq;
    p.dk = (uint16_t *)dk;
    p.dv = (uint16_t *)dv;
    p.dl = (float2 *)workspace;
    p.N = (int)N;
    p.Npad = (int)padded_rows(N);
    p.Hq = (int)Hq;
    p.Hkv = (int)Hkv;
    p.group = (int)(Hq / Hkv);
    p.window = mask == attnfwd::MASK_WINDOW ? (int)std::min<int64_t>(window, N) : 0;
    p.n_bh = (int)(B * Hq);
    p.n_bhk = (int)(B * Hkv);
    p.hsplit = 1;
    p.ws_dkv = (float *)((char *)workspace + dl_bytes(B, Hq, N));
    const Plan pl = make_plan(B, Hq, Hkv, N, d, mask);
    p.hsplit = pl.hsplit;
    p.n_qtiles = (int)((N + 32 * pl.nw_q - 1) / (32 * pl.nw_q));
    p.c2 = (float)((double)scale * 1.4426950408889634);
    p.scale = scale;
    if (pl.grid_kv > INT_MAX || pl.grid_q > INT_MAX || pl.grid_pre > INT_MAX) return ATTN_ERR_SHAPE;
    hipStream_t st = (hipStream_t)stream;
    hipError_t err;
    if (d == 64)
        err = dtype == ATTN_F16 ? launch_mask<64, 0>(mask, p, pl, st) : launch_mask<64, 1>(mask, p, pl, st);
    else
        err = dtype == ATTN_F16 ? launch_mask<128, 0>(mask, p, pl, st) : launch_mask<128, 1>(mask, p, pl, st);
    return bwd_status(err);
}

}  // extern "C"
