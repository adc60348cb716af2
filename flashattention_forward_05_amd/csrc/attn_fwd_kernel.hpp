// attn_fwd_kernel.hpp -- fused exact attention forward for gfx950 (MI355X).
//
// One workgroup computes one (batch, query head, query tile) of BM rows; its
// NW waves each own QB blocks of 32 query rows.  The workgroup walks the key /
// value tiles (BN keys each) that at least one of its rows can see, keeping a
// running row max, running row sum and an fp32 output accumulator per row, so
// the N x N score matrix never leaves the chip.  This is the tiled online
// softmax of "Optimizaciones de Atencion", section "FlashAttention: Nunca
// materializar la matriz de atencion", and the kernel body of "Lab 02 - Forward
// de flash attention en Triton", sections "La estructura del kernel" and
// "Bloque B" (query tile outer, key/value tiles inner, fp32 m / l / O, P cast
// to the value dtype before the P.V product, O divided by l and LSE = m + ln l
// at the end).
//
// gfx950 mapping (our design, not the pages'):
//  * Scores are formed transposed, S^T = K . Q^T, with v_mfma_f32_32x32x16
//    (fp16 or bf16 in, fp32 accumulate).  In the 32x32 accumulator a lane
//    holds one column, i.e. one query row, and 16 keys; the other 16 keys of
//    that 32-key block sit in lane ^ 32.  Row max and row sum are therefore
//    in-lane, plus one v_permlane32_swap for the max.
//  * K rows enter the MFMA A operand in the order pi(m) = m with bits 2 and 3
//    exchanged.  Then accumulator register r of lane half g holds key
//    16*(r/8) + 8*g + (r%8): registers 8*t .. 8*t+7 of a lane are 8
//    consecutive keys, which is exactly the B-operand layout of the next MFMA.
//    P^T therefore feeds O^T += V^T . P^T straight from registers.
//  * V stays row-major in LDS; ds_read_b64_tr_b16 returns, to lane j of each
//    16-lane group, column j of the 4 x 16 block the group addressed, which
//    is the V^T A-operand layout (8 consecutive keys of one channel per lane).
//  * K and V tiles are brought to LDS with direct global->LDS loads
//    (global_load_lds_dwordx4), double-buffered: tile t+1 is in flight while
//    tile t is used.  16-byte chunks are XOR-swizzled per row so that the
//    MFMA-operand reads of 16 consecutive rows hit distinct LDS banks.
//  * Softmax runs in base 2: c = |scale| * log2(e) is folded into one FMA per
//    score, p = v_exp_f32(s*c - m).  The running max m is only raised when a
//    row's new max exceeds it by more than TAU (log2 units); p is then at most
//    2^TAU, harmless in fp32 and in the 16-bit P, and the O rescale (an
//    exact algebraic no-op otherwise) is skipped for most tiles.
//  * Query tiles whose first row sees few keys use a two-term P (P_hi + P_lo,
//    both rounded to the 16-bit dtype, two MFMAs) so that the rounding of P
//    does not dominate the error of rows that average only a few values.
//  * Tiles no row of a wave can see are skipped; only tiles that cut the
//    causal diagonal, the window edge or the ragged tail evaluate masks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnfwd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define ATTN_LDS __attribute__((address_space(3)))

enum { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_WINDOW = 2 };

// Raise the running max only when a row's new max exceeds it by more than
// this many powers of two.
constexpr float TAU = 8.0f;

struct Params {
    const uint16_t *q;
    const uint16_t *k;
    const uint16_t *v;
    uint16_t *o;
    float *lse;          // may be null
    int Hq;
    int N;
    int group;           // Hq / Hkv
    int window;          // > 0 only with MASK_WINDOW
    int n_qtiles;        // ceil(N / BM)
    int n_bh;            // B * Hq
    int exact_below;     // a q-tile whose first row sees fewer keys uses two-term P
    float c;             // |scale| * log2(e), at least 2^-100
    uint32_t qsign;      // 0x80008000 when scale < 0 (flips the sign of Q), else 0
};

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 acc) {
    if constexpr (DT == 0)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// Two fp32 values to a packed pair of 16-bit values, round to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
    if constexpr (DT == 0) {
        f16x2 h = {(_Float16)x, (_Float16)y};
        return __builtin_bit_cast(uint32_t, h);
    } else {
        bf16x2 h = {(__bf16)x, (__bf16)y};
        return __builtin_bit_cast(uint32_t, h);
    }
}

template <int DT>
__device__ __forceinline__ float lo_half(uint32_t u) {
    if constexpr (DT == 0)
        return (float)__builtin_bit_cast(f16x2, u)[0];
    else
        return __uint_as_float(u << 16);
}

template <int DT>
__device__ __forceinline__ float hi_half(uint32_t u) {
    if constexpr (DT == 0)
        return (float)__builtin_bit_cast(f16x2, u)[1];
    else
        return __uint_as_float(u & 0xffff0000u);
}

// Max of a value over lanes l and l ^ 32.
__device__ __forceinline__ float max_halves(float x) {
    uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum of a value over lanes l and l ^ 32.
__device__ __forceinline__ float sum_halves(float x) {
    uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row order of K in the QK^T A operand: bits 2 and 3 exchanged.
__device__ __forceinline__ int key_perm(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// XOR swizzle of the 16-byte chunk index within a K/V row in LDS.  For D=128
// a row is 256 B (all 64 banks); for D=64 two rows share the 64 banks.  The
// choice makes both the MFMA A-operand reads of K (16 consecutive rows, same
// chunk) and the transposing reads of V (4 consecutive rows x 4 chunks per
// half-wave) touch distinct banks.
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128)
        return ((row & 3) << 2) | ((row >> 2) & 3);
    else
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

__device__ __forceinline__ void wait_vmem_all() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int D, int DT, int MASK, int QB, int NW, int BN>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(Params p) {
    constexpr int BM = NW * QB * 32;
    constexpr int KT = D / 16;         // 16-wide d steps of S^T = K Q^T
    constexpr int CB = D / 32;         // 32-channel blocks of O^T
    constexpr int KB = BN / 32;        // 32-key blocks of S^T
    constexpr int KS = BN / 16;        // 16-key steps of O^T += V^T P^T
    constexpr int ROWB = D * 2;        // bytes per K/V row
    constexpr int TILEB = BN * ROWB;   // bytes per K or V tile
    constexpr int CHUNKS_PER_ROW = D / 8;
    constexpr int LOADS = (BN * CHUNKS_PER_ROW) / (64 * NW);   // 16-B loads per lane per tensor
    static_assert((BN * CHUNKS_PER_ROW) % (64 * NW) == 0, "tile must split evenly over the waves");
    static_assert(BN % 32 == 0 && (D == 64 || D == 128), "unsupported tile");

    __shared__ __attribute__((aligned(1024))) char smem[2][2][TILEB];   // [stage][K or V]

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5;
    const int l32 = lane & 31;
    const int N = p.N;

    // ---- which (batch*head, query tile) this workgroup owns; for masked
    // runs the heaviest query tiles (most visible keys) are dispatched first.
    const int bid = blockIdx.x;
    const int bh = bid % p.n_bh;
    const int rank = bid / p.n_bh;
    const int qt = (MASK == MASK_NONE) ? rank : (p.n_qtiles - 1 - rank);
    const int b = bh / p.Hq;
    const int h = bh - b * p.Hq;
    const int hkv = (p.Hq / p.group);
    const int64_t kvhead = (int64_t)b * hkv + h / p.group;
    const uint16_t *qp = p.q + (int64_t)bh * N * D;
    const uint16_t *kp = p.k + kvhead * N * D;
    const uint16_t *vp = p.v + kvhead * N * D;

    const int q_tile0 = qt * BM;
    const int qw0 = q_tile0 + wave * QB * 32;             // first row of this wave
    const int w_last = min(qw0 + QB * 32, N) - 1;          // last valid row of this wave
    const bool wave_live = qw0 < N;

    // ---- Q fragments (MFMA B operand): lane holds row qw0 + 32*qb + l32,
    // channels 16*kk + 8*g .. +7.  Rows past N are zero.
    u32x4 qf[QB][KT];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = qw0 + qb * 32 + l32;
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (row < N) {
                x = *(const u32x4 *)(qp + (int64_t)row * D + kk * 16 + g * 8);
                x ^= p.qsign;
            }
            qf[qb][kk] = x;
        }
    }

    // ---- key range seen by the workgroup
    const int q_last = min(q_tile0 + BM, N) - 1;
    int kv_lo = 0, kv_hi = N - 1;
    if constexpr (MASK != MASK_NONE) kv_hi = q_last;
    if constexpr (MASK == MASK_WINDOW) kv_lo = max(0, q_tile0 - p.window + 1);
    const int t_begin = kv_lo / BN;
    const int t_end = kv_hi / BN + 1;

    // ---- two-term P for query tiles whose first row sees few keys
    int min_vis = N;
    if constexpr (MASK != MASK_NONE) min_vis = min(N, q_tile0 + 1);
    if constexpr (MASK == MASK_WINDOW) min_vis = min(min_vis, p.window);
    const bool exact = min_vis < p.exact_below;

    f32x16 oacc[QB][CB];
    float mrun[QB], lsum[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        mrun[qb] = -__builtin_inff();
        lsum[qb] = 0.0f;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][cb][r] = 0.0f;
    }

    // ---- global -> LDS tile loader.  Each wave instruction fills 1 KiB of
    // LDS linearly (lane * 16 B); the lane picks the global chunk that belongs
    // at that swizzled LDS position.  Rows past N read row N-1 (finite data,
    // masked later).
    auto load_tile = [&](int t, int stage) {
        const int j0 = t * BN;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int slot = (i * NW + wave) * 64 + lane;
            const int row = slot / CHUNKS_PER_ROW;
            const int chp = slot % CHUNKS_PER_ROW;
            const int ch = chp ^ swz<D>(row);
            const int64_t grow = min(j0 + row, N - 1);
            const int64_t off = grow * D + ch * 8;
            ATTN_LDS void *kd = (ATTN_LDS void *)(&smem[stage][0][(i * NW + wave) * 1024]);
            ATTN_LDS void *vd = (ATTN_LDS void *)(&smem[stage][1][(i * NW + wave) * 1024]);
            __builtin_amdgcn_global_load_lds((const void *)(kp + off), kd, 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(vp + off), vd, 16, 0, 0);
        }
    };

    load_tile(t_begin, 0);
    wait_vmem_all();
    __syncthreads();

    const float c = p.c;
    for (int t = t_begin; t < t_end; ++t) {
        const int stage = (t - t_begin) & 1;
        if (t + 1 < t_end) load_tile(t + 1, stage ^ 1);

        const int j0 = t * BN;
        bool any = wave_live;
        if constexpr (MASK != MASK_NONE) any = any && (j0 <= w_last);
        if constexpr (MASK == MASK_WINDOW) any = any && (j0 + BN - 1 >= qw0 - p.window + 1);

        if (any) {
            bool edge = (j0 + BN > N);
            if constexpr (MASK != MASK_NONE) edge = edge || (j0 + BN - 1 > qw0);
            if constexpr (MASK == MASK_WINDOW) edge = edge || (j0 < w_last - p.window + 1);

            const char *kl = smem[stage][0];
            const char *vl = smem[stage][1];

            // ---- S^T = K . Q^T
            f32x16 s[KB][QB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < KT; ++kk) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const int row = kb * 32 + key_perm(l32);
                    const int ch = (2 * kk + g) ^ swz<D>(row);
                    const u32x4 a = *(const ATTN_LDS u32x4 *)((const ATTN_LDS char *)kl + row * ROWB + ch * 16);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32<DT>(a, qf[qb][kk], s[kb][qb]);
                }
            }

            // ---- online softmax, one lane per query row
            u32x4 ph[QB][KS], pl[QB][KS];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int qi = qw0 + qb * 32 + l32;
                // visible iff lo <= key offset <= hi, offsets relative to j0 + 8g
                int hi = N - 1 - (j0 + 8 * g);
                int lo = -(1 << 30);
                if (edge) {
                    if constexpr (MASK != MASK_NONE) hi = min(hi, qi - (j0 + 8 * g));
                    if constexpr (MASK == MASK_WINDOW) lo = qi - p.window + 1 - (j0 + 8 * g);
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int off = kb * 32 + 16 * (r / 8) + (r % 8);
                            if (off > hi || off < lo) s[kb][qb][r] = -__builtin_inff();
                        }
                }
                float mx = -__builtin_inff();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
                mx = max_halves(mx);
                const float mxc = mx * c;
                const bool need = mxc > mrun[qb] + TAU;
                if (__builtin_amdgcn_ballot_w64(need) != 0) {
                    const float alpha = need ? __builtin_amdgcn_exp2f(mrun[qb] - mxc) : 1.0f;
                    mrun[qb] = need ? mxc : mrun[qb];
                    lsum[qb] *= alpha;
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[qb][cb][r] *= alpha;
                }
                // a row that has seen no key yet keeps m = -inf; use 0 so that
                // masked scores (-inf) still give p = 0
                const float msub = (mrun[qb] == -__builtin_inff()) ? 0.0f : mrun[qb];
                float rs = 0.0f;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r], c, -msub));
                        s[kb][qb][r] = e;
                        rs += e;
                    }
                lsum[qb] += rs;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int kb = ks / 2, r0 = 8 * (ks % 2);
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        ph[qb][ks][w] = pack2<DT>(s[kb][qb][r0 + 2 * w], s[kb][qb][r0 + 2 * w + 1]);
                }
                if (exact) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int kb = ks / 2, r0 = 8 * (ks % 2);
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const uint32_t hw = ph[qb][ks][w];
                            pl[qb][ks][w] = pack2<DT>(s[kb][qb][r0 + 2 * w] - lo_half<DT>(hw),
                                                      s[kb][qb][r0 + 2 * w + 1] - hi_half<DT>(hw));
                        }
                    }
                }
            }

            // ---- O^T += V^T . P^T
            const int hgrp = lane >> 4;
            const int tt = lane & 15;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const int row0 = ks * 16 + 8 * (hgrp >> 1) + (tt >> 2);
                    const int colb = cb * 64 + 32 * (hgrp & 1) + 8 * (tt & 3);
                    const int ch = colb >> 4, within = colb & 15;
                    const ATTN_LDS char *v0 = (const ATTN_LDS char *)vl + row0 * ROWB +
                                              ((ch ^ swz<D>(row0)) << 4) + within;
                    const ATTN_LDS char *v1 = (const ATTN_LDS char *)vl + (row0 + 4) * ROWB +
                                              ((ch ^ swz<D>(row0 + 4)) << 4) + within;
                    const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)v0);
                    const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)v1);
                    const u32x2 a0 = __builtin_bit_cast(u32x2, t0);
                    const u32x2 a1 = __builtin_bit_cast(u32x2, t1);
                    const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        oacc[qb][cb] = mfma32<DT>(a, ph[qb][ks], oacc[qb][cb]);
                        if (exact) oacc[qb][cb] = mfma32<DT>(a, pl[qb][ks], oacc[qb][cb]);
                    }
                }
            }
        }

        wait_vmem_all();
        __syncthreads();
    }

    // ---- epilogue: O = acc / l, rounded once; LSE = ln 2 * (m + log2 l)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = sum_halves(lsum[qb]);
        const int qi = qw0 + qb * 32 + l32;
        if (qi < N) {
            const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
            uint16_t *orow = p.o + ((int64_t)bh * N + qi) * D;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const int ch = cb * 32 + 8 * j4 + 4 * g;
                    u32x2 w;
                    w[0] = pack2<DT>(oacc[qb][cb][4 * j4 + 0] * inv, oacc[qb][cb][4 * j4 + 1] * inv);
                    w[1] = pack2<DT>(oacc[qb][cb][4 * j4 + 2] * inv, oacc[qb][cb][4 * j4 + 3] * inv);
                    *(u32x2 *)(orow + ch) = w;
                }
            if (p.lse != nullptr && g == 0) {
                const float l2 = lt > 0.0f ? __builtin_amdgcn_logf(lt) : -__builtin_inff();
                p.lse[(int64_t)bh * N + qi] = (mrun[qb] + l2) * 0.69314718055994530942f;
            }
        }
    }
}

}  // namespace attnfwd
