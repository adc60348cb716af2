// attn_fwd_common.hpp -- pieces shared by the attention-forward kernels for
// gfx950: parameter block, MFMA and conversion wrappers, cross-half lane
// reductions, the K row order of the S^T MFMA, the LDS swizzle and the
// vector-memory wait helpers.  The layout facts these rely on are described in
// attn_fwd_kernel.hpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
    int N;               // query rows per head
    int Nk;              // keys per head (= N except for the split-KV entry point)
    int q_off;           // Nk - N: query row i sits at sequence position i + q_off
    int pack_nq;         // > 0: a "head" is one K/V head's G query heads stacked (G * pack_nq
                         // rows); row r then sits at position q_off + r % pack_nq
    int n_splits;        // key splits over workgroups (1 = none; lockstep kernel only)
    int split_tiles;     // key tiles per split
    int split_t0;        // first key tile of split 0 (the first tile any query row sees)
    float *ws_o;         // n_splits > 1: partial outputs (n_splits, B*Hq, N, d), O/l in fp32
    float *ws_ml;        // n_splits > 1: partial log2-sum-exp (n_splits, B*Hq, N), m + log2 l
    // paged K/V (paged = 1): k and v are page pools (num_pages, Hkv, page_size, d);
    // key j of batch b lives in page block_table[b * max_pages + j / page_size] at
    // slot j % page_size; batch b has min(seq_lens[b], Nk) keys
    const int32_t *block_table;
    const int32_t *seq_lens;
    int paged;
    int page_shift;      // log2(page_size), page_size >= 8
    int max_pages;       // block-table entries per batch
    int num_pages;       // pages in each pool (page ids are clamped to it)
    int Hkv;
    int group;           // Hq / Hkv
    int window;          // > 0 only with MASK_WINDOW
    int n_qtiles;        // ceil(N / BM)
    int n_bh;            // B * Hq
    int exact_below;     // a q-tile whose first row sees fewer keys uses two-term P
    int xcd_kv;          // 1 = place all query heads of a K/V head on one XCD (see bh_of)
    int zigzag;          // masked runs: 1 = ranks 0 .. n/2-1 take the tiles heavy-first and the
                         // rest light-first (pairs a heavy and a light tile per compute unit
                         // when two workgroups share one), 0 = heavy-first throughout;
                         // 2 = (128-row configuration, causal) the workgroup of rank r takes
                         // the 64-row query tiles r and ceil(N/64) - 1 - r (equal work)
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

// 2^x on the FMA pipe instead of the transcendental unit: x = n + f with
// n = floor(x) and f in [0, 1) (Cody and Waite's argument reduction), 2^f by
// a cubic fitted for least maximum relative error on [0, 1) (Lawson's
// iteration of weighted least squares, from the mathematics of 2^f alone),
// then 2^n applied by v_ldexp_f32.  Relative error below 7.6e-5 over the
// range the softmax feeds it, far under the 16-bit rounding of P; an x below
// -149 gives 0.  Six VALU instructions against one v_exp_f32.  Built with
// -DATTN_EXP2_POLY_EVERY=k, the steady-state softmax takes the second
// exponential of every k-th packed pair from it; measured slower at every
// share, so the default build uses none.
#ifndef ATTN_EXP2_POLY_EVERY
#define ATTN_EXP2_POLY_EVERY 0
#endif
constexpr int kPolyEvery = ATTN_EXP2_POLY_EVERY > 0 ? ATTN_EXP2_POLY_EVERY : 1 << 20;
__device__ __forceinline__ float exp2_poly(float x) {
    int n;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(n) : "v"(x));
    const float f = __builtin_amdgcn_fractf(x);
    const float p = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(0x1.3f96a4p-4f, f, 0x1.cefc4cp-3f), f,
                                                  0x1.64444cp-1f), f, 0x1.fff632p-1f);
    return __builtin_amdgcn_ldexpf(p, n);
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

// Max / sum of a value over lanes l and l ^ 32.
__device__ __forceinline__ float max_halves(float x) {
    uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

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

// One 16-byte-per-lane direct load from global memory into LDS: lane i's 16
// bytes land at lds_addr + 16 * i (lds_addr is wave-uniform).  Issued as
// inline assembly so that the compiler does not treat it as an LDS store:
// otherwise it waits for every such load in flight before any LDS read whose
// target it cannot attribute to one LDS object, which cancels the
// prefetching.  Completion is instead tracked by the explicit vmcnt waits in
// the kernels, placed before the barrier that publishes a tile.  Nothing else
// in these kernels uses m0.
__device__ __forceinline__ void lds_dma16(const void *gptr, uint32_t lds_addr) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr) : "memory", "m0");
#pragma clang diagnostic pop
}

// The same load with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit
// byte offset (the buffer must be smaller than 4 GiB).
__device__ __forceinline__ void lds_dma16_s(const void *sbase, uint32_t voff, uint32_t lds_addr) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
                 : "memory", "m0");
#pragma clang diagnostic pop
}

// The same two loads with the LDS address given as a wave-uniform base plus
// a compile-time byte offset, added into m0 by the load sequence itself: the
// compiler then keeps one base per ring stage live instead of one address per
// load slot (which otherwise runs the kernels out of scalar registers).
template <int OFF>
__device__ __forceinline__ void lds_dma16_at(const void *gptr, uint32_t lds_base) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_add_u32 m0, %1, %2\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_base), "i"(OFF)
                 : "memory", "m0", "scc");
#pragma clang diagnostic pop
}

template <int OFF>
__device__ __forceinline__ void lds_dma16_s_at(const void *sbase, uint32_t voff, uint32_t lds_base) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base),
                 "i"(OFF)
                 : "memory", "m0", "scc");
#pragma clang diagnostic pop
}

// LDS byte address of a pointer into an LDS object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const ATTN_LDS void *)p;
}

// (batch * query head) handled by workgroup index j (mod n_bh).  Workgroups
// are dealt to the 8 XCDs round-robin by index, so with xcd_kv the index is
// permuted to keep every query head of one K/V head on the same XCD, where
// its K/V tiles then stay in that XCD's L2: j -> XCD j % 8, which owns the
// K/V heads kvg with kvg % 8 == j % 8.  Needs (number of K/V heads over the
// batch) % 8 == 0; bh = kvg * group + index within the group.
__device__ __forceinline__ int bh_of(int j, int n_bh, int group, int xcd_kv) {
    if (!xcd_kv) return j;
    const int x = j % 8, r = j / 8;
    const int kvg = (r / group) * 8 + x;
    return kvg * group + r % group;
}

// Query tile of a masked run for dispatch rank `rank` of n tiles: the tiles
// with the most visible keys (the last ones) go first; with zigzag the second
// half of the ranks walks back up from the lightest tile.
__device__ __forceinline__ int masked_qtile(int rank, int n, int zigzag) {
    const int h = (n + 1) / 2;
    if (!zigzag || rank < h) return n - 1 - rank;
    return rank - h;
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time
// indices for template arguments inside an unrolled loop).
template <int I, int N, class F>
__device__ __forceinline__ void static_for_from(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_from<I + 1, N>(f);
    }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_from<0, N>(f);
}

// Workgroup barrier with no memory-counter waits; the compiler may not move
// memory accesses across it.
__device__ __forceinline__ void block_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt immediate with only the vector-memory counter constrained.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most `younger` tiles (of LPT loads each) of this wave are
// still in flight.
template <int LPT>
__device__ __forceinline__ void wait_tiles(int younger) {
    if (younger >= 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPT));
    else if (younger == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPT));
    else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// Online-softmax update of one wave's tile of scores.  s holds S^T for KB
// blocks of 32 keys (lane = query row, register r of block kb = key
// 32*kb + 16*(r/8) + 8*g + (r%8)); m and l are the row's running max (log2
// units, scaled by c) and its lane-half share of the running sum; o is the
// O^T accumulator.  Writes the packed 16-bit P^T (and for EXACT the rounding
// residual P_lo) in the B-operand layout of O^T += V^T . P^T.
//
// Steady state skips the tile max: p = 2^(s*c - m) against the running max,
// accepted when every lane-half sum stays <= 2^15 (so every p fits the 16-bit
// P and nothing overflows); this is the same algebra with a stale reference
// point, as exact as the rescaled form.  Otherwise -- first tile of a row,
// tiles that cut a mask, two-term P, or a sum out of range -- the tile max is
// taken, m is raised when it grows by more than TAU, and O and l are rescaled.
// On edge tiles a key is visible iff lo <= (key offset from j0 + 8g) <= hi.
template <int DT, int KB, int CB, bool EXACT>
__device__ __forceinline__ void online_softmax_full(f32x16 (&s)[KB], f32x16 (&o)[CB], float &m, float &l,
                                                    u32x4 (&ph)[2 * KB], u32x4 (&pl)[2 * KB], float c,
                                                    bool edge, int hi, int lo);

template <int DT, int KB, int CB, bool EXACT>
__device__ __forceinline__ void online_softmax(f32x16 (&s)[KB], f32x16 (&o)[CB], float &m, float &l,
                                               u32x4 (&ph)[2 * KB], u32x4 (&pl)[2 * KB], float c,
                                               bool edge, int hi, int lo) {
    if constexpr (!EXACT) {
        if (!edge && __builtin_amdgcn_ballot_w64(m == -__builtin_inff()) == 0) {
            float rs = 0.0f, rs1 = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 2 * KB; ++ks) {
                const int kb = ks / 2, r0 = 8 * (ks % 2);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r0 + 2 * q], c, -m));
                    const float x1 = __builtin_fmaf(s[kb][r0 + 2 * q + 1], c, -m);
                    float e1;
                    if ((4 * ks + q) % kPolyEvery == kPolyEvery - 1)
                        e1 = exp2_poly(x1);
                    else
                        e1 = __builtin_amdgcn_exp2f(x1);
                    const uint32_t pk = pack2<DT>(e0, e1);
                    ph[ks][q] = pk;
                    if constexpr (DT == 0) {
                        // fp16: sum the packed pair with one dot product
                        // against (1, 1); the rounding of p moves the row's
                        // log-sum-exp by at most the fp16 unit roundoff.  The
                        // pair is taken from the scalar pk: this compiler
                        // miscompiles __builtin_bit_cast of an element of an
                        // ext_vector_type lvalue (it reads element 0).
                        float &acc = (q & 1) ? rs1 : rs;
                        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk),
                                                     __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
                    } else {
                        rs += e0;
                        rs += e1;
                    }
                }
            }
            rs += rs1;
            if (__builtin_amdgcn_ballot_w64(!(rs <= 32768.0f)) == 0) {
                l += rs;
                return;
            }
        }
    }
    online_softmax_full<DT, KB, CB, EXACT>(s, o, m, l, ph, pl, c, edge, hi, lo);
}

// The general update: mask (edge tiles), tile max, lazy raise of the running
// max with the O / l rescale, then p = 2^(s*c - m).
template <int DT, int KB, int CB, bool EXACT>
__device__ __forceinline__ void online_softmax_full(f32x16 (&s)[KB], f32x16 (&o)[CB], float &m, float &l,
                                                    u32x4 (&ph)[2 * KB], u32x4 (&pl)[2 * KB], float c,
                                                    bool edge, int hi, int lo) {
    if (edge) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int off = kb * 32 + 16 * (r / 8) + (r % 8);
                if (off > hi || off < lo) s[kb][r] = -__builtin_inff();
            }
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = max_halves(mx);
    const float mxc = mx * c;
    const bool need = mxc > m + TAU;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m - mxc) : 1.0f;
        m = need ? mxc : m;
        l *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[cb][r] *= alpha;
    }
    // a row that has seen no key yet keeps m = -inf; use 0 so that masked
    // scores (-inf) still give p = 0
    const float msub = (m == -__builtin_inff()) ? 0.0f : m;
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -msub));
            s[kb][r] = e;
            rs += e;
        }
    l += rs;
#pragma unroll
    for (int ks = 0; ks < 2 * KB; ++ks) {
        const int kb = ks / 2, r0 = 8 * (ks % 2);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t hw = pack2<DT>(s[kb][r0 + 2 * q], s[kb][r0 + 2 * q + 1]);
            ph[ks][q] = hw;
            if constexpr (EXACT)
                pl[ks][q] = pack2<DT>(s[kb][r0 + 2 * q] - lo_half<DT>(hw), s[kb][r0 + 2 * q + 1] - hi_half<DT>(hw));
        }
    }
}

}  // namespace attnfwd
