// attn_fwd_pingpong.hpp -- attention forward for gfx950 with two wave groups
// whose matrix and vector phases alternate ("ping-pong").
//
// Same computation as attn_fwd_kernel.hpp (tiled online softmax; see the
// sources cited there), same operand layouts (S^T = K . Q^T on 32x32x16
// MFMA, P^T straight from the accumulator, V^T through ds_read_b64_tr_b16,
// K/V in LDS through direct global->LDS loads with per-row XOR swizzle).
// What differs is the schedule.
//
// Every wave works on one tile t in two phases:
//   M_t : O^T += V^T . P^T for tile t-1, then S^T = K . Q^T for tile t, on
//         operands already in registers (matrix cores; for d = 128 the V^T
//         operand is read here, the register file cannot hold it ahead)
//   S_t : online softmax of S^T -> P^T, running max / sum, lazy O rescale
//         (vector ALU), plus the LDS reads of K of tile t+1 (and for d = 64
//         of V of tile t) for the next matrix phase
// The workgroup holds two groups of NWG waves, one wave of each per SIMD.
// Group A runs M_0 S_0 M_1 S_1 ...; group B runs the same sequence one
// barrier later, so in every phase one group feeds the matrix cores of a SIMD
// while the other keeps its vector ALU busy, instead of both waves of a SIMD
// asking for the same unit at the same time.
//
// Two ways to split the workgroup's work between the groups:
//  ROWS: the groups own different query rows (BM = 2 * 32 * NWG) and share one
//        K/V ring that group A alone loads;
//  KEYS: the groups own the same rows (BM = 32 * NWG) and split the key range,
//        each with its own ring; their partial (m, l, O) are merged in LDS at
//        the end with the rescale-and-add that "Optimizaciones de Atencion",
//        section "FlashDecoding", uses to combine key chunks.  For small grids.
//
// Putting every LDS read in the softmax phase spreads the operand traffic
// evenly: with 32-row waves a matrix phase would otherwise ask LDS for about
// as many bytes per clock as it delivers.
//
// The ring has four stages.  At M_t a group's stages hold tile t-1 and tile t
// (already read into registers or being read in S_t), tile t+1 (landed before
// S_t) and the stage of tile t-2, refilled with tile t+2 right after the M_t
// barrier.
#pragma once

#include "attn_fwd_common.hpp"

namespace attnfwd {

template <int D, int DT, int MASK, int NWG, bool ROWS, int BN>
struct PingPong {
    static constexpr int NSTAGE = 4;
    static constexpr int QROWS = NWG * 32;               // query rows per group
    static constexpr int BM = ROWS ? 2 * QROWS : QROWS;   // query rows per workgroup
    static constexpr int NWAVES = 2 * NWG;
    static constexpr int KT = D / 16;
    static constexpr int CB = D / 32;
    static constexpr int KB = BN / 32;
    static constexpr int KS = BN / 16;
    static constexpr int ROWB = 2 * D;
    static constexpr int TILEB = BN * ROWB;
    static constexpr int CPR = D / 8;                     // 16-B chunks per K/V row
    static constexpr int LOADS = BN * CPR / (64 * NWG);   // loads per lane per tensor per tile
    static constexpr int LPT = 2 * LOADS;
    static constexpr int RINGS = ROWS ? 1 : 2;
    static constexpr int STAGEB = RINGS * TILEB;          // bytes of one stage array
    // V^T operands are read ahead in the softmax phase when registers allow
    // (d = 64); for d = 128 the matrix phase reads them itself.
    static constexpr bool VPRE = (D == 64);
    static_assert((BN * CPR) % (64 * NWG) == 0, "tile must split evenly over the loading waves");
    static_assert(BN % 32 == 0 && (D == 64 || D == 128), "unsupported tile");

    struct W {
        const uint16_t *kp, *vp;
        int N, window, lane, g, l32, wq, grp;
        int qw0, w_last;          // first / last valid query row of this wave
        int my_begin, my_count;   // this group's key tiles (absolute first, count)
        int T;                    // number of tiles in the (workgroup-uniform) phase sequence
        bool loader;
        float c;
        int ring_off;
        int koff[KT];             // per-lane LDS byte offsets of the K operand reads
        int voff[2 * CB];         // ... and of the V^T transposing reads
        char *kst[NSTAGE], *vst[NSTAGE];
    };
    struct St {
        u32x4 qf[KT];
        f32x16 o[CB];
        f32x16 s[KB];
        u32x4 ph[KS], pl[KS];
        u32x4 ka[KT][KB];         // K operand of the next S^T, read during a softmax phase
        u32x4 va[KS][CB];         // V^T operand of the next P.V, read during a softmax phase
        float m, l;
    };

    static __device__ __forceinline__ bool visible(const W &w, int abs_tile) {
        bool any = w.qw0 < w.N;
        if constexpr (MASK != MASK_NONE) any = any && (abs_tile * BN <= w.w_last);
        if constexpr (MASK == MASK_WINDOW) any = any && (abs_tile * BN + BN - 1 >= w.qw0 - w.window + 1);
        return any;
    }

    // direct loads of tile (absolute index) into the given stage arrays
    static __device__ __forceinline__ void load_tile(const W &w, int abs_tile, char *kdst, char *vdst) {
        const int j0 = abs_tile * BN;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int slot = (i * NWG + w.wq) * 64 + w.lane;
            const int row = slot / CPR;
            const int ch = (slot % CPR) ^ swz<D>(row);
            const int64_t grow = min(j0 + row, w.N - 1);
            const int64_t off = grow * D + ch * 8;
            const int lds_off = w.ring_off + (i * NWG + w.wq) * 1024;
            lds_dma16(w.kp + off, __builtin_amdgcn_readfirstlane(lds_addr(kdst + lds_off)));
            lds_dma16(w.vp + off, __builtin_amdgcn_readfirstlane(lds_addr(vdst + lds_off)));
        }
    }

    // LDS -> registers: the K operand of a tile (kl) ...
    static __device__ __forceinline__ void read_k(const W &w, St &st, const char *kl) {
#pragma unroll
        for (int kk = 0; kk < KT; ++kk)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                st.ka[kk][kb] = *(const ATTN_LDS u32x4 *)((const ATTN_LDS char *)kl + w.koff[kk] + kb * 32 * ROWB);
    }

    // ... and the V^T operand (vl), two transposing reads per fragment
    static __device__ __forceinline__ void read_v(const W &w, St &st, const char *vl) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const ATTN_LDS char *b = (const ATTN_LDS char *)vl + ks * 16 * ROWB;
                const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)(b + w.voff[2 * cb]));
                const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)(b + w.voff[2 * cb + 1]));
                const u32x2 a0 = __builtin_bit_cast(u32x2, t0);
                const u32x2 a1 = __builtin_bit_cast(u32x2, t1);
                st.va[ks][cb] = u32x4{a0[0], a0[1], a1[0], a1[1]};
            }
    }

    // S^T = K . Q^T from registers
    static __device__ __forceinline__ void qk(St &st) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) st.s[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KT; ++kk)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) st.s[kb] = mfma32<DT>(st.ka[kk][kb], st.qf[kk], st.s[kb]);
    }

    // O^T += V^T . P^T from registers (P_lo as well when EXACT)
    template <bool EXACT>
    static __device__ __forceinline__ void pv(St &st) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                st.o[cb] = mfma32<DT>(st.va[ks][cb], st.ph[ks], st.o[cb]);
                if constexpr (EXACT) st.o[cb] = mfma32<DT>(st.va[ks][cb], st.pl[ks], st.o[cb]);
            }
    }

    // online softmax of st.s (tile abs_tile) -> st.ph / st.pl
    template <bool EXACT>
    static __device__ __forceinline__ void softmax(const W &w, St &st, int abs_tile) {
        const int j0 = abs_tile * BN;
        bool edge = (j0 + BN > w.N);
        if constexpr (MASK != MASK_NONE) edge = edge || (j0 + BN - 1 > w.qw0);
        if constexpr (MASK == MASK_WINDOW) edge = edge || (j0 < w.w_last - w.window + 1);
        const int qi = w.qw0 + w.l32;
        int hi = w.N - 1 - (j0 + 8 * w.g);
        int lo = -(1 << 30);
        if constexpr (MASK != MASK_NONE) hi = min(hi, qi - (j0 + 8 * w.g));
        if constexpr (MASK == MASK_WINDOW) lo = qi - w.window + 1 - (j0 + 8 * w.g);
        online_softmax<DT, KB, CB, EXACT>(st.s, st.o, st.m, st.l, st.ph, st.pl, w.c, edge, hi, lo);
    }

    // One tile period: M_t then (unless t == T) S_t.  J = t mod 4 picks the
    // ring stages at compile time.  M_t touches no LDS: P.V of tile t-1 and
    // S^T of tile t run on operands read during S_{t-1}.  S_t does the
    // softmax of tile t and reads V of tile t and K of tile t+1.  Returns true
    // after the last M phase.
    template <int J, bool EXACT>
    static __device__ __forceinline__ bool period(W &w, St &st, int t, bool &act_prev) {
        block_sync();
        if (w.loader && t + 2 < w.my_count)
            load_tile(w, w.my_begin + t + 2, w.kst[(J + 2) % NSTAGE], w.vst[(J + 2) % NSTAGE]);
        if (t >= 1 && act_prev) {
            if constexpr (!VPRE) read_v(w, st, w.vst[(J + 3) % NSTAGE] + w.ring_off);
            pv<EXACT>(st);
        }
        const bool cur = t < w.my_count && visible(w, w.my_begin + t);
        if (cur) qk(st);
        if (t == w.T) return true;
        // tile t+1 must have landed (tile t+2 may still be in flight)
        if (w.loader && t + 1 < w.my_count) wait_tiles<LPT>(t + 2 < w.my_count ? 1 : 0);
        block_sync();
        if constexpr (VPRE)
            if (cur) read_v(w, st, w.vst[J] + w.ring_off);
        if (t + 1 < w.my_count && visible(w, w.my_begin + t + 1))
            read_k(w, st, w.kst[(J + 1) % NSTAGE] + w.ring_off);
        if (cur) softmax<EXACT>(w, st, w.my_begin + t);
        act_prev = cur;
        return false;
    }

    template <bool EXACT>
    static __device__ __forceinline__ void loop(W &w, St &st) {
        bool act_prev = false;
        if (w.grp == 1) block_sync();      // group B runs one phase behind
        for (int t = 0;; t += NSTAGE) {
            if (period<0, EXACT>(w, st, t, act_prev)) break;
            if (period<1, EXACT>(w, st, t + 1, act_prev)) break;
            if (period<2, EXACT>(w, st, t + 2, act_prev)) break;
            if (period<3, EXACT>(w, st, t + 3, act_prev)) break;
        }
        if (w.grp == 0) block_sync();      // same barrier count as group B
    }

    static __device__ __forceinline__ void run(const Params &p, char *const (&kst)[NSTAGE],
                                               char *const (&vst)[NSTAGE], float *ml) {
        W w;
        w.lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        w.grp = wave / NWG;
        w.wq = wave % NWG;
        w.g = w.lane >> 5;
        w.l32 = w.lane & 31;
        w.N = p.N;
        w.window = p.window;
        w.c = p.c;
#pragma unroll
        for (int s = 0; s < NSTAGE; ++s) {
            w.kst[s] = kst[s];
            w.vst[s] = vst[s];
        }
        const int N = p.N;

        const int bid = blockIdx.x;
        const int bh = bh_of(bid % p.n_bh, p.n_bh, p.group, p.xcd_kv);
        const int rank = bid / p.n_bh;
        const int qt = (MASK == MASK_NONE) ? rank : masked_qtile(rank, p.n_qtiles, p.zigzag);
        const int b = bh / p.Hq;
        const int h = bh - b * p.Hq;
        const int hkv = p.Hq / p.group;
        const int64_t kvhead = (int64_t)b * hkv + h / p.group;
        const uint16_t *qp = p.q + (int64_t)bh * N * D;
        w.kp = p.k + kvhead * N * D;
        w.vp = p.v + kvhead * N * D;

        const int q_tile0 = qt * BM;
        w.qw0 = q_tile0 + (ROWS ? w.grp * QROWS : 0) + w.wq * 32;
        w.w_last = min(w.qw0 + 32, N) - 1;

        // per-lane LDS offsets (independent of the tile and of the stage)
        {
            const int row = key_perm(w.l32);
#pragma unroll
            for (int kk = 0; kk < KT; ++kk) w.koff[kk] = row * ROWB + (((2 * kk + w.g) ^ swz<D>(row)) << 4);
            const int hgrp = w.lane >> 4, tt = w.lane & 15;
            const int row0 = 8 * (hgrp >> 1) + (tt >> 2);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int colb = cb * 64 + 32 * (hgrp & 1) + 8 * (tt & 3);
                const int ch = colb >> 4, within = colb & 15;
                w.voff[2 * cb] = row0 * ROWB + ((ch ^ swz<D>(row0)) << 4) + within;
                w.voff[2 * cb + 1] = (row0 + 4) * ROWB + ((ch ^ swz<D>(row0 + 4)) << 4) + within;
            }
        }

        St st;
        {
            const int row = w.qw0 + w.l32;
#pragma unroll
            for (int kk = 0; kk < KT; ++kk) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (row < N) {
                    v = *(const u32x4 *)(qp + (int64_t)row * D + kk * 16 + w.g * 8);
                    v ^= p.qsign;
                }
                st.qf[kk] = v;
            }
            st.m = -__builtin_inff();
            st.l = 0.0f;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) st.o[cb][r] = 0.0f;
        }

        // key tiles of the workgroup and of this group
        const int q_last = min(q_tile0 + BM, N) - 1;
        int kv_lo = 0, kv_hi = N - 1;
        if constexpr (MASK != MASK_NONE) kv_hi = q_last;
        if constexpr (MASK == MASK_WINDOW) kv_lo = max(0, q_tile0 - p.window + 1);
        const int t_begin = kv_lo / BN;
        const int n_tiles = kv_hi / BN + 1 - t_begin;
        if constexpr (ROWS) {
            w.my_begin = t_begin;
            w.my_count = n_tiles;
            w.T = n_tiles;
            w.loader = (w.grp == 0);
            w.ring_off = 0;
        } else {
            const int half = (n_tiles + 1) / 2;
            w.my_begin = t_begin + w.grp * half;
            w.my_count = max(0, min(half, n_tiles - w.grp * half));
            w.T = half;
            w.loader = true;
            w.ring_off = w.grp * TILEB;
        }

        int min_vis = N;
        if constexpr (MASK != MASK_NONE) min_vis = min(N, q_tile0 + 1);
        if constexpr (MASK == MASK_WINDOW) min_vis = min(min_vis, p.window);
        const bool exact = min_vis < p.exact_below;

        if (w.loader) {
            if (0 < w.my_count) load_tile(w, w.my_begin, w.kst[0], w.vst[0]);
            if (1 < w.my_count) load_tile(w, w.my_begin + 1, w.kst[1], w.vst[1]);
            if (0 < w.my_count) wait_tiles<LPT>(1 < w.my_count ? 1 : 0);
        }
        block_sync();
        if (0 < w.my_count && visible(w, w.my_begin)) read_k(w, st, w.kst[0] + w.ring_off);

        if (exact)
            loop<true>(w, st);
        else
            loop<false>(w, st);

        if constexpr (!ROWS) {
            // merge the key groups through the idle ring: channel block cb of
            // group B's O goes to ring array cb, its (m, l) to ml
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __syncthreads();
            char *ring[2 * NSTAGE];
#pragma unroll
            for (int s2 = 0; s2 < NSTAGE; ++s2) {
                ring[2 * s2] = w.kst[s2];
                ring[2 * s2 + 1] = w.vst[s2];
            }
            if (w.grp == 1) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    float *dst = (float *)ring[cb];
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[(w.wq * 16 + r) * 64 + w.lane] = st.o[cb][r];
                }
                ml[(w.wq * 2 + 0) * 64 + w.lane] = st.m;
                ml[(w.wq * 2 + 1) * 64 + w.lane] = st.l;
            }
            __syncthreads();
            if (w.grp == 1) return;
            const float m1 = ml[(w.wq * 2 + 0) * 64 + w.lane];
            const float l1 = ml[(w.wq * 2 + 1) * 64 + w.lane];
            const float m = fmaxf(st.m, m1);
            const float a0 = (st.m == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(st.m - m);
            const float a1 = (m1 == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
            st.m = m;
            st.l = st.l * a0 + l1 * a1;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const float *src = (const float *)ring[cb];
#pragma unroll
                for (int r = 0; r < 16; ++r) st.o[cb][r] = st.o[cb][r] * a0 + src[(w.wq * 16 + r) * 64 + w.lane] * a1;
            }
        }

        // epilogue: O = acc / l rounded once; LSE = ln 2 * (m + log2 l)
        const float lt = sum_halves(st.l);
        const int qi = w.qw0 + w.l32;
        if (qi < N) {
            const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
            uint16_t *orow = p.o + ((int64_t)bh * N + qi) * D;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const int ch = cb * 32 + 8 * j4 + 4 * w.g;
                    u32x2 v;
                    v[0] = pack2<DT>(st.o[cb][4 * j4 + 0] * inv, st.o[cb][4 * j4 + 1] * inv);
                    v[1] = pack2<DT>(st.o[cb][4 * j4 + 2] * inv, st.o[cb][4 * j4 + 3] * inv);
                    *(u32x2 *)(orow + ch) = v;
                }
            if (p.lse != nullptr && w.g == 0) {
                const float l2 = lt > 0.0f ? __builtin_amdgcn_logf(lt) : -__builtin_inff();
                p.lse[(int64_t)bh * N + qi] = (st.m + l2) * 0.69314718055994530942f;
            }
        }
    }
};

template <int D, int DT, int MASK, int NWG, bool ROWS, int BN>
__global__ __launch_bounds__(2 * NWG * 64) void attn_fwd_pingpong_kernel(Params p) {
    using K = PingPong<D, DT, MASK, NWG, ROWS, BN>;
    constexpr int SB = K::STAGEB;
    __shared__ __attribute__((aligned(1024))) char k0[SB];
    __shared__ __attribute__((aligned(1024))) char v0[SB];
    __shared__ __attribute__((aligned(1024))) char k1[SB];
    __shared__ __attribute__((aligned(1024))) char v1[SB];
    __shared__ __attribute__((aligned(1024))) char k2[SB];
    __shared__ __attribute__((aligned(1024))) char v2[SB];
    __shared__ __attribute__((aligned(1024))) char k3[SB];
    __shared__ __attribute__((aligned(1024))) char v3[SB];
    static_assert(ROWS || (D / 32 <= 8 && NWG * 16 * 64 * 4 <= SB), "ring too small for the key-group merge");
    __shared__ __attribute__((aligned(16))) float ml[ROWS ? 4 : NWG * 2 * 64];
    char *kst[4] = {k0, k1, k2, k3};
    char *vst[4] = {v0, v1, v2, v3};
    K::run(p, kst, vst, ml);
}

}  // namespace attnfwd
