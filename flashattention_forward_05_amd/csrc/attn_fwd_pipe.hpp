// attn_fwd_pipe.hpp -- attention forward for gfx950 in which every wave
// interleaves the matrix work of neighbouring key tiles with the softmax of
// the tile in between.
//
// Same computation and operand layouts as attn_fwd_kernel.hpp (tiled online
// softmax of "Optimizaciones de Atencion", section "FlashAttention: Nunca
// materializar la matriz de atencion"; S^T = K . Q^T on 32x32x16 MFMA, P^T
// straight from the accumulator, V^T through ds_read_b64_tr_b16, K/V in LDS
// through direct global->LDS loads with the per-row XOR swizzle).  What
// differs is the order of work inside a wave.  In iteration t a wave issues
//     S_{t+1}^T = K_{t+1} . Q^T        and        O^T += V_{t-1}^T . P_{t-1}^T
// on the matrix cores and, in the same instruction stream, the online softmax
// of S_t (exponentials, 16-bit P_t, row sums) on the vector ALU.  The two
// streams share no registers -- the steady-state softmax (max-free, see
// online_softmax) never touches O -- so the exponentials run under the MFMAs.
// On gfx950 a wave's MFMAs overlap well with its own vector instructions,
// while an MFMA-only wave beside a VALU-only wave on one SIMD overlaps poorly
// (measured), so the overlap is built inside the wave.  Iterations whose tile
// needs the general update (the first tile of a row, tiles cut by a mask or
// past the key range, and everything after a running max that had to move)
// take the same steps without the interleaving.  Query tiles whose rows see
// few keys (two-term P) are not run here: the host sends them to the lockstep
// kernel of attn_fwd_kernel.hpp.
//
// K and V have separate three-stage LDS rings.  Iteration t reads K of tile
// t+1 and V of tile t-1; after its barrier it issues the loads of K_{t+3}
// (into the stage K_t held) and V_{t+1} (into the stage V_{t-2} held), so a
// tile has two iterations to arrive and the wait before the barrier is always
// "all but the previous iteration's loads".
//
// With KSPLIT = 2 a second set of NWQ waves takes the second half of the key
// range and the partial (m, l, O) are merged in LDS at the end (the
// rescale-and-add of section "FlashDecoding" of the same page).
#pragma once

#include "attn_fwd_common.hpp"

namespace attnfwd {

// s_waitcnt immediate that waits for all LDS reads (lgkmcnt = 0) only.
constexpr int kLgkmZero = 15 | (3 << 14) | (7 << 4);

template <int D, int DT, int MASK, int QB, int NWQ, int KSPLIT, int BN>
struct Pipe {
    static constexpr int NS = 3;                          // stages of each ring
    static constexpr int BM = NWQ * QB * 32;              // query rows per workgroup
    static constexpr int NWAVES = NWQ * KSPLIT;
    static constexpr int KT = D / 16;                     // 16-wide d steps of S^T = K Q^T
    static constexpr int CB = D / 32;                     // 32-channel blocks of O^T
    static constexpr int KB = BN / 32;                    // 32-key blocks of S^T
    static constexpr int KS = BN / 16;                    // 16-key steps of O^T += V^T P^T
    static constexpr int ROWB = 2 * D;                    // bytes per K/V row
    static constexpr int TILEB = BN * ROWB;               // bytes per K or V tile of one key group
    static constexpr int CPR = D / 8;                     // 16-byte chunks per row
    static constexpr int LOADS = BN * CPR / (64 * NWQ);   // 16-byte loads per lane per tile
    static constexpr int STAGEB = KSPLIT * TILEB;         // bytes of one stage
    static constexpr int RINGB = 2 * NS * STAGEB;         // bytes of both rings
    static_assert((BN * CPR) % (64 * NWQ) == 0 && LOADS >= 1, "tile must split evenly over the waves");
    static_assert(BN % 32 == 0 && (D == 64 || D == 128) && (KSPLIT == 1 || KSPLIT == 2), "unsupported tile");
    static_assert(KSPLIT == 1 || STAGEB >= NWQ * 16 * 64 * 4, "stage too small for the key-group merge");

    struct W {
        const uint16_t *kp, *vp;  // this head's K and V (wave-uniform)
        int N, window, lane, g, l32, wq, kgroup;
        int qw0, w_last;          // first / last query row of this wave
        int my_begin, my_count;   // this key group's tiles (absolute first, count)
        float c;
        uint32_t goff[LOADS];     // byte offset within a tile of this lane's chunk in load i
        uint32_t gend;            // byte offset of the tensor's last 16-byte chunk
        int koff[KT];             // LDS byte offsets (within a stage) of the K operand reads
        int voff[2 * CB];         // ... and of the V^T transposing reads
        ATTN_LDS char *ring;      // 2 * NS stages: K stages 0 .. NS-1, then V stages
    };

    static __device__ __forceinline__ ATTN_LDS char *kstage(const W &w, int s) { return w.ring + s * STAGEB; }
    static __device__ __forceinline__ ATTN_LDS char *vstage(const W &w, int s) { return w.ring + (NS + s) * STAGEB; }

    struct St {
        u32x4 qf[QB][KT];         // Q^T operand (MFMA B), resident
        f32x16 o[QB][CB];         // O^T accumulators
        float m[QB], l[QB];       // running max (log2 units) and this lane-half's running sum
        f32x16 s[2][KB][QB];      // S^T of tile t (being normalised) and t+1 (being formed)
        u32x4 ph[2][QB][KS];      // 16-bit P^T of tile t-1 (being consumed) and t (being formed)
        u32x4 pl[2][QB][KS];      // unused here (two-term P runs on the lockstep kernel)
    };

    // Does any row of this wave see a key of tile a?
    static __device__ __forceinline__ bool vis(const W &w, int a) {
        bool any = w.qw0 < w.N;
        if constexpr (MASK != MASK_NONE) any = any && (a * BN <= w.w_last);
        if constexpr (MASK == MASK_WINDOW) any = any && (a * BN + BN - 1 >= w.qw0 - w.window + 1);
        return any;
    }

    // Does tile a need masking for some row of this wave?
    static __device__ __forceinline__ bool edge(const W &w, int a) {
        const int j0 = a * BN;
        bool e = j0 + BN > w.N;
        if constexpr (MASK != MASK_NONE) e = e || (j0 + BN - 1 > w.qw0);
        if constexpr (MASK == MASK_WINDOW) e = e || (j0 < w.w_last - w.window + 1);
        return e;
    }

    // Direct loads of this wave's share of tile a of one tensor into a stage.
    static __device__ __forceinline__ void load(const W &w, const uint16_t *base, int a, ATTN_LDS char *stage) {
        const uint32_t t0 = (uint32_t)a * TILEB;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            // chunks of rows past N read the tensor's last chunk instead (any
            // finite data: those keys are masked)
            const uint32_t off = min(t0 + w.goff[i], w.gend);
            const int lds_off = w.kgroup * TILEB + (i * NWQ + w.wq) * 1024;
            lds_dma16_s(base, off, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(stage + lds_off)));
        }
    }

    static __device__ __forceinline__ u32x4 k_frag(const W &w, const ATTN_LDS char *kl, int kk, int kb) {
        return *(const ATTN_LDS u32x4 *)(kl + w.koff[kk] + kb * 32 * ROWB);
    }

    static __device__ __forceinline__ u32x4 v_frag(const W &w, const ATTN_LDS char *vl, int ks, int cb) {
        const ATTN_LDS char *b = vl + ks * 16 * ROWB;
        const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)(b + w.voff[2 * cb]));
        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)(b + w.voff[2 * cb + 1]));
        const u32x2 a0 = __builtin_bit_cast(u32x2, t0);
        const u32x2 a1 = __builtin_bit_cast(u32x2, t1);
        return u32x4{a0[0], a0[1], a1[0], a1[1]};
    }

    // S^T of the next tile into s[(J + 1) & 1].
    template <int J>
    static __device__ __forceinline__ void qk(const W &w, St &st, const ATTN_LDS char *kl) {
        constexpr int NX = (J + 1) & 1;
        u32x4 ka[KT][KB];
#pragma unroll
        for (int kk = 0; kk < KT; ++kk)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) ka[kk][kb] = k_frag(w, kl, kk, kb);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) st.s[NX][kb][qb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KT; ++kk)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) st.s[NX][kb][qb] = mfma32<DT>(ka[kk][kb], st.qf[qb][kk], st.s[NX][kb][qb]);
    }

    // O^T += V^T . P^T of the previous tile (P in ph / pl[(J + 1) & 1]).
    template <int J, bool EXACT>
    static __device__ __forceinline__ void pv(const W &w, St &st, const ATTN_LDS char *vl) {
        constexpr int PP = (J + 1) & 1;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const u32x4 va = v_frag(w, vl, ks, cb);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    st.o[qb][cb] = mfma32<DT>(va, st.ph[PP][qb][ks], st.o[qb][cb]);
                    if constexpr (EXACT) st.o[qb][cb] = mfma32<DT>(va, st.pl[PP][qb][ks], st.o[qb][cb]);
                }
            }
    }

    // The steady-state iteration is written out as NMF steps, one MFMA each
    // (P.V of tile t-1 in (ks, cb, qb) order, then S^T of tile t+1 in
    // (kk, kb, qb) order).  Step i issues the LDS reads of the operand
    // fragments first used LA steps later, its MFMA, the packing and row sum
    // of the softmax pairs of step i-1 and the exponentials of its own pairs;
    // a scheduling fence after each step keeps this order, so the
    // exponentials run while the matrix core works and every LDS read has LA
    // MFMAs of time.
    static constexpr int NPV = KS * CB * QB;
    static constexpr int NQK = KT * KB * QB;
    static constexpr int NMF = NPV + NQK;
    static constexpr int NVF = KS * CB;                 // V^T fragments (two transposing reads each)
    static constexpr int NF = NVF + KT * KB;            // + K fragments (one 16-byte read each)
    static constexpr int NPAIR = QB * KS * 4;           // softmax pairs per lane
    static constexpr int LA = 3;
    // Step i runs P.V MFMA pv_index(i) or S^T MFMA qk_index(i): the two kinds
    // alternate in proportion, so that O stays in use across the whole step
    // sequence (its registers then stay put).
    static constexpr bool is_pv(int i) { return (i * NPV) / NMF != ((i + 1) * NPV) / NMF; }
    static constexpr int pv_index(int i) { return (i * NPV) / NMF; }
    static constexpr int qk_index(int i) { return i - (i * NPV) / NMF - (is_pv(i) ? 0 : 0); }
    static constexpr int step_of_pv(int n) {
        for (int i = 0; i < NMF; ++i)
            if (is_pv(i) && pv_index(i) == n) return i;
        return NMF;
    }
    static constexpr int step_of_qk(int n) {
        for (int i = 0; i < NMF; ++i)
            if (!is_pv(i) && qk_index(i) == n) return i;
        return NMF;
    }
    static constexpr int first_use(int j) { return j < NVF ? step_of_pv(j * QB) : step_of_qk((j - NVF) * QB); }
    static constexpr int pair_begin(int i) { return i <= 0 ? 0 : (i >= NMF ? NPAIR : (i * NPAIR) / NMF); }

    // Operand fragment j from per-lane base addresses formed once per
    // iteration (ka: K row, one per d-step; va: the two V^T read rows, per
    // channel block); the key-block / key-step offsets are immediates.
    static __device__ __forceinline__ u32x4 frag(const ATTN_LDS char *const (&ka)[KT],
                                                 const ATTN_LDS char *const (&va)[2 * CB], int j) {
        if (j < NVF) {
            const int ks = j / CB, cb = j % CB;
            const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)(va[2 * cb] + ks * 16 * ROWB));
            const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)(va[2 * cb + 1] + ks * 16 * ROWB));
            const u32x2 a0 = __builtin_bit_cast(u32x2, t0);
            const u32x2 a1 = __builtin_bit_cast(u32x2, t1);
            return u32x4{a0[0], a0[1], a1[0], a1[1]};
        }
        const int kk = (j - NVF) / KB, kb = (j - NVF) % KB;
        return *(const ATTN_LDS u32x4 *)(ka[kk] + kb * 32 * ROWB);
    }

    // Steady-state iteration: P.V of tile t-1 and S^T of tile t+1 on the
    // matrix cores, interleaved with the max-free softmax of tile t.  Returns
    // false when some row's partial sum left the accepted range (or the row
    // has not seen a key yet); the caller then runs the general update.
    template <int J>
    static __device__ __forceinline__ bool fast(const W &w, St &st, const ATTN_LDS char *kl, const ATTN_LDS char *vl) {
        constexpr int C = J & 1, NX = (J + 1) & 1;
        u32x4 fr[NF];
        f32x16 sn[KB][QB];
        float ex[NPAIR][2];
        float rs[QB][2];
        float nm[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            nm[qb] = -st.m[qb];
            rs[qb][0] = 0.0f;
            rs[qb][1] = 0.0f;
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sn[kb][qb] = f32x16{};
        // one address per distinct lane offset; the empty asm keeps the
        // compiler from re-associating the stage base into every read
        const ATTN_LDS char *ka[KT];
        const ATTN_LDS char *va[2 * CB];
        const uint32_t kb0 = (uint32_t)(uintptr_t)kl, vb0 = (uint32_t)(uintptr_t)vl;
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
            uint32_t a = kb0 + (uint32_t)w.koff[kk];
            asm volatile("" : "+v"(a));
            ka[kk] = (const ATTN_LDS char *)(uintptr_t)a;
        }
#pragma unroll
        for (int j = 0; j < 2 * CB; ++j) {
            uint32_t a = vb0 + (uint32_t)w.voff[j];
            asm volatile("" : "+v"(a));
            va[j] = (const ATTN_LDS char *)(uintptr_t)a;
        }
#pragma unroll
        for (int j = 0; j < NF; ++j)
            if (first_use(j) < LA) fr[j] = frag(ka, va, j);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
#pragma unroll
            for (int j = 0; j < NF; ++j)
                if (first_use(j) == i + LA) fr[j] = frag(ka, va, j);
            if (is_pv(i)) {
                const int n = pv_index(i), f = n / QB, qb = n % QB, ks = f / CB, cb = f % CB;
                st.o[qb][cb] = mfma32<DT>(fr[f], st.ph[NX][qb][ks], st.o[qb][cb]);
            } else {
                const int n = qk_index(i), f = n / QB, qb = n % QB, kk = f / KB, kb = f % KB;
                sn[kb][qb] = mfma32<DT>(fr[NVF + f], st.qf[qb][kk], sn[kb][qb]);
            }
            // pack and sum the pairs of the previous step
#pragma unroll
            for (int p = pair_begin(i - 1); p < pair_begin(i); ++p) {
                const int qb = p / (KS * 4), ks = (p / 4) % KS, q = p % 4;
                st.ph[C][qb][ks][q] = pack2<DT>(ex[p][0], ex[p][1]);
                rs[qb][q & 1] += ex[p][0] + ex[p][1];
            }
            // p = 2^(s*c - m) against the running max for this step's pairs
#pragma unroll
            for (int p = pair_begin(i); p < pair_begin(i + 1); ++p) {
                const int qb = p / (KS * 4), ks = (p / 4) % KS, q = p % 4;
                const int kb = ks >> 1, r = 8 * (ks & 1) + 2 * q;
                ex[p][0] = __builtin_amdgcn_exp2f(__builtin_fmaf(st.s[C][kb][qb][r], w.c, nm[qb]));
                ex[p][1] = __builtin_amdgcn_exp2f(__builtin_fmaf(st.s[C][kb][qb][r + 1], w.c, nm[qb]));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int p = pair_begin(NMF - 1); p < NPAIR; ++p) {
            const int qb = p / (KS * 4), ks = (p / 4) % KS, q = p % 4;
            st.ph[C][qb][ks][q] = pack2<DT>(ex[p][0], ex[p][1]);
            rs[qb][q & 1] += ex[p][0] + ex[p][1];
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) st.s[NX][kb][qb] = sn[kb][qb];
        bool bad = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            bad = bad || !(rs[qb][0] + rs[qb][1] <= 32768.0f) || st.m[qb] == -__builtin_inff();
        if (__builtin_amdgcn_ballot_w64(bad) != 0) return false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) st.l[qb] += rs[qb][0] + rs[qb][1];
        return true;
    }

    // Wait until K_{t+1} and V_{t-1} (issued in iteration t-2) have landed --
    // only the loads of iteration t-1 (K_{t+2}, V_t) may still be in flight --
    // then barrier and issue the loads of iteration t: K_{t+3} into the stage
    // K_t held, V_{t+1} into the stage V_{t-2} held.  Stage of tile j: j mod 3.
    static __device__ __forceinline__ void ring_step(const W &w, int t) {
        const int mc = w.my_count;
        const int pend = (t + 2 < mc ? 1 : 0) + (t < mc ? 1 : 0);
        if (pend == 2)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LOADS));
        else if (pend == 1)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_waitcnt(kLgkmZero);
        block_sync();
        if (t + 3 < mc) load(w, w.kp, w.my_begin + t + 3, kstage(w, t % 3));
        if (t + 1 < mc) load(w, w.vp, w.my_begin + t + 1, vstage(w, (t + 1) % 3));
    }

    // Mask S^T of tile a (in s[J & 1]) for the rows of this wave; with
    // all = true every key is masked (tile not seen by this wave, or past the
    // key group's range).
    template <int J>
    static __device__ __forceinline__ void mask(const W &w, St &st, int a, bool all) {
        constexpr int C = J & 1;
        const int j0 = a * BN;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int qi = w.qw0 + qb * 32 + w.l32;
            int hi = w.N - 1 - (j0 + 8 * w.g);
            int lo = -(1 << 30);
            if constexpr (MASK != MASK_NONE) hi = min(hi, qi - (j0 + 8 * w.g));
            if constexpr (MASK == MASK_WINDOW) lo = qi - w.window + 1 - (j0 + 8 * w.g);
            if (all) hi = -(1 << 30);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kb * 32 + 16 * (r / 8) + (r % 8);
                    if (off > hi || off < lo) st.s[C][kb][qb][r] = -__builtin_inff();
                }
        }
    }

    // General update of the (already masked) tile in s[J & 1]: tile max,
    // lazy raise of the running max with the O / l rescale, then p.
    template <int J, bool EXACT>
    static __device__ __forceinline__ void general(const W &w, St &st) {
        constexpr int C = J & 1;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            f32x16 sq[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sq[kb] = st.s[C][kb][qb];
            online_softmax_full<DT, KB, CB, EXACT>(sq, st.o[qb], st.m[qb], st.l[qb], st.ph[C][qb], st.pl[C][qb],
                                                   w.c, false, 0, 0);
        }
    }

    // Iteration t, 0 <= t <= T, any tile, without the interleaving: S^T of
    // tile t+1, P.V of tile t-1, then the (masked where needed) general
    // update of tile t.  Iteration 0 skips the P.V (nothing to multiply yet);
    // iteration T forms an unused S^T and a fully masked softmax.
    template <int J>
    static __device__ __forceinline__ void body(W &w, St &st, int t) {
        ring_step(w, t);
        qk<J>(w, st, kstage(w, (t + 1) % 3));
        if (t > 0) pv<J, false>(w, st, vstage(w, (t + 2) % 3));
        const int a = w.my_begin + t;
        const bool seen = t < w.my_count && vis(w, a);
        if (!seen || edge(w, a)) mask<J>(w, st, a, !seen);
        general<J, false>(w, st);
    }

    // Iteration t of the fast range (tile t visible and unmasked for every
    // row of this wave).  Returns false after a rejected tile, which has then
    // been finished by the general update.
    template <int J>
    static __device__ __forceinline__ bool body_fast(W &w, St &st, int t) {
        ring_step(w, t);
        if (fast<J>(w, st, kstage(w, (t + 1) % 3), vstage(w, (t + 2) % 3))) return true;
        general<J, false>(w, st);
        return false;
    }

    // Iterations t .. t_end-1 with the general body.
    static __device__ __forceinline__ int run_any(W &w, St &st, int t, int t_end) {
        if (t < t_end && (t & 1)) body<1>(w, st, t++);
        for (; t + 1 < t_end; t += 2) {
            body<0>(w, st, t);
            body<1>(w, st, t + 1);
        }
        if (t < t_end) body<0>(w, st, t++);
        return t;
    }

    // Iterations t .. t_end-1 of the fast range; stops after the first
    // rejected tile.  O is only touched by MFMAs here, so it keeps one set of
    // registers through the loop.
    static __device__ __forceinline__ int run_fast(W &w, St &st, int t, int t_end) {
        if (t < t_end && (t & 1))
            if (!body_fast<1>(w, st, t++)) return t;
        for (; t + 1 < t_end; t += 2) {
            if (!body_fast<0>(w, st, t)) return t + 1;
            if (!body_fast<1>(w, st, t + 1)) return t + 2;
        }
        if (t < t_end)
            if (!body_fast<0>(w, st, t++)) return t;
        return t;
    }

    // First and last+1 iteration whose tile every row of this wave sees in
    // full (no mask), within [1, my_count).
    static __device__ __forceinline__ void fast_range(const W &w, int &t_fb, int &t_fe) {
        int a_end = w.N / BN;                                   // tiles past it are ragged
        if constexpr (MASK != MASK_NONE) a_end = min(a_end, (w.qw0 + 1) / BN);
        int a_beg = 0;
        if constexpr (MASK == MASK_WINDOW) a_beg = (max(0, w.w_last - w.window + 1) + BN - 1) / BN;
        t_fb = max(1, a_beg - w.my_begin);
        t_fe = max(t_fb, min(w.my_count, a_end - w.my_begin));
        if (w.qw0 >= w.N) t_fe = t_fb;
    }

    static __device__ __forceinline__ void loop(W &w, St &st, int T) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) st.ph[1][qb][ks] = u32x4{0u, 0u, 0u, 0u};   // P_{-1}
        int t_fb, t_fe;
        fast_range(w, t_fb, t_fe);
        t_fb = min(t_fb, T);
        t_fe = min(t_fe, T);
        int t = run_any(w, st, 0, t_fb);
        t = run_fast(w, st, t, t_fe);
        run_any(w, st, t, T + 1);
    }

    static __device__ __forceinline__ void run(const Params &p, ATTN_LDS char *ring, float *ml) {
        W w;
        w.lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        w.wq = wave % NWQ;
        w.kgroup = wave / NWQ;
        w.g = w.lane >> 5;
        w.l32 = w.lane & 31;
        w.N = p.N;
        w.window = p.window;
        w.c = p.c;
        w.ring = ring;
        const int N = p.N;

        // ---- (batch*head, query tile) of this workgroup; masked runs take
        // the heaviest query tiles first
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
        w.qw0 = q_tile0 + w.wq * QB * 32;
        w.w_last = min(w.qw0 + QB * 32, N) - 1;

        // ---- per-lane offsets that do not change with the tile
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int slot = (i * NWQ + w.wq) * 64 + w.lane;
            const int row = slot / CPR;
            w.goff[i] = row * ROWB + ((slot % CPR) ^ swz<D>(row)) * 16;
        }
        w.gend = (uint32_t)N * ROWB - 16;
        {
            const int row = key_perm(w.l32);
#pragma unroll
            for (int kk = 0; kk < KT; ++kk)
                w.koff[kk] = w.kgroup * TILEB + row * ROWB + (((2 * kk + w.g) ^ swz<D>(row)) << 4);
            const int hgrp = w.lane >> 4, tt = w.lane & 15;
            const int row0 = 8 * (hgrp >> 1) + (tt >> 2);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int colb = cb * 64 + 32 * (hgrp & 1) + 8 * (tt & 3);
                const int ch = colb >> 4, within = colb & 15;
                w.voff[2 * cb] = w.kgroup * TILEB + row0 * ROWB + ((ch ^ swz<D>(row0)) << 4) + within;
                w.voff[2 * cb + 1] = w.kgroup * TILEB + (row0 + 4) * ROWB + ((ch ^ swz<D>(row0 + 4)) << 4) + within;
            }
        }

        St st;
        // ---- Q fragments (MFMA B operand): lane holds row qw0 + 32*qb + l32,
        // channels 16*kk + 8*g .. +7.  Rows past N are zero.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int row = w.qw0 + qb * 32 + w.l32;
#pragma unroll
            for (int kk = 0; kk < KT; ++kk) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (row < N) {
                    v = *(const u32x4 *)(qp + (int64_t)row * D + kk * 16 + w.g * 8);
                    v ^= p.qsign;
                }
                st.qf[qb][kk] = v;
            }
            st.m[qb] = -__builtin_inff();
            st.l[qb] = 0.0f;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) st.o[qb][cb][r] = 0.0f;
        }

        // ---- key tiles of the workgroup, split between the key groups; both
        // groups run the same number of iterations (barriers must match)
        const int q_last = min(q_tile0 + BM, N) - 1;
        int kv_lo = 0, kv_hi = N - 1;
        if constexpr (MASK != MASK_NONE) kv_hi = q_last;
        if constexpr (MASK == MASK_WINDOW) kv_lo = max(0, q_tile0 - p.window + 1);
        const int t_begin = kv_lo / BN;
        const int n_tiles = kv_hi / BN + 1 - t_begin;
        const int T = (n_tiles + KSPLIT - 1) / KSPLIT;
        w.my_begin = t_begin + w.kgroup * T;
        w.my_count = max(0, min(T, n_tiles - w.kgroup * T));

        // ---- the matrix work of an iteration runs whatever the tile: stages
        // never loaded must hold finite values (zero), so that a zero P times
        // a stale V stays zero and a stale S^T is masked away
        {
            const u32x4 z = {0u, 0u, 0u, 0u};
            for (int i = threadIdx.x; i < RINGB / 16; i += NWAVES * 64) ((ATTN_LDS u32x4 *)ring)[i] = z;
            __syncthreads();
        }

        // ---- prologue: K_0, K_1, then what iteration -1 would issue (K_2,
        // V_0); wait for K_0 and form S^T of tile 0
        const int mc = w.my_count;
        if (0 < mc) load(w, w.kp, w.my_begin + 0, kstage(w, 0));
        if (1 < mc) load(w, w.kp, w.my_begin + 1, kstage(w, 1));
        if (2 < mc) load(w, w.kp, w.my_begin + 2, kstage(w, 2));
        if (0 < mc) load(w, w.vp, w.my_begin + 0, vstage(w, 0));
        {
            const int after = (1 < mc ? 1 : 0) + (2 < mc ? 1 : 0) + (0 < mc ? 1 : 0);
            if (after == 3)
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * LOADS));
            else if (after == 2)
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LOADS));
            else if (after == 1)
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
            else
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        block_sync();
        qk<1>(w, st, kstage(w, 0));   // as iteration -1: S^T of tile 0 into s[0]

        // ---- main loop; one instance per P mode
        loop(w, st, T);

        // ---- merge the key groups: group 1 hands (m, l, O) to group 0
        // through the idle rings, one (qb, cb) block per stage array per round
        if constexpr (KSPLIT == 2) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __syncthreads();
            if (w.kgroup == 1) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    ml[((w.wq * QB + qb) * 2 + 0) * 64 + w.lane] = st.m[qb];
                    ml[((w.wq * QB + qb) * 2 + 1) * 64 + w.lane] = st.l[qb];
                }
            }
            float a0[QB], a1[QB];
            constexpr int NBLK = QB * CB;
#pragma unroll
            for (int r0 = 0; r0 < NBLK; r0 += 2 * NS) {
                if (w.kgroup == 1) {
#pragma unroll
                    for (int j = 0; j < 2 * NS; ++j)
                        if (r0 + j < NBLK) {
                            const int qb = (r0 + j) / CB, cb = (r0 + j) % CB;
                            ATTN_LDS float *dst = (ATTN_LDS float *)(ring + j * STAGEB);
#pragma unroll
                            for (int r = 0; r < 16; ++r) dst[(w.wq * 16 + r) * 64 + w.lane] = st.o[qb][cb][r];
                        }
                }
                __syncthreads();
                if (w.kgroup == 0) {
                    if (r0 == 0) {
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) {
                            const float m1 = ml[((w.wq * QB + qb) * 2 + 0) * 64 + w.lane];
                            const float l1 = ml[((w.wq * QB + qb) * 2 + 1) * 64 + w.lane];
                            const float m0 = st.m[qb];
                            const float m = fmaxf(m0, m1);
                            a0[qb] = (m0 == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m0 - m);
                            a1[qb] = (m1 == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
                            st.m[qb] = m;
                            st.l[qb] = st.l[qb] * a0[qb] + l1 * a1[qb];
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 2 * NS; ++j)
                        if (r0 + j < NBLK) {
                            const int qb = (r0 + j) / CB, cb = (r0 + j) % CB;
                            const ATTN_LDS float *src = (const ATTN_LDS float *)(ring + j * STAGEB);
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                st.o[qb][cb][r] = st.o[qb][cb][r] * a0[qb] + src[(w.wq * 16 + r) * 64 + w.lane] * a1[qb];
                        }
                }
                if (r0 + 2 * NS < NBLK) __syncthreads();
            }
            if (w.kgroup == 1) return;
        }

        // ---- epilogue: O = acc / l, rounded once; LSE = ln 2 * (m + log2 l)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float lt = sum_halves(st.l[qb]);
            const int qi = w.qw0 + qb * 32 + w.l32;
            if (qi < N) {
                const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
                uint16_t *orow = p.o + ((int64_t)bh * N + qi) * D;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const int ch = cb * 32 + 8 * j4 + 4 * w.g;
                        u32x2 v;
                        v[0] = pack2<DT>(st.o[qb][cb][4 * j4 + 0] * inv, st.o[qb][cb][4 * j4 + 1] * inv);
                        v[1] = pack2<DT>(st.o[qb][cb][4 * j4 + 2] * inv, st.o[qb][cb][4 * j4 + 3] * inv);
                        *(u32x2 *)(orow + ch) = v;
                    }
                if (p.lse != nullptr && w.g == 0) {
                    const float l2 = lt > 0.0f ? __builtin_amdgcn_logf(lt) : -__builtin_inff();
                    p.lse[(int64_t)bh * N + qi] = (st.m[qb] + l2) * 0.69314718055994530942f;
                }
            }
        }
    }
};

template <int D, int DT, int MASK, int QB, int NWQ, int KSPLIT, int BN>
__global__ __launch_bounds__(NWQ * KSPLIT * 64) void attn_fwd_pipe_kernel(Params p) {
    using K = Pipe<D, DT, MASK, QB, NWQ, KSPLIT, BN>;
    __shared__ __attribute__((aligned(1024))) char ring[K::RINGB];
    __shared__ __attribute__((aligned(16))) float ml[KSPLIT == 2 ? NWQ * QB * 2 * 64 : 4];
    K::run(p, (ATTN_LDS char *)ring, ml);
}

}  // namespace attnfwd
