// attn_fwd_pp.hpp -- attention forward for gfx950 with two wave groups whose
// matrix and vector phases alternate ("ping-pong").
//
// Same computation as attn_fwd_kernel.hpp: the tiled online softmax of
// "Optimizaciones de Atencion", section "FlashAttention: Nunca materializar
// la matriz de atencion", and the kernel body of "Lab 02 - Forward de flash
// attention en Triton", sections "La estructura del kernel" and "Bloque B";
// same operand layouts (S^T = K . Q^T on 32x32x16 MFMA, P^T straight from the
// accumulator, V^T through ds_read_b64_tr_b16, K/V in LDS through direct
// global->LDS loads with a per-row XOR swizzle).  What differs is the
// schedule.
//
// Measured on the MI355X (microbench.hip): one wave alone issues a vector
// instruction only about every 8 clocks, while a matrix instruction of one
// wave and vector instructions of the other wave on the same SIMD overlap by
// 80-86%.  When both waves of a SIMD run the same phase at once (the lockstep
// kernel), the matrix core idles during the softmax.  Here the workgroup has
// two groups of four waves, one wave of each group per SIMD, owning different
// query rows (BM = 256) and sharing one K/V ring.  Each wave works on its key
// tiles in two phases:
//   M_i : O^T += V^T . P^T of tile i-1, then S^T = K . Q^T of tile i, with the
//         operands read from LDS right ahead of their MFMAs (matrix core);
//   S_i : online softmax of S^T -> P^T, running max / sum, lazy O rescale
//         (vector ALU).
// Group A runs M_0 S_0 M_1 S_1 ... M_T; group B runs the same sequence one
// barrier later, so in every phase one wave of a SIMD feeds the matrix core
// while the other keeps the vector ALU busy.
//
// K/V ring: four stages.  Group A issues the loads of tile i+2 right after the
// barrier that opens its M_i (into the stage of tile i-2, which group B last
// read in its M_{i-1}, before that barrier) and waits for tile i+1 at the end
// of its S_i, before the barrier that opens M_{i+1} for A (and S_{i+1}... for
// B, whose M_{i+1} follows one barrier later).
//
// Only the plain square forward runs here (no key splits, no paging, no
// stacked heads), and no two-term P: the host sends the query tiles whose
// first row sees few keys to the lockstep kernel with the same 256-row tiling.
#pragma once

#include "attn_fwd_common.hpp"

namespace attnfwd {

template <int D, int DT, int MASK>
struct PingPong {
    static constexpr int NWG = 4;                 // waves per group (one per SIMD)
    static constexpr int BN = 64;                 // keys per tile
    static constexpr int NSTAGE = 4;
    static constexpr int QROWS = NWG * 32;        // query rows per group
    static constexpr int BM = 2 * QROWS;          // query rows per workgroup
    static constexpr int KT = D / 16;             // 16-wide d steps of S^T = K Q^T
    static constexpr int CB = D / 32;             // 32-channel blocks of O^T
    static constexpr int KB = BN / 32;            // 32-key blocks of S^T
    static constexpr int KS = BN / 16;            // 16-key steps of O^T += V^T P^T
    static constexpr int ROWB = 2 * D;            // bytes per K/V row
    static constexpr int TILEB = BN * ROWB;       // bytes per K or V tile
    static constexpr int CPR = D / 8;             // 16-byte chunks per row
    static constexpr int LOADS = BN * CPR / (64 * NWG);   // per lane per tensor per tile
    static constexpr int LPT = 2 * LOADS;
    static_assert((BN * CPR) % (64 * NWG) == 0 && (D == 64 || D == 128), "unsupported tile");

    struct W {
        const uint16_t *kp, *vp;
        int N, window, lane, g, l32, wq, grp;
        int qw0, w_last;   // first / last valid query row of this wave
        int t_begin, T;    // the workgroup's first key tile and tile count
        float c;
        char *ring;           // K stages 0..3, then V stages 0..3, TILEB bytes each
        // Per-lane operand offsets in the ring, kept as a base and an XOR
        // term: the K operand of d-step kk (key block 0, stage 0) is at
        // kb_ + (32 * kk ^ ks_), the two transposing V^T reads h = 0, 1 of
        // channel block cb (16-key step 0, stage 0) at va_[h] + (64 * cb ^ vs_[h]).
        uint32_t kb_, ks_, va_[2], vs_[2];
    };

    // The per-lane offsets of one matrix phase, rebuilt from the six values
    // above after an empty asm that hides them from the optimiser: every read
    // then adds its stage and step as an immediate offset, and only those six
    // registers stay live through the softmax (a precomputed address per
    // (stage, fragment), or even the sixteen offsets, would not fit beside
    // the accumulators at d = 128).
    struct Off {
        uint32_t k[KT], v[2 * CB];
    };
    static __device__ __forceinline__ Off offsets(const W &w, int kstage, int vstage) {
        uint32_t kb = w.kb_, ks = w.ks_, va0 = w.va_[0], va1 = w.va_[1], vs0 = w.vs_[0], vs1 = w.vs_[1];
        asm volatile("" : "+v"(kb), "+v"(ks), "+v"(va0), "+v"(va1), "+v"(vs0), "+v"(vs1));
        kb += kstage * TILEB;
        va0 += vstage * TILEB;
        va1 += vstage * TILEB;
        Off o;
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) o.k[kk] = ((32u * kk) ^ ks) + kb;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            o.v[2 * cb] = ((64u * cb) ^ vs0) + va0;
            o.v[2 * cb + 1] = ((64u * cb) ^ vs1) + va1;
        }
        return o;
    }

    // Operand fragments the vector phase reads ahead for the next matrix
    // phase: the first NPV V^T fragments (in P.V order, j -> ks = j / CB,
    // cb = j % CB) and the first NPK K fragments (j -> kk = j / KB, kb = j %
    // KB).  A wave alone issues a transposing 8-byte LDS read only about every
    // 16 clocks, so the 2 * NPAIR of them would otherwise pace the matrix
    // phase; the vector phase has the LDS issue slots to spare.
    static constexpr int NPAIR = KS * CB;
    static constexpr int NPV = D == 128 ? 8 : NPAIR;
    static constexpr int NPK = D == 128 ? 2 : 4;

    struct St {
        u32x4 qf[KT];
        f32x16 o[CB];
        f32x16 s[KB];
        u32x4 ph[KS];
        u32x4 vpre[NPV], kpre[NPK];
        float m, l;
    };

    static __device__ __forceinline__ bool visible(const W &w, int abs_tile) {
        bool any = w.qw0 < w.N;
        if constexpr (MASK != MASK_NONE) any = any && (abs_tile * BN <= w.w_last);
        if constexpr (MASK == MASK_WINDOW) any = any && (abs_tile * BN + BN - 1 >= w.qw0 - w.window + 1);
        return any;
    }

    // Group A's direct loads of one tile: lane `lane` of wave wq moves 16-byte
    // slot (i * NWG + wq) * 64 + lane of K and of V; the slot's row keeps its
    // chunks XOR-swizzled (swz) so that the operand reads hit distinct banks.
    static __device__ __forceinline__ void load_tile(const W &w, int abs_tile, int stage) {
        const int j0 = abs_tile * BN;
        const uint32_t kb = __builtin_amdgcn_readfirstlane(lds_addr(w.ring + stage * TILEB + w.wq * 1024));
        const uint32_t vb = __builtin_amdgcn_readfirstlane(lds_addr(w.ring + (NSTAGE + stage) * TILEB + w.wq * 1024));
        static_for<LOADS>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const int slot = (i * NWG + w.wq) * 64 + w.lane;
            const int row = slot / CPR;
            const int ch = (slot % CPR) ^ swz<D>(row);
            const int64_t off = (int64_t)min(j0 + row, w.N - 1) * D + ch * 8;
            lds_dma16_at<i * NWG * 1024>(w.kp + off, kb);
            lds_dma16_at<i * NWG * 1024>(w.vp + off, vb);
        });
    }

    // K operand of d-step kk, key block kb (rows in the key_perm order, chunks
    // swizzled by swz); the stage is in the offsets.
    static __device__ __forceinline__ u32x4 k_frag(const W &w, const Off &o, int kk, int kb) {
        return *(const ATTN_LDS u32x4 *)((const ATTN_LDS char *)w.ring + o.k[kk] + kb * 32 * ROWB);
    }

    // V^T operand of 16-key step ks, channel block cb: two transposing reads
    // of 4 keys x 16 channels per 16-lane group.
    static __device__ __forceinline__ u32x4 v_frag(const W &w, const Off &o, int ks, int cb) {
        const ATTN_LDS char *base = (const ATTN_LDS char *)w.ring + ks * 16 * ROWB;
        const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)(base + o.v[2 * cb]));
        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)(base + o.v[2 * cb + 1]));
        const u32x2 a0 = __builtin_bit_cast(u32x2, t0);
        const u32x2 a1 = __builtin_bit_cast(u32x2, t1);
        return u32x4{a0[0], a0[1], a1[0], a1[1]};
    }

    // O^T += V^T . P^T for the tile in vl alone (the last matrix phase); the
    // reads of step ks+1 are scheduled ahead of the MFMAs of step ks.
    static __device__ __forceinline__ void pv(const W &w, St &st, int stage) {
        const Off o = offsets(w, 0, stage);
        u32x4 va[KS][CB];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) va[ks][cb] = v_frag(w, o, ks, cb);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) st.o[cb] = mfma32<DT>(va[ks][cb], st.ph[ks], st.o[cb]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * CB, 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2 * CB, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, CB, 1);
        }
    }

    // S^T = K . Q^T for the tile in kl alone (the first matrix phase).
    static __device__ __forceinline__ void qk(const W &w, St &st, int stage) {
        const Off o = offsets(w, stage, 0);
        u32x4 ka[KT][KB];
#pragma unroll
        for (int kk = 0; kk < KT; ++kk)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) ka[kk][kb] = k_frag(w, o, kk, kb);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) st.s[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KT; ++kk)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) st.s[kb] = mfma32<DT>(ka[kk][kb], st.qf[kk], st.s[kb]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * KB, 2);
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
            if (kk + 2 < KT) __builtin_amdgcn_sched_group_barrier(0x100, KB, 2);
            __builtin_amdgcn_sched_group_barrier(0x008, KB, 2);
        }
    }

    // The steady matrix phase: O^T += V^T . P^T of the previous tile and
    // S^T = K . Q^T of this one, their MFMAs alternating.  The fragments not
    // read ahead by the vector phase are read here, in the order the MFMAs
    // use them, PF pairs ahead.
    static_assert(NPAIR == KT * KB, "P.V and S^T must have the same MFMA count to alternate");
    static constexpr int PF = 2;
    // LDS read instructions of MFMA pair j (two per V^T fragment, one per K fragment)
    static constexpr int reads_of(int j) { return (j >= NPV ? 2 : 0) + (j >= NPK ? 1 : 0); }
    static constexpr int reads_before(int n) {
        int r = 0;
        for (int j = 0; j < n && j < NPAIR; ++j) r += reads_of(j);
        return r;
    }
    static __device__ __forceinline__ void pv_qk(const W &w, St &st, int vstage, int kstage) {
        const Off o = offsets(w, kstage, vstage);
        u32x4 va[NPAIR], ka[NPAIR];
#pragma unroll
        for (int j = 0; j < NPAIR; ++j) {
            va[j] = j < NPV ? st.vpre[j < NPV ? j : 0] : v_frag(w, o, j / CB, j % CB);
            ka[j] = j < NPK ? st.kpre[j < NPK ? j : 0] : k_frag(w, o, j / KB, j % KB);
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) st.s[kb] = f32x16{};
#pragma unroll
        for (int j = 0; j < NPAIR; ++j) {
            st.o[j % CB] = mfma32<DT>(va[j], st.ph[j / CB], st.o[j % CB]);
            st.s[j % KB] = mfma32<DT>(ka[j], st.qf[j / KB], st.s[j % KB]);
        }
        if constexpr (reads_before(PF) > 0) __builtin_amdgcn_sched_group_barrier(0x100, reads_before(PF), 3);
        static_for<NPAIR>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr (j + PF < NPAIR && reads_of(j + PF) > 0)
                __builtin_amdgcn_sched_group_barrier(0x100, reads_of(j + PF), 3);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 3);
        });
    }

    // The vector phase's reads ahead: V^T of the tile in vstage (used by the
    // next matrix phase's P.V) and K of the tile in kstage (its S^T).
    static __device__ __forceinline__ void read_ahead(const W &w, St &st, int vstage, int kstage) {
        const Off o = offsets(w, kstage, vstage);
#pragma unroll
        for (int j = 0; j < NPV; ++j) st.vpre[j] = v_frag(w, o, j / CB, j % CB);
#pragma unroll
        for (int j = 0; j < NPK; ++j) st.kpre[j] = k_frag(w, o, j / KB, j % KB);
    }

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
        u32x4 unused[KS];
        online_softmax<DT, KB, CB, false>(st.s, st.o, st.m, st.l, st.ph, unused, w.c, edge, hi, lo);
    }

    // The vector phase of tile i: the softmax when some row of the wave sees
    // the tile, else a zero P (the next matrix phase then adds nothing).
    static __device__ __forceinline__ void sphase(const W &w, St &st, int i) {
        // tile i (its V) and tile i+1 (its K, when there is one: group A
        // waited for it before the barrier that opened this phase) are in LDS
        if (i + 1 < w.T) read_ahead(w, st, i % NSTAGE, (i + 1) % NSTAGE);
        if (visible(w, w.t_begin + i)) {
            softmax(w, st, w.t_begin + i);
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) st.ph[ks] = u32x4{0u, 0u, 0u, 0u};
        }
    }

    // Tile period 1 <= i < T (ring stage i mod 4): barrier, M_i (P.V of tile
    // i-1 with S^T of tile i), barrier, S_i.  Group A issues the loads of
    // tile i+2 after the first barrier and waits for tile i+1 before the
    // second.  The loop over periods is not unrolled: the stage is a scalar
    // added into the operand offsets, and the accumulators keep one register
    // assignment.
    static __device__ __forceinline__ void period(const W &w, St &st, int i) {
        block_sync();
        if (w.grp == 0 && i + 2 < w.T) load_tile(w, w.t_begin + i + 2, (i + 2) % NSTAGE);
        pv_qk(w, st, (i + 3) % NSTAGE, i % NSTAGE);
        if (w.grp == 0 && i + 1 < w.T) wait_tiles<LPT>(i + 2 < w.T ? 1 : 0);
        block_sync();
        sphase(w, st, i);
    }

    static __device__ __forceinline__ void run(const Params &p, char *ring) {
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
        w.ring = ring;
        {
            // K: lane (l32, g) reads row kb * 32 + key_perm(l32), logical chunk
            // 2 * kk + g stored at chunk (2 * kk + g) ^ swz(row); 16 * that is
            // (32 * kk) ^ (16 * g ^ 16 * swz(row)) since 32 * kk has no bit 4.
            const int row = key_perm(w.l32);
            w.kb_ = row * ROWB;
            w.ks_ = (16 * w.g) ^ (16 * swz<D>(row));
            // V^T: lane tt of 16-lane group hgrp reads rows row0 + 4h (plus 16 *
            // ks), bytes colb .. colb + 7 of the row with colb = 64 * cb + c0;
            // chunk (colb >> 4) ^ swz(r) splits into (4 * cb) ^ (swz(r) & 12) and
            // (c0 >> 4) ^ (swz(r) & 3) on disjoint bits.  Offsets count from the
            // ring start, past the NSTAGE K stages.
            const int hgrp = w.lane >> 4, tt = w.lane & 15;
            const int row0 = 8 * (hgrp >> 1) + (tt >> 2);
            const int c0 = 32 * (hgrp & 1) + 8 * (tt & 3);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = row0 + 4 * h;
                const int sz = swz<D>(r);
                w.va_[h] = NSTAGE * TILEB + r * ROWB + ((((c0 >> 4) ^ (sz & 3))) << 4) + (c0 & 15);
                w.vs_[h] = (sz & 12) << 4;
            }
        }
        const int N = p.N;

        // (batch * head, query tile) of this workgroup; masked runs take the
        // heaviest query tiles first (n_qtiles counts down from the last)
        const int bid = blockIdx.x;
        const int bh = bh_of(bid % p.n_bh, p.n_bh, p.group, p.xcd_kv);
        const int rank = bid / p.n_bh;
        const int qt = (MASK == MASK_NONE) ? rank : p.n_qtiles - 1 - rank;
        const int b = bh / p.Hq;
        const int h = bh - b * p.Hq;
        const int hkv = p.Hq / p.group;
        const int64_t kvhead = (int64_t)b * hkv + h / p.group;
        const uint16_t *qp = p.q + (int64_t)bh * N * D;
        w.kp = p.k + kvhead * N * D;
        w.vp = p.v + kvhead * N * D;

        const int q_tile0 = qt * BM;
        w.qw0 = q_tile0 + w.grp * QROWS + w.wq * 32;
        w.w_last = min(w.qw0 + 32, N) - 1;

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

        // key tiles seen by some row of the workgroup
        const int q_last = min(q_tile0 + BM, N) - 1;
        int kv_lo = 0, kv_hi = N - 1;
        if constexpr (MASK != MASK_NONE) kv_hi = q_last;
        if constexpr (MASK == MASK_WINDOW) kv_lo = max(0, q_tile0 - p.window + 1);
        w.t_begin = kv_lo / BN;
        w.T = kv_hi / BN + 1 - w.t_begin;

        if (w.grp == 0) {
            load_tile(w, w.t_begin, 0);
            if (1 < w.T) load_tile(w, w.t_begin + 1, 1);
            wait_tiles<LPT>(1 < w.T ? 1 : 0);
        }

        if (w.grp == 1) block_sync();   // group B runs one phase behind
        // period 0: S^T of the first tile only
        block_sync();
        if (w.grp == 0 && 2 < w.T) load_tile(w, w.t_begin + 2, 2);
        qk(w, st, 0);
        if (w.grp == 0 && 1 < w.T) wait_tiles<LPT>(2 < w.T ? 1 : 0);
        block_sync();
        sphase(w, st, 0);
#pragma unroll 1
        for (int i = 1; i < w.T; ++i) period(w, st, i);
        // M_T: the P.V of the last tile
        block_sync();
        pv(w, st, (w.T + 3) % NSTAGE);
        if (w.grp == 0) block_sync();   // same barrier count as group B

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

template <int D, int DT, int MASK>
__global__ __launch_bounds__(512) void attn_fwd_pp_kernel(Params p) {
    using K = PingPong<D, DT, MASK>;
    // one LDS object: the four K stages, then the four V stages, so that a
    // wave's per-lane operand offsets serve every stage of a tensor with the
    // stage in the 16-bit immediate offset of the read (K stages within the
    // first 64 KiB, V stages within 64 KiB of the first V stage)
    __shared__ __attribute__((aligned(1024))) char ring[2 * K::NSTAGE * K::TILEB];
    K::run(p, ring);
}

}  // namespace attnfwd
