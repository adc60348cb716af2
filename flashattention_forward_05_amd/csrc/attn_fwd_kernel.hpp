// attn_fwd_kernel.hpp -- fused exact attention forward for gfx950 (MI355X).
//
// One workgroup computes one (batch, query head, query tile) of BM rows.  Its
// NWQ query waves each own QB blocks of 32 query rows; with KSPLIT = 2 or 4,
// further sets of NWQ waves own the same rows and take later parts of the
// key range, and the partial results are merged in LDS at the end (the
// rescale-and-add of partial softmax results that "Optimizaciones de
// Atencion", section "FlashDecoding", uses to combine key chunks).  A wave
// walks its key/value tiles (BN keys each) keeping a running row max, running
// row sum and an fp32 output accumulator per row, so the N x N score matrix
// never leaves the chip.  This is the tiled online softmax of that page's
// section "FlashAttention: Nunca materializar la matriz de atencion" and the
// kernel body of "Lab 02 - Forward de flash attention en Triton", sections "La
// estructura del kernel" and "Bloque B" (query tile outer, key/value tiles
// inner, fp32 m / l / O, P cast to the value dtype before P.V, O divided by l
// and LSE = m + ln l at the end).
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
//  * K and V tiles are brought to LDS by direct global->LDS loads
//    (global_load_lds_dwordx4; with eight waves, issued by waves 0-3 alone,
//    see LOADERS) into an NSTAGE-deep ring: tiles i+1 ..
//    i+NSTAGE-2 are in flight while tile i is used (a four-stage ring
//    instead loads two tiles at a time and synchronises once per pair).  The loop is unrolled
//    over the stages and the ring is one K and one V object, so each lane
//    keeps one LDS address per distinct read and reaches every stage, key
//    block and key step through the instruction's immediate offset.  The
//    waits for landed tiles are explicit partial vmcnt waits followed by a
//    bare s_barrier.  16-byte chunks are XOR-swizzled per row so that the
//    MFMA-operand reads of 16 consecutive rows hit distinct LDS banks.
//  * Softmax runs in base 2: c = |scale| * log2(e) is folded into one FMA per
//    score, p = v_exp_f32(s*c - m).  In steady state the tile max is not even
//    taken: p is formed against the running max and accepted while every
//    partial row sum stays <= 2^15; otherwise the tile max is taken and the
//    running max raised when it grows by more than TAU (log2 units).  Both are
//    the same algebra with a different reference point, so the O rescale is
//    skipped for most tiles (online_softmax in attn_fwd_common.hpp).
//  * Query tiles whose first row sees few keys use a two-term P (P_hi + P_lo,
//    both rounded to the 16-bit dtype, two MFMAs) so that the rounding of P
//    does not dominate the error of rows that average only a few values.
//  * Tiles no row of a wave can see are skipped; only tiles that cut the
//    causal diagonal, the window edge or the ragged tail evaluate masks.
#pragma once

#include "attn_fwd_common.hpp"

namespace attnfwd {

template <int D, int DT, int MASK, int QB, int NWQ, int KSPLIT, int BN, int NSTAGE, bool PAGED = false>
struct Kernel {
    static constexpr int BM = NWQ * QB * 32;
    static constexpr int NWAVES = NWQ * KSPLIT;
    static constexpr int KT = D / 16;          // 16-wide d steps of S^T = K Q^T
    static constexpr int CB = D / 32;          // 32-channel blocks of O^T
    static constexpr int KB = BN / 32;         // 32-key blocks of S^T
    static constexpr int KS = BN / 16;         // 16-key steps of O^T += V^T P^T
    static constexpr int ROWB = D * 2;         // bytes per K/V row
    static constexpr int TILEB = BN * ROWB;    // bytes per K or V tile
    static constexpr int CHUNKS_PER_ROW = D / 8;
    static constexpr int LOADS = (BN * CHUNKS_PER_ROW) / (64 * NWQ);   // 16-B loads per lane per tensor
    static constexpr int LPT = 2 * LOADS;                              // loads per lane per tile
    static constexpr int STAGEB = KSPLIT * TILEB;                      // one stage of K (or V), all groups
    static_assert((BN * CHUNKS_PER_ROW) % (64 * NWQ) == 0, "tile must split evenly over the waves");
    static_assert(BN % 32 == 0 && (D == 64 || D == 128), "unsupported tile");
    static_assert(NSTAGE >= 2 && NSTAGE <= 4 && (KSPLIT == 1 || KSPLIT == 2 || KSPLIT == 4), "unsupported pipeline");

    // per-wave state
    struct State {
        u32x4 qf[QB][KT];
        f32x16 oacc[QB][CB];
        float mrun[QB];
        float lsum[QB];
    };

    // Nq / Nk: query rows and keys; qw0: first query row of the wave; pw0 and
    // w_last: lowest and highest sequence position of the wave's valid rows
    // (row + q_off, or q_off + row % pack_nq for stacked heads), and lpos the
    // position of this lane's rows: what the masks compare keys against.
    struct Ctx {
        const uint16_t *kp, *vp;
        int Nq, Nk, window, lane, g, l32, wave_q, kgroup;
        int qw0, pw0, w_last, q_off;
        int tstride;             // key tiles of one group: my_begin + i * tstride
        bool loader;   // LOADERS: this wave issues its partner's loads as well
        int lpos[QB];
        // paged K/V: this batch's block-table row, the K/V head and the page geometry
        const int32_t *bt;
        int64_t kvh;
        int page_shift, num_pages, Hkv;
        int max_pages;
        float c;
        char *kst[NSTAGE];
        char *vst[NSTAGE];
        // LDS byte addresses of this lane's operand reads in ring stage 0,
        // without the key block / key step (added as immediates, as is the
        // stage): koff[kk] for the K row of d-step kk, voff[2*cb+h] for the
        // two V^T reads of channel block cb
        uint32_t koff[KT];
        uint32_t voff[2 * CB];
    };

    // Sequence position of query row r, and the lowest / highest position
    // over rows a .. b (a <= b): with stacked heads the rows of one range can
    // wrap from one query head to the next.
    static __device__ __forceinline__ int pos_of(const Params &p, int q_off, int r) {
        return q_off + (p.pack_nq > 0 ? r % p.pack_nq : r);
    }
    static __device__ __forceinline__ void pos_range(const Params &p, int q_off, int a, int b, int &lo, int &hi) {
        b = max(a, b);
        if (p.pack_nq > 0 && (b - a + 1 >= p.pack_nq || a / p.pack_nq != b / p.pack_nq)) {
            lo = q_off;
            hi = q_off + p.pack_nq - 1;
        } else {
            lo = pos_of(p, q_off, a);
            hi = pos_of(p, q_off, b);
        }
    }

    // Paged K/V: one direct-load instruction covers 64 / CHUNKS_PER_ROW (4 or
    // 8) consecutive rows starting at a multiple of that count, so with pages
    // of at least 8 keys its rows share one page and the page id is a scalar
    // (a scalar-cache read of the block table: it does not count against the
    // vector-memory waits that track the tile loads).  Rows at or past the
    // batch's length read the last key instead (in the same page, or the last
    // key's page when the whole group is past it), so masked rows still hold
    // finite data.  paged_page gives the (clamped) page id of a group,
    // paged_slot the slot of a lane's key in it.
    static __device__ __forceinline__ int paged_page(const Ctx &x, int row_first) {
        const int prow = __builtin_amdgcn_readfirstlane(min(row_first, x.Nk - 1));
        const int page = ((const __attribute__((address_space(4))) int32_t *)x.bt)[prow >> x.page_shift];
        return min(max(page, 0), x.num_pages - 1);
    }
    static __device__ __forceinline__ int paged_slot(const Ctx &x, int row) {
        return min(row, x.Nk - 1) & ((1 << x.page_shift) - 1);
    }

    // Issue the direct loads of tile t (keys t*BN ..) into ring stage dst.
    // Paged tile loads with PPT consecutive block-table entries per tile
    // (page_size = BN / PPT, or PPT = 1 when a page holds the whole tile):
    // when the tile's entries lie inside the batch's table row they are read
    // with one wide scalar load; group i then takes entry
    // min(its first row, last key) / page_size of that window.  Otherwise
    // (the last entries of a row) each group reads its own entry.
    template <int PPT>
    static __device__ __forceinline__ void load_tile_paged(const Ctx &x, int j0, char *kdst, char *vdst) {
        const int e_first = j0 >> x.page_shift;
        const int e_last = (x.Nk - 1) >> x.page_shift;
        int page[LOADS];
        if (e_first + PPT <= x.max_pages) {
            int pw[PPT];
            const __attribute__((address_space(4))) int32_t *bt =
                (const __attribute__((address_space(4))) int32_t *)x.bt + e_first;
#pragma unroll
            for (int k = 0; k < PPT; ++k) pw[k] = min(max(bt[k], 0), x.num_pages - 1);
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int e = min((j0 + ((i * NWQ + x.wave_q) * 64) / CHUNKS_PER_ROW) >> x.page_shift, e_last);
                int pg = pw[0];
#pragma unroll
                for (int k = 1; k < PPT; ++k) pg = (e - e_first == k) ? pw[k] : pg;
                page[i] = pg;
            }
        } else {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) page[i] = paged_page(x, j0 + ((i * NWQ + x.wave_q) * 64) / CHUNKS_PER_ROW);
        }
        const uint32_t kb = lds_base(x, kdst), vb = lds_base(x, vdst);
        static_for<LOADS>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const int slot = (i * NWQ + x.wave_q) * 64 + x.lane;
            const int row = slot / CHUNKS_PER_ROW;
            const int ch = (slot % CHUNKS_PER_ROW) ^ swz<D>(row);
            const int64_t pbase = ((int64_t)page[i] * x.Hkv + x.kvh) << x.page_shift;   // in rows
            const uint32_t voff = (uint32_t)(paged_slot(x, j0 + row) * (D * 2) + ch * 16);
            lds_dma16_s_at<i * NWQ * 1024>(x.kp + pbase * D, voff, kb);
            lds_dma16_s_at<i * NWQ * 1024>(x.vp + pbase * D, voff, vb);
        });
    }

    // Wave-uniform LDS address of this wave's first load slot in a ring
    // stage; slot i is at + i * NWQ * 1024.
    static __device__ __forceinline__ uint32_t lds_base(const Ctx &x, const char *stage) {
        return __builtin_amdgcn_readfirstlane(lds_addr(stage + x.kgroup * TILEB + x.wave_q * 1024));
    }

    // Contiguous K/V: tile t into the load slots of query wave wq of this
    // wave's key group.
    static __device__ __forceinline__ void load_tile_as(const Ctx &x, int t, char *kdst, char *vdst, int wq) {
        const int j0 = t * BN;
        const uint32_t kb = __builtin_amdgcn_readfirstlane(lds_addr(kdst + x.kgroup * TILEB + wq * 1024));
        const uint32_t vb = __builtin_amdgcn_readfirstlane(lds_addr(vdst + x.kgroup * TILEB + wq * 1024));
        static_for<LOADS>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const int slot = (i * NWQ + wq) * 64 + x.lane;
            const int row = slot / CHUNKS_PER_ROW;
            const int chp = slot % CHUNKS_PER_ROW;
            const int ch = chp ^ swz<D>(row);
            const int64_t grow = min(j0 + row, x.Nk - 1);
            const int64_t off = grow * D + ch * 8;
            lds_dma16_at<i * NWQ * 1024>(x.kp + off, kb);
            lds_dma16_at<i * NWQ * 1024>(x.vp + off, vb);
        });
    }

    // Eight-wave configurations (waves w and w + 4 on one SIMD): the waves
    // w + 4 lose the SIMD's issue to the waves w and set the pace, while the
    // waves w wait at the barrier.  So waves 0-3 issue every tile load, their
    // own slots and those of wave w + 4, right after the barrier, and waves
    // 4-7 issue none.
    // With two key groups (the 128-row configuration) the waves are numbered
    // group-minor (key group = wave % 2) so that waves w and w + 4 share a key
    // group, and the same scheme applies.
    static constexpr bool LOADERS = !PAGED && NWQ * KSPLIT == 8 && (KSPLIT == 1 || KSPLIT == 2);

    // Tile t into this wave's load slots (and, for a loader, its partner's).
    static __device__ __forceinline__ void load_tile_step(const Ctx &x, int t, char *kdst, char *vdst) {
        if constexpr (LOADERS) {
            if (x.loader) {
                load_tile_as(x, t, kdst, vdst, x.wave_q);
                load_tile_as(x, t, kdst, vdst, x.wave_q + NWQ / 2);
            }
        } else {
            load_tile(x, t, kdst, vdst);
        }
    }

    static __device__ __forceinline__ void load_tile(const Ctx &x, int t, char *kdst, char *vdst) {
        const int j0 = t * BN;
        if constexpr (PAGED) {
            const int ppt = BN >> x.page_shift;   // 0 when a page is longer than a tile
            if constexpr (BN >= 64) {
                if (ppt >= 8) return load_tile_paged<8>(x, j0, kdst, vdst);
            }
            if (ppt >= 4) return load_tile_paged<4>(x, j0, kdst, vdst);
            if (ppt >= 2) return load_tile_paged<2>(x, j0, kdst, vdst);
            return load_tile_paged<1>(x, j0, kdst, vdst);
        }
        const uint32_t kb = lds_base(x, kdst), vb = lds_base(x, vdst);
        static_for<LOADS>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const int slot = (i * NWQ + x.wave_q) * 64 + x.lane;
            const int row = slot / CHUNKS_PER_ROW;
            const int chp = slot % CHUNKS_PER_ROW;
            const int ch = chp ^ swz<D>(row);
            const int64_t grow = min(j0 + row, x.Nk - 1);
            const int64_t off = grow * D + ch * 8;
            lds_dma16_at<i * NWQ * 1024>(x.kp + off, kb);
            lds_dma16_at<i * NWQ * 1024>(x.vp + off, vb);
        });
    }

    // The per-lane read offsets of Ctx (the ring is one K and one V object,
    // so every stage is a fixed distance from stage 0).  K: the lane reads
    // row key_perm(l32) of each 32-key block, 16-byte chunk 2*kk + g; the
    // swizzle depends only on the row's low four bits, which the key block
    // does not change.  V: in each 16-lane group lane tt reads rows
    // 8*(group/2) + tt/4 (+4) of each 16-key step at column 8*(tt%4) of its
    // half of channel block cb; again the step does not change the low row
    // bits.  The offsets are made opaque to the compiler so that it keeps
    // one register each rather than one per ring stage.
    static __device__ __forceinline__ void set_offsets(Ctx &x) {
        const uint32_t kb0 = lds_addr(x.kst[0] + x.kgroup * TILEB);
        const uint32_t vb0 = lds_addr(x.vst[0] + x.kgroup * TILEB);
        const int krow = key_perm(x.l32);
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
            x.koff[kk] = kb0 + (uint32_t)(krow * ROWB + (((2 * kk + x.g) ^ swz<D>(krow)) << 4));
            asm volatile("" : "+v"(x.koff[kk]));
        }
        const int hgrp = x.lane >> 4;
        const int tt = x.lane & 15;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 8 * (hgrp >> 1) + (tt >> 2) + 4 * h;
                const int colb = cb * 64 + 32 * (hgrp & 1) + 8 * (tt & 3);
                const int ch = colb >> 4, within = colb & 15;
                x.voff[2 * cb + h] = vb0 + (uint32_t)(row * ROWB + ((ch ^ swz<D>(row)) << 4) + within);
                asm volatile("" : "+v"(x.voff[2 * cb + h]));
            }
    }

    // V^T A-operand fragment of ring stage S for 16-key step ks and channel
    // block cb: two transposing reads of 4 keys x 16 channels per 16-lane
    // group.
    template <int S>
    static __device__ __forceinline__ u32x4 v_frag(const Ctx &x, int ks, int cb) {
        constexpr int IMM0 = S * STAGEB;
        const uint32_t a0 = x.voff[2 * cb] + (uint32_t)(IMM0 + ks * 16 * ROWB);
        const uint32_t a1 = x.voff[2 * cb + 1] + (uint32_t)(IMM0 + ks * 16 * ROWB);
        const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)(uintptr_t)a0);
        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4 *)(uintptr_t)a1);
        const u32x2 b0 = __builtin_bit_cast(u32x2, t0);
        const u32x2 b1 = __builtin_bit_cast(u32x2, t1);
        return u32x4{b0[0], b0[1], b1[0], b1[1]};
    }

    // O^T += V^T . P^T over one tile in ring stage S (P_lo as well when
    // EXACT).  The reads of step ks+1 are scheduled ahead of the MFMAs of
    // step ks.
    template <bool EXACT, int S>
    static __device__ __forceinline__ void pv(const Ctx &x, State &st, const u32x4 (&ph)[QB][KS],
                                              const u32x4 (&pl)[QB][KS]) {
        u32x4 va[KS][CB];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) va[ks][cb] = v_frag<S>(x, ks, cb);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    st.oacc[qb][cb] = mfma32<DT>(va[ks][cb], ph[qb][ks], st.oacc[qb][cb]);
                    if constexpr (EXACT) st.oacc[qb][cb] = mfma32<DT>(va[ks][cb], pl[qb][ks], st.oacc[qb][cb]);
                }
        constexpr int RD = 2 * CB;                        // transposing reads per step
        constexpr int MF = CB * QB * (EXACT ? 2 : 1);     // MFMAs per step
        __builtin_amdgcn_sched_group_barrier(0x100, RD, 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) __builtin_amdgcn_sched_group_barrier(0x100, RD, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, MF, 1);
        }
    }

    // S^T = K . Q^T for the tile in ring stage S; K fragments are read two
    // d-steps ahead.
    template <int S>
    static __device__ __forceinline__ void qk(const Ctx &x, const State &st, f32x16 (&s)[KB][QB]) {
        u32x4 ka[KT][KB];
#pragma unroll
        for (int kk = 0; kk < KT; ++kk)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const uint32_t a = x.koff[kk] + (uint32_t)(S * STAGEB + kb * 32 * ROWB);
                ka[kk][kb] = *(const ATTN_LDS u32x4 *)(uintptr_t)a;
            }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KT; ++kk)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma32<DT>(ka[kk][kb], st.qf[qb][kk], s[kb][qb]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * KB, 0);
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
            if (kk + 2 < KT) __builtin_amdgcn_sched_group_barrier(0x100, KB, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, KB * QB, 0);
        }
    }

    // Does tile t need masks for some row of this wave (causal diagonal,
    // window edge or the ragged tail)?
    static __device__ __forceinline__ bool edge_tile(const Ctx &x, int t) {
        const int j0 = t * BN;
        bool edge = (j0 + BN > x.Nk);
        if constexpr (MASK != MASK_NONE) edge = edge || (j0 + BN - 1 > x.pw0);
        if constexpr (MASK == MASK_WINDOW) edge = edge || (j0 < x.w_last - x.window + 1);
        return edge;
    }

    // Does some row of this wave see a key of tile t?
    static __device__ __forceinline__ bool visible_tile(const Ctx &x, int t) {
        bool any = x.qw0 < x.Nq;
        if constexpr (MASK != MASK_NONE) any = any && (t * BN <= x.w_last);
        if constexpr (MASK == MASK_WINDOW) any = any && (t * BN + BN - 1 >= x.pw0 - x.window + 1);
        return any;
    }

    // The online-softmax update of one tile for every query block of the
    // wave (masks on edge tiles).
    template <bool EXACT>
    static __device__ __forceinline__ void softmax(const Ctx &x, State &st, int t, f32x16 (&s)[KB][QB], bool edge,
                                                   u32x4 (&ph)[QB][KS], u32x4 (&pl)[QB][KS]) {
        const int j0 = t * BN;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int qi = x.lpos[qb];
            int hi = x.Nk - 1 - (j0 + 8 * x.g);
            int lo = -(1 << 30);
            if constexpr (MASK != MASK_NONE) hi = min(hi, qi - (j0 + 8 * x.g));
            if constexpr (MASK == MASK_WINDOW) lo = qi - x.window + 1 - (j0 + 8 * x.g);
            f32x16 sq[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sq[kb] = s[kb][qb];
            online_softmax<DT, KB, CB, EXACT>(sq, st.oacc[qb], st.mrun[qb], st.lsum[qb], ph[qb], pl[qb], x.c, edge,
                                              hi, lo);
        }
    }

    // Everything one wave does with the landed tile t in ring stage S.
    template <bool EXACT, int S>
    static __device__ __forceinline__ void compute_tile(const Ctx &x, State &st, int t) {
        const bool edge = edge_tile(x, t);

        // ---- S^T = K . Q^T
        f32x16 s[KB][QB];
        qk<S>(x, st, s);

        // ---- online softmax, one lane per query row
        u32x4 ph[QB][KS], pl[QB][KS];
        softmax<EXACT>(x, st, t, s, edge, ph, pl);

        // ---- O^T += V^T . P^T
        pv<EXACT, S>(x, st, ph, pl);
    }

    // With a four-stage ring the workgroup meets once per pair of tiles: at
    // the even step i both tiles i and i+1 have landed, so a wave that is
    // ahead runs on into tile i+1 instead of waiting at a barrier, and the
    // loads of tiles i+2 and i+3 go to the two stages the previous pair held.
    static constexpr bool PAIR = NSTAGE == 4;

    // Paired 64-row query tiles (causal, 128-row configuration): the key
    // groups take alternate tiles, so the few tiles of the light rows are
    // shared by both groups.
    static constexpr bool PAIRABLE = MASK == MASK_CAUSAL && !PAGED && NWQ == 4 && KSPLIT == 2 && QB == 1;
    static __device__ __forceinline__ int tile_at(const Ctx &x, int my_begin, int i) {
        if constexpr (PAIRABLE) return my_begin + i * x.tstride;
        return my_begin + i;
    }

    // One pipeline step on ring stage S: wait for tile i, barrier, prefetch
    // tile i + NSTAGE - 1 into the stage that held tile i - 1, compute tile i
    // (with PAIR: the barrier and the loads of two tiles on even steps only).
    template <int S, bool EXACT>
    static __device__ __forceinline__ void step(const Ctx &x, State &st, int i, int my_begin, int my_count) {
        if constexpr (PAIR) {
            if constexpr (S % 2 == 0) {
                // tiles i and i+1 are the only loads in flight: both landed
                // for every wave, and tiles i-2, i-1 are no longer read
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                block_sync();
                if (i + 2 < my_count) load_tile_step(x, tile_at(x, my_begin, i + 2), x.kst[(S + 2) % 4], x.vst[(S + 2) % 4]);
                if (i + 3 < my_count) load_tile_step(x, tile_at(x, my_begin, i + 3), x.kst[(S + 3) % 4], x.vst[(S + 3) % 4]);
            }
            if (i < my_count) {
                const int t = tile_at(x, my_begin, i);
                if (visible_tile(x, t)) compute_tile<EXACT, S>(x, st, t);
            }
            return;
        }
        // a loader issues the loads of two waves per tile
        wait_tiles<(LOADERS ? 2 : 1) * LPT>(min(NSTAGE - 2, my_count - 1 - i));
        block_sync();
        constexpr int SN = (S + NSTAGE - 1) % NSTAGE;
        if (i + NSTAGE - 1 < my_count) load_tile_step(x, tile_at(x, my_begin, i + NSTAGE - 1), x.kst[SN], x.vst[SN]);
        if (i < my_count) {
            const int t = tile_at(x, my_begin, i);
            if (visible_tile(x, t)) compute_tile<EXACT, S>(x, st, t);
        }
    }

    template <bool EXACT>
    static __device__ __forceinline__ void loop(const Ctx &x, State &st, int half, int my_begin, int my_count) {
        for (int i = 0; i < half; i += NSTAGE) {
            step<0, EXACT>(x, st, i, my_begin, my_count);
            if (i + 1 < half) step<1 % NSTAGE, EXACT>(x, st, i + 1, my_begin, my_count);
            if constexpr (NSTAGE > 2)
                if (i + 2 < half) step<2 % NSTAGE, EXACT>(x, st, i + 2, my_begin, my_count);
            if constexpr (NSTAGE > 3)
                if (i + 3 < half) step<3 % NSTAGE, EXACT>(x, st, i + 3, my_begin, my_count);
        }
    }

    static __device__ __forceinline__ void run(const Params &p, char *const (&kst)[NSTAGE],
                                               char *const (&vst)[NSTAGE], float *ml) {
        Ctx x;
        x.lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        x.wave_q = (LOADERS && KSPLIT == 2) ? wave / 2 : wave % NWQ;
        x.kgroup = (LOADERS && KSPLIT == 2) ? wave % 2 : wave / NWQ;
        x.g = x.lane >> 5;
        x.l32 = x.lane & 31;
        x.Nq = p.N;
        x.window = p.window;
        x.c = p.c;
        for (int s = 0; s < NSTAGE; ++s) {
            x.kst[s] = kst[s];
            x.vst[s] = vst[s];
        }
        set_offsets(x);
        const int N = p.N;

        // ---- which (batch*head, key split, query tile) this workgroup owns;
        // for masked runs the heaviest query tiles (most visible keys) are
        // dispatched first.
        const int bid = blockIdx.x;
        const int bh = bh_of(bid % p.n_bh, p.n_bh, p.group, p.xcd_kv);
        const int rest = bid / p.n_bh;
        const int split = rest % p.n_splits;
        const int rank = rest / p.n_splits;
        const int qt = (MASK == MASK_NONE) ? rank : masked_qtile(rank, p.n_qtiles, p.zigzag);
        const int b = bh / p.Hq;
        const int h = bh - b * p.Hq;
        const int hkv = p.Hq / p.group;
        const int64_t kvhead = (int64_t)b * hkv + h / p.group;
        const uint16_t *qp = p.q + (int64_t)bh * N * D;
        // keys of this batch, and the position offset of its query rows
        int Nk = p.Nk;
        int q_off = p.q_off;
        if constexpr (PAGED) {
            Nk = min(max(((const __attribute__((address_space(4))) int32_t *)p.seq_lens)[b], 0), p.Nk);
            q_off = Nk - (p.pack_nq > 0 ? p.pack_nq : N);
            x.bt = p.block_table + (int64_t)b * p.max_pages;
            x.kvh = h / p.group;
            x.page_shift = p.page_shift;
            x.num_pages = p.num_pages;
            x.max_pages = p.max_pages;
            x.Hkv = p.Hkv;
            x.kp = p.k;
            x.vp = p.v;
        } else {
            x.kp = p.k + kvhead * Nk * D;
            x.vp = p.v + kvhead * Nk * D;
        }
        x.Nk = Nk;
        x.q_off = q_off;

        const int q_tile0 = qt * BM;
        x.qw0 = q_tile0 + x.wave_q * QB * 32;
        int row_lo = q_tile0, row_hi = min(q_tile0 + BM, N) - 1;
        if constexpr (MASK == MASK_CAUSAL && !PAGED && NWQ == 4 && KSPLIT == 2 && QB == 1) {
            if (p.zigzag == 2) {
                // query waves 0-1 take 64-row tile n64 - 1 - rank, waves 2-3 tile rank
                // (none when the two coincide); the key range covers both
                const int n64 = (N + 63) >> 6;
                const int heavy = n64 - 1 - rank, light = rank;
                const bool upper = x.wave_q < NWQ / 2;
                x.qw0 = upper ? heavy * 64 + x.wave_q * 32
                              : (light < heavy ? light * 64 + (x.wave_q - NWQ / 2) * 32 : N);
                row_lo = light * 64;
                row_hi = min(heavy * 64 + 63, N - 1);
            }
        }
        pos_range(p, q_off, x.qw0, min(x.qw0 + QB * 32, N) - 1, x.pw0, x.w_last);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) x.lpos[qb] = pos_of(p, q_off, x.qw0 + qb * 32 + x.l32);

        State st;
        // ---- Q fragments (MFMA B operand): lane holds row qw0 + 32*qb + l32,
        // channels 16*kk + 8*g .. +7.  Rows past N are zero.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int row = x.qw0 + qb * 32 + x.l32;
#pragma unroll
            for (int kk = 0; kk < KT; ++kk) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (row < N) {
                    v = *(const u32x4 *)(qp + (int64_t)row * D + kk * 16 + x.g * 8);
                    v ^= p.qsign;
                }
                st.qf[qb][kk] = v;
            }
            st.mrun[qb] = -__builtin_inff();
            st.lsum[qb] = 0.0f;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) st.oacc[qb][cb][r] = 0.0f;
        }

        // ---- key tiles seen by the workgroup (within its key split), divided
        // between the key groups
        int p_first, p_last;
        pos_range(p, q_off, row_lo, row_hi, p_first, p_last);
        int kv_lo = 0, kv_hi = Nk - 1;
        if constexpr (MASK != MASK_NONE) kv_hi = min(kv_hi, p_last);
        if constexpr (MASK == MASK_WINDOW) kv_lo = max(0, p_first - p.window + 1);
        const int s_first = p.split_t0 + split * p.split_tiles;
        const int t_begin = max(kv_lo / BN, s_first);
        const int t_last = min(kv_hi / BN, s_first + p.split_tiles - 1);
        const int n_tiles = Nk > 0 ? max(0, t_last + 1 - t_begin) : 0;
        const int half = (n_tiles + KSPLIT - 1) / KSPLIT;
        int my_begin = t_begin + x.kgroup * half;
        int my_count = max(0, min(half, n_tiles - x.kgroup * half));
        x.tstride = 1;

        // ---- two-term P for query tiles whose first row sees few keys
        int min_vis = Nk;
        if constexpr (MASK != MASK_NONE) min_vis = min(Nk, p_first + 1);
        if constexpr (MASK == MASK_WINDOW) min_vis = min(min_vis, p.window);
        if constexpr (PAIRABLE) {
            if (p.zigzag == 2) {
                // alternate tiles per key group; the P mode follows the wave's own rows
                my_begin = t_begin + x.kgroup;
                my_count = max(0, (n_tiles - x.kgroup + 1) / 2);
                x.tstride = 2;
                min_vis = min(Nk, x.pw0 + 1);
            }
        }
        const bool exact = min_vis < p.exact_below;

        // ---- prologue: the first NSTAGE-1 tiles (two with PAIR) in flight, then the main
        // loop, unrolled over the ring stages; one instance per P mode
        x.loader = x.wave_q < NWQ / 2;
#pragma unroll
        for (int s = 0; s < (PAIR ? 2 : NSTAGE - 1); ++s)
            if (s < my_count) load_tile_step(x, tile_at(x, my_begin, s), x.kst[s], x.vst[s]);
        if (exact)
            loop<true>(x, st, half, my_begin, my_count);
        else
            loop<false>(x, st, half, my_begin, my_count);

        // ---- merge the key groups: groups 1 .. KSPLIT-1 hand (m, l, O) to
        // group 0.  The ring is idle now; channel block cb of O of group g
        // goes to ring array cb at slot g - 1.
        if constexpr (KSPLIT > 1) {
            constexpr int SLOT = NWQ * QB * 16 * 64;   // floats of one group's channel block
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __syncthreads();
            char *ring[2 * NSTAGE];
#pragma unroll
            for (int s2 = 0; s2 < NSTAGE; ++s2) {
                ring[2 * s2] = x.kst[s2];
                ring[2 * s2 + 1] = x.vst[s2];
            }
            if (x.kgroup != 0) {
                const int slot = x.kgroup - 1;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int base = (x.wave_q * QB + qb);
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        float *dst = (float *)ring[cb] + slot * SLOT;
#pragma unroll
                        for (int r = 0; r < 16; ++r) dst[(base * 16 + r) * 64 + x.lane] = st.oacc[qb][cb][r];
                    }
                    ml[((slot * NWQ * QB + base) * 2 + 0) * 64 + x.lane] = st.mrun[qb];
                    ml[((slot * NWQ * QB + base) * 2 + 1) * 64 + x.lane] = st.lsum[qb];
                }
            }
            __syncthreads();
            if (x.kgroup != 0) return;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int base = (x.wave_q * QB + qb);
                float mg[KSPLIT], lg[KSPLIT];
                mg[0] = st.mrun[qb];
                lg[0] = st.lsum[qb];
                float m = mg[0];
#pragma unroll
                for (int g2 = 1; g2 < KSPLIT; ++g2) {
                    mg[g2] = ml[(((g2 - 1) * NWQ * QB + base) * 2 + 0) * 64 + x.lane];
                    lg[g2] = ml[(((g2 - 1) * NWQ * QB + base) * 2 + 1) * 64 + x.lane];
                    m = fmaxf(m, mg[g2]);
                }
                float a[KSPLIT];
                float l = 0.0f;
#pragma unroll
                for (int g2 = 0; g2 < KSPLIT; ++g2) {
                    a[g2] = (mg[g2] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mg[g2] - m);
                    l += lg[g2] * a[g2];
                }
                st.mrun[qb] = m;
                st.lsum[qb] = l;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const float *src = (const float *)ring[cb];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float acc = st.oacc[qb][cb][r] * a[0];
#pragma unroll
                        for (int g2 = 1; g2 < KSPLIT; ++g2)
                            acc += src[(g2 - 1) * SLOT + (base * 16 + r) * 64 + x.lane] * a[g2];
                        st.oacc[qb][cb][r] = acc;
                    }
                }
            }
        }

        // ---- epilogue of one key split: O / l in fp32 and m + log2 l go to
        // the workspace for the merge kernel (a row that saw no key of this
        // split gives O = 0 and -inf)
        if (p.n_splits > 1) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float lt = sum_halves(st.lsum[qb]);
                const int qi = x.qw0 + qb * 32 + x.l32;
                if (qi < N) {
                    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
                    const int64_t prow = ((int64_t)split * p.n_bh + bh) * N + qi;
                    float *orow = p.ws_o + prow * D;
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                        for (int j4 = 0; j4 < 4; ++j4) {
                            const int ch = cb * 32 + 8 * j4 + 4 * x.g;
                            float4 w;
                            w.x = st.oacc[qb][cb][4 * j4 + 0] * inv;
                            w.y = st.oacc[qb][cb][4 * j4 + 1] * inv;
                            w.z = st.oacc[qb][cb][4 * j4 + 2] * inv;
                            w.w = st.oacc[qb][cb][4 * j4 + 3] * inv;
                            *(float4 *)(orow + ch) = w;
                        }
                    if (x.g == 0)
                        p.ws_ml[prow] = lt > 0.0f ? st.mrun[qb] + __builtin_amdgcn_logf(lt) : -__builtin_inff();
                }
            }
            return;
        }

        // ---- epilogue: O = acc / l, rounded once; LSE = ln 2 * (m + log2 l)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float lt = sum_halves(st.lsum[qb]);
            const int qi = x.qw0 + qb * 32 + x.l32;
            if (qi < N) {
                const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
                uint16_t *orow = p.o + ((int64_t)bh * N + qi) * D;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4) {
                        const int ch = cb * 32 + 8 * j4 + 4 * x.g;
                        u32x2 w;
                        w[0] = pack2<DT>(st.oacc[qb][cb][4 * j4 + 0] * inv, st.oacc[qb][cb][4 * j4 + 1] * inv);
                        w[1] = pack2<DT>(st.oacc[qb][cb][4 * j4 + 2] * inv, st.oacc[qb][cb][4 * j4 + 3] * inv);
                        *(u32x2 *)(orow + ch) = w;
                    }
                if (p.lse != nullptr && x.g == 0) {
                    const float l2 = lt > 0.0f ? __builtin_amdgcn_logf(lt) : -__builtin_inff();
                    p.lse[(int64_t)bh * N + qi] = (st.mrun[qb] + l2) * 0.69314718055994530942f;
                }
            }
        }
    }
};

// Ring-stage LDS objects are declared one by one so that each stage is a
// distinct object to the compiler's alias analysis.
template <int D, int DT, int MASK, int QB, int NWQ, int KSPLIT, int BN, int NSTAGE, bool PAGED = false>
__global__ __launch_bounds__(NWQ * KSPLIT * 64) void attn_fwd_kernel(Params p) {
    using K = Kernel<D, DT, MASK, QB, NWQ, KSPLIT, BN, NSTAGE, PAGED>;
    constexpr int SB = K::STAGEB;
    // one K and one V object for all ring stages: every stage is a
    // compile-time distance from stage 0, so reads address it by immediate
    __shared__ __attribute__((aligned(1024))) char kring[NSTAGE * SB];
    __shared__ __attribute__((aligned(1024))) char vring[NSTAGE * SB];
    // the merge of the key groups keeps O in the ring and (m, l) here
    static_assert(KSPLIT == 1 || (D / 32 <= 2 * NSTAGE && (KSPLIT - 1) * NWQ * QB * 16 * 64 * 4 <= SB),
                  "ring too small to hold the key-group merge");
    static_assert((NSTAGE - 1) * SB + (BN - 16) * D * 2 < 65536, "stage offsets must fit the 16-bit LDS immediate");
    __shared__ __attribute__((aligned(16))) float ml[KSPLIT > 1 ? (KSPLIT - 1) * NWQ * QB * 2 * 64 : 4];
    char *kst[NSTAGE];
    char *vst[NSTAGE];
#pragma unroll
    for (int s = 0; s < NSTAGE; ++s) {
        kst[s] = kring + s * SB;
        vst[s] = vring + s * SB;
    }
    K::run(p, kst, vst, ml);
}

}  // namespace attnfwd
