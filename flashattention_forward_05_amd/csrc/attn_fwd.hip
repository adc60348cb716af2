// attn_fwd.hip -- C ABI of the fused attention forward (declared in
// include/attn_fwd.h): argument checks, tile-configuration choice and launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "attn_fwd.h"
#include "attn_fwd_launch.hpp"
#include "attn_fwd_lockstep.hpp"
#include "attn_fwd_merge.hpp"

namespace {

using attnfwd::Params;

// Tile configurations compiled into the library (all of the lockstep kernel,
// attn_fwd_kernel.hpp).  qb: 32-row query blocks per wave; nwq: query waves
// per workgroup; ksplit: key groups per workgroup (2 or 4 = further sets of
// waves take later parts of the key range, merged in LDS); bn: keys per K/V
// tile; nstage: depth of the LDS tile ring.  The same id may use a smaller
// tile for d = 128 so that LDS and registers fit.  Each is the automatic
// choice of some workload (see auto_config and splitkv_auto_config).
struct TileCfg {
    int qb, nwq, ksplit, bn, nstage;
    int bm() const { return qb * nwq * 32; }
    int waves() const { return nwq * ksplit; }
};
constexpr int kNumConfigs = 5;
constexpr TileCfg kCfg64[kNumConfigs] = {
    {1, 4, 2, 64, 3},   // 0: 128 rows, 8 waves (two key groups)
    {1, 8, 1, 64, 4},   // 1: 256 rows, 8 waves (four stages: one barrier per two tiles)
    {1, 2, 2, 64, 2},   // 2: 64 rows, 4 waves (two key groups), two workgroups per CU
    {1, 1, 1, 64, 3},   // 3: 32 rows, 1 wave (few query rows: decoding)
    {1, 1, 4, 64, 2},   // 4: 32 rows, 4 waves in four key groups (small grids)
};
constexpr TileCfg kCfg128[kNumConfigs] = {
    {1, 4, 2, 64, 2},
    {1, 8, 1, 64, 4},
    {1, 2, 2, 32, 2},
    {1, 1, 1, 32, 3},
    {1, 1, 4, 32, 2},
};
const TileCfg &tile_cfg(int64_t d, int id) { return d == 64 ? kCfg64[id] : kCfg128[id]; }


// Query tiles whose first row sees fewer keys than this use the two-term P.
constexpr int kExactBelow = 256;

// Causal runs of the 128-row configuration pair 64-row query tiles r and
// n - 1 - r per workgroup (equal work) while the grid fits one resident round;
// on larger grids heavy-first dispatch balances the load and the paired
// layout, whose light waves finish early, is slower.
constexpr int64_t kPairMaxGrid = 256;

constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxSplits = 1024;
constexpr int64_t kMaxHeads = int64_t(1) << 24;

bool ranges_overlap(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

int mask_mode(int causal, int64_t window) {
    if (!causal) return attnfwd::MASK_NONE;
    return window > 0 ? attnfwd::MASK_WINDOW : attnfwd::MASK_CAUSAL;
}

int check_sizes(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                int64_t window, float scale, int dtype) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 0 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
    if (N > kMaxN || B > kMaxHeads || Hq > kMaxHeads || B * Hq > kMaxHeads) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (window < 0 || (window > 0 && !causal)) return ATTN_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return ATTN_ERR_ARG;
    return ATTN_OK;
}

// Automatic choice (measured on MI355X).  d = 128 with at least two 256-row
// workgroups per compute unit runs 8 query waves of 32 rows (1); smaller
// d = 128 grids run 128-row workgroups with two key groups (0).  For d = 64,
// 64-row workgroups, two per compute unit (2), win on small grids and on
// masked runs, where they spread the uneven causal work over twice as many
// workgroups; larger unmasked grids keep the 128-row workgroups (0).  When
// even 32-row workgroups are at most one per compute unit, 32 rows with four
// key groups (4) keep every SIMD busy.
int auto_config(int64_t B, int64_t Hq, int64_t N, int64_t d, int mask, bool pairs = true) {
    const int64_t wg128 = B * Hq * ((N + 127) / 128);
    if (d == 128) {
        const int64_t wg256 = B * Hq * ((N + 255) / 256);
        return wg256 >= 512 ? 1 : 0;
    }
    if (B * Hq * ((N + 31) / 32) <= 256) return 4;
    // causal: below about one 128-row workgroup per compute unit the 64-row
    // workgroups fill more units; up to one resident round configuration 0 with
    // paired 64-row tiles of equal work (where the launch can pair them: not for
    // paged K/V or stacked heads); on large grids the 256-row workgroups
    if (mask == attnfwd::MASK_CAUSAL && pairs) {
        if (wg128 < 128) return 2;
        if (B * Hq * ((N + 255) / 256) >= 1024) return 1;
        return 0;
    }
    if (mask != attnfwd::MASK_NONE) return wg128 <= 512 ? 2 : 0;
    return wg128 < 128 ? 2 : 0;
}

// Routes a launch to the translation unit that holds its instantiation.
hipError_t launch(int64_t d, int dtype, int mask, int cfg, const Params &p, int64_t grid,
                  hipStream_t stream) {
    const int dt = dtype == ATTN_F16 ? 0 : 1;
    if (p.paged)
        return d == 64 ? attnfwd::launch_lockstep_paged64(dt, mask, cfg, p, grid, stream)
                       : attnfwd::launch_lockstep_paged128(dt, mask, cfg, p, grid, stream);
    if (d == 64) return attnfwd::launch_lockstep_d64(dt, mask, cfg, p, grid, stream);
    return attnfwd::launch_lockstep_d128(dt, mask, cfg, p, grid, stream);
}

// Number of query tiles (from the first) whose first row sees fewer than
// kExactBelow keys.
int64_t exact_tiles(int64_t N, int causal, int64_t window, int bm) {
    const int64_t ntiles = (N + bm - 1) / bm;
    if (!causal) return N < kExactBelow ? ntiles : 0;
    int64_t n = 0;
    for (int64_t t = 0; t < ntiles; ++t) {
        int64_t vis = std::min<int64_t>(N, t * bm + 1);
        if (window > 0) vis = std::min<int64_t>(vis, window);
        if (vis < kExactBelow) ++n;
    }
    return n;
}

// The merge kernel: groups of D/4 lanes, 256 / (D/4) per workgroup; sg of
// them (the largest power of two <= min(chunks, groups)) share a row.
template <int D, int DT>
hipError_t launch_merge_t(const attnfwd::MergeParams &mp, hipStream_t stream) {
    constexpr int G = 256 / (D / 4);
    attnfwd::MergeParams args = mp;
    args.sg = 1;
    while (args.sg * 2 <= std::min(G, mp.n_splits)) args.sg *= 2;
    const int64_t rows_per_block = G / args.sg;
    void *argv[] = {&args};
    return hipLaunchKernel((const void *)&attnfwd::attn_fwd_merge_kernel<D, DT>,
                           dim3((unsigned)((mp.rows + rows_per_block - 1) / rows_per_block)), dim3(256), argv, 0,
                           stream);
}

hipError_t launch_merge(int64_t d, int dtype, const attnfwd::MergeParams &mp, hipStream_t stream) {
    if (d == 64)
        return dtype == ATTN_F16 ? launch_merge_t<64, 0>(mp, stream) : launch_merge_t<64, 1>(mp, stream);
    return dtype == ATTN_F16 ? launch_merge_t<128, 0>(mp, stream) : launch_merge_t<128, 1>(mp, stream);
}

int status_of(hipError_t err) {
    if (err == hipErrorNoBinaryForGpu || err == hipErrorInvalidDeviceFunction || err == hipErrorNoDevice ||
        err == hipErrorInvalidDevice)
        return ATTN_ERR_DEVICE;
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Kernel parameters shared by the plain and the split-KV entry points.
Params make_params(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                   int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t window, int mask, float scale,
                   int64_t ntiles) {
    Params p;
    p.q = (const uint16_t *)q;
    p.k = (const uint16_t *)k;
    p.v = (const uint16_t *)v;
    p.o = (uint16_t *)o;
    p.lse = lse;
    p.Hq = (int)Hq;
    p.N = (int)Nq;
    p.Nk = (int)Nk;
    p.q_off = (int)(Nk - Nq);
    p.pack_nq = 0;
    p.n_splits = 1;
    p.split_tiles = INT_MAX / 2;
    p.split_t0 = 0;
    p.ws_o = nullptr;
    p.ws_ml = nullptr;
    p.block_table = nullptr;
    p.seq_lens = nullptr;
    p.paged = 0;
    p.page_shift = 0;
    p.max_pages = 0;
    p.num_pages = 0;
    p.Hkv = (int)Hkv;
    p.group = (int)(Hq / Hkv);
    p.window = mask == attnfwd::MASK_WINDOW ? (int)std::min<int64_t>(window, Nk) : 0;
    p.n_qtiles = (int)ntiles;
    p.n_bh = (int)(B * Hq);
    p.exact_below = kExactBelow;
    p.zigzag = 0;
    p.xcd_kv = (p.group > 1 && (B * Hkv) % 8 == 0) ? 1 : 0;
    // fold |scale| * log2(e) into one multiplier; a negative scale flips the
    // sign of Q instead (exact for 16-bit values).  A zero or vanishing scale
    // is raised to 2^-100: every score then maps to an exponent that rounds
    // to 0 in fp32, exactly what scale = 0 gives.
    const double cabs = std::fabs((double)scale) * 1.4426950408889634;
    p.c = (float)std::min(std::max(cabs, std::ldexp(1.0, -100)), (double)FLT_MAX);
    p.qsign = scale < 0.0f ? 0x80008000u : 0u;
    return p;
}

// ---- split-KV ("FlashDecoding"): Nq queries against Nk keys, the key range
// cut into chunks over workgroups, partial results merged by a second kernel.

int check_sizes_kv(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int causal,
                   int64_t window, float scale, int dtype) {
    if (Nk < 0 || Nk > kMaxN || (Nq > 0 && Nk == 0)) return ATTN_ERR_SHAPE;
    if (causal && Nq > Nk) return ATTN_ERR_SHAPE;
    return check_sizes(B, Hq, Hkv, Nq, d, causal, window, scale, dtype);
}

// Stacked heads: with few query rows (decoding) and G > 1, the G query heads
// of one K/V head are processed as one head of G * Nq rows, so that each K/V
// tile is brought on chip once for all of them.  Because q and o are
// (B, Hq, Nq, d) with the G heads of a K/V group adjacent, those rows are
// already contiguous: the kernel only needs to know that row r sits at
// position Nk - Nq + r % Nq.
constexpr int64_t kStackMaxNq = 16;

struct KvView {
    int64_t Hq, Nq;   // heads and rows per head as launched
    int pack_nq;      // 0, or Nq when the heads are stacked
};

KvView kv_view(int64_t Hq, int64_t Hkv, int64_t Nq) {
    const int64_t G = Hq / Hkv;
    if (G > 1 && Nq > 0 && Nq <= kStackMaxNq) return {Hkv, G * Nq, (int)Nq};
    return {Hq, Nq, 0};
}

// Automatic choice for split-KV calls (from measurement): one-wave 32-row
// workgroups (3) while a (stacked) head has fewer than 32 rows (GQA decoding:
// few rows, many K/V heads, so many workgroups); at 32 rows and more, with few
// K/V heads (MQA decoding), the 8-wave workgroups of configuration 0 keep
// more loads in flight per compute unit; longer query blocks take the choice
// of the plain forward, with 64-row workgroups (2) in place of the four-key-
// group ones (4): key chunks already spread a small grid.
int splitkv_auto_config(int64_t B, int64_t Hq, int64_t Nq, int64_t d, int mask, bool pairs) {
    if (Nq < 32) return 3;
    if (Nq <= 128) return 0;
    const int id = auto_config(B, Hq, Nq, d, mask, pairs);
    return id == 4 ? 2 : id;
}

struct SplitPlan {
    int64_t ntiles, grid, n_splits, split_tiles, t0, ws_bytes;
};

// Chunks of whole K/V tiles over the tiles some query row sees (with a
// window, the first row's window start bounds them below).  num_splits = 0
// picks, from measurement: for a few rows per (stacked) head, enough chunks
// for about 512 workgroups with at least four tiles each; for longer query
// blocks no split unless the grid has fewer than 64 workgroups (the partial
// results and the merge cost more than they save on larger grids).  The
// count used is ceil(visible tiles / tiles per chunk), so no chunk is empty
// for every row.
SplitPlan plan_split(int64_t B, int64_t Hq, int64_t Nq, int64_t Nk, int64_t q_first, int causal, int64_t window,
                     int64_t d, int64_t num_splits, int id) {
    SplitPlan sp;
    const TileCfg &tc = tile_cfg(d, id);
    sp.ntiles = (Nq + tc.bm() - 1) / tc.bm();
    const int64_t lo = (causal && window > 0) ? std::max<int64_t>(0, q_first - window + 1) : 0;
    sp.t0 = lo / tc.bn;
    const int64_t n_kt = std::max<int64_t>(1, (Nk + tc.bn - 1) / tc.bn - sp.t0);
    int64_t want = num_splits;
    if (want == 0) {
        const int64_t wgs = std::max<int64_t>(1, B * Hq * sp.ntiles);
        const int64_t target = Nq <= 32 ? 512 : (wgs < 64 ? 128 : 1);
        want = std::min<int64_t>((target + wgs - 1) / wgs, std::max<int64_t>(1, n_kt / 4));
    }
    want = std::max<int64_t>(1, std::min(want, n_kt));
    sp.split_tiles = (n_kt + want - 1) / want;
    sp.n_splits = (n_kt + sp.split_tiles - 1) / sp.split_tiles;
    sp.grid = B * Hq * sp.ntiles * sp.n_splits;
    sp.ws_bytes = sp.n_splits > 1 ? sp.n_splits * B * Hq * Nq * (d + 1) * 4 : 0;
    return sp;
}

}  // namespace

namespace attnfwd {

hipError_t launch_lockstep_d64(int dt, int mask, int cfg, const Params &p, int64_t grid, hipStream_t stream) {
    return launch_lockstep_d<64, false>(dt, mask, cfg, p, grid, stream);
}

}  // namespace attnfwd

extern "C" {

const char *attn_status_str(int status) {
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer argument";
    case ATTN_ERR_SHAPE: return "invalid or too large shape";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dim, dtype or mask";
    case ATTN_ERR_ARG: return "scale is not finite";
    case ATTN_ERR_ALIGN: return "pointer not aligned";
    case ATTN_ERR_ALIAS: return "output overlaps an input or the other output";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_DEVICE: return "no usable gfx950 device";
    case ATTN_ERR_WORKSPACE: return "workspace smaller than attn_fwd_splitkv_workspace_size";
    case ATTN_ERR_SCRATCH: return "split-KV partials larger than the fixed scratch of attn_fwd_splitkv_noalloc";
    default: return "unknown status";
    }
}

int attn_fwd_validate(const void *q, const void *k, const void *v, const void *o,
                      const float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                      int64_t d, int causal, int64_t window, float scale, int dtype) {
    if (N > 0 && (!q || !k || !v || !o)) return ATTN_ERR_NULL;
    const int rc = check_sizes(B, Hq, Hkv, N, d, causal, window, scale, dtype);
    if (rc != ATTN_OK) return rc;
    const uintptr_t mis = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o;
    if ((mis & 15) != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_ALIGN;
    const int64_t qbytes = B * Hq * N * d * 2;
    const int64_t kvbytes = B * Hkv * N * d * 2;
    const int64_t lbytes = B * Hq * N * 4;
    if (N > 0) {
        if (ranges_overlap(o, qbytes, q, qbytes) || ranges_overlap(o, qbytes, k, kvbytes) ||
            ranges_overlap(o, qbytes, v, kvbytes))
            return ATTN_ERR_ALIAS;
        if (lse && (ranges_overlap(lse, lbytes, q, qbytes) || ranges_overlap(lse, lbytes, k, kvbytes) ||
                    ranges_overlap(lse, lbytes, v, kvbytes) || ranges_overlap(lse, lbytes, o, qbytes)))
            return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

int attn_fwd_num_configs(void) { return kNumConfigs; }

int attn_fwd_config_desc(int id, int64_t d, int64_t *desc) {
    if (id < 0 || id >= kNumConfigs || !desc || (d != 64 && d != 128)) return ATTN_ERR_ARG;
    const TileCfg &tc = tile_cfg(d, id);
    desc[0] = tc.qb;
    desc[1] = tc.waves();
    desc[2] = tc.bn;
    desc[3] = tc.bm();
    desc[4] = tc.ksplit;
    desc[5] = tc.nstage;
    return ATTN_OK;
}

int attn_fwd_plan_ex(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                     int64_t window, int dtype, int config_id, int64_t *cfg) {
    const int rc = check_sizes(B, Hq, Hkv, N, d, causal, window, 1.0f, dtype);
    if (rc != ATTN_OK) return rc;
    if (config_id < -1 || config_id >= kNumConfigs) return ATTN_ERR_ARG;
    const int id = config_id >= 0 ? config_id : auto_config(B, Hq, N, d, mask_mode(causal, window));
    const TileCfg &tc = tile_cfg(d, id);
    if (cfg) {
        cfg[0] = tc.bm();
        cfg[1] = tc.bn;
        cfg[2] = tc.waves();
        cfg[3] = B * Hq * ((N + tc.bm() - 1) / tc.bm());
        cfg[4] = exact_tiles(N, causal, window, tc.bm());
        cfg[5] = mask_mode(causal, window);
        cfg[6] = id;
    }
    return ATTN_OK;
}

int attn_fwd_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                  int64_t window, int dtype, int64_t *cfg) {
    int64_t full[7];
    const int rc = attn_fwd_plan_ex(B, Hq, Hkv, N, d, causal, window, dtype, -1, full);
    if (rc == ATTN_OK && cfg)
        for (int i = 0; i < 6; ++i) cfg[i] = full[i];
    return rc;
}

int attn_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal, int64_t window,
                float scale, int dtype, int config_id, void *stream) {
    int rc = attn_fwd_validate(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, dtype);
    if (rc != ATTN_OK) return rc;
    if (config_id < -1 || config_id >= kNumConfigs) return ATTN_ERR_ARG;
    if (N == 0) return ATTN_OK;

    const int id = config_id >= 0 ? config_id : auto_config(B, Hq, N, d, mask_mode(causal, window));
    const TileCfg &tc = tile_cfg(d, id);
    const int bm = tc.bm();
    const int64_t ntiles = (N + bm - 1) / bm;
    const int64_t grid = B * Hq * ntiles;
    if (grid > INT_MAX) return ATTN_ERR_SHAPE;

    const int mask = mask_mode(causal, window);
    Params p = make_params(q, k, v, o, lse, B, Hq, Hkv, N, N, window, mask, scale, ntiles);
    // two 64-row workgroups share a compute unit: pair heavy and light tiles;
    // causal, 128 rows: two 64-row tiles of equal combined work per workgroup
    // (ceil(ceil(N / 64) / 2) = ceil(N / 128) pairs: the grid is the same)
    p.zigzag = (id == 2) ? 1 : (id == 0 && mask == attnfwd::MASK_CAUSAL && grid <= kPairMaxGrid) ? 2 : 0;
    const hipError_t err = launch(d, dtype, mask, id, p, grid, (hipStream_t)stream);
    return status_of(err);
}

int attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
             int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal, int64_t window, float scale,
             int dtype, void *stream) {
    return attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, dtype, -1, stream);
}

int attn_fwd_splitkv_validate(const void *q, const void *k, const void *v, const void *o,
                              const float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                              int64_t Nk, int64_t d, int causal, int64_t window, float scale, int dtype,
                              int64_t num_splits, int config_id, const void *workspace,
                              int64_t workspace_bytes) {
    if (Nq > 0 && (!q || !k || !v || !o)) return ATTN_ERR_NULL;
    const int rc = check_sizes_kv(B, Hq, Hkv, Nq, Nk, d, causal, window, scale, dtype);
    if (rc != ATTN_OK) return rc;
    if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_ARG;
    if (config_id < -1 || config_id >= kNumConfigs) return ATTN_ERR_ARG;
    const KvView kv = kv_view(Hq, Hkv, Nq);
    const int id = config_id >= 0 ? config_id : splitkv_auto_config(B, kv.Hq, kv.Nq, d, mask_mode(causal, window), kv.pack_nq == 0);
    const uintptr_t mis = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)workspace;
    if ((mis & 15) != 0 || ((uintptr_t)lse & 3) != 0) return ATTN_ERR_ALIGN;
    if (Nq == 0) return ATTN_OK;
    const SplitPlan sp = plan_split(B, kv.Hq, kv.Nq, Nk, Nk - Nq, causal, window, d, num_splits, id);
    if (sp.grid > INT_MAX) return ATTN_ERR_SHAPE;
    if (sp.n_splits > 1 && B * Hq * Nq > INT_MAX) return ATTN_ERR_SHAPE;   // merge grid
    if (sp.n_splits > 1) {
        if (!workspace) return ATTN_ERR_NULL;
        if (workspace_bytes < sp.ws_bytes) return ATTN_ERR_WORKSPACE;
    }
    const int64_t qbytes = B * Hq * Nq * d * 2;
    const int64_t kvbytes = B * Hkv * Nk * d * 2;
    const int64_t lbytes = B * Hq * Nq * 4;
    if (ranges_overlap(o, qbytes, q, qbytes) || ranges_overlap(o, qbytes, k, kvbytes) ||
        ranges_overlap(o, qbytes, v, kvbytes))
        return ATTN_ERR_ALIAS;
    if (lse && (ranges_overlap(lse, lbytes, q, qbytes) || ranges_overlap(lse, lbytes, k, kvbytes) ||
                ranges_overlap(lse, lbytes, v, kvbytes) || ranges_overlap(lse, lbytes, o, qbytes)))
        return ATTN_ERR_ALIAS;
    if (sp.n_splits > 1) {
        const void *bufs[5] = {q, k, v, o, lse};
        const int64_t sizes[5] = {qbytes, kvbytes, kvbytes, qbytes, lse ? lbytes : 0};
        for (int i = 0; i < 5; ++i)
            if (sizes[i] > 0 && ranges_overlap(workspace, sp.ws_bytes, bufs[i], sizes[i])) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

int attn_fwd_splitkv_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                          int causal, int64_t window, int dtype, int64_t num_splits, int config_id,
                          int64_t *plan) {
    const int rc = check_sizes_kv(B, Hq, Hkv, Nq, Nk, d, causal, window, 1.0f, dtype);
    if (rc != ATTN_OK) return rc;
    if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_ARG;
    if (config_id < -1 || config_id >= kNumConfigs) return ATTN_ERR_ARG;
    const KvView kv = kv_view(Hq, Hkv, Nq);
    const int id = config_id >= 0 ? config_id : splitkv_auto_config(B, kv.Hq, kv.Nq, d, mask_mode(causal, window), kv.pack_nq == 0);
    const TileCfg &tc = tile_cfg(d, id);
    const SplitPlan sp = plan_split(B, kv.Hq, kv.Nq, Nk, Nk - Nq, causal, window, d, num_splits, id);
    if (plan) {
        plan[0] = tc.bm();
        plan[1] = tc.bn;
        plan[2] = tc.waves();
        plan[3] = Nq > 0 ? sp.grid : 0;
        plan[4] = sp.n_splits;
        plan[5] = sp.split_tiles;
        plan[6] = id;
        plan[7] = Nq > 0 ? sp.ws_bytes : 0;
        plan[8] = kv.pack_nq > 0 ? 1 : 0;
    }
    return ATTN_OK;
}

int64_t attn_fwd_splitkv_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                                        int64_t d, int causal, int64_t window, int dtype,
                                        int64_t num_splits, int config_id) {
    int64_t plan[9];
    const int rc = attn_fwd_splitkv_plan(B, Hq, Hkv, Nq, Nk, d, causal, window, dtype, num_splits,
                                         config_id, plan);
    return rc == ATTN_OK ? plan[7] : -(int64_t)rc;
}

int attn_fwd_splitkv_ex(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                        int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int causal,
                        int64_t window, float scale, int dtype, int64_t num_splits, int config_id,
                        void *workspace, int64_t workspace_bytes, void *stream) {
    const int rc = attn_fwd_splitkv_validate(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, scale,
                                             dtype, num_splits, config_id, workspace, workspace_bytes);
    if (rc != ATTN_OK) return rc;
    if (Nq == 0) return ATTN_OK;
    const int mask = mask_mode(causal, window);
    const KvView kv = kv_view(Hq, Hkv, Nq);
    const int id = config_id >= 0 ? config_id : splitkv_auto_config(B, kv.Hq, kv.Nq, d, mask, kv.pack_nq == 0);
    const SplitPlan sp = plan_split(B, kv.Hq, kv.Nq, Nk, Nk - Nq, causal, window, d, num_splits, id);
    // stacked heads: B * Hkv heads of G * Nq rows, each its own K/V head
    Params p = make_params(q, k, v, o, lse, B, kv.Hq, kv.pack_nq > 0 ? kv.Hq : Hkv, kv.Nq, Nk, window, mask,
                           scale, sp.ntiles);
    p.q_off = (int)(Nk - Nq);
    p.pack_nq = kv.pack_nq;
    p.zigzag = (id == 2) ? 1
               : (id == 0 && mask == attnfwd::MASK_CAUSAL && kv.pack_nq == 0 && sp.grid <= kPairMaxGrid) ? 2 : 0;
    p.n_splits = (int)sp.n_splits;
    p.split_tiles = (int)sp.split_tiles;
    p.split_t0 = (int)sp.t0;
    const int64_t rows = B * Hq * Nq;
    if (sp.n_splits > 1) {
        p.ws_o = (float *)workspace;
        p.ws_ml = (float *)workspace + sp.n_splits * rows * d;
    }
    hipError_t err = launch(d, dtype, mask, id, p, sp.grid, (hipStream_t)stream);
    if (err == hipSuccess && sp.n_splits > 1) {
        attnfwd::MergeParams mp;
        mp.ws_o = p.ws_o;
        mp.ws_ml = p.ws_ml;
        mp.o = (uint16_t *)o;
        mp.lse = lse;
        mp.rows = rows;
        mp.n_splits = (int)sp.n_splits;
        err = launch_merge(d, dtype, mp, (hipStream_t)stream);
    }
    return status_of(err);
}

}  // extern "C"

// ---- split-KV without allocation -----------------------------------------
// attn_fwd_splitkv_noalloc keeps its chunk partials in this fixed array
// instead of a caller workspace.  Each device holds its own copy from module
// load to process exit.  Host code must never pass `scratch` itself to a
// kernel: on the host the name is a stand-in, not the device address, which
// is looked up once per device with hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's `scratch`, looked up on the first
// call on that device (with it current) and kept.
int scratch_ptr(void **out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return status_of(err);
    if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_DEVICE;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (err != hipSuccess || !p) return err != hipSuccess ? status_of(err) : ATTN_ERR_DEVICE;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                             int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int causal,
                             int64_t window, float scale, int dtype, int64_t num_splits, int config_id,
                             void *stream) {
    // every host check that needs no device first, so an oversized call fails
    // before any HIP call
    int64_t plan[9];
    int rc = attn_fwd_splitkv_plan(B, Hq, Hkv, Nq, Nk, d, causal, window, dtype, num_splits, config_id, plan);
    if (rc != ATTN_OK) return rc;
    if (plan[7] > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
    if (Nq == 0) return attn_fwd_splitkv_validate(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, scale,
                                                  dtype, num_splits, config_id, nullptr, 0);
    void *ws = nullptr;
    if (plan[7] > 0) {
        rc = scratch_ptr(&ws);
        if (rc != ATTN_OK) return rc;
    }
    return attn_fwd_splitkv_ex(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, scale, dtype, num_splits,
                               config_id, ws, ws ? ATTN_NOALLOC_SCRATCH_BYTES : 0, stream);
}

// ---- tile-configuration tuning ------------------------------------------

int attn_fwd_autotune(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B, int64_t Hq,
                      int64_t Hkv, int64_t N, int64_t d, int causal, int64_t window, float scale, int dtype,
                      int reps, int *best_config, float *ms, void *stream) {
    if (!best_config) return ATTN_ERR_NULL;
    if (reps < 1 || reps > 10000) return ATTN_ERR_ARG;
    int rc = attn_fwd_validate(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, dtype);
    if (rc != ATTN_OK) return rc;
    *best_config = auto_config(B, Hq, N, d, mask_mode(causal, window));
    if (ms)
        for (int id = 0; id < kNumConfigs; ++id) ms[id] = -1.0f;
    if (N == 0) return ATTN_OK;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return ATTN_ERR_LAUNCH;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return ATTN_ERR_LAUNCH;
    }
    const hipStream_t st = (hipStream_t)stream;
    float best = -1.0f;
    rc = ATTN_OK;
    for (int id = 0; id < kNumConfigs && rc == ATTN_OK; ++id) {
        // one untimed call, then `reps` back-to-back calls between two events
        rc = attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, dtype, id, stream);
        if (rc != ATTN_OK) break;
        if (hipEventRecord(e0, st) != hipSuccess) rc = ATTN_ERR_LAUNCH;
        for (int r = 0; r < reps && rc == ATTN_OK; ++r)
            rc = attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, dtype, id, stream);
        if (rc == ATTN_OK && hipEventRecord(e1, st) != hipSuccess) rc = ATTN_ERR_LAUNCH;
        if (rc == ATTN_OK && hipEventSynchronize(e1) != hipSuccess) rc = ATTN_ERR_LAUNCH;
        float t = 0.0f;
        if (rc == ATTN_OK && hipEventElapsedTime(&t, e0, e1) != hipSuccess) rc = ATTN_ERR_LAUNCH;
        if (rc != ATTN_OK) break;
        t /= (float)reps;
        if (ms) ms[id] = t;
        if (best < 0.0f || t < best) {
            best = t;
            *best_config = id;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return rc;
}

// ---- paged K/V ---------------------------------------------------------

static int paged_geometry(int64_t page_size, int64_t num_pages, int64_t max_pages, int64_t max_seq_len) {
    if (page_size < 8 || page_size > 256 || (page_size & (page_size - 1)) != 0) return ATTN_ERR_UNSUPPORTED;
    if (num_pages < 1 || num_pages > INT_MAX || max_pages < 1 || max_pages > INT_MAX) return ATTN_ERR_SHAPE;
    if (max_seq_len < 1 || max_seq_len > kMaxN || max_seq_len > max_pages * page_size) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

int attn_fwd_paged_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t d, int64_t page_size,
                        int64_t num_pages, int64_t max_pages, int64_t max_seq_len, int causal, int64_t window,
                        int dtype, int64_t num_splits, int config_id, int64_t *plan) {
    int rc = paged_geometry(page_size, num_pages, max_pages, max_seq_len);
    if (rc != ATTN_OK) return rc;
    rc = check_sizes(B, Hq, Hkv, Nq, d, causal, window, 1.0f, dtype);
    if (rc != ATTN_OK) return rc;
    if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_ARG;
    if (config_id < -1 || config_id >= kNumConfigs) return ATTN_ERR_ARG;
    const KvView kv = kv_view(Hq, Hkv, Nq);
    const int id = config_id >= 0 ? config_id : splitkv_auto_config(B, kv.Hq, kv.Nq, d, mask_mode(causal, window), false);
    const TileCfg &tc = tile_cfg(d, id);
    // lengths differ per batch: chunks cover [0, max_seq_len)
    const SplitPlan sp = plan_split(B, kv.Hq, kv.Nq, max_seq_len, 0, 0, 0, d, num_splits, id);
    if (plan) {
        plan[0] = tc.bm();
        plan[1] = tc.bn;
        plan[2] = tc.waves();
        plan[3] = Nq > 0 ? sp.grid : 0;
        plan[4] = sp.n_splits;
        plan[5] = sp.split_tiles;
        plan[6] = id;
        plan[7] = Nq > 0 ? sp.ws_bytes : 0;
        plan[8] = kv.pack_nq > 0 ? 1 : 0;
    }
    return ATTN_OK;
}

int64_t attn_fwd_paged_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t d, int64_t page_size,
                                      int64_t num_pages, int64_t max_pages, int64_t max_seq_len, int causal,
                                      int64_t window, int dtype, int64_t num_splits, int config_id) {
    int64_t plan[9];
    const int rc = attn_fwd_paged_plan(B, Hq, Hkv, Nq, d, page_size, num_pages, max_pages, max_seq_len, causal,
                                       window, dtype, num_splits, config_id, plan);
    return rc == ATTN_OK ? plan[7] : -(int64_t)rc;
}

int attn_fwd_paged_validate(const void *q, const void *k_pool, const void *v_pool, const int32_t *block_table,
                            const int32_t *seq_lens, const void *o, const float *lse, int64_t B, int64_t Hq,
                            int64_t Hkv, int64_t Nq, int64_t d, int64_t page_size, int64_t num_pages,
                            int64_t max_pages, int64_t max_seq_len, int causal, int64_t window, float scale,
                            int dtype, int64_t num_splits, int config_id, const void *workspace,
                            int64_t workspace_bytes) {
    if (Nq > 0 && (!q || !k_pool || !v_pool || !block_table || !seq_lens || !o)) return ATTN_ERR_NULL;
    int rc = paged_geometry(page_size, num_pages, max_pages, max_seq_len);
    if (rc != ATTN_OK) return rc;
    rc = check_sizes(B, Hq, Hkv, Nq, d, causal, window, scale, dtype);
    if (rc != ATTN_OK) return rc;
    if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_ARG;
    if (config_id < -1 || config_id >= kNumConfigs) return ATTN_ERR_ARG;
    int64_t plan[9];
    rc = attn_fwd_paged_plan(B, Hq, Hkv, Nq, d, page_size, num_pages, max_pages, max_seq_len, causal, window, dtype,
                             num_splits, config_id, plan);
    if (rc != ATTN_OK) return rc;
    const uintptr_t mis = (uintptr_t)q | (uintptr_t)k_pool | (uintptr_t)v_pool | (uintptr_t)o | (uintptr_t)workspace;
    if ((mis & 15) != 0 || ((uintptr_t)lse & 3) != 0 || ((uintptr_t)block_table & 3) != 0 ||
        ((uintptr_t)seq_lens & 3) != 0)
        return ATTN_ERR_ALIGN;
    if (Nq == 0) return ATTN_OK;
    if (plan[3] > INT_MAX || (plan[4] > 1 && B * Hq * Nq > INT_MAX)) return ATTN_ERR_SHAPE;
    if (plan[4] > 1) {
        if (!workspace) return ATTN_ERR_NULL;
        if (workspace_bytes < plan[7]) return ATTN_ERR_WORKSPACE;
    }
    const int64_t qbytes = B * Hq * Nq * d * 2;
    const int64_t poolbytes = num_pages * Hkv * page_size * d * 2;
    const int64_t btbytes = B * max_pages * 4;
    const int64_t slbytes = B * 4;
    const int64_t lbytes = B * Hq * Nq * 4;
    const void *ins[5] = {q, k_pool, v_pool, block_table, seq_lens};
    const int64_t insz[5] = {qbytes, poolbytes, poolbytes, btbytes, slbytes};
    for (int i = 0; i < 5; ++i) {
        if (ranges_overlap(o, qbytes, ins[i], insz[i])) return ATTN_ERR_ALIAS;
        if (lse && ranges_overlap(lse, lbytes, ins[i], insz[i])) return ATTN_ERR_ALIAS;
        if (plan[4] > 1 && ranges_overlap(workspace, plan[7], ins[i], insz[i])) return ATTN_ERR_ALIAS;
    }
    if (lse && ranges_overlap(lse, lbytes, o, qbytes)) return ATTN_ERR_ALIAS;
    if (plan[4] > 1 && (ranges_overlap(workspace, plan[7], o, qbytes) ||
                        (lse && ranges_overlap(workspace, plan[7], lse, lbytes))))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

int attn_fwd_paged_ex(const void *q, const void *k_pool, const void *v_pool, const int32_t *block_table,
                      const int32_t *seq_lens, void *o, float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                      int64_t d, int64_t page_size, int64_t num_pages, int64_t max_pages, int64_t max_seq_len,
                      int causal, int64_t window, float scale, int dtype, int64_t num_splits, int config_id,
                      void *workspace, int64_t workspace_bytes, void *stream) {
    const int rc = attn_fwd_paged_validate(q, k_pool, v_pool, block_table, seq_lens, o, lse, B, Hq, Hkv, Nq, d,
                                           page_size, num_pages, max_pages, max_seq_len, causal, window, scale,
                                           dtype, num_splits, config_id, workspace, workspace_bytes);
    if (rc != ATTN_OK) return rc;
    if (Nq == 0) return ATTN_OK;
    const int mask = mask_mode(causal, window);
    const KvView kv = kv_view(Hq, Hkv, Nq);
    const int id = config_id >= 0 ? config_id : splitkv_auto_config(B, kv.Hq, kv.Nq, d, mask, false);
    const SplitPlan sp = plan_split(B, kv.Hq, kv.Nq, max_seq_len, 0, 0, 0, d, num_splits, id);
    Params p = make_params(q, k_pool, v_pool, o, lse, B, kv.Hq, kv.pack_nq > 0 ? kv.Hq : Hkv, kv.Nq, max_seq_len,
                           window, mask, scale, sp.ntiles);
    p.q_off = (int)(max_seq_len - Nq);   // replaced per batch from seq_lens in the kernel
    p.pack_nq = kv.pack_nq;
    p.zigzag = (id == 2) ? 1 : 0;
    p.n_splits = (int)sp.n_splits;
    p.split_tiles = (int)sp.split_tiles;
    p.split_t0 = 0;
    p.paged = 1;
    p.block_table = block_table;
    p.seq_lens = seq_lens;
    int shift = 0;
    while ((int64_t(1) << shift) < page_size) ++shift;
    p.page_shift = shift;
    p.max_pages = (int)max_pages;
    p.num_pages = (int)num_pages;
    p.Hkv = (int)Hkv;
    const int64_t rows = B * Hq * Nq;
    if (sp.n_splits > 1) {
        p.ws_o = (float *)workspace;
        p.ws_ml = (float *)workspace + sp.n_splits * rows * d;
    }
    hipError_t err = launch(d, dtype, mask, id, p, sp.grid, (hipStream_t)stream);
    if (err == hipSuccess && sp.n_splits > 1) {
        attnfwd::MergeParams mp;
        mp.ws_o = p.ws_o;
        mp.ws_ml = p.ws_ml;
        mp.o = (uint16_t *)o;
        mp.lse = lse;
        mp.rows = rows;
        mp.n_splits = (int)sp.n_splits;
        err = launch_merge(d, dtype, mp, (hipStream_t)stream);
    }
    return status_of(err);
}

int attn_fwd_paged(const void *q, const void *k_pool, const void *v_pool, const int32_t *block_table,
                   const int32_t *seq_lens, void *o, float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                   int64_t d, int64_t page_size, int64_t num_pages, int64_t max_pages, int64_t max_seq_len,
                   int causal, int64_t window, float scale, int dtype, int64_t num_splits, void *workspace,
                   int64_t workspace_bytes, void *stream) {
    return attn_fwd_paged_ex(q, k_pool, v_pool, block_table, seq_lens, o, lse, B, Hq, Hkv, Nq, d, page_size,
                             num_pages, max_pages, max_seq_len, causal, window, scale, dtype, num_splits, -1,
                             workspace, workspace_bytes, stream);
}

int attn_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse, int64_t B,
                     int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int causal, int64_t window,
                     float scale, int dtype, int64_t num_splits, void *workspace, int64_t workspace_bytes,
                     void *stream) {
    return attn_fwd_splitkv_ex(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, scale, dtype,
                               num_splits, -1, workspace, workspace_bytes, stream);
}

}  // extern "C"
