// attn_fwd_merge.hpp -- combine kernel of the split-KV forward.
//
// The attention kernel, run with the keys cut into n_splits chunks, leaves for
// every (chunk p, query row) the chunk's partial output O_p = (sum_j p_j v_j)
// / l_p in fp32 and its base-2 log-sum-exp L_p = m_p + log2 l_p (-inf when the
// row sees no key of the chunk).  This kernel forms the exact result, the
// global reduction of "Optimizaciones de Atencion", section "FlashDecoding":
// with M = max_p L_p, each partial output is weighted by 2^(L_p - M) (that is
// exp(m_p - m) * l_p up to the common factor 2^(m - M)), the weighted outputs
// are summed and divided by the sum of the weights, and the row's log-sum-exp
// is M + log2 of that sum (stored as a natural log).
//
// Work split: a group of D/4 lanes owns one row, four channels per lane, so
// each partial-output read is 16 bytes per lane over consecutive channels.
// `sg` groups share a row and take every sg-th chunk each (the chunk loop is a
// chain of dependent-latency loads otherwise); each group keeps its own
// running max, weight sum and weighted sum in one pass over its chunks, and
// the first group of the row combines the sg results through LDS with the
// same rescale.  The output is rounded to the
// 16-bit type once.
#pragma once

#include "attn_fwd_common.hpp"

namespace attnfwd {

struct MergeParams {
    const float *ws_o;   // (n_splits, rows, D)
    const float *ws_ml;  // (n_splits, rows)
    uint16_t *o;         // (rows, D)
    float *lse;          // (rows,), may be null
    int64_t rows;        // B * Hq * Nq
    int n_splits;
    int sg;              // groups per row: a power of two <= 256 / (D / 4)
};

template <int D, int DT>
__global__ __launch_bounds__(256) void attn_fwd_merge_kernel(MergeParams mp) {
    constexpr int LPR = D / 4;      // lanes per group
    constexpr int G = 256 / LPR;    // groups per workgroup
    __shared__ float sm_m[G];
    __shared__ float sm_w[G];
    __shared__ float4 sm_acc[256];

    const int sg = mp.sg;
    const int grp = threadIdx.x / LPR;
    const int c4 = threadIdx.x % LPR;
    const int rloc = grp / sg;
    const int part = grp % sg;
    const int64_t row = (int64_t)blockIdx.x * (G / sg) + rloc;
    const bool live = row < mp.rows;

    // one pass over the group's chunks with a running max: the loads of a
    // chunk do not wait on the max of the earlier ones, so the unrolled loop
    // issues them together
    float m = -__builtin_inff();
    float w = 0.0f;
    float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (live) {
#pragma unroll 8
        for (int s = part; s < mp.n_splits; s += sg) {
            const float ls = mp.ws_ml[s * mp.rows + row];
            const float4 x = *(const float4 *)(mp.ws_o + (s * mp.rows + row) * D + 4 * c4);
            const float nm = fmaxf(m, ls);
            const float f = (m == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m - nm);
            const float e = (ls == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(ls - nm);
            m = nm;
            w = w * f + e;
            acc.x = acc.x * f + e * x.x;
            acc.y = acc.y * f + e * x.y;
            acc.z = acc.z * f + e * x.z;
            acc.w = acc.w * f + e * x.w;
        }
    }
    if (c4 == 0) {
        sm_m[grp] = m;
        sm_w[grp] = w;
    }
    sm_acc[threadIdx.x] = acc;
    __syncthreads();
    if (!live || part != 0) return;

    const int g0 = rloc * sg;
    float mx = -__builtin_inff();
    for (int g = 0; g < sg; ++g) mx = fmaxf(mx, sm_m[g0 + g]);
    float wsum = 0.0f;
    float4 tot = {0.0f, 0.0f, 0.0f, 0.0f};
    if (mx != -__builtin_inff()) {
        for (int g = 0; g < sg; ++g) {
            const float mg = sm_m[g0 + g];
            if (mg == -__builtin_inff()) continue;
            const float f = __builtin_amdgcn_exp2f(mg - mx);
            const float4 a = sm_acc[(g0 + g) * LPR + c4];
            wsum += f * sm_w[g0 + g];
            tot.x += f * a.x;
            tot.y += f * a.y;
            tot.z += f * a.z;
            tot.w += f * a.w;
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    u32x2 out;
    out[0] = pack2<DT>(tot.x * inv, tot.y * inv);
    out[1] = pack2<DT>(tot.z * inv, tot.w * inv);
    *(u32x2 *)(mp.o + row * D + 4 * c4) = out;
    if (mp.lse != nullptr && c4 == 0)
        mp.lse[row] = wsum > 0.0f ? (mx + __builtin_amdgcn_logf(wsum)) * 0.69314718055994530942f
                                  : -__builtin_inff();
}

}  // namespace attnfwd
