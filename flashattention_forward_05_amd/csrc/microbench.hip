// microbench.hip -- measured ceilings of an MI355X (gfx950) compute unit, next
// to which the attention kernels' throughput is judged: the dense MFMA rate,
// the rates of v_exp_f32 and v_fma_f32, whether the vector ALU of one wave runs
// while another wave on the same SIMD keeps the matrix core busy, the LDS read
// bandwidth and the HBM copy bandwidth.  Also the shader clock under load.
//
// Every kernel is launched with 8 waves (512 lanes) per workgroup and enough
// LDS that one workgroup fills a compute unit: waves w and w + 4 share a SIMD
// (recorded from HW_ID so that the host can check it).  Wave w runs the loop
// `kind_lo` if w < 4, else `kind_hi`, for its own iteration count, and lane 0
// records the shader-clock and real-time counters around the loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum Kind {
    K_MFMA32 = 0, K_EXP = 1, K_FMA = 2, K_IDLE = 3, K_MFMA16 = 4, K_EXPFMA = 5, K_LDS = 6,
    K_MFMA32_DEP2 = 7, K_MFMA32_DEP1 = 8, K_LDS_TR = 9, K_MFMA_FMA4 = 10, K_MFMA_EXP2 = 11, K_MFMA_LDS = 12,
    K_GLOAD = 13, K_GLOAD_LDS = 14
};

// Per wave: [t0, t1] of the shader clock, [r0, r1] of the 100 MHz real-time
// counter, then the HW_ID and XCC_ID registers.
struct Rec {
    long long t0, t1, r0, r1;
    int hw_id, xcc_id, pad0, pad1;
};

__device__ __forceinline__ void loop_mfma32(int iters, float seed, float *sink) {
    const bf16x8 a = {(__bf16)seed, (__bf16)1.0f, (__bf16)0.5f, (__bf16)0.25f,
                      (__bf16)seed, (__bf16)1.0f, (__bf16)0.5f, (__bf16)0.25f};
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c3, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c3, 0, 0, 0);
    }
    const float r = c0[0] + c1[1] + c2[2] + c3[3];
    if (r == 1234.5f) sink[threadIdx.x] = r;
}

// The same MFMAs on two accumulators (each MFMA depends on the one issued two
// before it) and on one (each depends on the previous): dependent-issue
// latency of the matrix core.
__device__ __forceinline__ void loop_mfma32_dep(int iters, float seed, float *sink, int chains) {
    const bf16x8 a = {(__bf16)seed, (__bf16)1.0f, (__bf16)0.5f, (__bf16)0.25f,
                      (__bf16)seed, (__bf16)1.0f, (__bf16)0.5f, (__bf16)0.25f};
    f32x16 c0 = {}, c1 = {};
    if (chains == 2) {
#pragma unroll 1
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c1, 0, 0, 0);
            }
        }
    } else {
#pragma unroll 1
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int j = 0; j < 8; ++j) c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c0, 0, 0, 0);
        }
    }
    const float r = c0[0] + c1[1];
    if (r == 1234.5f) sink[threadIdx.x] = r;
}

// One wave interleaving its own work: 8 MFMAs per iteration, each followed
// by independent vector instructions (4 v_fma_f32, or 2 v_exp_f32) or by one
// 16-byte LDS read.  If a wave keeps issuing while its MFMA executes, this
// takes about as long as the MFMAs alone.
template <int KIND>
__device__ __forceinline__ void loop_mfma_mixed(int iters, float seed, const char *lds, float *sink) {
    const bf16x8 a = {(__bf16)seed, (__bf16)1.0f, (__bf16)0.5f, (__bf16)0.25f,
                      (__bf16)seed, (__bf16)1.0f, (__bf16)0.5f, (__bf16)0.25f};
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = seed + 0.01f * j;
    const float y = 0.999f - 1e-7f * seed, z = 1e-3f * seed;
    const int lane = threadIdx.x & 63;
    int row = (threadIdx.x >> 6) * 8;
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            f32x16 &c = (j % 4 == 0) ? c0 : (j % 4 == 1) ? c1 : (j % 4 == 2) ? c2 : c3;
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c, 0, 0, 0);
            if constexpr (KIND == K_MFMA_FMA4) {
#pragma unroll
                for (int u = 0; u < 4; ++u) x[(4 * j + u) % 16] = __builtin_fmaf(x[(4 * j + u) % 16], y, z);
            } else if constexpr (KIND == K_MFMA_EXP2) {
#pragma unroll
                for (int u = 0; u < 2; ++u) x[(2 * j + u) % 16] = __builtin_amdgcn_exp2f(-x[(2 * j + u) % 16]);
            } else {
                const u32x4 v = *(const u32x4 *)(lds + ((row + j) & 63) * 1024 + lane * 16);
                asm volatile("" ::"v"(v));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        row += 8;
    }
    float r = c0[0] + c1[1] + c2[2] + c3[3];
#pragma unroll
    for (int j = 0; j < 16; ++j) r += x[j];
    if (r == 1234.5f) sink[threadIdx.x] = r;
}

__device__ __forceinline__ void loop_mfma16(int iters, float seed, float *sink) {
    const bf16x8 a = {(__bf16)seed, (__bf16)1.0f, (__bf16)0.5f, (__bf16)0.25f,
                      (__bf16)seed, (__bf16)1.0f, (__bf16)0.5f, (__bf16)0.25f};
    f32x4 c[8] = {};
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, c[j], 0, 0, 0);
    }
    float r = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) r += c[j][j & 3];
    if (r == 1234.5f) sink[threadIdx.x] = r;
}

// 16 independent chains x = 2^-x per iteration (one v_exp_f32 each, the
// negation folded into the source modifier).
__device__ __forceinline__ void loop_exp(int iters, float seed, float *sink) {
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = seed + 0.01f * j;
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
    }
    float r = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) r += x[j];
    if (r == 1234.5f) sink[threadIdx.x] = r;
}

// 16 independent chains x = x * y + z per iteration (one v_fma_f32 each).
__device__ __forceinline__ void loop_fma(int iters, float seed, float *sink) {
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = seed + 0.01f * j;
    const float y = 0.999f - 1e-7f * seed, z = 1e-3f * seed;
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = __builtin_fmaf(x[j], y, z);
    }
    float r = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) r += x[j];
    if (r == 1234.5f) sink[threadIdx.x] = r;
}

// One wave alternating the two: 8 exps and 8 fmas per iteration.
__device__ __forceinline__ void loop_expfma(int iters, float seed, float *sink) {
    float x[8], u[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        x[j] = seed + 0.01f * j;
        u[j] = seed - 0.01f * j;
    }
    const float y = 0.999f - 1e-7f * seed, z = 1e-3f * seed;
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            x[j] = __builtin_amdgcn_exp2f(-x[j]);
            u[j] = __builtin_fmaf(u[j], y, z);
        }
    }
    float r = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) r += x[j] + u[j];
    if (r == 1234.5f) sink[threadIdx.x] = r;
}

// 16-byte LDS reads: 8 per iteration, each lane at its own 16 bytes of a
// 1 KiB row, rows walking through a 64 KiB buffer (no bank conflicts).  The
// values are consumed by an empty asm statement, so no vector ALU work paces
// the loop: it measures the LDS path alone.
__device__ __forceinline__ void loop_lds(int iters, const char *lds, float *sink) {
    const int lane = threadIdx.x & 63;
    int row = (threadIdx.x >> 6) * 8;
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = *(const u32x4 *)(lds + ((row + j) & 63) * 1024 + lane * 16);
#pragma unroll
        for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(v[j]));
        row += 8;
    }
    (void)sink;
}

// 8-byte transposing LDS reads (ds_read_b64_tr_b16): 8 per iteration, lane
// i at byte 8 * i of a 512-byte row; consumed the same way.
__device__ __forceinline__ void loop_lds_tr(int iters, const char *lds, float *sink) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63;
    int row = (threadIdx.x >> 6) * 8;
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
        i16x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4 *)(lds + ((row + j) & 127) * 512 + lane * 8));
#pragma unroll
        for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(v[j]));
        row += 8;
    }
    (void)sink;
}

// Global loads from a small (L2-resident) buffer: 8 per iteration of 16 bytes
// per lane, then a wait for all of them; into registers (K_GLOAD) or
// straight into LDS (K_GLOAD_LDS, global_load_lds_dwordx4, the attention
// kernels' K/V staging).  Each lane reads its own 16 bytes of a 1 KiB row of
// 64 rows; LDS slots are this wave's own 8 KiB.
__device__ __forceinline__ void loop_gload(int iters, const u32x4 *src, char *lds, float *sink, bool to_lds) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    u32x4 acc = {0u, 0u, 0u, 0u};
    const uint32_t lbase = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)(lds + wave * 8192));
#pragma unroll 1
    for (int i = 0; i < iters; ++i) {
        const u32x4 *row = src + ((i * 8) & 63) * 64 + lane;
        if (to_lds) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
                asm volatile("s_add_u32 m0, %1, %2\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(row + j * 64), "s"(lbase),
                             "i"(j * 1024)
                             : "memory", "m0", "scc");
#pragma clang diagnostic pop
            }
            __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));   // vmcnt(0)
        } else {
            u32x4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(row + j * 64);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc ^= v[j];
        }
    }
    if (acc[0] == 0x12345678u && acc[1] == 0x9abcdef0u) sink[threadIdx.x] = (float)acc[2];
}

__device__ __forceinline__ void run_kind(int kind, int iters, float seed, char *lds, float *sink,
                                         const u32x4 *gsrc) {
    switch (kind) {
    case K_GLOAD: loop_gload(iters, gsrc, lds, sink, false); break;
    case K_GLOAD_LDS: loop_gload(iters, gsrc, lds, sink, true); break;
    case K_MFMA32: loop_mfma32(iters, seed, sink); break;
    case K_EXP: loop_exp(iters, seed, sink); break;
    case K_FMA: loop_fma(iters, seed, sink); break;
    case K_MFMA16: loop_mfma16(iters, seed, sink); break;
    case K_EXPFMA: loop_expfma(iters, seed, sink); break;
    case K_LDS: loop_lds(iters, lds, sink); break;
    case K_MFMA32_DEP2: loop_mfma32_dep(iters, seed, sink, 2); break;
    case K_MFMA32_DEP1: loop_mfma32_dep(iters, seed, sink, 1); break;
    case K_LDS_TR: loop_lds_tr(iters, lds, sink); break;
    case K_MFMA_FMA4: loop_mfma_mixed<K_MFMA_FMA4>(iters, seed, lds, sink); break;
    case K_MFMA_EXP2: loop_mfma_mixed<K_MFMA_EXP2>(iters, seed, lds, sink); break;
    case K_MFMA_LDS: loop_mfma_mixed<K_MFMA_LDS>(iters, seed, lds, sink); break;
    default: break;
    }
}

// HW_ID (hardware register 4) and XCC_ID (20), full 32 bits each:
// s_getreg immediate = (size - 1) << 11 | offset << 6 | id.
constexpr int kHwIdImm = (31 << 11) | 4;
constexpr int kXccIdImm = (31 << 11) | 20;

__global__ __launch_bounds__(512) void mb_kernel(int kind_lo, int kind_hi, int iters_lo, int iters_hi, Rec *rec,
                                                 float *sink, const u32x4 *gsrc) {
    // 96 KiB: one workgroup per compute unit
    __shared__ __attribute__((aligned(16))) char lds[96 * 1024];
    const int wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 64 * 1024 / 4; i += 512) ((uint32_t *)lds)[i] = (uint32_t)i * 2654435761u;
    __syncthreads();
    const bool lo = wave < 4;
    const int kind = lo ? kind_lo : kind_hi;
    const int iters = lo ? iters_lo : iters_hi;
    const float seed = (float)(threadIdx.x & 63) * 1e-3f + 0.5f;
    const long long t0 = __builtin_amdgcn_s_memtime();
    const long long r0 = __builtin_amdgcn_s_memrealtime();
    run_kind(kind, iters, seed, lds, sink, gsrc);
    const long long t1 = __builtin_amdgcn_s_memtime();
    const long long r1 = __builtin_amdgcn_s_memrealtime();
    if ((threadIdx.x & 63) == 0) {
        Rec r;
        r.t0 = t0;
        r.t1 = t1;
        r.r0 = r0;
        r.r1 = r1;
        r.hw_id = __builtin_amdgcn_s_getreg(kHwIdImm);
        r.xcc_id = __builtin_amdgcn_s_getreg(kXccIdImm);
        r.pad0 = kind;
        r.pad1 = iters;
        rec[blockIdx.x * 8 + wave] = r;
    }
}

// Grid-stride 16-byte copy.
__global__ __launch_bounds__(256) void mb_copy(const u32x4 *src, u32x4 *dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

// Size in bytes of one per-wave record.
int attn_mb_record_bytes(void) { return (int)sizeof(Rec); }

// Launch `grid` workgroups of 8 waves: waves 0-3 run loop kind_lo for iters_lo
// iterations, waves 4-7 loop kind_hi for iters_hi (kinds: 0 = 8 MFMA
// 32x32x16 bf16, 1 = 16 v_exp_f32, 2 = 16 v_fma_f32, 3 = nothing, 4 = 8 MFMA
// 16x16x32 bf16, 5 = 8 exp + 8 fma, 6 = 8 16-byte LDS reads, 7 = 8 MFMA
// 32x32x16 on two accumulators, 8 = the same on one accumulator, 9 = 8
// transposing 8-byte LDS reads, 10 = 8 MFMAs each followed by 4 v_fma_f32,
// 11 = the same with 2 v_exp_f32, 12 = with one 16-byte LDS read, 13 = 8
// 16-byte global loads into registers, 14 = the same straight into LDS).
// gsrc is a device buffer of at least 64 KiB (the global loads' source).
// rec receives grid * 8 records (attn_mb_record_bytes each) and sink 512
// floats (written only on an impossible value).  Returns 0, or 1 for bad
// arguments, 2 if the launch failed.
int attn_mb_launch(int kind_lo, int kind_hi, int iters_lo, int iters_hi, int64_t grid, void *rec, void *sink,
                   const void *gsrc, void *stream) {
    if (grid < 1 || grid > (1 << 20) || !rec || !sink || !gsrc || iters_lo < 0 || iters_hi < 0 || kind_lo < 0 ||
        kind_lo > 14 || kind_hi < 0 || kind_hi > 14)
        return 1;
    hipLaunchKernelGGL(mb_kernel, dim3((unsigned)grid), dim3(512), 0, (hipStream_t)stream, kind_lo, kind_hi, iters_lo,
                       iters_hi, (Rec *)rec, (float *)sink, (const u32x4 *)gsrc);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Copy `bytes` (a multiple of 16) from src to dst (16-byte aligned).
int attn_mb_copy(const void *src, void *dst, int64_t bytes, int64_t grid, void *stream) {
    if (!src || !dst || bytes < 16 || (bytes & 15) || grid < 1 || grid > (1 << 20) || (((uintptr_t)src | (uintptr_t)dst) & 15))
        return 1;
    hipLaunchKernelGGL(mb_copy, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, (const u32x4 *)src,
                       (u32x4 *)dst, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
