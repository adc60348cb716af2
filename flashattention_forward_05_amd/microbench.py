"""Measured ceilings of the GPU the attention kernels run on.

Runs the kernels of ``csrc/microbench.hip`` (library ``lib/libattn_microbench.so``)
and reports, for one MI355X:

- the dense bf16 MFMA rate (32x32x16 and 16x16x32 forms), the number the
  attention forward's matrix work is measured against beside the published
  peak;
- v_exp_f32 and v_fma_f32 rates per compute unit and clock;
- whether a wave's vector instructions run while another wave on the same
  SIMD keeps the matrix core busy (and exp beside fma);
- 16-byte LDS read bandwidth per compute unit and clock;
- the HBM copy bandwidth;
- the shader clock under each load (shader-clock counter over the 100 MHz
  real-time counter, both read in the kernel).

``python -m flashattention_forward_05_amd.microbench`` prints the results as JSON.
"""
from __future__ import annotations

import ctypes
import json
import os
import statistics

_LIB = None
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libattn_microbench.so")

(K_MFMA32, K_EXP, K_FMA, K_IDLE, K_MFMA16, K_EXPFMA, K_LDS, K_MFMA32_DEP2, K_MFMA32_DEP1, K_LDS_TR,
 K_MFMA_FMA4, K_MFMA_EXP2, K_MFMA_LDS, K_GLOAD, K_GLOAD_LDS) = range(15)
# work per wave per loop iteration
_OPS = {K_MFMA32: 8 * 32 * 32 * 16 * 2, K_MFMA16: 8 * 16 * 16 * 32 * 2, K_EXP: 16 * 64, K_FMA: 16 * 64,
        K_EXPFMA: 16 * 64, K_LDS: 8 * 64 * 16, K_IDLE: 0, K_MFMA32_DEP2: 8 * 32 * 32 * 16 * 2,
        K_MFMA32_DEP1: 8 * 32 * 32 * 16 * 2, K_LDS_TR: 8 * 64 * 8, K_MFMA_FMA4: 8 * 32 * 32 * 16 * 2,
        K_MFMA_EXP2: 8 * 32 * 32 * 16 * 2, K_MFMA_LDS: 8 * 32 * 32 * 16 * 2, K_GLOAD: 8 * 64 * 16,
        K_GLOAD_LDS: 8 * 64 * 16}
REALTIME_HZ = 100e6


def load_library():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run flashattention_forward_05_amd/build.py)")
        lib = ctypes.CDLL(LIB_PATH)
        lib.attn_mb_record_bytes.restype = ctypes.c_int
        lib.attn_mb_launch.restype = ctypes.c_int
        lib.attn_mb_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.attn_mb_copy.restype = ctypes.c_int
        lib.attn_mb_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_void_p]
        _LIB = lib
    return _LIB


def _cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def _run(kind_lo, kind_hi, iters_lo, iters_hi, grid=None):
    """One launch (after an untimed one); returns event ms and per-wave records."""
    import numpy as np
    import torch

    lib = load_library()
    grid = grid or _cus()
    rb = lib.attn_mb_record_bytes()
    rec = torch.zeros(grid * 8 * rb, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(512, dtype=torch.float32, device="cuda")
    gsrc = torch.ones(1 << 16, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        rc = lib.attn_mb_launch(kind_lo, kind_hi, iters_lo, iters_hi, grid, rec.data_ptr(), sink.data_ptr(),
                                gsrc.data_ptr(), st)
        b.record()
        if rc != 0:
            raise RuntimeError(f"attn_mb_launch failed ({rc})")
        torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    raw = rec.cpu().numpy().view(np.int64).reshape(grid * 8, rb // 8)
    t = raw[:, 1] - raw[:, 0]
    r = raw[:, 3] - raw[:, 2]
    ids = rec.cpu().numpy().view(np.int32).reshape(grid * 8, rb // 4)
    return ms, t, r, ids[:, 8], ids[:, 9]


def _clock_ghz(t, r):
    ok = r > 0
    return float(statistics.median((t[ok] / (r[ok] / REALTIME_HZ)) / 1e9)) if ok.any() else None


def _per_cu_clk(kind, iters, t, waves):
    """Work per compute unit per shader clock, over the waves running `kind`."""
    import numpy as np
    t = t.reshape(-1, 8)[:, waves]
    return float(_OPS[kind] * iters * len(waves) / np.median(t.max(axis=1)))


def measure(quick: bool = False) -> dict:
    """All measurements; quick=True only the 32x32x16 MFMA rate."""
    import numpy as np
    import torch

    cus = _cus()
    out = {"compute_units": cus}
    it_m = 4000 if quick else 20000
    ms, t, r, hw, xcc = _run(K_MFMA32, K_MFMA32, it_m, it_m)
    flops = cus * 8 * it_m * _OPS[K_MFMA32]
    out["mfma_32x32x16_bf16_tflops"] = flops / (ms * 1e-3) / 1e12
    out["mfma_32x32x16_flop_per_clk_cu"] = _per_cu_clk(K_MFMA32, it_m, t, list(range(8)))
    out["clock_ghz_mfma"] = _clock_ghz(t, r)
    simd = (hw >> 4) & 3
    out["waves_w_and_w4_share_simd"] = bool(np.all(simd.reshape(-1, 8)[:, :4] == simd.reshape(-1, 8)[:, 4:]))
    out["xcd_of_workgroup_is_index_mod_8"] = bool(np.all((xcc.reshape(-1, 8)[:, 0] & 7) == np.arange(cus) % 8))
    if quick:
        return out

    ms, t, r, _, _ = _run(K_MFMA16, K_MFMA16, it_m, it_m)
    out["mfma_16x16x32_bf16_tflops"] = cus * 8 * it_m * _OPS[K_MFMA16] / (ms * 1e-3) / 1e12

    it_v = 20000
    ms, t, r, _, _ = _run(K_EXP, K_EXP, it_v, it_v)
    out["exp_f32_per_clk_cu"] = _per_cu_clk(K_EXP, it_v, t, list(range(8)))
    out["clock_ghz_exp"] = _clock_ghz(t, r)
    ms, t, r, _, _ = _run(K_FMA, K_FMA, it_v, it_v)
    out["fma_f32_per_clk_cu"] = _per_cu_clk(K_FMA, it_v, t, list(range(8)))
    ms, t, r, _, _ = _run(K_EXPFMA, K_EXPFMA, it_v, it_v)
    out["exp_and_fma_in_one_wave_per_clk_cu"] = _per_cu_clk(K_EXPFMA, it_v, t, list(range(8)))

    # overlap: one wave per SIMD of each kind alone, then both together
    def pair(k_lo, it_lo, k_hi, it_hi):
        a = _run(k_lo, K_IDLE, it_lo, 0)[1].reshape(-1, 8)[:, :4].max(axis=1)
        b = _run(K_IDLE, k_hi, 0, it_hi)[1].reshape(-1, 8)[:, 4:].max(axis=1)
        c = _run(k_lo, k_hi, it_lo, it_hi)[1].reshape(-1, 8).max(axis=1)
        ta, tb, tc = float(np.median(a)), float(np.median(b)), float(np.median(c))
        # 1.0 = fully overlapped (time of the longer), 0.0 = serialised (sum)
        return {"alone_cycles": [ta, tb], "together_cycles": tc,
                "overlap": (ta + tb - tc) / min(ta, tb)}

    out["overlap_mfma_with_exp"] = pair(K_MFMA32, 4000, K_EXP, 8000)
    out["overlap_mfma_with_fma"] = pair(K_MFMA32, 4000, K_FMA, 32000)
    out["overlap_exp_with_fma"] = pair(K_EXP, 8000, K_FMA, 32000)
    # waves that mix kinds, as the attention kernels' waves do: an MFMA chain
    # whose operands come from LDS, or with vector work between the MFMAs,
    # beside a wave of exponentials or of the same mix
    out["overlap_mfma_lds_with_exp"] = pair(K_MFMA_LDS, 4000, K_EXP, 8000)
    out["overlap_mfma_fma4_with_exp"] = pair(K_MFMA_FMA4, 4000, K_EXP, 8000)
    out["overlap_mfma_exp2_with_mfma_exp2"] = pair(K_MFMA_EXP2, 4000, K_MFMA_EXP2, 4000)
    out["overlap_mfma_with_mfma_exp2"] = pair(K_MFMA32, 4000, K_MFMA_EXP2, 4000)

    ms, t, r, _, _ = _run(K_LDS, K_LDS, it_v, it_v)
    out["lds_read_b128_bytes_per_clk_cu"] = _per_cu_clk(K_LDS, it_v, t, list(range(8)))
    ms, t, r, _, _ = _run(K_LDS, K_IDLE, it_v, 0)
    out["lds_read_b128_bytes_per_clk_cu_one_wave_per_simd"] = _per_cu_clk(K_LDS, it_v, t, list(range(4)))
    ms, t, r, _, _ = _run(K_LDS_TR, K_LDS_TR, it_v, it_v)
    out["lds_read_b64_tr_bytes_per_clk_cu"] = _per_cu_clk(K_LDS_TR, it_v, t, list(range(8)))
    ms, t, r, _, _ = _run(K_LDS_TR, K_IDLE, it_v, 0)
    out["lds_read_b64_tr_bytes_per_clk_cu_one_wave_per_simd"] = _per_cu_clk(K_LDS_TR, it_v, t, list(range(4)))
    # the attention kernels' mix: one wave per SIMD reading while the other
    # keeps the matrix core busy
    ms, t, r, _, _ = _run(K_LDS, K_MFMA32, it_v, 4000)
    out["lds_read_b128_bytes_per_clk_cu_beside_mfma"] = _per_cu_clk(K_LDS, it_v, t, list(range(4)))

    # clocks per 32x32x16 MFMA of one wave per SIMD with 4, 2 and 1
    # independent accumulators (full rate is 32)
    for kind, name in ((K_MFMA32, "4"), (K_MFMA32_DEP2, "2"), (K_MFMA32_DEP1, "1")):
        t = _run(kind, K_IDLE, 4000, 0)[1].reshape(-1, 8)[:, :4].max(axis=1)
        out[f"mfma32_clk_per_instr_one_wave_{name}_accumulators"] = float(np.median(t)) / (4000 * 8)

    # one wave per SIMD interleaving its own MFMAs with independent vector or
    # LDS work: clocks per MFMA (32 = the other work fully hidden), alone and
    # beside a second wave doing the same
    for kind, name in ((K_MFMA_FMA4, "4fma"), (K_MFMA_EXP2, "2exp"), (K_MFMA_LDS, "1lds")):
        t = _run(kind, K_IDLE, 4000, 0)[1].reshape(-1, 8)[:, :4].max(axis=1)
        out[f"mfma32_plus_{name}_clk_per_mfma_one_wave"] = float(np.median(t)) / (4000 * 8)
        t = _run(kind, kind, 4000, 4000)[1].reshape(-1, 8).max(axis=1)
        out[f"mfma32_plus_{name}_clk_per_mfma_two_waves"] = float(np.median(t)) / (4000 * 8 * 2)

    # 16-byte global loads (8 per iteration, then a wait) from an L2-resident
    # buffer: into registers and straight into LDS; clocks per instruction of
    # one wave, with one wave per SIMD and with two
    for kind, name in ((K_GLOAD, "global_load_dwordx4"), (K_GLOAD_LDS, "global_load_lds_dwordx4")):
        t = _run(kind, K_IDLE, 2000, 0)[1].reshape(-1, 8)[:, :4].max(axis=1)
        out[f"{name}_clk_per_instr_one_wave_per_simd"] = float(np.median(t)) / (2000 * 8)
        t = _run(kind, kind, 2000, 2000)[1].reshape(-1, 8).max(axis=1)
        out[f"{name}_clk_per_instr_two_waves_per_simd"] = float(np.median(t)) / (2000 * 8)

    lib = load_library()
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream().cuda_stream
    grid = cus * 16
    for _ in range(2):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        if lib.attn_mb_copy(src.data_ptr(), dst.data_ptr(), nbytes, grid, st) != 0:
            raise RuntimeError("attn_mb_copy failed")
        b.record()
        torch.cuda.synchronize()
    out["hbm_copy_gbs"] = 2 * nbytes / (a.elapsed_time(b) * 1e-3) / 1e9
    return out


if __name__ == "__main__":
    print(json.dumps(measure(), indent=1))
