"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same bytes, and compare with the stated tolerances."""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from attn_inputs import make_qkv, to_bits

# Max-abs tolerances against the fp64 oracle (strict <): output 1e-3 for fp16
# and 1e-2 for bf16, log-sum-exp 1e-3 for both.  An output element whose
# exact value is large enough that one unit in the last place of the 16-bit
# output type exceeds that bound (|o| >= 2 in fp16 or bf16: a row averaging
# only a few keys) is held to one such unit instead: even the correctly
# rounded value can miss 1e-3 there (at |o| in [4, 8) fp16 rounds to steps of
# 3.9e-3).
TOL_O = {"f16": 1e-3, "bf16": 1e-2}
TOL_LSE = 1e-3
DT_CODE = {"f16": 0, "bf16": 1}
MANT = {"f16": 10, "bf16": 7}     # explicit mantissa bits of the output type


def ulp16(x: np.ndarray, dtype: str) -> np.ndarray:
    """One unit in the last place of the 16-bit type at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    return 2.0 ** (e - MANT[dtype])


def output_bound(o_ref: np.ndarray, dtype: str) -> np.ndarray:
    """Per-element output bound: TOL_O, or one 16-bit ulp of the exact value
    when that is larger."""
    return np.maximum(TOL_O[dtype], ulp16(o_ref, dtype))


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import flashattention_forward_05_amd as fa
    fa.load_library()          # raises if the HIP library is missing
    return fa


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def run_gpu(q, k, v, *, causal, window=0, scale=None, config_id=-1, poison=True):
    """Host fp16/bf16 tensors in, (o, lse) host tensors out, via attn_fwd_ex."""
    import flashattention_forward_05_amd as fa
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    if poison:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    dtype = DT_CODE["f16" if q.dtype == torch.float16 else "bf16"]
    fa.attn_fwd_ex(qd, kd, vd, o, lse, B, Hq, Hkv, N, d, causal, window, scale, dtype, config_id,
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def run_gpu_splitkv(q, k, v, *, causal, window=0, scale=None, num_splits=0, config_id=-1, poison=True,
                    workspace=None):
    """Host tensors q (B,Hq,Nq,d), k/v (B,Hkv,Nk,d) in, (o, lse) host tensors
    out, via attn_fwd_splitkv_ex.  The workspace is allocated here (filled
    with NaN bit patterns when poison is set) unless one is passed."""
    import flashattention_forward_05_amd as fa
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    dtype = DT_CODE["f16" if q.dtype == torch.float16 else "bf16"]
    need = fa.attn_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal, window, dtype, num_splits,
                                              config_id)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        if poison:
            workspace.fill_(0xFF)
    if poison:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    fa.attn_fwd_splitkv_ex(qd, kd, vd, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, scale, dtype,
                           num_splits, config_id, workspace, workspace.numel(),
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def oracle_full(q, k, v, *, causal, window=0, scale=None):
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dt = "f16" if q.dtype == torch.float16 else "bf16"
    return oracle.oracle_fwd(to_bits(q), to_bits(k), to_bits(v), scale=float(np.float32(scale)),
                             causal=causal, window=window, dtype=dt)


def oracle_sampled(q, k, v, rows, *, causal, window=0, scale=None):
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dt = "f16" if q.dtype == torch.float16 else "bf16"
    return oracle.oracle_rows(to_bits(q), to_bits(k), to_bits(v), rows, scale=float(np.float32(scale)),
                              causal=causal, window=window, dtype=dt)


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    og = o_gpu.to(torch.float64).numpy()
    lg = lse_gpu.to(torch.float64).numpy()
    assert np.isfinite(og).all(), "non-finite output element"
    assert np.isfinite(lg).all(), "non-finite log-sum-exp"
    eo = np.abs(og - o_ref)
    el = np.abs(lg - lse_ref)
    return float(eo.max()) if eo.size else 0.0, float(el.max()) if el.size else 0.0, eo, el


def check(label, o_gpu, lse_gpu, o_ref, lse_ref, dtype):
    eo, el, eo_all, _ = errors(o_gpu, lse_gpu, o_ref, lse_ref)
    say(f"  {label}: max|dO| = {eo:.3e} (tol {TOL_O[dtype]:.0e}), max|dLSE| = {el:.3e} (tol {TOL_LSE:.0e})")
    if eo_all.size:
        bound = output_bound(np.asarray(o_ref), dtype)
        worst = np.unravel_index(np.argmax(eo_all - bound), eo_all.shape)
        assert (eo_all < bound).all(), (f"{label}: output error {eo_all[worst]:.3e} at {worst} (exact "
                                        f"{np.asarray(o_ref)[worst]:.6f}) >= {bound[worst]:.3e}")
    assert el < TOL_LSE, f"{label}: lse error {el:.3e} >= {TOL_LSE}"
    return eo, el


def sample_rows(B, Hq, N, n_random=96, seed=0, block=128):
    """Flat row ids: the first rows, rows around query-tile edges, the last
    rows, and random rows, spread over all (b, h)."""
    rng = np.random.default_rng(seed)
    pick = set()
    heads = [(b, h) for b in range(B) for h in range(Hq)]
    special = [0, 1, 2, 3, 31, 32, 63, 64, block - 1, block, block + 1, 2 * block - 1, 2 * block,
               N // 2, N - 2, N - 1]
    for idx, (b, h) in enumerate(heads):
        if idx % max(1, len(heads) // 8) == 0 or idx == len(heads) - 1:
            for i in special:
                if 0 <= i < N:
                    pick.add((b * Hq + h) * N + i)
    for _ in range(n_random):
        b, h = heads[rng.integers(len(heads))]
        pick.add((b * Hq + h) * N + int(rng.integers(N)))
    return np.array(sorted(pick), dtype=np.int64)


def inputs(B, Hq, Hkv, N, d, dtype, seed=0, amplitude=1.0):
    return make_qkv(B, Hq, Hkv, N, d, dtype, seed, amplitude)
