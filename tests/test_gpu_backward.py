"""GPU parity of the backward pass (attn_bwd through the C ABI) against the
fp64 oracle's gradients of sum(dO * O), on the same seeded inputs.

Where the whole tensors are checked, the backward is handed the oracle's O
(rounded to the 16-bit type) and lse, so that it is tested on its own; the
full-size sampled cases and test_bwd_after_hip_forward hand it the HIP
forward's o and lse, as a caller would.  The oracle differentiates the exact
forward.  Tolerance, per output tensor X in {dq, dk, dv}: max|X_gpu - X_ref|
< 4 u max|X_ref|, with u the unit roundoff of the 16-bit type (2^-11 fp16,
2^-8 bf16).  The kernels round P and dS to that type as MFMA operands and
round the outputs once; a numpy model of exactly that scheme
(bwd_rounding_model) against the same oracle stays below 1.6 u on every case
with random inputs here, so 4 u leaves a margin of more than 2 while any
error in a term (a wrong mask, scale, head map or transposed operand) shows
up at the size of the gradient itself.  On the score profiles with nearly
one-hot P the model's own dq error is far larger, and the bound follows it
(check_grads).  Each row of dq and each key's row of dk and dv is also
held to a bound of its own (check_slices below), so that an error confined
to rows with small gradients shows up too.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from attn_inputs import SCORE_PATTERNS, make_dout, make_qkv, make_score_pattern, to_bits
from bwd_rounding_model import model_bwd, oracle_forward_inputs
from gpu_helpers import DT_CODE, need_gpu, say

pytestmark = pytest.mark.gpu

TOL_BWD = {"f16": 4 * 2.0 ** -11, "bf16": 4 * 2.0 ** -8}


@pytest.fixture(scope="module")
def fa():
    return need_gpu()


def run_bwd(q, k, v, do, *, causal, window=0, scale=None, poison=True, o=None, lse=None):
    """Host tensors in; HIP backward on the given o and lse (host tensors), or
    on the HIP forward's when they are None; host (dq, dk, dv) out."""
    import flashattention_forward_05_amd as fa
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    dt = DT_CODE["f16" if q.dtype == torch.float16 else "bf16"]
    stream = torch.cuda.current_stream().cuda_stream
    if o is None:
        o = torch.empty_like(qd)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
        fa.attn_fwd(qd, kd, vd, o, lse, B, Hq, Hkv, N, d, causal, window, scale, dt, stream)
    else:
        assert o.shape == q.shape and o.dtype == q.dtype and lse.shape == (B, Hq, N) and lse.dtype == torch.float32
        o, lse = o.to(dev), lse.to(dev)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    need = fa.attn_bwd_workspace_size(B, Hq, Hkv, N, d)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if poison:
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        ws.fill_(0xFF)
    fa.attn_bwd(qd, kd, vd, o, dod, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, window, scale, dt, ws, ws.numel(),
                stream)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


# Per slice -- a row of dq, a key's row of dk or dv -- the error is also held
# against that slice's own largest gradient, floored at a fraction of the
# tensor's largest (a row whose gradient cancels to about zero, such as the
# first causal row, gets the floor): SLICE_TOL gives (multiple of u, floor).
# dq and dk are sums of the rounded dS = P (dP - D), whose terms cancel, the
# more so the fewer keys a row sees and the sharper the softmax: the rounding
# model of the kernels (bwd_rounding_model) reaches 31.2 u on dk with a 2-key
# window at scale 0.2, 9.9 u (dq) and 9.5 u (dk) at scale 0.3, and stays below
# 7.5 u at the default scale 1/sqrt(d) with no window or one of 64 keys or
# more.  So where the whole tensors are checked, and the model and the kernels
# receive the same O and lse, a slice's bound is twice the model's own error
# on that slice plus MODEL_SLACK u of the slice's scale.  Where nearly every
# row's P is one-hot and the keys are long and alike (the score profiles of
# make_score_pattern), dq is mostly rounding of dS: the model's median row is
# 4-38 u and its worst 33-350 u, and the rows that carry the most noise differ
# between the model and the kernels; there (median above MODEL_SLACK u) every
# slice may reach twice the model's worst slice.  The fixed multiples
# hold the cases that take the HIP forward's O: at the default scale with no
# short window.  (The forward rounds P before P.V, so its O differs from the
# correctly rounded one in a few last bits; through D = rowsum(dO * O) that
# moves a row's dS by a common amount, which shows in rows whose dq cancels,
# and more so with a sharp softmax.)  dv sums the positive P and stays
# below 2 u.  Below the floor these bounds are many times tighter than the
# tensor-wide one: an error confined to rows with small gradients (a mask or
# an index off by one near the diagonal) reaches the size of the slice's
# gradient itself and cannot hide under the largest gradient.
SLICE_TOL = {"dq": (20, 0.1), "dk": (20, 0.05), "dv": (6, 0.05)}
MODEL_SLACK = 4


def check_slices(label, name, g, r, dtype, m=None):
    """Worst slice error in units of u of the slice's scale; g, r and the
    model's values m are (slices, d).  Asserted below SLICE_TOL's multiple,
    or with m given, below 2 |m - r| + MODEL_SLACK u per slice."""
    u = TOL_BWD[dtype] / 4
    mult, floor = SLICE_TOL[name]
    gmax = float(np.abs(r).max()) if r.size else 0.0
    if gmax == 0.0:
        return 0.0
    err = np.abs(g - r).max(axis=-1)
    ref = np.maximum(np.abs(r).max(axis=-1), floor * gmax)
    if m is None:
        bound = mult * u * ref
    else:
        merr = np.abs(m - r).max(axis=-1)
        bound = 2 * merr + MODEL_SLACK * u * ref
        # slices that are mostly rounding noise (the model's median slice error
        # above MODEL_SLACK u): which of them carry the most noise differs
        # between the model and the kernels, so each may reach twice the
        # model's worst slice
        rel = merr / ref
        if np.median(rel) > MODEL_SLACK * u:
            bound = np.maximum(bound, 2 * rel.max() * ref)
    bad = np.flatnonzero(err >= bound)
    worst = float((err / ref).max() / u)
    if bad.size:
        i = int(bad[np.argmax(err[bad] / bound[bad])])
        raise AssertionError(f"{label}: {name} slice {i} error {err[i] / ref[i] / u:.2f} u of the slice's scale "
                             f"(largest |ref| {np.abs(r[i]).max():.3e}, floor {floor} x max|ref|) >= bound "
                             f"{bound[i] / ref[i] / u:.2f} u")
    return worst


def check_grads(label, got, ref, dtype, model=None):
    """Tensor-wide and per-slice bounds.  With the rounding model's values,
    the tensor-wide bound is also at least twice the model's own error: where
    every row's P is nearly one-hot and the keys are long and alike, dq is a
    small difference of large terms and the rounding of dS dominates it."""
    worst, slices = [], []
    for t, (name, g, r) in enumerate(zip(("dq", "dk", "dv"), got, ref)):
        gd = g.to(torch.float64).numpy().reshape(r.shape)
        assert np.isfinite(gd).all(), f"{label}: non-finite {name}"
        scale = float(np.abs(r).max()) if r.size else 0.0
        err = float(np.abs(gd - r).max()) if r.size else 0.0
        rel = err / scale if scale > 0 else err
        worst.append(rel)
        tol = TOL_BWD[dtype]
        if model is not None and scale > 0:
            tol = max(tol, 2 * float(np.abs(model[t] - r).max()) / scale)
        assert rel < tol, f"{label}: {name} error {err:.3e} = {rel:.2e} x max|ref| >= {tol:.2e}"
        d = r.shape[-1] if r.ndim else 1
        m = None if model is None else model[t].reshape(-1, d)
        slices.append(check_slices(label, name, gd.reshape(-1, d), np.asarray(r).reshape(-1, d), dtype, m))
    say(f"  {label}: max error / max|ref|: dq {worst[0]:.2e}, dk {worst[1]:.2e}, dv {worst[2]:.2e} "
        f"(tol {TOL_BWD[dtype]:.2e}); worst slice in u: dq {slices[0]:.2f}, dk {slices[1]:.2f}, dv {slices[2]:.2f}")
    return worst


def full_case(B, Hq, Hkv, N, d, dtype, causal, window=0, seed=0, scale=None, hip_forward=False):
    q, k, v = make_qkv(B, Hq, Hkv, N, d, dtype, seed=seed)
    do = make_dout(B, Hq, N, d, dtype, seed=seed)
    label = f"bwd B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} {dtype} causal={causal} W={window} seed={seed}"
    if scale is not None:
        label += f" scale={scale}"
    return check_case(label, q, k, v, do, dtype, causal, window, scale, hip_forward)


def check_case(label, q, k, v, do, dtype, causal, window=0, scale=None, hip_forward=False):
    """Whole tensors of the HIP backward against the oracle (and, unless the
    HIP forward's o and lse are used, the rounding model's slice bounds)."""
    d = q.shape[-1]
    if hip_forward:
        label += " (HIP forward's o, lse)"
    say(f"case {label}")
    s = 1.0 / math.sqrt(d) if scale is None else scale
    s32 = float(np.float32(s))
    ref = oracle.oracle_bwd(to_bits(q), to_bits(k), to_bits(v), to_bits(do), scale=s32, causal=causal,
                            window=window, dtype=dtype)
    if hip_forward:
        got = run_bwd(q, k, v, do, causal=causal, window=window, scale=s)
        return check_grads(label, got, ref, dtype)
    o, lse = oracle_forward_inputs(q, k, v, scale=s32, causal=causal, window=window, dtype=dtype)
    got = run_bwd(q, k, v, do, causal=causal, window=window, scale=s, o=o, lse=lse)
    model = model_bwd(q, k, v, do, o, lse, scale=s32, causal=causal, window=window, dtype=dtype)
    return check_grads(label, got, ref, dtype, model)


# ---- the lab shapes (2, 4, N, 64) fp16, causal and not, with a ragged tail
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [64, 256, 1000])
def test_bwd_lab(fa, N, causal):
    full_case(2, 4, 4, N, 64, "f16", causal)


# ---- GQA / MQA, d = 128, bf16 and fp16, every mask, ragged lengths
@pytest.mark.parametrize("mask", [(False, 0), (True, 0), (True, 100), (True, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_bwd_gqa_d128(fa, dtype, mask):
    causal, window = mask
    full_case(1, 8, 2, 333, 128, dtype, causal, window)


@pytest.mark.parametrize("mask", [(False, 0), (True, 0), (True, 77)])
def test_bwd_mqa(fa, mask):
    causal, window = mask
    full_case(2, 4, 1, 257, 128, "bf16", causal, window, seed=3)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 63, 65, 130])
def test_bwd_short_and_ragged(fa, N, d):
    full_case(1, 2, 1, N, d, "f16", True, seed=N)
    full_case(1, 2, 2, N, d, "bf16", False, seed=N + 1)


def test_bwd_window_d64(fa):
    full_case(2, 4, 2, 700, 64, "bf16", True, 129, seed=5)


def test_bwd_negative_and_odd_scale(fa):
    full_case(1, 4, 2, 200, 64, "f16", True, scale=-0.1, seed=6)
    full_case(1, 4, 4, 200, 128, "bf16", False, scale=0.3, seed=7)


# ---- forward then backward, both HIP, at the default scale
@pytest.mark.parametrize("case", [(2, 4, 4, 1000, 64, "f16", True, 0), (1, 8, 2, 333, 128, "bf16", True, 100),
                                  (2, 4, 1, 257, 128, "bf16", False, 0)])
def test_bwd_after_hip_forward(fa, case):
    full_case(*case, seed=12, hip_forward=True)


# ---- a seeded sweep: shapes, head groupings, dtypes, masks (windows of 1 and 2
# keys included) and scales (negative and sharp ones included)
def test_bwd_random_sweep(fa):
    rng = np.random.default_rng(31)
    for n in range(40):
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["f16", "bf16"]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 3))
        N = int(rng.choice([int(rng.integers(1, 130)), int(rng.integers(130, 600))]))
        causal = bool(rng.integers(0, 3) > 0)
        window = int(rng.choice([0, 0, 1, 2, 33, 100])) if causal else 0
        scale = float(rng.choice([1.0 / math.sqrt(d), 1.0 / math.sqrt(d), -0.1, 0.2]))
        full_case(B, G * Hkv, Hkv, N, d, dt, causal, window, seed=7000 + n, scale=scale)


# ---- the score profiles that drive the forward's online softmax (a running max
# raised on every tile, a stale one, underflow, spikes at tile edges): here they
# give rows whose P is nearly one-hot, where dS cancels hardest
@pytest.mark.parametrize("pattern", SCORE_PATTERNS)
@pytest.mark.parametrize("d,dtype", [(64, "f16"), (128, "bf16")])
def test_bwd_score_patterns(fa, pattern, d, dtype):
    N = 500
    for n_case, causal in enumerate((False, True)):
        q, k, v = make_score_pattern(pattern, N, d, dtype, seed=23 + n_case)
        do = make_dout(1, q.shape[1], N, d, dtype, seed=23 + n_case)
        check_case(f"bwd score pattern {pattern} N{N} d{d} {dtype} causal={causal}", q, k, v, do, dtype, causal)


def test_bwd_deterministic(fa):
    q, k, v = make_qkv(1, 8, 2, 500, 128, "bf16", seed=9)
    do = make_dout(1, 8, 500, 128, "bf16", seed=9)
    say("case bwd determinism (1, 8/2, 500, 128) bf16 causal")
    a = run_bwd(q, k, v, do, causal=True)
    b = run_bwd(q, k, v, do, causal=True, poison=False)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


# ---- full size, sampled: dq rows and dk / dv keys the oracle computes one by one
def sampled_case(B, Hq, Hkv, N, d, dtype, causal, window=0, seed=0, n_rows=48, n_keys=24):
    q, k, v = make_qkv(B, Hq, Hkv, N, d, dtype, seed=seed)
    do = make_dout(B, Hq, N, d, dtype, seed=seed)
    label = f"bwd sampled B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} {dtype} causal={causal} W={window}"
    say(f"case {label}")
    dq, dk, dv = run_bwd(q, k, v, do, causal=causal, window=window)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, N - 1, N // 2], rng.integers(0, B * Hq * N, n_rows)]))
    # keys of one (batch, K/V head) group: the oracle's forward runs per group
    grp = int(rng.integers(0, B * Hkv))
    keys = np.unique(np.concatenate([[0, 1, 63, 64, N - 1], rng.integers(0, N, n_keys)])) + grp * N
    s = float(np.float32(1.0 / math.sqrt(d)))
    kw = dict(scale=s, causal=causal, window=window, dtype=dtype)
    bits = [to_bits(t) for t in (q, k, v, do)]
    rq = oracle.oracle_bwd_rows(*bits, rows, **kw)
    rk, rv = oracle.oracle_bwd_keys(*bits, keys, **kw)
    # the scale of each tensor is taken over the sampled reference entries
    check_grads(label, (dq.reshape(-1, d)[rows], dk.reshape(-1, d)[keys], dv.reshape(-1, d)[keys]),
                (rq, rk, rv), dtype)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_lab_n4096_sampled(fa, causal):
    sampled_case(2, 4, 4, 4096, 64, "f16", causal)


def test_bwd_gqa_n8192_sampled(fa):
    sampled_case(4, 32, 8, 8192, 128, "bf16", True, n_rows=32, n_keys=12)


# ---- MQA long context at full size: the oracle cannot form every row's
# normaliser for the per-key check here, so dq is checked on sampled rows and
# dk, dv through identities that hold at any size (rows of P sum to 1, rows
# of dS sum to 0): sum_j dv_j equals the sum of dO over every row of every
# query head, and sum_j dk_j = 0, per channel.  The bound on each sum is 4 u
# times the sum of the magnitudes it adds up (u as above).
@pytest.mark.parametrize("window", [0, 4096])
def test_bwd_mqa_n32768_properties(fa, window):
    B, Hq, Hkv, N, d, dtype = 1, 32, 1, 32768, 128, "bf16"
    q, k, v = make_qkv(B, Hq, Hkv, N, d, dtype, seed=0)
    do = make_dout(B, Hq, N, d, dtype, seed=0)
    label = f"bwd MQA (1, 32/1, 32768, 128) bf16 causal W={window}"
    say(f"case {label}")
    dq, dk, dv = run_bwd(q, k, v, do, causal=True, window=window)
    s = float(np.float32(1.0 / math.sqrt(d)))
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, 4095, 4096, N - 1, 5 * N + 77], rng.integers(0, B * Hq * N, 24)]))
    rq = oracle.oracle_bwd_rows(to_bits(q), to_bits(k), to_bits(v), to_bits(do), rows, scale=s, causal=True,
                                window=window, dtype=dtype)
    gq = dq.reshape(-1, d)[rows].to(torch.float64).numpy()
    rel = float(np.abs(gq - rq).max() / np.abs(rq).max())
    u = TOL_BWD[dtype] / 4
    dvd = dv.to(torch.float64).numpy()[0, 0]
    dkd = dk.to(torch.float64).numpy()[0, 0]
    assert np.isfinite(dvd).all() and np.isfinite(dkd).all(), f"{label}: non-finite dk or dv"
    want_dv = do.to(torch.float64).numpy().sum(axis=(0, 1, 2))
    err_dv = np.abs(dvd.sum(0) - want_dv)
    bound_dv = 4 * u * np.abs(dvd).sum(0)
    err_dk = np.abs(dkd.sum(0))
    bound_dk = 4 * u * np.abs(dkd).sum(0)
    say(f"  {label}: dq rows {rel:.2e} x max|ref|; max |sum dv - sum dO| / bound {float((err_dv / bound_dv).max()):.2e}; "
        f"max |sum dk| / bound {float((err_dk / bound_dk).max()):.2e}")
    assert rel < TOL_BWD[dtype], f"{label}: dq error {rel:.2e} x max|ref|"
    assert (err_dv < bound_dv).all(), f"{label}: sum of dv differs from the sum of dO"
    assert (err_dk < bound_dk).all(), f"{label}: sum of dk is not 0"


# ---- MQA long context at full size, key by key: dk and dv of keys in the
# last 136 positions (both sides of the last 128- and 64-key block edges),
# checked elementwise.  Only the query rows at or after the earliest of them
# see these keys, so the oracle forms just those rows' normalisers (32 heads x
# 136 rows) instead of the whole forward.
@pytest.mark.timeout(400)
def test_bwd_mqa_n32768_keys(fa):
    B, Hq, Hkv, N, d, dtype = 1, 32, 1, 32768, 128, "bf16"
    q, k, v = make_qkv(B, Hq, Hkv, N, d, dtype, seed=0)
    do = make_dout(B, Hq, N, d, dtype, seed=0)
    label = f"bwd MQA (1, 32/1, 32768, 128) bf16 causal, late keys"
    say(f"case {label}")
    dq, dk, dv = run_bwd(q, k, v, do, causal=True)
    rng = np.random.default_rng(11)
    edges = [N - 136, N - 129, N - 128, N - 127, N - 65, N - 64, N - 63, N - 33, N - 32, N - 2, N - 1]
    keys = np.unique(np.concatenate([edges, rng.integers(N - 136, N, 20)]))
    assert keys.size >= 24
    s = float(np.float32(1.0 / math.sqrt(d)))
    bits = [to_bits(t) for t in (q, k, v, do)]
    say(f"  oracle for {keys.size} keys")
    rk, rv = oracle.oracle_bwd_keys(*bits, keys, scale=s, causal=True, window=0, dtype=dtype)
    gk = dk.reshape(-1, d)[keys].to(torch.float64).numpy()
    gv = dv.reshape(-1, d)[keys].to(torch.float64).numpy()
    assert np.isfinite(gk).all() and np.isfinite(gv).all(), f"{label}: non-finite dk or dv"
    assert np.abs(rk).max() > 0 and np.abs(gk).max() > 0, f"{label}: dk is all zero"
    ek = float(np.abs(gk - rk).max() / np.abs(rk).max())
    ev = float(np.abs(gv - rv).max() / np.abs(rv).max())
    say(f"  {label}: {keys.size} keys, max error / max|ref|: dk {ek:.2e}, dv {ev:.2e} (tol {TOL_BWD[dtype]:.2e})")
    assert ek < TOL_BWD[dtype], f"{label}: dk error {ek:.2e} x max|ref|"
    assert ev < TOL_BWD[dtype], f"{label}: dv error {ev:.2e} x max|ref|"
    sk = check_slices(label, "dk", gk, rk, dtype)
    sv = check_slices(label, "dv", gv, rv, dtype)
    say(f"  {label}: worst key in u: dk {sk:.2f}, dv {sv:.2f}")


# ---- d=64 on a grid of at least 512 128-row workgroups (B*Hq*ceil(N/128)),
# ragged N, causal and not, sampled rows and keys against the oracle
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_d64_large_grid_sampled(fa, causal):
    B, Hq, Hkv, N = 4, 16, 4, 1000
    assert B * Hq * -(-N // 128) >= 512
    sampled_case(B, Hq, Hkv, N, 64, "f16", causal, seed=5, n_rows=48, n_keys=24)
