"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element, with the stated tolerances."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

from attn_inputs import SCORE_PATTERNS, WORKLOADS, make_score_pattern, make_workload
from gpu_helpers import (DT_CODE, TOL_LSE, TOL_O, check, errors, inputs, need_gpu, oracle_full,
                         oracle_sampled, run_gpu, run_gpu_splitkv, sample_rows, say)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def fa():
    return need_gpu()


# ---- the pages' correctness protocol: (2, 4, N, 64) fp16, causal and not
LAB = json.load(open(os.path.join(GOLDEN, "lab_protocol.json")))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N", [64, 256, 1000, 1024])
def test_lab_protocol_full(fa, N, causal):
    q, k, v = inputs(LAB["B"], LAB["H"], LAB["H"], N, LAB["d"], "f16", seed=0)
    o, lse = run_gpu(q, k, v, causal=causal)
    ro, rl = oracle_full(q, k, v, causal=causal)
    check(f"lab N={N} causal={causal}", o, lse, ro, rl, "f16")


@pytest.mark.parametrize("causal", [True, False])
def test_lab_protocol_n4096_sampled(fa, causal):
    q, k, v = inputs(2, 4, 4, 4096, 64, "f16", seed=0)
    o, lse = run_gpu(q, k, v, causal=causal)
    rows = sample_rows(2, 4, 4096, n_random=256)
    ro, rl = oracle_sampled(q, k, v, rows, causal=causal)
    check(f"lab N=4096 causal={causal} ({len(rows)} rows)", o.reshape(-1, 64)[rows],
          lse.reshape(-1)[rows], ro, rl, "f16")


@pytest.mark.parametrize("seed", range(1, 10))
def test_lab_seeds_causal(fa, seed):
    """The error margin depends on the data; ten seeds of the causal case."""
    q, k, v = inputs(2, 4, 4, 1024, 64, "f16", seed=seed)
    o, lse = run_gpu(q, k, v, causal=True)
    ro, rl = oracle_full(q, k, v, causal=True)
    check(f"lab N=1024 causal seed={seed}", o, lse, ro, rl, "f16")


def test_tiny_anchor(fa):
    w = WORKLOADS["tiny"]
    q, k, v = make_workload(w, seed=0)
    o, lse = run_gpu(q, k, v, causal=w.causal)
    ro, rl = oracle_full(q, k, v, causal=w.causal)
    check("tiny (1,12,64,64) causal", o, lse, ro, rl, "f16")


@pytest.mark.parametrize("name", ["stress_full", "stress_causal"])
def test_stress_anchor(fa, name):
    w = WORKLOADS[name]
    q, k, v = make_workload(w, seed=0)
    o, lse = run_gpu(q, k, v, causal=w.causal)
    rows = sample_rows(w.B, w.Hq, w.N, n_random=256)
    ro, rl = oracle_sampled(q, k, v, rows, causal=w.causal)
    check(f"{name} ({len(rows)} rows)", o.reshape(-1, w.d)[rows], lse.reshape(-1)[rows], ro, rl, w.dtype)


# ---- every tile configuration on ragged shapes, both head dims and dtypes
CASES = [
    # B, Hq, Hkv, N, d, dtype, causal, window
    (1, 2, 2, 1, 64, "f16", False, 0),
    (1, 2, 2, 1, 128, "bf16", True, 0),
    (1, 2, 1, 2, 64, "f16", True, 0),
    (2, 3, 3, 63, 64, "f16", False, 0),
    (1, 4, 2, 65, 128, "bf16", True, 0),
    (1, 2, 2, 127, 64, "bf16", True, 0),
    (1, 2, 2, 129, 128, "f16", False, 0),
    (1, 4, 4, 300, 64, "f16", True, 1),
    (1, 4, 1, 300, 128, "bf16", True, 2),
    (1, 2, 2, 333, 64, "f16", True, 17),
    (2, 8, 2, 520, 128, "bf16", True, 200),
    (1, 6, 3, 777, 128, "f16", True, 0),
    (1, 2, 2, 1000, 64, "bf16", False, 0),
    (1, 4, 2, 1100, 64, "f16", True, 0),
    (1, 2, 1, 900, 128, "bf16", True, 300),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_N{}_d{}_{}_c{}_w{}".format(*c))
def test_ragged_all_configs(fa, case):
    B, Hq, Hkv, N, d, dt, causal, window = case
    q, k, v = inputs(B, Hq, Hkv, N, d, dt, seed=N)
    ro, rl = oracle_full(q, k, v, causal=causal, window=window)
    for cfg in range(fa.attn_fwd_num_configs()):
        o, lse = run_gpu(q, k, v, causal=causal, window=window, config_id=cfg)
        check(f"cfg{cfg}", o, lse, ro, rl, dt)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5, 1e-30])
def test_unusual_scales(fa, scale):
    q, k, v = inputs(1, 2, 2, 200, 64, "f16", seed=3)
    for causal in (False, True):
        o, lse = run_gpu(q, k, v, causal=causal, scale=scale)
        ro, rl = oracle_full(q, k, v, causal=causal, scale=scale)
        check(f"scale={scale} causal={causal}", o, lse, ro, rl, "f16")


# ---- full-size workloads, sampled rows, in the launch configuration the
# benchmark times (the automatic choice)
@pytest.mark.parametrize("name", ["gqa", "mqa_window", "mqa_causal"])
def test_full_size_sampled(fa, name):
    w = WORKLOADS[name]
    say(f"  generating {w.label()}")
    q, k, v = make_workload(w, seed=0)
    o, lse = run_gpu(q, k, v, causal=w.causal, window=w.window)
    rows = sample_rows(w.B, w.Hq, w.N, n_random=160)
    ro, rl = oracle_sampled(q, k, v, rows, causal=w.causal, window=w.window)
    check(f"{name} ({len(rows)} rows)", o.reshape(-1, w.d)[rows], lse.reshape(-1)[rows], ro, rl, w.dtype)
    # whole-output properties that hold at any size
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


# ---- identities and robustness
def test_gqa_equals_repeated_heads_bitwise(fa):
    q, k, v = inputs(2, 8, 2, 333, 128, "bf16", seed=7)
    o1, l1 = run_gpu(q, k, v, causal=True)
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    o2, l2 = run_gpu(q, kr, vr, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_wide_window_equals_causal(fa):
    q, k, v = inputs(1, 4, 4, 400, 64, "f16", seed=8)
    o1, l1 = run_gpu(q, k, v, causal=True)
    for w in (400, 4096):
        o2, l2 = run_gpu(q, k, v, causal=True, window=w)
        eo = (o1.float() - o2.float()).abs().max().item()
        el = (l1 - l2).abs().max().item()
        assert eo <= 1e-3 and el <= 1e-5, (w, eo, el)


def test_window_one_returns_own_value_row(fa):
    q, k, v = inputs(1, 2, 2, 150, 128, "f16", seed=9)
    o, _ = run_gpu(q, k, v, causal=True, window=1)
    assert torch.equal(o, v)


def test_causal_row0_is_v0(fa):
    q, k, v = inputs(2, 4, 2, 257, 64, "bf16", seed=10)
    o, _ = run_gpu(q, k, v, causal=True)
    assert torch.equal(o[:, :, 0], v.repeat_interleave(2, dim=1)[:, :, 0])


def test_deterministic(fa):
    q, k, v = inputs(1, 8, 8, 1500, 64, "f16", seed=11)
    o1, l1 = run_gpu(q, k, v, causal=True)
    o2, l2 = run_gpu(q, k, v, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_guard_bands_untouched(fa):
    import flashattention_forward_05_amd as fa_mod
    B, H, N, d = 1, 3, 211, 64
    q, k, v = inputs(B, H, H, N, d, "f16", seed=12)
    dev = torch.device("cuda:0")
    pad = 4096
    obuf = torch.full((B * H * N * d + 2 * pad,), 7.0, dtype=torch.float16, device=dev)
    lbuf = torch.full((B * H * N + 2 * pad,), 7.0, dtype=torch.float32, device=dev)
    o = obuf[pad:pad + B * H * N * d]
    lse = lbuf[pad:pad + B * H * N]
    fa_mod.attn_fwd(q.to(dev), k.to(dev), v.to(dev), o, lse, B, H, H, N, d, 1, 0, 0.125, 0)
    torch.cuda.synchronize()
    assert (obuf[:pad] == 7.0).all() and (obuf[-pad:] == 7.0).all()
    assert (lbuf[:pad] == 7.0).all() and (lbuf[-pad:] == 7.0).all()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_lse_may_be_null(fa):
    import flashattention_forward_05_amd as fa_mod
    q, k, v = inputs(1, 2, 2, 100, 64, "f16", seed=13)
    dev = torch.device("cuda:0")
    o = torch.empty_like(q, device=dev)
    fa_mod.attn_fwd(q.to(dev), k.to(dev), v.to(dev), o, None, 1, 2, 2, 100, 64, 0, 0, 0.125, 0)
    torch.cuda.synchronize()
    ro, _ = oracle_full(q, k, v, causal=False)
    eo = np.abs(o.cpu().double().numpy() - ro).max()
    assert eo < TOL_O["f16"]


def test_empty_sequence(fa):
    q = torch.empty(1, 2, 0, 64, dtype=torch.float16, device="cuda")
    o, lse = fa.flash_attn_forward(q, q, q, causal=True)
    assert o.shape == (1, 2, 0, 64) and lse.shape == (1, 2, 0)


def test_flash_attn_forward_wrapper(fa):
    q, k, v = inputs(1, 4, 2, 96, 128, "bf16", seed=14)
    o, lse = fa.flash_attn_forward(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle_full(q, k, v, causal=True)
    check("wrapper", o.cpu(), lse.cpu(), ro, rl, "bf16")


# ---- tile-configuration tuning
@pytest.mark.parametrize("d,dt", [(64, "f16"), (128, "bf16")])
def test_autotune(fa, d, dt):
    import flashattention_forward_05_amd as fa_mod
    B, H, N = 1, 4, 700
    q, k, v = inputs(B, H, H, N, d, dt, seed=31)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    best, ms = fa_mod.attn_fwd_autotune(qd, kd, vd, o, lse, B, H, H, N, d, True, 0, d ** -0.5,
                                        DT_CODE[dt], reps=5)
    built = list(range(fa_mod.attn_fwd_num_configs()))
    assert sorted(ms) == built and best in ms and ms[best] == min(ms.values())
    ro, rl = oracle_full(q, k, v, causal=True)
    check(f"after tuning (last config run)", o.cpu(), lse.cpu(), ro, rl, dt)
    # the wrapper tunes a shape once and then uses the fastest configuration
    for _ in range(2):
        o2, l2 = fa_mod.flash_attn_forward(qd, kd, vd, causal=True, tune=True)
        torch.cuda.synchronize()
        check("tuned wrapper", o2.cpu(), l2.cpu(), ro, rl, dt)
    assert any(key[1:6] == (B, H, H, N, d) for key in fa_mod.tuned_configs())


def test_plain_random_shapes(fa):
    """Seeded random shapes, masks and tile configurations of the plain forward."""
    rng = np.random.default_rng(99)
    for n in range(16):
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["f16", "bf16"]))
        Hkv = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 3))
        N = int(rng.integers(1, 1500))
        causal = bool(rng.integers(0, 3) > 0)
        window = int(rng.choice([0, 0, 1, 33, 700])) if causal else 0
        cfgs = list(range(fa.attn_fwd_num_configs()))
        cfg = int(rng.choice([-1] + cfgs))
        q, k, v = inputs(B, G * Hkv, Hkv, N, d, dt, seed=300 + n)
        ro, rl = oracle_full(q, k, v, causal=causal, window=window)
        o, lse = run_gpu(q, k, v, causal=causal, window=window, config_id=cfg)
        check(f"#{n} B{B} Hq{G * Hkv}/{Hkv} N{N} d{d} {dt} c{int(causal)} w{window} cfg{cfg}", o, lse, ro, rl, dt)


def test_random_sweep(fa):
    """A seeded sweep over shapes, head groupings, masks (short windows
    included, where a row averages a few keys and |o| can pass 2), dtypes,
    tile configurations and the split-KV entry point with forced chunk
    counts, against the oracle."""
    rng = np.random.default_rng(2024)
    for n in range(80):
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["f16", "bf16"]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 3))
        N = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(200, 1100)),
                            int(rng.choice([64, 128, 255, 256, 257, 511, 512, 513, 767, 1024]))]))
        causal = bool(rng.integers(0, 3) > 0)
        window = int(rng.choice([0, 0, 1, 2, 31, 64, 65, 127, 300, 1000])) if causal else 0
        cfgs = list(range(fa.attn_fwd_num_configs()))
        cfg = int(rng.choice([-1] + cfgs))
        split = bool(rng.integers(0, 4) == 0)
        q, k, v = inputs(B, G * Hkv, Hkv, N, d, dt, seed=1000 + n)
        ro, rl = oracle_full(q, k, v, causal=causal, window=window)
        label = f"#{n} B{B} Hq{G * Hkv}/{Hkv} N{N} d{d} {dt} c{int(causal)} w{window} cfg{cfg}"
        if split:
            nsp = int(rng.choice([0, 2, 3, 7]))
            o, lse = run_gpu_splitkv(q, k, v, causal=causal, window=window, num_splits=nsp, config_id=cfg)
            label += f" split-KV {nsp}"
        else:
            o, lse = run_gpu(q, k, v, causal=causal, window=window, config_id=cfg)
        check(label, o, lse, ro, rl, dt)


# ---- inputs built to drive the online softmax's own logic ("Optimizaciones de
# Atencion", section "FlashAttention: Nunca materializar la matriz de atencion":
# the running max and the rescale of the sum and accumulator when it grows;
# make_score_pattern gives the profiles): rising raises the running max on
# nearly every 64-key tile; slow grows below the raise threshold, so tiles are
# accepted against a stale max until the growth adds up; falling lets later
# tiles underflow to zero; spikes put a few dominant keys on both sides of tile
# edges.
@pytest.mark.parametrize("pattern", SCORE_PATTERNS)
@pytest.mark.parametrize("d,dtype", [(64, "f16"), (64, "bf16"), (128, "bf16"), (128, "f16")])
def test_softmax_stress_patterns(fa, pattern, d, dtype):
    N = 1000
    for n_case, causal in enumerate((False, True)):
        forced = (SCORE_PATTERNS.index(pattern) + d // 64 + 2 * n_case
                  + (dtype == "bf16")) % fa.attn_fwd_num_configs()
        for cfg in (-1, forced):
            q, k, v = make_score_pattern(pattern, N, d, dtype, seed=17 + n_case)
            ro, rl = oracle_full(q, k, v, causal=causal)
            o, lse = run_gpu(q, k, v, causal=causal, config_id=cfg)
            check(f"softmax stress {pattern} d{d} {dtype} causal={causal} cfg{cfg}", o, lse, ro, rl, dtype)


def test_causal_128_row_layouts(fa):
    """Configuration 0, causal: paired 64-row query tiles on grids of at most
    256 workgroups, heavy-first 128-row tiles above (B=2, 65 and 64 heads of
    N=640: 650 and 640 workgroups; B=1, 2 heads: 10)."""
    for B, Hq, N, dt in ((2, 65, 640, "f16"), (2, 64, 640, "bf16"), (1, 2, 640, "bf16")):
        plan = fa.attn_fwd_plan_ex(B, Hq, Hq, N, 64, 1, 0, 0 if dt == "f16" else 1, 0)
        q, k, v = inputs(B, Hq, Hq, N, 64, dt, seed=B * 1000 + Hq)
        ro, rl = oracle_full(q, k, v, causal=True, window=0)
        o, lse = run_gpu(q, k, v, causal=True, window=0, config_id=0)
        check(f"B{B} Hq{Hq} N{N} {dt} grid {plan['grid']}", o, lse, ro, rl, dt)
