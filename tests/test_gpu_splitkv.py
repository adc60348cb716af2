"""GPU parity of the split-KV forward ("Optimizaciones de Atencion", section
"FlashDecoding"): Nq queries against Nk keys, the keys cut into chunks over
workgroups, partial results merged by a second kernel.  Checked through the C
ABI against the fp64 oracle on the same seeded inputs, with the tolerances of
the plain forward."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from attn_inputs import SCORE_PATTERNS, WORKLOADS, make_qkv, make_score_pattern, make_workload
from gpu_helpers import (TOL_LSE, TOL_O, check, need_gpu, oracle_full, oracle_sampled, run_gpu,
                         run_gpu_splitkv, sample_rows, say)

pytestmark = pytest.mark.gpu

CONFIGS = (0, 1, 2, 3, 4)


@pytest.fixture(scope="module")
def fa():
    return need_gpu()


def qkv(B, Hq, Hkv, Nq, Nk, d, dt, seed):
    return make_qkv(B, Hq, Hkv, Nq, d, dt, seed=seed, nk=Nk)


# B, Hq, Hkv, Nq, Nk, d, dtype, causal, window
CASES = [
    (1, 4, 1, 1, 1, 64, "f16", True, 0),          # one key
    (2, 8, 2, 1, 77, 128, "bf16", True, 0),       # ragged single tile
    (1, 4, 4, 1, 1000, 64, "f16", True, 0),
    (1, 8, 2, 3, 1000, 128, "bf16", True, 0),     # a few new tokens: bottom-right causal
    (1, 4, 2, 5, 2049, 64, "bf16", True, 100),    # window inside the cache
    (1, 4, 1, 1, 3001, 128, "f16", True, 1),      # window of one key: the last value row
    (2, 4, 4, 2, 513, 64, "f16", False, 0),
    (1, 2, 2, 40, 1500, 64, "f16", True, 0),      # more than one 32-row tile
    (1, 8, 2, 16, 700, 64, "bf16", True, 0),      # stacked heads: 64 rows, a tile holds two heads
    (1, 32, 1, 3, 1111, 128, "f16", True, 50),    # stacked MQA: heads wrap inside a 32-row tile
    (2, 8, 2, 17, 600, 128, "f16", True, 0),      # one row too many to stack
    (1, 2, 1, 300, 300, 128, "bf16", True, 0),    # square: the plain forward's function
    (1, 3, 3, 257, 257, 64, "f16", True, 64),
    # several 64-row query tiles below a longer cache: the 128-row
    # configuration pairs tiles r and n - 1 - r with a query offset
    (1, 2, 2, 333, 2000, 64, "f16", True, 0),
    (1, 4, 2, 200, 900, 128, "bf16", True, 0),
]


def case_id(c):
    return "B{}_Hq{}_Hkv{}_Nq{}_Nk{}_d{}_{}_c{}_w{}".format(*c)


@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_splitkv_all_configs_and_chunk_counts(fa, case):
    B, Hq, Hkv, Nq, Nk, d, dt, causal, window = case
    q, k, v = qkv(B, Hq, Hkv, Nq, Nk, d, dt, seed=Nq * 7 + Nk)
    ro, rl = oracle_full(q, k, v, causal=causal, window=window)
    for cfg in CONFIGS:
        for splits in (0, 1, 2, 3, 1024):
            o, lse = run_gpu_splitkv(q, k, v, causal=causal, window=window, num_splits=splits, config_id=cfg)
            plan = fa.attn_fwd_splitkv_plan(B, Hq, Hkv, Nq, Nk, d, causal, window, 0 if dt == "f16" else 1,
                                            splits, cfg)
            check(f"cfg{cfg} splits={splits}->{plan['n_splits']}", o, lse, ro, rl, dt)


def test_splitkv_unknown_config_rejected(fa):
    q, k, v = qkv(1, 2, 2, 1, 100, 64, "f16", seed=1)
    with pytest.raises(fa.AttnError) as e:
        run_gpu_splitkv(q, k, v, causal=True, config_id=fa.attn_fwd_num_configs())
    assert e.value.status == 4


def test_window_one_is_last_value_row(fa):
    q, k, v = qkv(1, 4, 2, 3, 700, 128, "bf16", seed=2)
    o, _ = run_gpu_splitkv(q, k, v, causal=True, window=1, num_splits=5)
    want = v.repeat_interleave(2, dim=1)[:, :, -3:, :]
    assert torch.equal(o, want)


def test_square_split_matches_plain_forward(fa):
    """With Nq = Nk the split path computes the plain forward's function; both
    meet the oracle, and differ from each other only by rounding."""
    q, k, v = qkv(2, 4, 4, 1024, 1024, 64, "f16", seed=3)
    for causal in (False, True):
        o1, l1 = run_gpu(q, k, v, causal=causal)
        o2, l2 = run_gpu_splitkv(q, k, v, causal=causal, num_splits=4)
        ro, rl = oracle_full(q, k, v, causal=causal)
        check(f"plain causal={causal}", o1, l1, ro, rl, "f16")
        check(f"split causal={causal}", o2, l2, ro, rl, "f16")
        assert (o1.float() - o2.float()).abs().max().item() < 2e-3


def test_workspace_reuse_and_determinism(fa):
    """Two calls in a row on one workspace (the second with other shapes and
    fewer chunks), then the first again: the results do not depend on what
    the workspace held, and repeat bit for bit."""
    dev = torch.device("cuda:0")
    ws = torch.full((1 << 22,), 0xFF, dtype=torch.uint8, device=dev)
    a = qkv(1, 8, 2, 1, 4096, 128, "bf16", seed=4)
    b = qkv(2, 4, 4, 2, 1000, 64, "f16", seed=5)
    o1, l1 = run_gpu_splitkv(*a, causal=True, num_splits=16, workspace=ws)
    o2, l2 = run_gpu_splitkv(*b, causal=True, num_splits=3, workspace=ws)
    o3, l3 = run_gpu_splitkv(*a, causal=True, num_splits=16, workspace=ws)
    ra = oracle_full(*a, causal=True)
    rb = oracle_full(*b, causal=True)
    check("first", o1, l1, *ra, "bf16")
    check("second", o2, l2, *rb, "f16")
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_workspace_guard_bands(fa):
    """The kernels write only the documented workspace bytes and outputs."""
    import flashattention_forward_05_amd as fa_mod
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 2, 900, 64
    q, k, v = qkv(B, Hq, Hkv, Nq, Nk, d, "f16", seed=6)
    need = fa_mod.attn_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, 1, 0, 0, 5, -1)
    assert need > 0
    dev = torch.device("cuda:0")
    pad = 4096
    wbuf = torch.full((need + 2 * pad,), 0x5A, dtype=torch.uint8, device=dev)
    obuf = torch.full((B * Hq * Nq * d + 2 * pad,), 7.0, dtype=torch.float16, device=dev)
    o = obuf[pad:pad + B * Hq * Nq * d]
    lse = torch.empty(B * Hq * Nq, dtype=torch.float32, device=dev)
    fa_mod.attn_fwd_splitkv_ex(q.to(dev), k.to(dev), v.to(dev), o, lse, B, Hq, Hkv, Nq, Nk, d, 1, 0, 0.125,
                               0, 5, -1, wbuf[pad:pad + need], need)
    torch.cuda.synchronize()
    assert (wbuf[:pad] == 0x5A).all() and (wbuf[pad + need:] == 0x5A).all()
    assert (obuf[:pad] == 7.0).all() and (obuf[-pad:] == 7.0).all()
    ro, rl = oracle_full(q, k, v, causal=True, scale=0.125)
    check("guarded", o.view(B, Hq, Nq, d).cpu(), lse.view(B, Hq, Nq).cpu(), ro, rl, "f16")


# ---- the decoding workloads, whole output (one query row per head), in the
# launch configuration the benchmark times (the automatic choice)
@pytest.mark.parametrize("name", ["decode_gqa", "decode_mqa", "decode_mqa_window"])
def test_decode_workloads(fa, name):
    w = WORKLOADS[name]
    say(f"  generating {w.label()}")
    q, k, v = make_workload(w, seed=0)
    o, lse = run_gpu_splitkv(q, k, v, causal=w.causal, window=w.window)
    ro, rl = oracle_full(q, k, v, causal=w.causal, window=w.window)
    plan = fa.attn_fwd_splitkv_plan(w.B, w.Hq, w.Hkv, w.N, w.nk, w.d, w.causal, w.window, 1)
    check(f"{name} ({plan['n_splits']} chunks)", o, lse, ro, rl, w.dtype)


def test_flash_attn_forward_splitkv_wrapper(fa):
    q, k, v = qkv(1, 8, 2, 4, 2000, 128, "bf16", seed=7)
    o, lse = fa.flash_attn_forward_splitkv(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle_full(q, k, v, causal=True)
    check("wrapper", o.cpu(), lse.cpu(), ro, rl, "bf16")


def test_splitkv_random_shapes(fa):
    """Seeded random shapes, masks, chunk counts and configurations."""
    rng = np.random.default_rng(1234)
    for n in range(16):
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["f16", "bf16"]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 3))
        Nk = int(rng.integers(1, 2500))
        Nq = int(min(Nk, rng.choice([1, 2, 5, 16, 17, 40, 100])))
        causal = bool(rng.integers(0, 4) > 0)
        window = int(rng.choice([0, 0, 1, 7, 300])) if causal else 0
        splits = int(rng.choice([0, 1, 2, 5, 64]))
        cfg = int(rng.choice([-1, 0, 1, 2, 3]))
        q, k, v = qkv(B, G * Hkv, Hkv, Nq, Nk, d, dt, seed=100 + n)
        ro, rl = oracle_full(q, k, v, causal=causal, window=window)
        o, lse = run_gpu_splitkv(q, k, v, causal=causal, window=window, num_splits=splits, config_id=cfg)
        check(f"#{n} B{B} Hq{G * Hkv}/{Hkv} Nq{Nq} Nk{Nk} d{d} {dt} c{int(causal)} w{window} s{splits} cfg{cfg}",
              o, lse, ro, rl, dt)


# ---- the score profiles of make_score_pattern: with scores rising by 120
# along the keys the later chunks outweigh the earlier ones by about e^120,
# with falling scores the reverse, and spikes sit on chunk edges; the merge's
# rescale ("Optimizaciones de Atencion", section "FlashDecoding") must take
# partial results whose maxima differ that much.  Decoding (4 new rows, two
# query heads stacked on one K/V head) and square shapes.
@pytest.mark.parametrize("pattern", SCORE_PATTERNS)
@pytest.mark.parametrize("d,dt", [(64, "f16"), (128, "bf16")])
def test_splitkv_score_patterns(fa, pattern, d, dt):
    N = 1000
    q, k, v = make_score_pattern(pattern, N, d, dt, seed=31)
    for nq in (4, N):
        qq = q[:, :, N - nq:].contiguous()
        ro, rl = oracle_full(qq, k, v, causal=True)
        for cfg, splits in ((-1, 0), (-1, 2), (-1, 7), (3, 40), (0, 5)):
            o, lse = run_gpu_splitkv(qq, k, v, causal=True, num_splits=splits, config_id=cfg)
            check(f"split-KV {pattern} Nq{nq} Nk{N} d{d} {dt} cfg{cfg} splits{splits}", o, lse, ro, rl, dt)
