"""GPU parity of the paged K/V forward: queries against K/V kept in page pools
behind a per-request page table ("00 - Por que la atencion domina la
inferencia", section "PagedAttention es un problema distinto"), checked
through the C ABI against the fp64 oracle's page-table walk on the same bytes.
Unused pool slots and spare pages hold NaN, so a read of anything but a
request's own keys would show in the output."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from attn_inputs import SCORE_PATTERNS, WORKLOADS, make_paged_cache, make_qkv, make_score_pattern, make_workload, to_bits
from gpu_helpers import DT_CODE, check, need_gpu, run_gpu_splitkv, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    return need_gpu()


def run_gpu_paged(q, kp, vp, bt, sl, *, max_seq_len, causal, window=0, scale=None, num_splits=0, config_id=-1):
    import flashattention_forward_05_amd as fa
    B, Hq, Nq, d = q.shape
    num_pages, Hkv, ps, _ = kp.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dev = torch.device("cuda:0")
    qd, kd, vd, btd, sld = (t.to(dev) for t in (q, kp, vp, bt, sl))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=dev)
    dt = DT_CODE["f16" if q.dtype == torch.float16 else "bf16"]
    need = fa.attn_fwd_paged_workspace_size(B, Hq, Hkv, Nq, d, ps, num_pages, bt.shape[1], max_seq_len, causal,
                                            window, dt, num_splits, config_id)
    ws = torch.full((max(16, need),), 0xFF, dtype=torch.uint8, device=dev)
    fa.attn_fwd_paged_ex(qd, kd, vd, btd, sld, o, lse, B, Hq, Hkv, Nq, d, ps, num_pages, bt.shape[1], max_seq_len,
                         causal, window, scale, dt, num_splits, config_id, ws, ws.numel(),
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def oracle_paged(q, kp, vp, bt, sl, *, causal, window=0, scale=None):
    d = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dt = "f16" if q.dtype == torch.float16 else "bf16"
    return oracle.oracle_paged(to_bits(q), to_bits(kp), to_bits(vp), bt.numpy(), sl.numpy(),
                               scale=float(np.float32(scale)), causal=causal, window=window, dtype=dt)


# B, Hq, Hkv, Nq, lens, d, dtype, page_size, causal, window
CASES = [
    (3, 4, 2, 1, (1, 100, 700), 64, "f16", 16, True, 0),
    (2, 8, 2, 1, (1000, 333), 128, "bf16", 16, True, 0),
    (2, 32, 1, 2, (2048, 513), 128, "bf16", 32, True, 256),     # stacked MQA with a window
    (1, 4, 4, 3, (777,), 64, "bf16", 8, True, 0),
    (2, 4, 2, 5, (129, 64), 128, "f16", 64, False, 0),
    (2, 6, 3, 1, (4100, 90), 64, "f16", 256, True, 0),
    (1, 8, 2, 40, (1500,), 128, "bf16", 16, True, 0),            # a longer query block, not stacked
]


def case_id(c):
    return "B{}_Hq{}_Hkv{}_Nq{}_L{}_d{}_{}_ps{}_c{}_w{}".format(c[0], c[1], c[2], c[3], "-".join(map(str, c[4])),
                                                               *c[5:])


@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_paged_against_oracle(fa, case):
    B, Hq, Hkv, Nq, lens, d, dt, ps, causal, window = case
    nmax = max(lens)
    q, k, v = make_qkv(B, Hq, Hkv, Nq, d, dt, seed=nmax + Nq, nk=nmax)
    kp, vp, bt, sl = make_paged_cache(k, v, ps, lens, seed=nmax)
    ro, rl = oracle_paged(q, kp, vp, bt, sl, causal=causal, window=window)
    max_seq_len = bt.shape[1] * ps
    for cfg in (-1, 0, 1, 2, 3):
        for splits in (0, 1, 3):
            o, lse = run_gpu_paged(q, kp, vp, bt, sl, max_seq_len=max_seq_len, causal=causal, window=window,
                                   num_splits=splits, config_id=cfg)
            check(f"cfg{cfg} splits={splits}", o, lse, ro, rl, dt)


def test_paged_equals_contiguous_bitwise(fa):
    """Pages in any order, all requests of the full length: the same tiles,
    chunks and arithmetic as the contiguous split-KV call, so the same bits.
    (With a window the contiguous call starts its chunks at the window while
    the paged one, whose lengths vary per request, starts at key 0: different
    chunk boundaries, so agreement there is to rounding only.)"""
    B, Hq, Hkv, Nq, N, d = 2, 8, 2, 1, 1024, 128
    q, k, v = make_qkv(B, Hq, Hkv, Nq, d, "bf16", seed=21, nk=N)
    kp, vp, bt, sl = make_paged_cache(k, v, 16, (N, N), seed=21, spare_pages=0)
    for causal, window in ((True, 0), (False, 0), (True, 200)):
        o1, l1 = run_gpu_paged(q, kp, vp, bt, sl, max_seq_len=N, causal=causal, window=window, num_splits=4)
        o2, l2 = run_gpu_splitkv(q, k, v, causal=causal, window=window, num_splits=4)
        if window == 0:
            assert torch.equal(o1, o2) and torch.equal(l1, l2), (causal, window)
        else:
            assert (o1.float() - o2.float()).abs().max().item() < 1e-2
            assert (l1 - l2).abs().max().item() < 1e-5


def test_paged_empty_request(fa):
    """A request with no cached keys gets O = 0 and LSE = -inf; the others are
    unaffected."""
    B, Hq, Hkv, Nq, d = 2, 4, 2, 1, 64
    q, k, v = make_qkv(B, Hq, Hkv, Nq, d, "f16", seed=22, nk=300)
    kp, vp, bt, sl = make_paged_cache(k, v, 16, (0, 300), seed=22)
    o, lse = run_gpu_paged(q, kp, vp, bt, sl, max_seq_len=bt.shape[1] * 16, causal=False, num_splits=2)
    assert torch.equal(o[0], torch.zeros_like(o[0])) and bool(torch.isneginf(lse[0]).all())
    ro, rl = oracle_paged(q[1:], kp, vp, bt[1:], sl[1:], causal=False)
    check("second request", o[1:], lse[1:], ro, rl, "f16")


@pytest.mark.parametrize("name", ["decode_gqa", "decode_mqa_window"])
def test_paged_decode_workloads(fa, name):
    """The decoding workloads with their caches in 16-token pages."""
    w = WORKLOADS[name]
    say(f"  generating {w.label()} in 16-token pages")
    q, k, v = make_workload(w, seed=0)
    kp, vp, bt, sl = make_paged_cache(k, v, 16, [w.nk] * w.B, seed=0)
    o, lse = run_gpu_paged(q, kp, vp, bt, sl, max_seq_len=w.nk, causal=w.causal, window=w.window)
    ro, rl = oracle_paged(q, kp, vp, bt, sl, causal=w.causal, window=w.window)
    check(name + " paged", o, lse, ro, rl, w.dtype)


def test_flash_attn_forward_paged_wrapper(fa):
    q, k, v = make_qkv(2, 8, 2, 1, 128, "bf16", seed=23, nk=900)
    kp, vp, bt, sl = make_paged_cache(k, v, 16, (900, 411), seed=23)
    o, lse = fa.flash_attn_forward_paged(q.cuda(), kp.cuda(), vp.cuda(), bt.cuda(), sl.cuda(), causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle_paged(q, kp, vp, bt, sl, causal=True)
    check("wrapper", o.cpu(), lse.cpu(), ro, rl, "bf16")


def test_paged_random_shapes(fa):
    """Seeded random requests, page sizes, masks, chunk counts and configurations."""
    rng = np.random.default_rng(4321)
    for n in range(48):
        d = int(rng.choice([64, 128]))
        dt = str(rng.choice(["f16", "bf16"]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 4, 8]))
        B = int(rng.integers(1, 4))
        Nq = int(rng.choice([1, 2, 3, 7, 16, 31, 32, 33, 100]))
        lens = [int(x) for x in rng.integers(Nq, 1800, size=B)]
        ps = int(rng.choice([8, 16, 32, 64, 128, 256]))
        causal = bool(rng.integers(0, 4) > 0)
        window = int(rng.choice([0, 0, 1, 2, 50, 300])) if causal else 0
        splits = int(rng.choice([0, 1, 2, 3, 40]))
        cfg = int(rng.choice([-1, 0, 1, 2, 3, 4]))
        nmax = max(lens)
        q, k, v = make_qkv(B, G * Hkv, Hkv, Nq, d, dt, seed=200 + n, nk=nmax)
        kp, vp, bt, sl = make_paged_cache(k, v, ps, lens, seed=200 + n)
        ro, rl = oracle_paged(q, kp, vp, bt, sl, causal=causal, window=window)
        o, lse = run_gpu_paged(q, kp, vp, bt, sl, max_seq_len=bt.shape[1] * ps, causal=causal, window=window,
                               num_splits=splits, config_id=cfg)
        check(f"#{n} B{B} Hq{G * Hkv}/{Hkv} Nq{Nq} lens{lens} ps{ps} d{d} {dt} c{int(causal)} w{window} "
              f"s{splits} cfg{cfg}", o, lse, ro, rl, dt)


# ---- the score profiles of make_score_pattern behind a block table (pages in
# seeded random order): chunk maxima that differ by up to e^120 and spikes on
# page and chunk edges, for decoding rows against one request of 1000 keys
@pytest.mark.parametrize("pattern", SCORE_PATTERNS)
@pytest.mark.parametrize("d,dt", [(64, "f16"), (128, "bf16")])
def test_paged_score_patterns(fa, pattern, d, dt):
    N = 1000
    q, k, v = make_score_pattern(pattern, N, d, dt, seed=37)
    qq = q[:, :, N - 4:].contiguous()
    for ps, splits in ((16, 0), (64, 7), (256, 2)):
        kp, vp, bt, sl = make_paged_cache(k, v, ps, [N], seed=37 + ps)
        ro, rl = oracle_paged(qq, kp, vp, bt, sl, causal=True)
        o, lse = run_gpu_paged(qq, kp, vp, bt, sl, max_seq_len=bt.shape[1] * ps, causal=True, num_splits=splits)
        check(f"paged {pattern} ps{ps} splits{splits} d{d} {dt}", o, lse, ro, rl, dt)
