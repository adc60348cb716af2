"""The benchmark's FLOP and byte accounting, pinned to the figures the pages
print (tests/golden/page_figures.json) and to brute-force counts.

Every TFLOP/s, roofline fraction and traffic ratio bench.py reports rests on
metric_flops, visible_keys and algorithmic_bytes; the pages' byte models
(page_naive_score_bytes, page_tiled_bytes) are reported beside them.
"""
import json
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_figures.json")
MIB, GIB = float(1 << 20), float(1 << 30)


@pytest.fixture(scope="module")
def fig():
    with open(GOLDEN) as f:
        return json.load(f)


def test_attention_flops_one_head(fig):
    # "00 - Por que la atencion domina la inferencia": 4 N^2 d ~ 1.07 GFLOP at N=2048, d=64
    g = fig["attention_flops_one_head"]
    got = bench.metric_flops(1, 1, g["N"], g["d"], False)
    assert abs(got - g["page_value"]) <= g["rel_tol"] * g["page_value"]
    assert bench.metric_flops(1, 1, g["N"], g["d"], True) == got / 2


def test_naive_and_tiled_traffic(fig):
    # the same page: 16 N^2 B (64 MiB) for the fp32 score matrix, ~16 FLOP/B;
    # N d (3 + 2 N / B_c) * 4 B (33 MiB) for the tiled kernel, ~30 FLOP/B
    n = fig["naive_score_traffic_bytes"]
    naive = bench.page_naive_score_bytes(n["N"])
    assert abs(naive / MIB - n["page_value_mib"]) <= n["rel_tol"] * n["page_value_mib"]
    flops = bench.metric_flops(1, 1, fig["attention_flops_one_head"]["N"], fig["attention_flops_one_head"]["d"], False)
    ni = fig["naive_intensity_flop_per_byte"]
    assert abs(flops / naive - ni["page_value"]) <= ni["rel_tol"] * ni["page_value"]
    t = fig["flash_traffic_bytes"]
    tiled = bench.page_tiled_bytes(t["N"], t["d"], t["B_c"])
    assert abs(tiled / MIB - t["page_value_mib"]) <= t["rel_tol"] * t["page_value_mib"]
    fi = fig["flash_intensity_flop_per_byte"]
    assert abs(flops / tiled - fi["page_value"]) <= fi["rel_tol"] * fi["page_value"]


def test_fp16_score_matrix_sizes(fig):
    # "Optimizaciones de Atencion": an fp16 score matrix per head is ~2 GiB at
    # 32K tokens and ~32 GiB at 128K (one of the four passes of the naive model)
    for e in fig["fp16_score_matrix_bytes"]:
        got = bench.page_naive_score_bytes(e["s"], elem=2) / 4 / GIB
        assert abs(got - e["page_value_gib"]) <= e["rel_tol"] * e["page_value_gib"]


def brute_pairs(N, causal, window, Nk=None):
    Nk = N if Nk is None else Nk
    n = 0
    for i in range(N):
        pos = Nk - N + i
        for j in range(Nk):
            if causal and j > pos:
                continue
            if window > 0 and pos - j >= window:
                continue
            n += 1
    return n


@pytest.mark.parametrize("N,causal,window", [(1, False, 0), (7, False, 0), (64, True, 0), (100, True, 0),
                                             (100, True, 1), (100, True, 13), (100, True, 99), (100, True, 100),
                                             (100, True, 250), (33, True, 32)])
def test_visible_pairs_brute_force(N, causal, window):
    pairs = sum(bench.visible_keys(i, N, causal, window) for i in range(N))
    assert pairs == brute_pairs(N, causal, window)
    if window > 0 and window < N:
        # the windowed metric counts exactly the visible pairs
        assert bench.metric_flops(1, 1, N, 1, True, window) == 4 * pairs
    if causal and window == 0 and N >= 64:
        # the causal metric is the stated N^2 / 2, within 1.6% of the exact pairs
        assert abs(bench.metric_flops(1, 1, N, 1, True) / 4 - pairs) <= 0.016 * pairs


@pytest.mark.parametrize("Nq,Nk,causal,window", [(1, 300, True, 0), (3, 300, True, 7), (5, 300, False, 0),
                                                  (300, 300, True, 0)])
def test_decode_pairs_brute_force(Nq, Nk, causal, window):
    assert sum(bench.visible_keys(i, Nq, causal, window, Nk) for i in range(Nq)) == brute_pairs(Nq, causal, window, Nk)


class W:
    def __init__(self, B, Hq, Hkv, N, d, causal, window, nk=None):
        self.B, self.Hq, self.Hkv, self.N, self.d, self.causal, self.window = B, Hq, Hkv, N, d, causal, window
        self.nk = N if nk is None else nk


@pytest.mark.parametrize("w", [W(2, 4, 4, 50, 64, False, 0), W(1, 8, 2, 77, 128, True, 0),
                               W(1, 4, 1, 90, 64, True, 10), W(2, 8, 2, 3, 128, True, 0, nk=200),
                               W(1, 4, 4, 2, 64, True, 30, nk=100)])
def test_algorithmic_bytes_brute_force(w):
    # every Q element read and O element written once (2 bytes), every K/V row
    # some query sees read once per K/V head (2 bytes per element), one fp32
    # LSE per query row
    seen = set()
    for i in range(w.N):
        pos = w.nk - w.N + i
        for j in range(w.nk):
            if w.causal and j > pos:
                continue
            if w.window > 0 and pos - j >= w.window:
                continue
            seen.add(j)
    want = (2 * w.B * w.Hq * w.N * w.d * 2 + 2 * w.B * w.Hkv * len(seen) * w.d * 2 + 4 * w.B * w.Hq * w.N)
    assert bench.algorithmic_bytes(w) == want
