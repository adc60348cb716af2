"""How much the row sum of the softmax may move when it is taken over the
16-bit P that feeds the P.V products (one v_dot2 per packed pair) instead of
over the fp32 weights.

The kernel forms p = 2^(s*c - m) in fp32 against the running max m and packs
pairs of p to the value dtype for the MFMA.  Summing those packed pairs with a
dot product against (1, 1) halves the adds but sums rounded values.  This
emulates, in numpy, the forward's per-tile softmax steps (first tile: tile
max; later tiles: against the stale running max, accepted while a lane-half
sum stays <= 2^15, otherwise the tile max and a raise of m by more than 8) on
the seeded inputs of the paged fp16 parity cases, both ways, and checks the
resulting log-sum-exps against each other and against the fp64 value.

What it shows: each packed value carries a relative rounding error of at
most the unit roundoff u of the 16-bit format (2^-11 for fp16, 2^-8 for bf16)
and the fp32 accumulation adds far less, so ln of the sum moves by at most
about u.  For fp16 that is below the 1e-3 LSE tolerance by a factor of two;
a log-sum-exp error of 0.13 cannot come from summing rounded fp16 weights.
For bf16 the bound is above the tolerance, and rows dominated by a few keys
reach it, so bf16 keeps the fp32 sums.  No GPU is used."""
from __future__ import annotations

import math

import numpy as np
import pytest

from attn_inputs import make_qkv

TAU = 8.0
BN = 64


def round16(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 -> 16-bit -> fp32, round to nearest even (fp16 via numpy, bf16 by
    rounding the fp32 bit pattern to its upper 16 bits)."""
    x = x.astype(np.float32)
    if dtype == "f16":
        with np.errstate(over="ignore"):          # above 65504: inf, as the hardware pack gives
            return x.astype(np.float16).astype(np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def half_of_key(j: np.ndarray) -> np.ndarray:
    """Lane half (0 or 1) that holds key j of a 64-key tile in the score
    accumulator: key 32*kb + 16*(r/8) + 8*g + r%8 sits in half g."""
    return (j >> 3) & 1


def emulate_lse(s: np.ndarray, c: float, packed: str | None) -> np.ndarray:
    """Log-sum-exp (natural log) of each row of s (rows x keys, fp32 scores)
    by the kernel's tile steps.  packed=None sums the fp32 p; packed='f16' or
    'bf16' sums the rounded p in pairs with one fp32 rounding per pair."""
    rows, n = s.shape
    m = np.full(rows, -np.inf, dtype=np.float32)
    l = np.zeros(rows, dtype=np.float32)
    for j0 in range(0, n, BN):
        t = s[:, j0:j0 + BN].astype(np.float32)
        halves = half_of_key(np.arange(t.shape[1]))

        def tile_sum(p):
            if packed is None:
                q = p
            else:
                q = round16(p, packed)
            # pairs of consecutive keys per half, each pair one fp32 rounding
            tot = np.zeros((rows, 2), dtype=np.float32)
            for h in (0, 1):
                qh = q[:, halves == h]
                if qh.shape[1] % 2:
                    qh = np.concatenate([qh, np.zeros((rows, 1), np.float32)], axis=1)
                pairs = (qh[:, 0::2].astype(np.float64) + qh[:, 1::2]).astype(np.float32)
                acc = np.zeros(rows, dtype=np.float32)
                for k in range(pairs.shape[1]):
                    acc = (acc.astype(np.float64) + pairs[:, k]).astype(np.float32)
                tot[:, h] = acc
            return tot

        fast_ok = np.isfinite(m)
        p_fast = np.exp2((t * np.float32(c) - m[:, None]).astype(np.float32)).astype(np.float32)
        hs = tile_sum(np.where(fast_ok[:, None], p_fast, 0).astype(np.float32))
        accept = fast_ok & np.all(hs <= 32768.0, axis=1)
        # rejected rows: tile max, lazy raise of m, rescale of l
        mx = (t.max(axis=1) * np.float32(c)).astype(np.float32)
        need = ~accept & (mx > m + TAU)
        alpha = np.where(need & np.isfinite(m), np.exp2(m - mx), 1.0).astype(np.float32)
        l = np.where(need, l * alpha, l).astype(np.float32)
        m = np.where(need, mx, m).astype(np.float32)
        p_full = np.exp2((t * np.float32(c) - m[:, None]).astype(np.float32)).astype(np.float32)
        hf = tile_sum(p_full)
        rs = np.where(accept[:, None], hs, hf).sum(axis=1, dtype=np.float32)
        l = (l + rs).astype(np.float32)
    return (m.astype(np.float64) + np.log2(l.astype(np.float64))) * math.log(2.0)


def scores(q, k):
    """fp32 unscaled scores q.k of 16-bit inputs (fp32 accumulate, as the
    MFMA does); the kernel folds the scale into c."""
    return (q.astype(np.float64) @ k.astype(np.float64).T).astype(np.float32)


def exact_lse(q, k, scale):
    s = q.astype(np.float64) @ k.astype(np.float64).T * scale
    mx = s.max(axis=1, keepdims=True)
    return (mx[:, 0] + np.log(np.exp(s - mx).sum(axis=1)))


# query rows x keys of the paged fp16 parity cases (one K/V head each), plus
# the same shapes with the scores eight times sharper (rows dominated by a
# few keys: the worst case for the rounding of P)
CASES = [(1, 700, 64, 1.0), (5, 129, 128, 1.0), (1, 4100, 64, 1.0), (1, 90, 64, 1.0),
         (1, 700, 64, 8.0), (1, 4100, 64, 8.0)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_packed_rowsum_moves_lse_by_at_most_the_unit_roundoff(dtype):
    u = 2.0 ** -11 if dtype == "f16" else 2.0 ** -8
    worst = 0.0
    for nq, nk, d, sharp in CASES:
        q, k, _ = make_qkv(1, 4, 1, nq, d, dtype, seed=nk + d, nk=nk)
        qn = q.float().numpy().reshape(-1, d)           # 4 heads share the K/V head
        kn = k.float().numpy()[0, 0]
        scale = sharp / math.sqrt(d)
        s = scores(qn, kn)
        c = float(np.float32(scale * math.log2(math.e)))
        l32 = emulate_lse(s, c, None)
        l16 = emulate_lse(s, c, dtype)
        ref = exact_lse(qn, kn, scale)
        assert np.max(np.abs(l32 - ref)) < 1e-4            # the fp32 sums: the kernel as built
        diff = float(np.max(np.abs(l16 - l32)))
        worst = max(worst, diff)
        assert diff <= 1.05 * u, (nq, nk, d, sharp, diff)
    print(f"{dtype}: largest LSE change from summing packed P = {worst:.3e} (unit roundoff {u:.3e})")
    if dtype == "f16":
        assert worst < 1e-3 / 2            # far inside the LSE tolerance: cannot explain an error of 0.13
    else:
        assert worst > 1e-3                # beyond the LSE tolerance: bf16 keeps the fp32 sums
