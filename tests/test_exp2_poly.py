"""The polynomial 2^x of the forward's softmax (exp2_poly in
attn_fwd_common.hpp, used for a share of the steady-state exponentials when
the library is built with -DATTN_EXP2_POLY_EVERY=k), emulated step by step in
numpy float32 and checked against float64 exp2.

The kernel's steps: n = floor(x) (v_cvt_flr_i32_f32), f = fract(x) (v_fract_f32:
x - floor(x), at most the largest float below 1), a cubic in f by three fused
multiply-adds, then v_ldexp_f32(p, n).  The error bound that matters is the
relative error on the exponents the softmax feeds it: x = s*c - m is at most
15 on an accepted tile (every partial row sum stays <= 2^15) and is unbounded
below.  The bound asserted here is a quarter of the fp16 unit roundoff 2^-11,
so the 16-bit rounding of P, not the polynomial, sets the error of P.  No GPU
is used."""
from __future__ import annotations

import os
import re

import numpy as np

HEADER = os.path.join(os.path.dirname(__file__), os.pardir, "flashattention_forward_05_amd", "csrc",
                      "attn_fwd_common.hpp")
F32_BELOW_ONE = np.float32(np.nextafter(np.float32(1.0), np.float32(0.0)))


def coefficients() -> list[float]:
    """c3, c2, c1, c0 in Horner order, read from the kernel source."""
    src = open(HEADER).read()
    body = src[src.index("float exp2_poly(float x)"):]
    body = body[:body.index("}")]
    hexes = re.findall(r"(0x1\.[0-9a-f]+p-?\d+)f", body)
    assert len(hexes) == 4, hexes
    return [float.fromhex(h) for h in hexes]


def fma32(a: np.ndarray, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    """float32 fused multiply-add: the product of two floats is exact in
    float64, so one float64 add and a rounding to float32 (a double rounding
    that can differ from the hardware's single rounding by one ulp, far below
    the bounds tested)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def exp2_poly(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32)
    fl = np.floor(x)
    n = np.clip(fl, -2.0 ** 31, 2.0 ** 31 - 1).astype(np.int64)   # the conversion saturates
    f = np.minimum((x - fl).astype(np.float32), F32_BELOW_ONE)
    c3, c2, c1, c0 = (np.float32(c) for c in coefficients())
    p = fma32(np.full_like(f, c3), f, np.full_like(f, c2))
    p = fma32(p, f, np.full_like(f, c1))
    p = fma32(p, f, np.full_like(f, c0))
    return np.ldexp(p.astype(np.float64), n).astype(np.float32)


def test_relative_error_on_the_softmax_range():
    rng = np.random.default_rng(7)
    xs = [np.linspace(-125.0, 15.999, 2_000_001, dtype=np.float64).astype(np.float32),
          rng.uniform(-30.0, 16.0, 1_000_000).astype(np.float32)]
    # both sides of every integer, where f jumps from just below 1 to 0
    ints = np.arange(-125, 16, dtype=np.float32)
    xs.append(np.concatenate([np.nextafter(ints, np.float32(-1e9)), ints, np.nextafter(ints, np.float32(1e9))]))
    x = np.concatenate(xs)
    got = exp2_poly(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(got - ref) / ref
    worst = float(rel.max())
    assert worst < 7.6e-5, worst
    assert worst < 2.0 ** -11 / 4


def test_underflow_and_sign():
    x = np.array([-126.5, -140.0, -149.5, -150.0, -1000.0, -3.0e38], dtype=np.float32)
    got = exp2_poly(x)
    assert np.all(got >= 0)
    # below 2^-126 the result is denormal or zero: never more than 2^-125
    assert np.all(got <= 2.0 ** -125)
    assert got[-1] == 0.0 and got[-2] == 0.0


def test_exact_at_zero_within_bound_and_monotone_steps():
    # 2^0 = 1 to the bound; consecutive integers differ by a factor of 2
    # within twice the bound (the same polynomial value, scaled by ldexp)
    ints = np.arange(-20, 16, dtype=np.float32)
    got = exp2_poly(ints).astype(np.float64)
    assert np.all(np.abs(got / np.exp2(ints.astype(np.float64)) - 1) < 7.6e-5)
    assert np.all(np.abs(got[1:] / got[:-1] - 2.0) == 0.0)


def lawson_cubic(nodes: int = 4000, iters: int = 300) -> np.ndarray:
    """The fit the kernel's cubic comes from: least maximum relative error of
    a cubic against 2^f on [0, 1), by Lawson's iteration (weighted least
    squares, each weight multiplied by that node's error) on Chebyshev nodes.
    Returns c0 .. c3."""
    f = (np.cos(np.pi * (np.arange(nodes) + 0.5) / nodes) + 1) / 2
    y = 2.0 ** f
    a = np.vstack([f ** i for i in range(4)]).T
    w = np.ones(nodes) / nodes
    for _ in range(iters):
        sw = np.sqrt(w) / y
        c, *_ = np.linalg.lstsq(a * sw[:, None], y * sw, rcond=None)
        e = np.abs((a @ c - y) / y)
        w = w * e
        w /= w.sum()
    return c


def test_coefficients_are_the_lawson_fit():
    c3, c2, c1, c0 = coefficients()
    fit = lawson_cubic()
    np.testing.assert_allclose([c0, c1, c2, c3], fit, rtol=2e-6)
    # and they sit close to the Taylor terms of 2^f = sum (f ln 2)^k / k!
    ln2 = np.log(2.0)
    taylor = [1.0, ln2, ln2 ** 2 / 2, ln2 ** 3 / 6]
    assert np.all(np.abs(np.array([c0, c1, c2, c3]) - taylor) < 0.03)
