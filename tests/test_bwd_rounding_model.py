"""The backward rounding model (bwd_rounding_model) against the fp64 oracle,
on the CPU: it must be a model of the same gradients (within a few u of the
oracle over each whole tensor, so no term is missing or misplaced), and on
the inputs where the per-slice cancellation is worst it must show that
cancellation, which is what lets the GPU tests bound a slice by the model's
own error instead of a fixed multiple of u."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from attn_inputs import make_dout, make_qkv, to_bits
from bwd_rounding_model import model_bwd, oracle_forward_inputs

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def model_and_ref(B, Hq, Hkv, N, d, dtype, causal, window, scale, seed):
    q, k, v = make_qkv(B, Hq, Hkv, N, d, dtype, seed=seed)
    do = make_dout(B, Hq, N, d, dtype, seed=seed)
    s = float(np.float32(scale if scale is not None else 1.0 / math.sqrt(d)))
    ref = oracle.oracle_bwd(to_bits(q), to_bits(k), to_bits(v), to_bits(do), scale=s, causal=causal,
                            window=window, dtype=dtype)
    o, lse = oracle_forward_inputs(q, k, v, scale=s, causal=causal, window=window, dtype=dtype)
    return model_bwd(q, k, v, do, o, lse, scale=s, causal=causal, window=window, dtype=dtype), ref


@pytest.mark.parametrize("case", [
    (2, 4, 4, 130, 64, "f16", True, 0, None, 1),
    (1, 4, 2, 97, 128, "bf16", True, 33, None, 2),
    (1, 4, 1, 80, 128, "bf16", False, 0, 0.3, 3),
    (1, 2, 2, 70, 64, "f16", True, 0, -0.1, 4),
])
def test_model_tracks_oracle(case):
    dtype = case[5]
    m, ref = model_and_ref(*case)
    for name, a, r in zip(("dq", "dk", "dv"), m, ref):
        rel = np.abs(a - r).max() / np.abs(r).max()
        assert rel < 2 * U[dtype], f"{case}: model {name} {rel / U[dtype]:.2f} u of max|ref|"


def test_model_window_one_is_zero():
    # one visible key per row: P = 1, O = v, so dS and the exact dq, dk vanish
    m, ref = model_and_ref(1, 2, 1, 40, 64, "bf16", True, 1, None, 5)
    assert np.abs(ref[0]).max() == 0 and np.abs(ref[1]).max() == 0
    assert np.abs(m[0]).max() < 1e-4 and np.abs(m[1]).max() < 1e-4
    assert np.abs(m[2] - ref[2]).max() < 2 * U["bf16"] * np.abs(ref[2]).max()


def test_model_slice_cancellation():
    # a 2-key window at scale 0.2: dk of some keys is mostly rounding of dS
    m, ref = model_and_ref(2, 2, 2, 157, 128, "bf16", True, 2, 0.2, 7015)
    r = ref[1].reshape(-1, 128)
    e = np.abs(m[1].reshape(-1, 128) - r).max(-1)
    den = np.maximum(np.abs(r).max(-1), 0.05 * np.abs(r).max())
    worst = (e / den).max() / U["bf16"]
    assert 25 < worst < 40, worst
