"""A numpy model of where the backward kernels round, used to bound their
error element by element (test infrastructure only).

The kernels form the gradients of sum(dO * O) with the scores recomputed from
the forward's log-sum-exp ("Optimizaciones de Atencion", section
"FlashAttention: Nunca materializar la matriz de atencion": the backward
recomputes from the stored statistics).  They take the products in fp32 from
the 16-bit inputs, form D = rowsum(dO * O) from the O they are handed, P and
dS = P (dP - D) in fp32, round P and dS to the 16-bit type as matrix-product
operands, accumulate in fp32 and round each output once.  This model does the
same steps on the CPU from the same inputs (O and lse included).

Where the terms of a gradient cancel -- a key or row with few visible
partners, or a sharp softmax -- the rounding of dS can dominate that
gradient, so no fixed multiple of u bounds an element against its own size.
The model's error against the fp64 oracle measures that effect for the very
inputs of a test; the kernels are then held to a small multiple of it."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from attn_inputs import to_bits

LOG2E = 1.4426950408889634


def round16(x: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float16 if dtype == "f16" else torch.bfloat16).to(torch.float32).numpy()


def model_bwd(q, k, v, do, o, lse, *, scale: float, causal: bool, window: int, dtype: str):
    """(dq, dk, dv) as float64 arrays with the kernels' rounding points;
    q, do, o (B, Hq, N, d) and k, v (B, Hkv, N, d) 16-bit host tensors, lse
    (B, Hq, N) float32 natural log, as the backward receives them."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    s32 = np.float32(scale)
    O = o.float().numpy()
    L = lse.float().numpy()
    qf, kf, vf, dof = (t.float().numpy() for t in (q, k, v, do))
    kk = np.repeat(kf, G, axis=1)
    vv = np.repeat(vf, G, axis=1)
    S = np.matmul(qf, np.swapaxes(kk, -1, -2)).astype(np.float32)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = np.ones((N, N), dtype=bool)
    if causal:
        vis &= j <= i
    if window:
        vis &= (i - j) < window
    c2 = np.float32(float(s32) * LOG2E)
    with np.errstate(over="ignore"):           # masked scores may overflow; they are dropped
        P = np.where(vis, np.exp2(S * c2 - L[..., None] * np.float32(LOG2E)), 0.0).astype(np.float32)
    dP = np.matmul(dof, np.swapaxes(vv, -1, -2)).astype(np.float32)
    D = (dof * O).sum(-1, dtype=np.float32)
    dS = (P * (dP - D[..., None])).astype(np.float32)
    Pr = round16(P, dtype).astype(np.float64)
    dSr = round16(dS, dtype).astype(np.float64)
    dV = np.matmul(np.swapaxes(Pr, -1, -2), dof.astype(np.float64)).reshape(B, Hkv, G, N, d).sum(2)
    dK = float(s32) * np.matmul(np.swapaxes(dSr, -1, -2), qf.astype(np.float64)).reshape(B, Hkv, G, N, d).sum(2)
    dQ = float(s32) * np.matmul(dSr, kk.astype(np.float64))
    return tuple(round16(x, dtype).astype(np.float64) for x in (dQ, dK, dV))


def oracle_forward_inputs(q, k, v, *, scale: float, causal: bool, window: int, dtype: str):
    """The oracle's O rounded to the 16-bit type and its lse in float32: the
    best inputs a forward can hand the backward."""
    o64, lse64 = oracle.oracle_fwd(to_bits(q), to_bits(k), to_bits(v), scale=scale, causal=causal,
                                   window=window, dtype=dtype)
    o = torch.from_numpy(o64.astype(np.float32)).to(q.dtype)
    return o, torch.from_numpy(lse64.astype(np.float32))
