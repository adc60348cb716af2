"""Pure-Python attention references for tiny inputs (TEST INFRASTRUCTURE ONLY).

Matrices are lists of rows of Python floats.  These exist to pin the C oracle
to things other than itself:

* ``batch_attention`` -- the plain definition (scores, mask, row softmax,
  weighted V sum, log-sum-exp) with every sum taken by ``math.fsum`` (exactly
  rounded), following "Lab 02 - Forward de flash attention en Triton",
  "Bloque C", and the standard branch of the demo in "Optimizaciones de
  Atencion", section "FlashAttention: Nunca materializar la matriz de
  atencion".
* ``online_attention`` -- the tiled online-softmax recurrence of that same demo
  (Q blocks outer, K/V blocks inner, a running max and running sum per row,
  previous partial results multiplied by exp(old_max - new_max), which is taken
  as 0 while the old max is still -inf).  The page states that the tiled and
  standard results agree to below 1e-10; the tests check this recurrence
  against ``batch_attention`` and the C oracle.
* ``batch_softmax`` / ``online_softmax`` -- the one-vector identity behind the
  recurrence ("Fase 27 - Optimizaciones de atencion moderna", reading order,
  lab 00: an online softmax in pure Python must equal the batch softmax).

Masking reading used throughout: causal keeps j <= i; a window W > 0 further
keeps i - j < W; a row with no visible key gives o = 0 and lse = -inf.
"""
from __future__ import annotations

import math

NEG_INF = float("-inf")


def visible(i: int, j: int, causal: bool, window: int) -> bool:
    """Key j is visible from query row i."""
    if causal and j > i:
        return False
    if window > 0 and i - j >= window:
        return False
    return True


def batch_softmax(xs):
    """Row softmax with the row max subtracted first."""
    m = max(xs)
    es = [math.exp(x - m) for x in xs]
    total = math.fsum(es)
    return [e / total for e in es]


def online_softmax(xs, block: int):
    """Softmax of xs built block by block with a running max and running sum;
    the exponentials are re-based to the final max at the end."""
    run_max = NEG_INF
    run_sum = 0.0
    for start in range(0, len(xs), block):
        chunk = xs[start:start + block]
        new_max = max(run_max, max(chunk))
        corr = math.exp(run_max - new_max) if run_max != NEG_INF else 0.0
        run_sum = run_sum * corr + math.fsum(math.exp(x - new_max) for x in chunk)
        run_max = new_max
    return [math.exp(x - run_max) / run_sum for x in xs]


def batch_attention(Q, K, V, scale: float, causal: bool = False, window: int = 0):
    """One head.  Q (n, d), K and V (n, d).  Returns (O, LSE)."""
    n = len(Q)
    out, lse = [], []
    for i in range(n):
        js = [j for j in range(len(K)) if visible(i, j, causal, window)]
        if not js:
            out.append([0.0] * len(V[0]))
            lse.append(NEG_INF)
            continue
        s = [scale * math.fsum(a * b for a, b in zip(Q[i], K[j])) for j in js]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        total = math.fsum(e)
        out.append([math.fsum(e[t] * V[j][c] for t, j in enumerate(js)) / total
                    for c in range(len(V[0]))])
        lse.append(m + math.log(total))
    return out, lse


def online_attention(Q, K, V, scale: float, block_q: int, block_k: int,
                     causal: bool = False, window: int = 0):
    """One head, tiled: Q blocks outer, K/V blocks inner, online softmax per
    row.  Returns (O, LSE)."""
    n, d = len(Q), len(V[0])
    out = [[0.0] * d for _ in range(n)]
    lse = [NEG_INF] * n
    for q0 in range(0, n, block_q):
        rows = range(q0, min(q0 + block_q, n))
        run_max = {i: NEG_INF for i in rows}
        run_sum = {i: 0.0 for i in rows}
        acc = {i: [0.0] * d for i in rows}
        for k0 in range(0, len(K), block_k):
            for i in rows:
                js = [j for j in range(k0, min(k0 + block_k, len(K))) if visible(i, j, causal, window)]
                if not js:
                    continue
                scores = [scale * sum(a * b for a, b in zip(Q[i], K[j])) for j in js]
                new_max = max(run_max[i], max(scores))
                corr = math.exp(run_max[i] - new_max) if run_max[i] != NEG_INF else 0.0
                run_sum[i] *= corr
                acc[i] = [x * corr for x in acc[i]]
                for t, j in enumerate(js):
                    w = math.exp(scores[t] - new_max)
                    run_sum[i] += w
                    for c in range(d):
                        acc[i][c] += w * V[j][c]
                run_max[i] = new_max
        for i in rows:
            if run_sum[i] > 0.0:
                out[i] = [x / run_sum[i] for x in acc[i]]
                lse[i] = run_max[i] + math.log(run_sum[i])
    return out, lse
