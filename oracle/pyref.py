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
* ``split_kv_attention`` -- the three steps of "Optimizaciones de Atencion",
  section "FlashDecoding": cut the keys into P chunks of about s/P tokens, form
  per chunk a local softmax (local max m_p, local sum l_p) and the partial
  output normalised within the chunk, then merge: global max m = max_p m_p,
  each partial output weighted by exp(m_p - m) * l_p, divided by the sum of
  those weights.  The method is exact, so this must equal
  ``batch_attention`` up to rounding; the tests check that.

Masking reading used throughout: causal keeps j <= i; a window W > 0 further
keeps i - j < W; a row with no visible key gives o = 0 and lse = -inf.  With
fewer queries than keys (nq < nk, decoding) query row i sits at position
nk - nq + i and the masks apply to that position (the pages leave the
alignment open; bottom-right is the reading taken).
"""
from __future__ import annotations

import math

NEG_INF = float("-inf")


def visible(i: int, j: int, causal: bool, window: int, offset: int = 0) -> bool:
    """Key j is visible from query row i, which sits at position i + offset."""
    pos = i + offset
    if causal and j > pos:
        return False
    if window > 0 and pos - j >= window:
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
    """One head.  Q (nq, d), K and V (nk, d).  Returns (O, LSE)."""
    n = len(Q)
    off = len(K) - n
    out, lse = [], []
    for i in range(n):
        js = [j for j in range(len(K)) if visible(i, j, causal, window, off)]
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
                js = [j for j in range(k0, min(k0 + block_k, len(K))) if visible(i, j, causal, window, len(K) - n)]
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


def split_kv_attention(Q, K, V, scale: float, n_splits: int,
                       causal: bool = False, window: int = 0):
    """One head, keys cut into n_splits chunks of ceil(nk / n_splits) tokens
    (trailing chunks may be empty); partial softmax per chunk, then the merge.
    Returns (O, LSE)."""
    nq, nk, d = len(Q), len(K), len(V[0])
    off = nk - nq
    size = -(-nk // n_splits) if nk else 0
    out, lse = [], []
    for i in range(nq):
        parts = []          # (m_p, l_p, partial output normalised by l_p)
        for p in range(n_splits):
            js = [j for j in range(p * size, min((p + 1) * size, nk)) if visible(i, j, causal, window, off)]
            if not js:
                parts.append((NEG_INF, 0.0, [0.0] * d))
                continue
            s = [scale * math.fsum(a * b for a, b in zip(Q[i], K[j])) for j in js]
            m_p = max(s)
            e = [math.exp(x - m_p) for x in s]
            l_p = math.fsum(e)
            o_p = [math.fsum(e[t] * V[j][c] for t, j in enumerate(js)) / l_p for c in range(d)]
            parts.append((m_p, l_p, o_p))
        m = max(mp for mp, _, _ in parts)
        if m == NEG_INF:
            out.append([0.0] * d)
            lse.append(NEG_INF)
            continue
        w = [math.exp(mp - m) * lp if lp > 0.0 else 0.0 for mp, lp, _ in parts]
        total = math.fsum(w)
        out.append([math.fsum(w[p] * parts[p][2][c] for p in range(n_splits)) / total for c in range(d)])
        lse.append(m + math.log(total))
    return out, lse
