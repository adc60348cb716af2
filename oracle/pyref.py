"""Pure-Python attention references for tiny inputs (TEST INFRASTRUCTURE ONLY).

Matrices are lists of rows of Python floats.  These exist to pin the C oracle
to things other than itself:

* ``batch_attention`` -- the plain definition (scores, mask, row softmax,
  weighted V sum, log-sum-exp) with every sum taken by ``math.fsum`` (exactly
  rounded), following "Lab 02 - Forward de flash attention en Triton",
  "Bloque C", and the standard branch of the demo in "Optimizaciones de
  Atencion", section "FlashAttention: Nunca materializar la matriz de
  atencion".
* ``online_attention`` -- the tiled computation that same demo checks: the
  keys of a row are taken one block at a time, and what a block contributes
  (its own max, its sum of exponentials against that max, its unnormalised
  weighted sum of V rows) is folded into the row's result so far.  The fold
  is the associative merge of two such triples, both re-based to the larger
  max (``merge_partials``); that re-basing is the recurrence of the page's
  running max and running sum, written here as a binary operator rather than
  an in-place update.  The page states that the tiled and standard results
  agree to below 1e-10; the tests check this against ``batch_attention`` and
  the C oracle.
* ``batch_softmax`` / ``online_softmax`` -- the one-vector identity behind the
  recurrence ("Fase 27 - Optimizaciones de atencion moderna", reading order,
  lab 00: an online softmax in pure Python must equal the batch softmax),
  the latter with the same merge on (max, sum) pairs.
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


def merge_partials(a, b):
    """Merge two partial softmax results (m, l, o) of disjoint key sets into the
    result of their union: m is a max of scores, l the sum of exp(score - m)
    and o (a list, possibly empty) the sum of exp(score - m) * value.  Both
    sides are re-based to the larger max; an empty side has m = -inf and
    contributes nothing.  The merge is associative and commutative."""
    ma, la, oa = a
    mb, lb, ob = b
    if mb == NEG_INF:
        return a
    if ma == NEG_INF:
        return b
    m = max(ma, mb)
    fa, fb = math.exp(ma - m), math.exp(mb - m)
    return m, la * fa + lb * fb, [x * fa + y * fb for x, y in zip(oa, ob)]


EMPTY = (NEG_INF, 0.0, [])


def online_softmax(xs, block: int):
    """Softmax of xs built from per-block (max, sum of exponentials) pairs,
    folded left to right with ``merge_partials``; the exponentials are then
    taken against the final max."""
    state = EMPTY
    for start in range(0, len(xs), block):
        chunk = xs[start:start + block]
        mb = max(chunk)
        state = merge_partials(state, (mb, math.fsum(math.exp(x - mb) for x in chunk), []))
    m, total, _ = state
    return [math.exp(x - m) / total for x in xs]


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


def _block_partial(q, K, V, js, scale: float):
    """(m, l, o) of one query row over the keys js: the block's own max score,
    its sum of exp(score - m) and its unnormalised weighted sum of V rows."""
    d = len(V[0])
    if not js:
        return NEG_INF, 0.0, [0.0] * d
    s = [scale * sum(a * b for a, b in zip(q, K[j])) for j in js]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    return m, math.fsum(w), [math.fsum(w[t] * V[j][c] for t, j in enumerate(js)) for c in range(d)]


def online_attention(Q, K, V, scale: float, block_q: int, block_k: int,
                     causal: bool = False, window: int = 0):
    """One head, tiled: query rows in blocks of block_q, keys in blocks of
    block_k.  Each row's result is the left fold of ``merge_partials`` over its
    key blocks' partials, then o / l and m + ln l.  Returns (O, LSE)."""
    n, nk, d = len(Q), len(K), len(V[0])
    off = nk - n
    key_blocks = [range(k0, min(k0 + block_k, nk)) for k0 in range(0, nk, block_k)]
    out, lse = [], []
    for q0 in range(0, n, block_q):
        for i in range(q0, min(q0 + block_q, n)):
            state = (NEG_INF, 0.0, [0.0] * d)
            for blk in key_blocks:
                js = [j for j in blk if visible(i, j, causal, window, off)]
                state = merge_partials(state, _block_partial(Q[i], K, V, js, scale))
            m, total, o = state
            if total > 0.0:
                out.append([x / total for x in o])
                lse.append(m + math.log(total))
            else:
                out.append([0.0] * d)
                lse.append(NEG_INF)
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
