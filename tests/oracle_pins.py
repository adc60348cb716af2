"""Pins of the fp64 oracle to things other than itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load_library``)
and raises AssertionError when the oracle disagrees with what the pages or the
mathematics fix.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with a planted
mistake and requires that some pin catch each one.

Kinds of pin used: exact library conversions (decoders), a worked example the
pages state (the tiled-vs-standard demo), closed forms derived by hand, special
cases that reduce to a plain mean or to one V row, invariants of softmax
(translation, permutation, normalisation, weight ratios), an equivalence that
fixes the GQA head map, brute force with exactly rounded sums, and the pages'
naive PyTorch recipe run in float64 on the CPU.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import pyref
from attn_inputs import make_dout, make_qkv, sine_matrix, to_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def lib_decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode bit patterns with library conversions (numpy float16, torch
    bfloat16), independent of the oracle's own decoders."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def run(lib, q, k, v, scale, causal=False, window=0, dtype="f64"):
    return oracle.oracle_fwd(q, k, v, scale=scale, causal=causal, window=window,
                             dtype=dtype, lib=lib)


def visible_lists(N: int, causal: bool, window: int):
    return [[j for j in range(N) if pyref.visible(i, j, causal, window)] for i in range(N)]


def close(a, b, tol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(same_inf, 0.0, np.abs(a - b))
    worst = float(np.nanmax(err)) if err.size else 0.0
    assert not np.isnan(err).any(), f"{what}: NaN mismatch"
    assert worst <= tol, f"{what}: max abs diff {worst:.3e} > {tol:.1e}"


MASKS = [(False, 0), (True, 0), (True, 1), (True, 3), (True, 7)]


# ---------------------------------------------------------------------------
def pin_decoders(lib):
    """Every fp16 and bf16 bit pattern decodes to what numpy/torch say."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dtype in ("f16", "bf16"):
        want = lib_decode(pats, dtype)
        got = np.array([lib.attn_oracle_decode(int(p), oracle.DTYPES[dtype]) for p in pats])
        nan = np.isnan(want)
        assert (np.isnan(got) == nan).all(), f"{dtype}: NaN patterns differ"
        assert (got[~nan] == want[~nan]).all(), f"{dtype}: decoded values differ"


def pin_tiled_demo(lib):
    """The demo of "Optimizaciones de Atencion": with its inputs the tiled
    online-softmax result equals the standard one to below 1e-10; the oracle
    must agree with both at that bound."""
    g = golden("tiled_demo.json")
    s, dk, blk, amp = g["s"], g["d_k"], g["block"], g["amplitude"]
    Q = sine_matrix(s, dk, g["seeds"]["Q"], amp)
    K = sine_matrix(s, dk, g["seeds"]["K"], amp)
    V = sine_matrix(s, dk, g["seeds"]["V"], amp)
    scale = 1.0 / math.sqrt(dk)
    tiled_o, tiled_lse = pyref.online_attention(Q, K, V, scale, blk, blk)
    std_o, _ = pyref.batch_attention(Q, K, V, scale)
    close(tiled_o, std_o, g["max_abs_diff_below"], "demo tiled vs standard (pure Python)")
    # the oracle receives the fp32-rounded scale, so feed the same to pyref
    scale32 = float(np.float32(scale))
    tiled_o, tiled_lse = pyref.online_attention(Q, K, V, scale32, blk, blk)
    o, lse = run(lib, f64(Q)[None, None], f64(K)[None, None], f64(V)[None, None], scale32)
    close(o[0, 0], tiled_o, g["max_abs_diff_below"], "demo oracle vs tiled")
    close(lse[0, 0], tiled_lse, g["max_abs_diff_below"], "demo oracle lse vs tiled")


def pin_two_key_closed_form(lib):
    """Hand-derived: d=1, keys ln(3)/scale and 0, values 4 and 8.
    Row 0 (q=1) weighs the keys 3:1, so o = 3/4*4 + 1/4*8 = 5, lse = ln 4.
    Row 1 (q=0) weighs them 1:1, so o = 6, lse = ln 2.  Causal: row 0 sees
    only key 0, so o = 4 and lse = ln 3."""
    for scale in (1.0, 0.5, 0.25):
        q = f64([[[[1.0], [0.0]]]])
        k = f64([[[[math.log(3.0) / scale], [0.0]]]])
        v = f64([[[[4.0], [8.0]]]])
        o, lse = run(lib, q, k, v, scale)
        close(o[0, 0, :, 0], [5.0, 6.0], 1e-14, f"two-key o, scale {scale}")
        close(lse[0, 0], [math.log(4.0), math.log(2.0)], 1e-14, f"two-key lse, scale {scale}")
        o, lse = run(lib, q, k, v, scale, causal=True)
        close(o[0, 0, :, 0], [4.0, 6.0], 1e-14, f"two-key causal o, scale {scale}")
        close(lse[0, 0], [math.log(3.0), math.log(2.0)], 1e-14, f"two-key causal lse, scale {scale}")
    # negative scale flips which key dominates: weights 1:3
    q = f64([[[[1.0], [0.0]]]])
    k = f64([[[[math.log(3.0)], [0.0]]]])
    v = f64([[[[4.0], [8.0]]]])
    o, lse = run(lib, q, k, v, -1.0)
    close(o[0, 0, :, 0], [1.0 + 6.0, 6.0], 1e-14, "two-key negative scale o")
    close(lse[0, 0], [math.log(4.0 / 3.0), math.log(2.0)], 1e-14, "two-key negative scale lse")


def pin_zero_scores_give_visible_mean(lib):
    """Q = 0 (or scale = 0): every visible key has score 0, so o_i is the mean
    of the visible V rows and lse_i = ln(number of visible keys)."""
    B, H, N, d = 2, 3, 37, 8
    for dtype in ("f16", "bf16"):
        q, k, v = (to_bits(t) for t in make_qkv(B, H, H, N, d, dtype, seed=11))
        vd = lib_decode(v, dtype)
        zero_q = np.zeros_like(q)
        for causal, window in MASKS:
            vis = visible_lists(N, causal, window)
            want_o = np.stack([vd[:, :, js, :].mean(axis=2) for js in vis], axis=2)
            want_lse = np.broadcast_to(np.log([len(js) for js in vis]), (B, H, N))
            for qq, sc in ((zero_q, 0.125), (q, 0.0)):
                o, lse = run(lib, qq, k, v, sc, causal, window, dtype)
                close(o, want_o, 1e-12, f"{dtype} mean o causal={causal} W={window}")
                close(lse, want_lse, 1e-12, f"{dtype} mean lse causal={causal} W={window}")


def pin_single_visible_key(lib):
    """Causal row 0 and every row under a width-1 window see one key: o_i is
    that V row exactly and lse_i is its scaled score."""
    B, H, N, d = 1, 2, 19, 16
    scale = 0.3
    for dtype in ("f16", "bf16"):
        q, k, v = (to_bits(t) for t in make_qkv(B, H, H, N, d, dtype, seed=5))
        qd, kd, vd = (lib_decode(x, dtype) for x in (q, k, v))
        s_self = np.array([[[scale32(scale) * math.fsum(qd[b, h, i] * kd[b, h, i]) for i in range(N)]
                            for h in range(H)] for b in range(B)])
        o, lse = run(lib, q, k, v, scale32(scale), True, 0, dtype)
        close(o[:, :, 0], vd[:, :, 0], 0.0, f"{dtype} causal row 0 o")
        close(lse[:, :, 0], s_self[:, :, 0], 1e-12, f"{dtype} causal row 0 lse")
        o, lse = run(lib, q, k, v, scale32(scale), True, 1, dtype)
        close(o, vd, 0.0, f"{dtype} window 1 o")
        close(lse, s_self, 1e-12, f"{dtype} window 1 lse")


def scale32(x: float) -> float:
    return float(np.float32(x))


def pin_wide_window_is_causal(lib):
    """A window at least N wide hides nothing beyond the causal mask."""
    q, k, v = (to_bits(t) for t in make_qkv(1, 2, 2, 23, 8, "f16", seed=3))
    base = run(lib, q, k, v, 0.35, True, 0, "f16")
    for w in (23, 24, 1000):
        got = run(lib, q, k, v, 0.35, True, w, "f16")
        close(got[0], base[0], 0.0, f"W={w} o")
        close(got[1], base[1], 0.0, f"W={w} lse")


def pin_softmax_rows(lib):
    """V = ones gives o = 1.  V = identity (d >= N) exposes the softmax rows
    in o: non-negative, summing to 1, exactly 0 where masked, and with weight
    ratios exp(s_ij - s_ik) for the scores s = scale * q.k."""
    B, H, N, d = 1, 2, 12, 16
    scale = scale32(0.4)
    q, k, _ = (to_bits(t) for t in make_qkv(B, H, H, N, d, "f16", seed=21))
    qd, kd = lib_decode(q, "f16"), lib_decode(k, "f16")
    ones = np.full((B, H, N, d), 0x3C00, np.uint16)            # fp16 1.0
    eye = np.zeros((B, H, N, d), np.uint16)
    for j in range(N):
        eye[:, :, j, j] = 0x3C00
    for causal, window in MASKS:
        o, _ = run(lib, q, k, ones, scale, causal, window, "f16")
        close(o, np.ones_like(o), 1e-14, f"V=1 causal={causal} W={window}")
        p, _ = run(lib, q, k, eye, scale, causal, window, "f16")
        assert (p >= 0).all()
        close(p[..., N:], np.zeros_like(p[..., N:]), 0.0, "columns past N")
        close(p[..., :N].sum(-1), np.ones((B, H, N)), 1e-14, f"row sums causal={causal} W={window}")
        vis = visible_lists(N, causal, window)
        for b in range(B):
            for h in range(H):
                for i in range(N):
                    js = vis[i]
                    hidden = [j for j in range(N) if j not in js]
                    assert (p[b, h, i, hidden] == 0).all(), "masked weight not zero"
                    s = [scale * math.fsum(qd[b, h, i] * kd[b, h, j]) for j in js]
                    ratio = np.log(p[b, h, i, js]) - math.log(p[b, h, i, js[0]])
                    close(ratio, np.array(s) - s[0], 1e-12, "weight ratios")


def pin_key_permutation(lib):
    """Without a mask, permuting K and V rows together changes nothing."""
    rng = np.random.default_rng(7)
    q, k, v = (to_bits(t) for t in make_qkv(2, 2, 2, 29, 16, "bf16", seed=8))
    o, lse = run(lib, q, k, v, 0.25, dtype="bf16")
    perm = rng.permutation(29)
    o2, lse2 = run(lib, q, np.ascontiguousarray(k[:, :, perm]), np.ascontiguousarray(v[:, :, perm]),
                   0.25, dtype="bf16")
    close(o2, o, 1e-13, "permuted o")
    close(lse2, lse, 1e-13, "permuted lse")


def pin_score_shift(lib):
    """With a constant column c in K (value kappa), adding delta to column c
    of q adds scale*delta*kappa to every score of that row: o is unchanged and
    lse shifts by that amount."""
    rng = np.random.default_rng(3)
    B, H, N, d, c, kappa, delta, scale = 1, 2, 17, 8, 5, 0.75, 1.5, 0.5
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    k[..., c] = kappa
    for causal, window in MASKS:
        o, lse = run(lib, f64(q), f64(k), f64(v), scale, causal, window)
        q2 = q.copy()
        q2[..., c] += delta
        o2, lse2 = run(lib, f64(q2), f64(k), f64(v), scale, causal, window)
        close(o2, o, 1e-13, "shifted o")
        close(lse2 - lse, np.full_like(lse, scale * delta * kappa), 1e-12, "shifted lse")


def pin_gqa_head_map(lib):
    """GQA with G query heads per K/V head equals MHA with every K/V head
    repeated G times contiguously (kv head = floor(h / G))."""
    B, Hq, Hkv, N, d = 2, 6, 2, 21, 16
    q, k, v = (to_bits(t) for t in make_qkv(B, Hq, Hkv, N, d, "f16", seed=4))
    G = Hq // Hkv
    k_rep = np.ascontiguousarray(np.repeat(k, G, axis=1))
    v_rep = np.ascontiguousarray(np.repeat(v, G, axis=1))
    for causal, window in MASKS:
        o, lse = run(lib, q, k, v, 0.25, causal, window, "f16")
        o2, lse2 = run(lib, q, k_rep, v_rep, 0.25, causal, window, "f16")
        close(o, o2, 0.0, "gqa o")
        close(lse, lse2, 0.0, "gqa lse")
    # MQA: one K/V head for all query heads
    q1, k1, v1 = (to_bits(t) for t in make_qkv(1, 4, 1, 9, 8, "bf16", seed=9))
    o, lse = run(lib, q1, k1, v1, 0.3, True, 0, "bf16")
    o2, lse2 = run(lib, q1, np.ascontiguousarray(np.repeat(k1, 4, 1)),
                   np.ascontiguousarray(np.repeat(v1, 4, 1)), 0.3, True, 0, "bf16")
    close(o, o2, 0.0, "mqa o")
    close(lse, lse2, 0.0, "mqa lse")


def pin_brute_force(lib):
    """Tiny random cases against the definition with exactly rounded sums."""
    cases = [(1, 2, 1, 1, 4), (1, 2, 2, 2, 8), (2, 4, 2, 7, 8), (1, 3, 1, 12, 5), (1, 2, 2, 16, 3)]
    for n_case, (B, Hq, Hkv, N, d) in enumerate(cases):
        for dtype in ("f16", "bf16"):
            q, k, v = (to_bits(t) for t in make_qkv(B, Hq, Hkv, N, d, dtype, seed=100 + n_case))
            qd, kd, vd = (lib_decode(x, dtype) for x in (q, k, v))
            scale = scale32(1.0 / math.sqrt(d))
            for causal, window in MASKS:
                o, lse = run(lib, q, k, v, scale, causal, window, dtype)
                for b in range(B):
                    for h in range(Hq):
                        hk = h // (Hq // Hkv)
                        want_o, want_lse = pyref.batch_attention(
                            qd[b, h].tolist(), kd[b, hk].tolist(), vd[b, hk].tolist(),
                            scale, causal, window)
                        close(o[b, h], want_o, 1e-13, f"brute o {dtype} {causal} {window}")
                        close(lse[b, h], want_lse, 1e-13, f"brute lse {dtype} {causal} {window}")


def torch_recipe(qd, kd, vd, scale, causal, window):
    """The naive recipe of "Lab 02", "Bloque C" in float64 on the CPU, with
    the window added as extra -inf entries; LSE via torch.logsumexp."""
    Q, K, V = (torch.from_numpy(x) for x in (qd, kd, vd))
    G = Q.shape[1] // K.shape[1]
    K = K.repeat_interleave(G, dim=1)
    V = V.repeat_interleave(G, dim=1)
    S = (Q @ K.transpose(-1, -2).contiguous()) * scale
    N = Q.shape[2]
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    hide = torch.zeros(N, N, dtype=torch.bool)
    if causal:
        hide |= j > i
    if window > 0:
        hide |= (i - j) >= window
    S = S.masked_fill(hide, float("-inf"))
    P = torch.softmax(S, dim=-1)
    return (P @ V).numpy(), torch.logsumexp(S, dim=-1).numpy()


def pin_torch_recipe(lib):
    """Moderate random cases against the pages' naive recipe in float64."""
    for (B, Hq, Hkv, N, d, dtype, seed) in [(2, 3, 3, 77, 64, "f16", 1), (1, 4, 2, 65, 128, "bf16", 2),
                                            (1, 2, 1, 130, 32, "f16", 3)]:
        q, k, v = (to_bits(t) for t in make_qkv(B, Hq, Hkv, N, d, dtype, seed=seed))
        qd, kd, vd = (lib_decode(x, dtype) for x in (q, k, v))
        scale = scale32(1.0 / math.sqrt(d))
        for causal, window in MASKS + [(True, 40)]:
            o, lse = run(lib, q, k, v, scale, causal, window, dtype)
            want_o, want_lse = torch_recipe(qd, kd, vd, scale, causal, window)
            close(o, want_o, 1e-12, f"recipe o {dtype} causal={causal} W={window}")
            close(lse, want_lse, 1e-12, f"recipe lse {dtype} causal={causal} W={window}")


def pin_row_entry(lib):
    """Selected-row entry gives exactly the rows of the full forward."""
    B, Hq, Hkv, N, d = 2, 4, 2, 33, 16
    q, k, v = (to_bits(t) for t in make_qkv(B, Hq, Hkv, N, d, "bf16", seed=6))
    rng = np.random.default_rng(0)
    ids = rng.choice(B * Hq * N, size=40, replace=False)
    for causal, window in MASKS:
        o, lse = run(lib, q, k, v, 0.2, causal, window, "bf16")
        ro, rlse = oracle.oracle_rows(q, k, v, ids, scale=0.2, causal=causal, window=window,
                                      dtype="bf16", lib=lib)
        close(ro, o.reshape(-1, d)[ids], 0.0, "rows o")
        close(rlse, lse.reshape(-1)[ids], 0.0, "rows lse")


def pin_online_matches_oracle(lib):
    """The tiled online recurrence (several block shapes, masks) agrees with
    the oracle on random fp16 input."""
    B, H, N, d = 1, 1, 13, 6
    q, k, v = (to_bits(t) for t in make_qkv(B, H, H, N, d, "f16", seed=31))
    qd, kd, vd = (lib_decode(x, "f16")[0, 0].tolist() for x in (q, k, v))
    scale = scale32(0.45)
    for causal, window in MASKS:
        o, lse = run(lib, q, k, v, scale, causal, window, "f16")
        for bq, bk in ((1, 1), (2, 3), (4, 4), (13, 5), (5, 13)):
            to, tl = pyref.online_attention(qd, kd, vd, scale, bq, bk, causal, window)
            close(o[0, 0], to, 1e-13, f"online o blocks {bq}x{bk}")
            close(lse[0, 0], tl, 1e-13, f"online lse blocks {bq}x{bk}")


def pin_large_scores(lib):
    """Scores far beyond exp()'s range must still give the exact softmax, as
    the stable form that subtracts the row max does: keys 0, 800, -800, 799
    with q = 1 give o = (v1 + e^-1 v3) / (1 + e^-1) up to terms of e^-799, and
    lse = 800 + ln(1 + e^-1)."""
    q = f64([[[[1.0]]]])
    k = f64([[[[0.0], [800.0], [-800.0], [799.0]]]])
    v = f64([[[[1.0], [2.0], [3.0], [5.0]]]])
    q4 = f64(np.repeat(q, 4, axis=2))
    o, lse = run(lib, q4, k, v, 1.0)
    w = math.exp(-1.0)
    close(o[0, 0, :, 0], [(2.0 + 5.0 * w) / (1.0 + w)] * 4, 1e-13, "large-score o")
    close(lse[0, 0], [800.0 + math.log1p(w)] * 4, 1e-12, "large-score lse")


def pin_decode_is_tail_of_square(lib):
    """Nq < Nk: the queries are the last Nq positions.  The result must equal
    the last Nq rows of the square Nk x Nk forward whose last Nq query rows
    are these queries (every mask, GQA, both dtypes)."""
    for (B, Hq, Hkv, Nq, Nk, d, dtype, seed) in [(2, 4, 2, 3, 29, 16, "f16", 41),
                                                 (1, 2, 1, 1, 40, 8, "bf16", 42),
                                                 (1, 3, 3, 7, 7, 8, "f16", 43)]:
        qf, k, v = (to_bits(t) for t in make_qkv(B, Hq, Hkv, Nk, d, dtype, seed=seed))
        q = np.ascontiguousarray(qf[:, :, Nk - Nq:, :])
        for causal, window in MASKS + [(True, 40)]:
            o, lse = run(lib, q, k, v, 0.3, causal, window, dtype)
            of, lf = run(lib, qf, k, v, 0.3, causal, window, dtype)
            close(o, of[:, :, Nk - Nq:, :], 0.0, f"tail o causal={causal} W={window}")
            close(lse, lf[:, :, Nk - Nq:], 0.0, f"tail lse causal={causal} W={window}")


def pin_decode_brute_force(lib):
    """Nq < Nk against the definition with exactly rounded sums, and the
    closed form for zero scores: the mean of the visible V rows (the last
    min(W, pos + 1) keys of row position pos) with LSE = ln(count)."""
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 3, 11, 8
    q, k, v = (to_bits(t) for t in make_qkv(B, Hq, Hkv, Nq, d, "f16", seed=44, nk=Nk))
    qd, kd, vd = (lib_decode(x, "f16") for x in (q, k, v))
    for causal, window in MASKS:
        o, lse = run(lib, q, k, v, 0.35, causal, window, "f16")
        for b in range(B):
            for h in range(Hq):
                hk = h // (Hq // Hkv)
                want_o, want_lse = pyref.batch_attention(qd[b, h].tolist(), kd[b, hk].tolist(),
                                                         vd[b, hk].tolist(), scale32(0.35), causal, window)
                close(o[b, h], want_o, 1e-13, f"decode brute o causal={causal} W={window}")
                close(lse[b, h], want_lse, 1e-13, f"decode brute lse causal={causal} W={window}")
        oz, lz = run(lib, q, k, v, 0.0, causal, window, "f16")
        for i in range(Nq):
            pos = Nk - Nq + i
            hi = pos if causal else Nk - 1
            lo = max(0, pos - window + 1) if window > 0 else 0
            close(oz[0, :, i, :], np.repeat(vd[0], Hq // Hkv, 0)[:, lo:hi + 1, :].mean(axis=1), 1e-14,
                  "decode zero-score mean")
            close(lz[0, :, i], [math.log(hi - lo + 1)] * Hq, 1e-14, "decode zero-score lse")


def pin_split_kv_merge(lib):
    """The chunked partial-softmax-and-merge of "Optimizaciones de Atencion",
    section "FlashDecoding", equals the plain definition for every chunk count
    (including more chunks than keys, so that some are empty), square and
    decoding shapes, every mask; and the oracle agrees with both."""
    for (nq, nk, d, seed) in [(1, 23, 6, 51), (4, 17, 5, 52), (9, 9, 4, 53)]:
        q, k, v = (to_bits(t) for t in make_qkv(1, 1, 1, nq, d, "bf16", seed=seed, nk=nk))
        qd, kd, vd = (lib_decode(x, "bf16")[0, 0].tolist() for x in (q, k, v))
        for causal, window in MASKS:
            o, lse = run(lib, q, k, v, 0.4, causal, window, "bf16")
            bo, bl = pyref.batch_attention(qd, kd, vd, scale32(0.4), causal, window)
            for n_splits in (1, 2, 3, 5, nk, nk + 3):
                so, sl = pyref.split_kv_attention(qd, kd, vd, scale32(0.4), n_splits, causal, window)
                close(so, bo, 1e-13, f"split o P={n_splits}")
                close(sl, bl, 1e-13, f"split lse P={n_splits}")
                close(o[0, 0], so, 1e-13, f"oracle vs split o P={n_splits}")
                close(lse[0, 0], sl, 1e-13, f"oracle vs split lse P={n_splits}")


def pin_paged_matches_contiguous(lib):
    """Walking a random page table gives exactly the result of the same keys
    laid out contiguously (ragged lengths per request, every mask, GQA, page
    sizes below and above the lengths); NaN-filled unused slots are never
    read."""
    from attn_inputs import make_paged_cache
    for (B, Hq, Hkv, Nq, lens, d, ps, dtype, seed) in [(3, 4, 2, 1, (37, 5, 64), 8, 16, "f16", 61),
                                                       (2, 2, 1, 3, (40, 17), 4, 8, "bf16", 62),
                                                       (1, 3, 3, 2, (9,), 8, 64, "f16", 63)]:
        nmax = max(lens)
        q, k, v = make_qkv(B, Hq, Hkv, Nq, d, dtype, seed=seed, nk=nmax)
        kp, vp, bt, sl = make_paged_cache(k, v, ps, lens, seed=seed)
        qb = to_bits(q)
        for causal, window in MASKS:
            o, lse = oracle.oracle_paged(qb, to_bits(kp), to_bits(vp), bt.numpy(), sl.numpy(), scale=0.3,
                                         causal=causal, window=window, dtype=dtype, lib=lib)
            assert np.isfinite(o).all()
            for b in range(B):
                kb = np.ascontiguousarray(to_bits(k)[b:b + 1, :, :lens[b]])
                vb = np.ascontiguousarray(to_bits(v)[b:b + 1, :, :lens[b]])
                ob, lb = run(lib, np.ascontiguousarray(qb[b:b + 1]), kb, vb, 0.3, causal, window, dtype)
                close(o[b:b + 1], ob, 0.0, f"paged o b={b} causal={causal} W={window}")
                close(lse[b:b + 1], lb, 0.0, f"paged lse b={b} causal={causal} W={window}")


def pin_paged_gather_order(lib):
    """Closed form that fixes the page walk: with K = 0 every visible key has
    the same weight, and V rows that encode (request, K/V head, key index)
    give O = the mean code over the visible keys of that request and head,
    LSE = ln(count).  A wrong page, slot or head shows up as a wrong mean."""
    B, Hq, Hkv, Nq, d, ps = 2, 4, 2, 2, 2, 8
    lens = (29, 11)
    nmax = max(lens)
    q = np.random.default_rng(5).standard_normal((B, Hq, Nq, d))
    k = torch.zeros((B, Hkv, nmax, d), dtype=torch.float64)
    v = torch.zeros((B, Hkv, nmax, d), dtype=torch.float64)
    for b in range(B):
        for hk in range(Hkv):
            for j in range(nmax):
                v[b, hk, j, 0] = 1000.0 * b + 100.0 * hk + j
                v[b, hk, j, 1] = j * j
    kp, vp, bt, sl = make_paged_cache_f64(k, v, ps, lens, seed=9)
    for causal, window in MASKS:
        o, lse = oracle.oracle_paged(f64(q), f64(kp), f64(vp), bt, sl, scale=0.7, causal=causal, window=window,
                                     dtype="f64", lib=lib)
        for b in range(B):
            for h in range(Hq):
                hk = h // (Hq // Hkv)
                for i in range(Nq):
                    pos = lens[b] - Nq + i
                    hi = pos if causal else lens[b] - 1
                    lo = max(0, pos - window + 1) if window > 0 else 0
                    js = list(range(lo, hi + 1))
                    want0 = sum(1000.0 * b + 100.0 * hk + j for j in js) / len(js)
                    want1 = sum(j * j for j in js) / len(js)
                    close([o[b, h, i, 0], o[b, h, i, 1]], [want0, want1], 1e-9, f"gather b={b} h={h} i={i}")
                    close([lse[b, h, i]], [math.log(len(js))], 1e-14, "gather lse")


def make_paged_cache_f64(k, v, ps, lens, seed):
    """make_paged_cache on float64 tensors, as numpy arrays."""
    from attn_inputs import make_paged_cache
    kp, vp, bt, sl = make_paged_cache(k, v, ps, lens, seed=seed)
    return kp.numpy(), vp.numpy(), bt.numpy(), sl.numpy()


# ---------------------------------------------------------------------------
# Backward: the gradients of sum(dO * O).  The pages leave the backward out of
# scope and print no formula for it, so every pin below is mathematics: finite
# differences of the (already pinned) forward, the chain rule run by torch
# autograd over the pages' naive recipe, a hand-derived closed form, and
# identities of the softmax Jacobian.

def run_bwd(lib, q, k, v, do, scale, causal=False, window=0, dtype="f64"):
    return oracle.oracle_bwd(q, k, v, do, scale=scale, causal=causal, window=window, dtype=dtype, lib=lib)


def _seeded_f64(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def pin_bwd_finite_differences(lib):
    """Central differences of L = sum(dO * O) through the forward oracle, one
    input element at a time, equal the backward oracle's gradients (error
    O(h^2) plus rounding, far below the tolerance)."""
    B, Hq, Hkv, N, d = 1, 2, 1, 5, 3
    q, k, v, do = (f64(_seeded_f64(s, 100 + i)) for i, s in enumerate(
        [(B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, Hq, N, d)]))
    scale, h = 0.7, 1e-5
    for causal, window in MASKS:
        dq, dk, dv = run_bwd(lib, q, k, v, do, scale, causal, window)
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                args_p[name], args_m[name] = xp, xm
                op, _ = run(lib, args_p["q"], args_p["k"], args_p["v"], scale, causal, window)
                om, _ = run(lib, args_m["q"], args_m["k"], args_m["v"], scale, causal, window)
                fd[idx] = ((op - om) * do).sum() / (2 * h)
            close(g, fd, 1e-7, f"finite differences d{name}, causal={causal} W={window}")


def pin_bwd_torch_autograd(lib):
    """The pages' naive recipe ("Lab 02", "Bloque C": Q K^T * scale, -inf
    mask, softmax, @ V) in torch float64 on the CPU, differentiated by
    autograd; K/V heads are repeated contiguously for GQA, so autograd sums
    dk and dv over each group.  Same bit patterns, both dtypes."""
    B, Hq, Hkv, N, d = 2, 4, 2, 19, 8
    for dtype in ("f16", "bf16"):
        q, k, v = (to_bits(t) for t in make_qkv(B, Hq, Hkv, N, d, dtype, seed=21))
        do = to_bits(make_dout(B, Hq, N, d, dtype, seed=22))
        scale = float(np.float32(1.0 / math.sqrt(d)))
        for causal, window in MASKS:
            tq, tk, tv = (torch.from_numpy(lib_decode(x, dtype)).requires_grad_() for x in (q, k, v))
            tdo = torch.from_numpy(lib_decode(do, dtype))
            kk = tk.repeat_interleave(Hq // Hkv, dim=1)
            vv = tv.repeat_interleave(Hq // Hkv, dim=1)
            s = (tq @ kk.transpose(-1, -2)) * scale
            i = torch.arange(N)[:, None]
            j = torch.arange(N)[None, :]
            hide = torch.zeros(N, N, dtype=torch.bool)
            if causal:
                hide |= j > i
            if window:
                hide |= (i - j) >= window
            o = torch.softmax(s.masked_fill(hide, float("-inf")), dim=-1) @ vv
            (o * tdo).sum().backward()
            dq, dk, dv = run_bwd(lib, q, k, v, do, scale, causal, window, dtype)
            what = f"{dtype} causal={causal} W={window}"
            close(dq, tq.grad.numpy(), 1e-12, f"autograd dq {what}")
            close(dk, tk.grad.numpy(), 1e-12, f"autograd dk {what}")
            close(dv, tv.grad.numpy(), 1e-12, f"autograd dv {what}")


def pin_bwd_two_key_closed_form(lib):
    """Hand-derived, d=1: q = (1, 0), k = (ln 3 / scale, 0), v = (4, 8),
    dO = (1, 2).  Row 0 weighs the keys 3:1: dP = (4, 8), D = 5,
    dS = (-3/4, 3/4), so dq_0 = -(3/4) ln 3, dk += scale * (-3/4, 3/4),
    dv += (3/4, 1/4).  Row 1 (q = 0) weighs them 1:1: dP = (8, 16), D = 12,
    dS = (-2, 2), dq_1 = -2 ln 3, dk += 0, dv += (1, 1).  Causal: row 0 sees
    key 0 alone, so dS = 0 and dv += (1, 0); row 1 is unchanged."""
    for scale in (1.0, 0.5, 0.25):
        q = f64([[[[1.0], [0.0]]]])
        k = f64([[[[math.log(3.0) / scale], [0.0]]]])
        v = f64([[[[4.0], [8.0]]]])
        do = f64([[[[1.0], [2.0]]]])
        dq, dk, dv = run_bwd(lib, q, k, v, do, scale)
        l3 = math.log(3.0)
        close(dq[0, 0, :, 0], [-0.75 * l3, -2.0 * l3], 1e-14, f"two-key dq, scale {scale}")
        close(dk[0, 0, :, 0], [-0.75 * scale, 0.75 * scale], 1e-14, f"two-key dk, scale {scale}")
        close(dv[0, 0, :, 0], [1.75, 1.25], 1e-14, f"two-key dv, scale {scale}")
        dq, dk, dv = run_bwd(lib, q, k, v, do, scale, causal=True)
        close(dq[0, 0, :, 0], [0.0, -2.0 * l3], 1e-14, f"two-key causal dq, scale {scale}")
        close(dk[0, 0, :, 0], [0.0, 0.0], 1e-14, f"two-key causal dk, scale {scale}")
        close(dv[0, 0, :, 0], [2.0, 1.0], 1e-14, f"two-key causal dv, scale {scale}")


def pin_bwd_identities(lib):
    """Identities of the softmax Jacobian, on GQA shapes under every mask:
    - rows of dS sum to 0, so sum_j dk_j = 0 for every (batch, K/V head);
    - rows of P sum to 1, so sum_j dv_j = sum over the group's rows of dO;
    - V rows all equal make dP constant along a row, so dq = dk = 0;
    - under W = 1 each row sees only itself: dq = dk = 0 and dv_j is the sum
      of dO row j over the group's heads."""
    B, Hq, Hkv, N, d = 2, 6, 2, 23, 8
    G = Hq // Hkv
    for dtype in ("f16", "bf16"):
        q, k, v = (to_bits(t) for t in make_qkv(B, Hq, Hkv, N, d, dtype, seed=31))
        do = to_bits(make_dout(B, Hq, N, d, dtype, seed=32))
        dod = lib_decode(do, dtype)
        group_do = dod.reshape(B, Hkv, G, N, d).sum(axis=2)
        scale = float(np.float32(1.0 / math.sqrt(d)))
        for causal, window in MASKS:
            what = f"{dtype} causal={causal} W={window}"
            dq, dk, dv = run_bwd(lib, q, k, v, do, scale, causal, window, dtype)
            close(dk.sum(axis=2), np.zeros((B, Hkv, d)), 1e-12, f"sum_j dk_j {what}")
            close(dv.sum(axis=2), group_do.sum(axis=2), 1e-11, f"sum_j dv_j {what}")
            vconst = np.ascontiguousarray(np.broadcast_to(v[:, :, :1, :], v.shape))
            dq, dk, dv = run_bwd(lib, q, k, vconst, do, scale, causal, window, dtype)
            close(dq, np.zeros_like(dq), 1e-12, f"constant V: dq {what}")
            close(dk, np.zeros_like(dk), 1e-12, f"constant V: dk {what}")
        dq, dk, dv = run_bwd(lib, q, k, v, do, scale, True, 1, dtype)
        close(dq, np.zeros_like(dq), 0.0, f"W=1 dq {dtype}")
        close(dk, np.zeros_like(dk), 0.0, f"W=1 dk {dtype}")
        close(dv, group_do, 1e-13, f"W=1 dv {dtype}")


def pin_bwd_sampled_entries(lib):
    """The per-row dq and per-key dk/dv entry points (used at full sizes)
    agree with the whole backward."""
    B, Hq, Hkv, N, d = 2, 4, 1, 29, 16
    q, k, v = (to_bits(t) for t in make_qkv(B, Hq, Hkv, N, d, "bf16", seed=41))
    do = to_bits(make_dout(B, Hq, N, d, "bf16", seed=42))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    rows = np.array([0, 5, N - 1, N + 3, 3 * N + 7, B * Hq * N - 1])
    keys = np.array([0, 1, N - 1, N + 2, B * Hkv * N - 1])
    for causal, window in MASKS:
        kw = dict(scale=scale, causal=causal, window=window, dtype="bf16", lib=lib)
        dq, dk, dv = oracle.oracle_bwd(q, k, v, do, **kw)
        what = f"causal={causal} W={window}"
        close(oracle.oracle_bwd_rows(q, k, v, do, rows, **kw), dq.reshape(-1, d)[rows], 1e-13, f"rows dq {what}")
        # the second set has only late keys: with a mask the key entry then
        # forms the normalisers of just the rows after them (any other row it
        # read would be NaN and show here)
        for ks in (keys, np.array([N - 3, N - 1, 2 * N - 5, 2 * N - 1])):
            sk, sv = oracle.oracle_bwd_keys(q, k, v, do, ks, **kw)
            close(sk, dk.reshape(-1, d)[ks], 1e-12, f"keys dk {what}")
            close(sv, dv.reshape(-1, d)[ks], 1e-12, f"keys dv {what}")


ALL_PINS = [
    pin_decoders,
    pin_tiled_demo,
    pin_two_key_closed_form,
    pin_zero_scores_give_visible_mean,
    pin_single_visible_key,
    pin_wide_window_is_causal,
    pin_softmax_rows,
    pin_key_permutation,
    pin_score_shift,
    pin_gqa_head_map,
    pin_brute_force,
    pin_torch_recipe,
    pin_row_entry,
    pin_online_matches_oracle,
    pin_large_scores,
    pin_decode_is_tail_of_square,
    pin_decode_brute_force,
    pin_split_kv_merge,
    pin_paged_matches_contiguous,
    pin_paged_gather_order,
    pin_bwd_finite_differences,
    pin_bwd_torch_autograd,
    pin_bwd_two_key_closed_form,
    pin_bwd_identities,
    pin_bwd_sampled_entries,
]
