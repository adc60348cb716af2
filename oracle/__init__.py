"""fp64 CPU oracle for exact scaled-dot-product attention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library
never imports, links or calls it, and it shares no code with the HIP library:
the two meet only in the seeded input generators of ``attn_inputs``.

``attn_oracle.c`` is the plain definition of attention in fp64 (naive scores,
mask, row softmax, weighted V sum, log-sum-exp), following "Lab 02 - Forward de
flash attention en Triton", section "Bloque C", and the standard branch of the
demo in "Optimizaciones de Atencion", section "FlashAttention: Nunca
materializar la matriz de atencion".  Its backward entry points are the
gradients of sum(dO * O) for that forward, written out by the chain rule
(the pages leave the backward out of scope and only say that it recomputes
the scores and uses the stored log-sum-exp).  ``pyref`` holds pure-Python versions for
tiny inputs: the same definition with exactly rounded sums, and the tiled
online-softmax recurrence of that demo, used to pin the C oracle.

Parity status of every function here is listed in the module docstrings of
``pyref`` and the tests that pin them; nothing in this package is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_attn.so")

DTYPES = {"f16": 0, "bf16": 1, "f64": 2}

_lib = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the C oracle with gcc (OpenMP, -O2, no fast-math)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, out)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.attn_oracle_fwd.restype = ctypes.c_int
    lib.attn_oracle_fwd.argtypes = [vp, vp, vp, dp, dp, i64, i64, i64, i64, i64,
                                    ctypes.c_int, i64, ctypes.c_float, ctypes.c_int]
    lib.attn_oracle_rows.restype = ctypes.c_int
    lib.attn_oracle_rows.argtypes = [vp, vp, vp, vp, i64, dp, dp, i64, i64, i64, i64, i64,
                                     ctypes.c_int, i64, ctypes.c_float, ctypes.c_int]
    lib.attn_oracle_fwd_qk.restype = ctypes.c_int
    lib.attn_oracle_fwd_qk.argtypes = [vp, vp, vp, dp, dp, i64, i64, i64, i64, i64, i64,
                                       ctypes.c_int, i64, ctypes.c_float, ctypes.c_int]
    lib.attn_oracle_rows_qk.restype = ctypes.c_int
    lib.attn_oracle_rows_qk.argtypes = [vp, vp, vp, vp, i64, dp, dp, i64, i64, i64, i64, i64, i64,
                                        ctypes.c_int, i64, ctypes.c_float, ctypes.c_int]
    lib.attn_oracle_fwd_paged.restype = ctypes.c_int
    lib.attn_oracle_fwd_paged.argtypes = [vp, vp, vp, vp, vp, dp, dp, i64, i64, i64, i64, i64, i64, i64, i64,
                                          ctypes.c_int, i64, ctypes.c_float, ctypes.c_int]
    lib.attn_oracle_bwd.restype = ctypes.c_int
    lib.attn_oracle_bwd.argtypes = [vp, vp, vp, vp, dp, dp, dp, i64, i64, i64, i64, i64,
                                    ctypes.c_int, i64, ctypes.c_float, ctypes.c_int]
    lib.attn_oracle_bwd_rows.restype = ctypes.c_int
    lib.attn_oracle_bwd_rows.argtypes = [vp, vp, vp, vp, vp, i64, dp, i64, i64, i64, i64, i64,
                                         ctypes.c_int, i64, ctypes.c_float, ctypes.c_int]
    lib.attn_oracle_bwd_keys.restype = ctypes.c_int
    lib.attn_oracle_bwd_keys.argtypes = [vp, vp, vp, vp, dp, dp, vp, i64, dp, dp, i64, i64, i64, i64, i64,
                                         ctypes.c_int, i64, ctypes.c_float, ctypes.c_int]
    lib.attn_oracle_decode.restype = ctypes.c_double
    lib.attn_oracle_decode.argtypes = [ctypes.c_uint16, ctypes.c_int]
    lib.attn_oracle_max_threads.restype = ctypes.c_int
    lib.attn_oracle_max_threads.argtypes = []
    return lib


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if absent or stale) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _as_input(x: np.ndarray, dtype: str) -> np.ndarray:
    want = np.float64 if dtype == "f64" else np.uint16
    if x.dtype != want:
        raise TypeError(f"oracle input for dtype {dtype} must be {np.dtype(want).name}, got {x.dtype}")
    return np.ascontiguousarray(x)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D (B, H, N, d)")
    B, Hq, Nq, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    Hkv, Nk = k.shape[1], k.shape[2]
    if Hkv < 1 or Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Nq, Nk, d


def oracle_fwd(q, k, v, *, scale: float, causal: bool = False, window: int = 0,
               dtype: str = "f16", lib: ctypes.CDLL | None = None):
    """Whole forward in fp64.  q (B,Hq,Nq,d), k/v (B,Hkv,Nk,d) as uint16 bit
    patterns (dtype "f16"/"bf16") or float64 ("f64").  With Nq < Nk the
    queries are the last Nq positions of the sequence (bottom-right causal
    alignment).  Returns (o, lse) as float64 arrays of shapes (B,Hq,Nq,d) and
    (B,Hq,Nq)."""
    lib = lib or load_library()
    q, k, v = (_as_input(x, dtype) for x in (q, k, v))
    B, Hq, Hkv, Nq, Nk, d = _check_shapes(q, k, v)
    o = np.zeros((B, Hq, Nq, d), np.float64)
    lse = np.zeros((B, Hq, Nq), np.float64)
    rc = lib.attn_oracle_fwd_qk(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                o.ctypes.data, lse.ctypes.data, B, Hq, Hkv, Nq, Nk, d,
                                int(bool(causal)), int(window), float(scale), DTYPES[dtype])
    if rc != 0:
        raise RuntimeError(f"attn_oracle_fwd failed with code {rc}")
    return o, lse


def oracle_rows(q, k, v, row_ids, *, scale: float, causal: bool = False, window: int = 0,
                dtype: str = "f16", lib: ctypes.CDLL | None = None):
    """Selected rows in fp64.  row_ids are flat (b*Hq + h)*Nq + i.  Returns
    (o (n, d), lse (n,)) as float64."""
    lib = lib or load_library()
    q, k, v = (_as_input(x, dtype) for x in (q, k, v))
    B, Hq, Hkv, Nq, Nk, d = _check_shapes(q, k, v)
    ids = np.ascontiguousarray(np.asarray(row_ids, dtype=np.int64))
    n = ids.shape[0]
    o = np.zeros((n, d), np.float64)
    lse = np.zeros((n,), np.float64)
    rc = lib.attn_oracle_rows_qk(q.ctypes.data, k.ctypes.data, v.ctypes.data, ids.ctypes.data, n,
                                 o.ctypes.data, lse.ctypes.data, B, Hq, Hkv, Nq, Nk, d,
                                 int(bool(causal)), int(window), float(scale), DTYPES[dtype])
    if rc != 0:
        raise RuntimeError(f"attn_oracle_rows failed with code {rc}")
    return o, lse


def oracle_paged(q, k_pool, v_pool, block_table, seq_lens, *, scale: float, causal: bool = False,
                 window: int = 0, dtype: str = "f16", lib: ctypes.CDLL | None = None):
    """Paged K/V forward in fp64.  q (B,Hq,Nq,d); pools (num_pages,Hkv,page_size,d)
    as uint16 bit patterns ("f16"/"bf16") or float64 ("f64"); block_table
    (B,max_pages) and seq_lens (B,) int32.  Returns (o (B,Hq,Nq,d), lse
    (B,Hq,Nq)) as float64."""
    lib = lib or load_library()
    q, k_pool, v_pool = (_as_input(x, dtype) for x in (q, k_pool, v_pool))
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B, Hq, Nq, d = q.shape
    num_pages, Hkv, page_size, dk = k_pool.shape
    if v_pool.shape != k_pool.shape or dk != d or bt.ndim != 2 or bt.shape[0] != B or sl.shape != (B,):
        raise ValueError("paged oracle: inconsistent shapes")
    o = np.zeros((B, Hq, Nq, d), np.float64)
    lse = np.zeros((B, Hq, Nq), np.float64)
    rc = lib.attn_oracle_fwd_paged(q.ctypes.data, k_pool.ctypes.data, v_pool.ctypes.data, bt.ctypes.data,
                                   sl.ctypes.data, o.ctypes.data, lse.ctypes.data, B, Hq, Hkv, Nq, d, page_size,
                                   num_pages, bt.shape[1], int(bool(causal)), int(window), float(scale),
                                   DTYPES[dtype])
    if rc != 0:
        raise RuntimeError(f"attn_oracle_fwd_paged failed with code {rc}")
    return o, lse


def oracle_bwd(q, k, v, dout, *, scale: float, causal: bool = False, window: int = 0,
               dtype: str = "f16", lib: ctypes.CDLL | None = None):
    """Whole backward in fp64: the gradients (dq, dk, dv) of sum(dout * O)
    for the forward O of ``oracle_fwd`` (Nq = Nk).  q and dout (B,Hq,N,d), k
    and v (B,Hkv,N,d), as uint16 bit patterns or float64.  dk and dv sum the
    contributions of every query head that shares a K/V head."""
    lib = lib or load_library()
    q, k, v, dout = (_as_input(x, dtype) for x in (q, k, v, dout))
    B, Hq, Hkv, Nq, Nk, d = _check_shapes(q, k, v)
    if Nq != Nk or dout.shape != q.shape:
        raise ValueError("backward oracle: needs Nq == Nk and dout shaped like q")
    dq = np.zeros(q.shape, np.float64)
    dk = np.zeros(k.shape, np.float64)
    dv = np.zeros(k.shape, np.float64)
    rc = lib.attn_oracle_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                             dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, B, Hq, Hkv, Nq, d,
                             int(bool(causal)), int(window), float(scale), DTYPES[dtype])
    if rc != 0:
        raise RuntimeError(f"attn_oracle_bwd failed with code {rc}")
    return dq, dk, dv


def oracle_bwd_rows(q, k, v, dout, row_ids, *, scale: float, causal: bool = False, window: int = 0,
                    dtype: str = "f16", lib: ctypes.CDLL | None = None):
    """dq of selected query rows (flat (b*Hq + h)*N + i), float64 (n, d)."""
    lib = lib or load_library()
    q, k, v, dout = (_as_input(x, dtype) for x in (q, k, v, dout))
    B, Hq, Hkv, Nq, Nk, d = _check_shapes(q, k, v)
    if Nq != Nk or dout.shape != q.shape:
        raise ValueError("backward oracle: needs Nq == Nk and dout shaped like q")
    ids = np.ascontiguousarray(np.asarray(row_ids, dtype=np.int64))
    dq = np.zeros((ids.shape[0], d), np.float64)
    rc = lib.attn_oracle_bwd_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                  ids.ctypes.data, ids.shape[0], dq.ctypes.data, B, Hq, Hkv, Nq, d,
                                  int(bool(causal)), int(window), float(scale), DTYPES[dtype])
    if rc != 0:
        raise RuntimeError(f"attn_oracle_bwd_rows failed with code {rc}")
    return dq


def _rows_seeing(keys_local, N: int, causal: bool, window: int) -> np.ndarray:
    """Query positions i (of a square N x N problem) that see at least one of
    the given key positions: every row without a mask; rows i >= j with the
    causal mask, and i < j + window with a window (visibility of the forward:
    0 <= i - j < window)."""
    if not causal:
        return np.arange(N, dtype=np.int64)
    seen = np.zeros(N, dtype=bool)
    for j in np.unique(keys_local):
        hi = N if window <= 0 else min(N, int(j) + window)
        seen[int(j):hi] = True
    return np.nonzero(seen)[0].astype(np.int64)


def oracle_bwd_keys(q, k, v, dout, key_ids, *, scale: float, causal: bool = False, window: int = 0,
                    dtype: str = "f16", lib: ctypes.CDLL | None = None):
    """dk and dv of selected keys (flat (b*Hkv + hk)*N + j), float64 (n, d)
    each.  A key's gradients need, for every query row that sees it, the row's
    log-sum-exp and the Jacobian term D = sum(dout * O); for each (batch, K/V
    head) that holds a selected key this forms them with the oracle's own
    forward over exactly those rows of that group's query heads (all rows
    without a mask; with a causal mask only rows at or after the earliest
    selected key, which keeps full-size checks of late keys cheap)."""
    lib = lib or load_library()
    q, k, v, dout = (_as_input(x, dtype) for x in (q, k, v, dout))
    B, Hq, Hkv, Nq, Nk, d = _check_shapes(q, k, v)
    if Nq != Nk or dout.shape != q.shape:
        raise ValueError("backward oracle: needs Nq == Nk and dout shaped like q")
    N, G = Nq, Hq // Hkv
    ids = np.asarray(key_ids, dtype=np.int64)
    if ids.size and (ids.min() < 0 or ids.max() >= B * Hkv * N):
        raise ValueError("key id out of range")
    dk = np.zeros((ids.shape[0], d), np.float64)
    dv = np.zeros((ids.shape[0], d), np.float64)
    table = None
    for grp in np.unique(ids // N):
        b, hk = divmod(int(grp), Hkv)
        sel = np.nonzero(ids // N == grp)[0]
        local = np.ascontiguousarray(ids[sel] % N)
        qs = np.ascontiguousarray(q[b:b + 1, hk * G:(hk + 1) * G])
        dos = np.ascontiguousarray(dout[b:b + 1, hk * G:(hk + 1) * G])
        ks = np.ascontiguousarray(k[b:b + 1, hk:hk + 1])
        vs = np.ascontiguousarray(v[b:b + 1, hk:hk + 1])
        pos = _rows_seeing(local, N, causal, window)
        rows = (np.arange(G, dtype=np.int64)[:, None] * N + pos[None, :]).reshape(-1)
        o, lse_rows = oracle_rows(qs, ks, vs, rows, scale=scale, causal=causal, window=window, dtype=dtype,
                                  lib=lib)
        if dtype == "f64":
            dof = dos.reshape(G * N, d)[rows]
        else:
            if table is None:
                table = np.array([lib.attn_oracle_decode(x, DTYPES[dtype]) for x in range(65536)], np.float64)
            dof = table[dos.reshape(G * N, d)[rows]]
        # the key routine reads lse and D only at rows that see a selected key
        lse = np.full(G * N, np.nan)
        drow = np.full(G * N, np.nan)
        lse[rows] = lse_rows
        drow[rows] = (dof * o).sum(-1)
        gk = np.zeros((sel.shape[0], d), np.float64)
        gv = np.zeros((sel.shape[0], d), np.float64)
        rc = lib.attn_oracle_bwd_keys(qs.ctypes.data, ks.ctypes.data, vs.ctypes.data, dos.ctypes.data,
                                      lse.ctypes.data, drow.ctypes.data, local.ctypes.data, local.shape[0],
                                      gk.ctypes.data, gv.ctypes.data, 1, G, 1, N, d,
                                      int(bool(causal)), int(window), float(scale), DTYPES[dtype])
        if rc != 0:
            raise RuntimeError(f"attn_oracle_bwd_keys failed with code {rc}")
        dk[sel], dv[sel] = gk, gv
    return dk, dv


def decode(bits: int, dtype: str, lib: ctypes.CDLL | None = None) -> float:
    """Exact value of one fp16/bf16 bit pattern, as the oracle decodes it."""
    lib = lib or load_library()
    return lib.attn_oracle_decode(int(bits) & 0xFFFF, DTYPES[dtype])


def max_threads(lib: ctypes.CDLL | None = None) -> int:
    lib = lib or load_library()
    return int(lib.attn_oracle_max_threads())
