"""Seeded synthetic inputs and the named workloads.

This module is the only code shared by the HIP path's tests/benchmark and the
CPU oracle: it draws inputs and describes shapes, and holds none of the
attention arithmetic.  Inputs are drawn on the host once, rounded to the
16-bit dtype, and the same bytes go to the GPU and (as bit patterns) to the
oracle.

Recipe: ``torch.Generator('cpu').manual_seed(seed)``; Q, K, V drawn in that
order with ``torch.randn(..., dtype=float32)`` (iid N(0,1)); multiplied by
``amplitude``; rounded to fp16/bf16 with ``.to(dtype)`` (round to nearest
even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """One attention-forward problem: shapes, dtype, masking and input scale."""
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str
    causal: bool
    window: int = 0
    amplitude: float = 1.0
    Nk: int = 0          # keys per head; 0 means N (N queries are then the last N positions)
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def nk(self) -> int:
        return self.Nk or self.N

    def label(self) -> str:
        mask = "causal" if self.causal else "full"
        if self.window:
            mask += f"_w{self.window}"
        n = f"N{self.N}" if self.nk == self.N else f"Nq{self.N}_Nk{self.nk}"
        return (f"{self.name}:B{self.B}_Hq{self.Hq}_Hkv{self.Hkv}_{n}_d{self.d}_"
                f"{self.dtype}_{mask}")


def _lab(N: int, causal: bool) -> Workload:
    return Workload("lab", 2, 4, 4, N, 64, "f16", causal,
                    note="Lab 02 (Triton flash forward), Bloque D correctness protocol")


# The pages' workloads (shapes from "Lab 02", "Bloque D"/"Condiciones de parada";
# the small-model anchor L=12, h=768, d=64, N=2048 of "00 - Por que la atencion
# domina la inferencia"; GQA/MQA and long context from the same pages).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 12, 12, 64, 64, "f16", True,
                     note="64-token anchor sequence, 12 heads of d=64"),
    **{f"lab_n{N}_{'causal' if c else 'full'}": _lab(N, c)
       for N in (256, 1000, 1024, 4096) for c in (False, True)},
    "stress_full": Workload("stress", 1, 12, 12, 2048, 64, "f16", False, amplitude=0.5,
                            note="small-model anchor scaled to N=2048, inputs x0.5"),
    "stress_causal": Workload("stress", 1, 12, 12, 2048, 64, "f16", True, amplitude=0.5,
                              note="small-model anchor scaled to N=2048, inputs x0.5"),
    "gqa": Workload("gqa", 4, 32, 8, 8192, 128, "bf16", True,
                    note="GQA prefill, 4 query heads per K/V head"),
    "mqa_window": Workload("mqa", 1, 32, 1, 32768, 128, "bf16", True, window=4096,
                           note="MQA long context, sliding window 4096"),
    "mqa_causal": Workload("mqa", 1, 32, 1, 32768, 128, "bf16", True,
                           note="MQA long context, full causal"),
    # decoding ("Optimizaciones de Atencion", section "FlashDecoding"): one new
    # query token per sequence against the cached K/V of the GQA and MQA shapes
    "decode_gqa": Workload("decode", 4, 32, 8, 1, 128, "bf16", True, Nk=8192,
                           note="GQA decode step: 1 query against 8192 cached keys"),
    "decode_mqa": Workload("decode", 1, 32, 1, 1, 128, "bf16", True, Nk=32768,
                           note="MQA decode step: 1 query against 32768 cached keys"),
    "decode_mqa_window": Workload("decode", 1, 32, 1, 1, 128, "bf16", True, window=4096, Nk=32768,
                                  note="MQA decode step with a 4096-token sliding window"),
}


def make_qkv(B: int, Hq: int, Hkv: int, N: int, d: int, dtype: str = "f16",
             seed: int = 0, amplitude: float = 1.0, nk: int | None = None):
    """Seeded host tensors q (B,Hq,N,d), k and v (B,Hkv,Nk,d) in fp16/bf16,
    with Nk = N unless nk is given (decoding shapes: N new queries against a
    cached sequence of nk keys)."""
    Nk = N if nk is None else int(nk)
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn(B, Hq, N, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, Hkv, Nk, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, Hkv, Nk, d, generator=g, dtype=torch.float32)
    if amplitude != 1.0:
        q, k, v = q * amplitude, k * amplitude, v * amplitude
    tdt = TORCH_DTYPES[dtype]
    return q.to(tdt).contiguous(), k.to(tdt).contiguous(), v.to(tdt).contiguous()


def make_dout(B: int, Hq: int, N: int, d: int, dtype: str = "f16", seed: int = 0,
              amplitude: float = 1.0) -> torch.Tensor:
    """Seeded upstream gradient dO (B,Hq,N,d) for the backward pass: iid
    N(0,1) times amplitude, rounded to the 16-bit dtype, drawn from its own
    generator (seed + 104729) so that it does not disturb the Q, K, V
    stream of the same seed."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 104729)
    do = torch.randn(B, Hq, N, d, generator=g, dtype=torch.float32)
    if amplitude != 1.0:
        do = do * amplitude
    return do.to(TORCH_DTYPES[dtype]).contiguous()


SCORE_PATTERNS = ("rising", "slow", "falling", "spikes")


def make_score_pattern(pattern: str, N: int, d: int, dtype: str = "f16", seed: int = 0, Hq: int = 2):
    """Host q (1,Hq,N,d), k and v (1,1,N,d) whose scores follow a set profile
    along the keys: every channel of q is about 1 and every channel of key j
    about target_j / sqrt(d), so with scale 1/sqrt(d) score (i, j) is about
    target_j, plus small noise; v is N(0,1).
      rising:  target grows by about 7.7 per 64 keys (0 .. 120 over N = 1000);
      slow:    it grows by about 2.6 per 64 keys (0 .. 40);
      falling: 120 .. 0, the first keys dominate;
      spikes:  0, except about 60 at keys 0, 63, 64, 127, 500, 501 and N-1."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    j = torch.arange(N, dtype=torch.float64)
    if pattern == "rising":
        target = 120.0 * j / N
    elif pattern == "slow":
        target = 40.0 * j / N
    elif pattern == "falling":
        target = 120.0 * (N - j) / N
    elif pattern == "spikes":
        target = torch.zeros(N, dtype=torch.float64)
        for s in (0, 63, 64, 127, 500, 501, N - 1):
            if s < N:
                target[s] = 60.0
    else:
        raise ValueError(f"unknown score pattern {pattern!r}")
    tdt = TORCH_DTYPES[dtype]
    q = (1.0 + 0.05 * torch.randn(1, Hq, N, d, generator=g, dtype=torch.float64)).to(tdt)
    k = (target[None, None, :, None] / math.sqrt(d)
         + 0.05 * torch.randn(1, 1, N, d, generator=g, dtype=torch.float64)).to(tdt)
    v = torch.randn(1, 1, N, d, generator=g, dtype=torch.float64).to(tdt)
    return q.contiguous(), k.contiguous(), v.contiguous()


def make_paged_cache(k: torch.Tensor, v: torch.Tensor, page_size: int, seq_lens, seed: int = 0,
                     spare_pages: int = 3):
    """Scatter contiguous host K/V (B, Hkv, Nmax, d) into page pools
    (num_pages, Hkv, page_size, d) through a seeded random page table, the
    layout of the paged forward: request b's keys 0 .. seq_lens[b]-1 fill
    ceil(seq_lens[b] / page_size) pages taken from a random permutation of
    the pool.  Slots past a request's length and spare pages hold NaN, so any
    read of them would show in the output; table entries past a request's
    pages are -1.  Returns (k_pool, v_pool, block_table int32 (B, max_pages),
    seq_lens int32 (B,))."""
    B, Hkv, nmax, d = k.shape
    lens = [int(x) for x in seq_lens]
    assert len(lens) == B and all(0 <= n <= nmax for n in lens)
    per = [-(-n // page_size) for n in lens]
    max_pages = max(1, -(-nmax // page_size))
    total = sum(per) + spare_pages
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 7919)
    perm = torch.randperm(total, generator=g).tolist()
    k_pool = torch.full((total, Hkv, page_size, d), float("nan"), dtype=k.dtype)
    v_pool = torch.full((total, Hkv, page_size, d), float("nan"), dtype=v.dtype)
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    n = 0
    for b in range(B):
        for pg in range(per[b]):
            page = perm[n]
            n += 1
            table[b, pg] = page
            lo, hi = pg * page_size, min((pg + 1) * page_size, lens[b])
            k_pool[page, :, :hi - lo] = k[b, :, lo:hi]
            v_pool[page, :, :hi - lo] = v[b, :, lo:hi]
    return k_pool.contiguous(), v_pool.contiguous(), table, torch.tensor(lens, dtype=torch.int32)


def make_workload(w: Workload, seed: int = 0):
    return make_qkv(w.B, w.Hq, w.Hkv, w.N, w.d, w.dtype, seed, w.amplitude,
                    nk=None if w.nk == w.N else w.nk)


def to_bits(t: torch.Tensor) -> np.ndarray:
    """The raw 16-bit patterns of a host fp16/bf16 tensor, as numpy uint16."""
    if t.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(f"expected fp16/bf16, got {t.dtype}")
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def sine_matrix(rows: int, cols: int, seed: float, amplitude: float = 0.5):
    """Deterministic input of the tiled-vs-standard demo in "Optimizaciones de
    Atencion" (section "FlashAttention: Nunca materializar la matriz de
    atencion"): entry (i, j) is amplitude * sin(seed + i*cols + j)."""
    return [[math.sin(seed + i * cols + j) * amplitude for j in range(cols)]
            for i in range(rows)]
