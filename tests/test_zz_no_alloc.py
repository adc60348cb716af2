"""The allocation-free split-KV entry point, attn_fwd_splitkv_noalloc, whose
chunk partials live in a fixed per-device array of the library instead of a
caller workspace.  Called through the C ABI and compared element by element
with attn_fwd_splitkv_ex on a caller workspace (same kernels, so the results
must be bitwise equal) and with the fp64 oracle at the usual tolerances, on
two calls in a row, the second smaller, so that it also runs over what the
first left in the array."""
from __future__ import annotations

import math

import pytest
import torch

from attn_inputs import make_qkv
from gpu_helpers import DT_CODE, check, need_gpu, oracle_full, run_gpu_splitkv, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    return need_gpu()


def run_noalloc(fa, q, k, v, *, causal, window, num_splits, config_id=-1):
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=dev)
    dtype = DT_CODE["f16" if q.dtype == torch.float16 else "bf16"]
    fa.attn_fwd_splitkv_noalloc(qd, kd, vd, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, 1.0 / math.sqrt(d),
                                dtype, num_splits, config_id, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


# B, Hq, Hkv, Nq, Nk, d, dtype, causal, window, num_splits -- the second is
# smaller in every size
CALLS = [
    (2, 16, 2, 4, 3000, 128, "bf16", True, 0, 16),
    (1, 4, 4, 1, 700, 64, "f16", True, 100, 3),
]


def test_noalloc_matches_workspace_entry_point_twice(fa):
    for B, Hq, Hkv, Nq, Nk, d, dt, causal, window, splits in CALLS:
        label = f"B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} {dt} causal={causal} w={window} splits={splits}"
        say("noalloc:", label)
        q, k, v = make_qkv(B, Hq, Hkv, Nq, d, dt, seed=Nk + Nq, nk=Nk)
        plan = fa.attn_fwd_splitkv_plan(B, Hq, Hkv, Nq, Nk, d, causal, window, DT_CODE[dt], splits, -1)
        assert plan["n_splits"] > 1 and 0 < plan["workspace_bytes"] <= fa.ATTN_NOALLOC_SCRATCH_BYTES
        o, lse = run_noalloc(fa, q, k, v, causal=causal, window=window, num_splits=splits)
        o_ws, lse_ws = run_gpu_splitkv(q, k, v, causal=causal, window=window, num_splits=splits)
        assert torch.equal(o, o_ws), label
        assert torch.equal(lse, lse_ws), label
        ro, rl = oracle_full(q, k, v, causal=causal, window=window)
        check(label, o, lse, ro, rl, dt)


def test_noalloc_single_chunk_and_empty(fa):
    q, k, v = make_qkv(1, 2, 1, 3, 64, "f16", seed=5, nk=200)
    o, lse = run_noalloc(fa, q, k, v, causal=True, window=0, num_splits=1)
    ro, rl = oracle_full(q, k, v, causal=True)
    check("one chunk", o, lse, ro, rl, "f16")
    e = torch.empty((1, 2, 0, 64), dtype=torch.float16, device="cuda:0")
    fa.attn_fwd_splitkv_noalloc(e, e, e, e, None, 1, 2, 2, 0, 0, 64, False, 0, 0.125, DT_CODE["f16"], 0, -1,
                                torch.cuda.current_stream().cuda_stream)


def test_noalloc_rejects_partials_beyond_scratch(fa):
    q = torch.zeros((1, 16, 512, 128), dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros((1, 16, 4096, 128), dtype=torch.bfloat16, device="cuda:0")
    o = torch.empty_like(q)
    need = fa.attn_fwd_splitkv_workspace_size(1, 16, 16, 512, 4096, 128, True, 0, DT_CODE["bf16"], 64, -1)
    assert need > fa.ATTN_NOALLOC_SCRATCH_BYTES
    with pytest.raises(fa.AttnError) as e:
        fa.attn_fwd_splitkv_noalloc(q, k, k, o, None, 1, 16, 16, 512, 4096, 128, True, 0, 0.1, DT_CODE["bf16"],
                                    64, -1, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == 10
