"""The C ABI on the CPU: the library loads, exports every declared symbol,
and its host-side argument checks return the documented codes.  No kernel is
launched here."""
import ctypes
import os
import re

import pytest

import flashattention_forward_05_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.library_path())
    names = declared_functions()
    assert "attn_fwd" in names and "attn_fwd_validate" in names and "attn_status_str" in names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def test_status_strings():
    for code in range(11):
        assert fa.attn_status_str(code) and fa.attn_status_str(code) != "unknown status"
    assert fa.attn_status_str(99) == "unknown status"


A = 1 << 20          # fake, aligned, disjoint addresses; nothing is dereferenced
GOOD = dict(q=A, k=2 * A, v=3 * A, o=4 * A, lse=5 * A, B=2, Hq=4, Hkv=2, N=100, d=64,
            causal=1, window=0, scale=0.125, dtype=0)


def validate(**over):
    a = dict(GOOD, **over)
    return fa.attn_fwd_validate(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                a["N"], a["d"], a["causal"], a["window"], a["scale"], a["dtype"])


@pytest.mark.parametrize("over,code", [
    ({}, 0),
    ({"lse": None}, 0),
    ({"N": 0, "q": None, "k": None, "v": None, "o": None}, 0),
    ({"q": None}, 1), ({"k": None}, 1), ({"v": None}, 1), ({"o": None}, 1),
    ({"B": 0}, 2), ({"Hq": 0}, 2), ({"Hkv": 0}, 2), ({"N": -1}, 2), ({"Hq": 3}, 2),
    ({"N": (1 << 24) + 1}, 2), ({"B": 1 << 13, "Hq": 1 << 12, "Hkv": 1 << 12}, 2),
    ({"d": 32}, 3), ({"d": 96}, 3), ({"d": 256}, 3), ({"dtype": 2}, 3), ({"dtype": -1}, 3),
    ({"window": -1}, 3), ({"window": 16, "causal": 0}, 3),
    ({"scale": float("inf")}, 4), ({"scale": float("nan")}, 4),
    ({"q": A + 8}, 5), ({"o": 4 * A + 2}, 5), ({"lse": 5 * A + 2}, 5),
    ({"o": A}, 6), ({"o": 2 * A + 64}, 6), ({"lse": 3 * A}, 6), ({"lse": 4 * A + 16}, 6),
])
def test_validate_codes(over, code):
    assert validate(**over) == code


def test_validate_accepts_edge_values():
    assert validate(scale=0.0) == 0
    assert validate(scale=-3.0) == 0
    assert validate(window=1) == 0
    assert validate(window=1 << 40) == 0
    assert validate(Hkv=1) == 0
    assert validate(d=128, dtype=1) == 0
    assert validate(q=2 * A, k=2 * A, v=2 * A) == 0      # inputs may alias each other


def test_plan_reports_tiles():
    p = fa.attn_fwd_plan(4, 32, 8, 8192, 128, 1, 0, 1)
    assert p["block_m"] * (8192 // p["block_m"]) == 8192
    assert p["grid"] == 4 * 32 * (8192 // p["block_m"])
    assert p["mask_mode"] == 1 and p["exact_tiles"] >= 1
    short = fa.attn_fwd_plan(1, 1, 1, 100, 64, 0, 0, 0)                     # short non-causal rows:
    assert short["exact_tiles"] == -(-100 // short["block_m"])             # every query tile two-term
    assert fa.attn_fwd_plan(1, 1, 1, 5000, 64, 0, 0, 0)["exact_tiles"] == 0
    assert fa.attn_fwd_plan(1, 32, 1, 32768, 128, 1, 4096, 1)["mask_mode"] == 2
    for d in (64, 128):
        for cid in range(fa.attn_fwd_num_configs()):
            desc = fa.attn_fwd_config_desc(cid, d)
            assert desc["block_m"] * desc["key_groups"] == 32 * desc["query_blocks_per_wave"] * desc["waves"]
            pe = fa.attn_fwd_plan_ex(2, 4, 4, 1000, d, 1, 0, 0, cid)
            assert pe["config_id"] == cid and pe["block_m"] == desc["block_m"]
            assert pe["block_n"] == desc["block_n"] and pe["waves"] == desc["waves"]
    with pytest.raises(fa.AttnError):
        fa.attn_fwd_config_desc(fa.attn_fwd_num_configs())
    with pytest.raises(fa.AttnError):
        fa.attn_fwd_config_desc(0, 96)
    with pytest.raises(fa.AttnError):
        fa.attn_fwd_plan(1, 3, 2, 10, 64, 1, 0, 0)


def test_launch_rejects_before_touching_the_gpu():
    # argument errors come back as exceptions without any HIP call
    with pytest.raises(fa.AttnError) as e:
        fa.attn_fwd_ex(None, 2 * A, 3 * A, 4 * A, None, 1, 1, 1, 8, 64, 0, 0, 0.1, 0, -1, 0)
    assert e.value.status == 1
    with pytest.raises(fa.AttnError) as e:
        fa.attn_fwd_ex(A, 2 * A, 3 * A, 4 * A, None, 1, 1, 1, 8, 64, 0, 0, 0.1, 0, 99, 0)
    assert e.value.status == 4


def test_auto_config_choice():
    """The automatic tile configuration follows the documented rule: for d=64,
    32-row workgroups with four key groups when there are at most 256 of
    them; else, causal, 64-row workgroups under 128 128-row ones, 256-row
    workgroups from 1024 of them, 128-row workgroups between (paired 64-row
    tiles up to 256 workgroups), with a window 64-row workgroups
    up to 512 128-row tiles, and unmasked 128-row workgroups unless the grid
    is small; 256-row workgroups for large d=128 grids."""
    auto = lambda *a: fa.attn_fwd_plan_ex(*a, -1)["config_id"]
    assert auto(2, 4, 4, 4096, 64, 1, 0, 0) == 0        # lab, causal: paired 64-row tiles
    assert auto(2, 4, 4, 4096, 64, 0, 0, 0) == 0        # lab, full
    assert auto(2, 4, 4, 1024, 64, 0, 0, 0) == 4        # small grid: 32 rows, four key groups
    assert auto(2, 4, 4, 1024, 64, 1, 0, 0) == 4
    assert auto(2, 4, 4, 256, 64, 1, 0, 0) == 4
    assert auto(2, 4, 4, 2048, 64, 1, 0, 0) == 0        # 512 32-row workgroups, 128 of 128 rows
    assert auto(1, 6, 6, 2048, 64, 1, 0, 0) == 2        # 96 of 128 rows: 64-row workgroups
    assert auto(2, 4, 4, 4096, 64, 1, 512, 0) == 2      # window
    assert auto(1, 12, 12, 2048, 64, 0, 0, 0) == 0      # stress, full
    assert auto(1, 12, 12, 2048, 64, 1, 0, 0) == 0      # stress, causal
    assert auto(1, 4, 4, 16384, 64, 1, 0, 0) == 0       # 256 256-row workgroups
    assert auto(4, 16, 16, 4096, 64, 1, 0, 0) == 1      # 1024 256-row workgroups
    assert auto(4, 32, 8, 8192, 128, 1, 0, 1) == 1      # GQA prefill
    assert auto(1, 32, 1, 32768, 128, 1, 4096, 1) == 1  # MQA with window
    assert auto(1, 2, 2, 512, 128, 1, 0, 1) == 0        # small d=128 grid


# ---- split-KV entry points (host checks, plan, workspace size)
G = 1 << 30          # room for every buffer of the split-KV shapes below
KV = dict(q=G, k=2 * G, v=3 * G, o=4 * G, lse=5 * G, B=2, Hq=8, Hkv=2, Nq=1, Nk=4096, d=128,
          causal=1, window=0, scale=0.125, dtype=1, num_splits=0, config_id=-1, workspace=6 * G,
          workspace_bytes=1 << 20)


def validate_kv(**over):
    a = dict(KV, **over)
    return fa.attn_fwd_splitkv_validate(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                        a["Nq"], a["Nk"], a["d"], a["causal"], a["window"], a["scale"],
                                        a["dtype"], a["num_splits"], a["config_id"], a["workspace"],
                                        a["workspace_bytes"])


@pytest.mark.parametrize("over,code", [
    ({}, 0),
    ({"lse": None}, 0),
    ({"Nq": 0, "q": None, "k": None, "v": None, "o": None, "workspace": None}, 0),
    ({"num_splits": 1, "workspace": None, "workspace_bytes": 0}, 0),      # one chunk: no workspace
    ({"Nq": 4096, "num_splits": 1, "workspace": None}, 0),
    ({"causal": 0, "Nq": 5000}, 0),                                     # non-causal may have Nq > Nk
    ({"q": None}, 1), ({"workspace": None}, 1),
    ({"Nk": 0}, 2), ({"Nk": -1}, 2), ({"Nq": 4097}, 2), ({"Nk": (1 << 24) + 1}, 2), ({"Hq": 3}, 2),
    ({"d": 96}, 3), ({"window": 8, "causal": 0}, 3), ({"config_id": 4}, 0),
    ({"num_splits": -1}, 4), ({"num_splits": 1025}, 4), ({"config_id": 5}, 4), ({"scale": float("nan")}, 4),
    ({"workspace": 6 * G + 8}, 5), ({"q": G + 2}, 5),
    ({"o": 2 * G}, 6), ({"workspace": 3 * G}, 6), ({"workspace": 5 * G}, 6), ({"workspace": 4 * G - 64}, 6),
    ({"workspace_bytes": 64}, 9),
])
def test_splitkv_validate_codes(over, code):
    assert validate_kv(**over) == code


def test_splitkv_plan_and_workspace():
    # decoding: the 4 query heads of each K/V head stacked into one 32-row
    # workgroup per chunk, automatic chunk count
    p = fa.attn_fwd_splitkv_plan(4, 32, 8, 1, 8192, 128, 1, 0, 1)
    assert p["config_id"] == 3 and p["block_m"] == 32 and p["waves"] == 1 and p["stacked"] == 1
    key_tiles = 8192 // p["block_n"]
    assert p["n_splits"] > 1 and p["split_tiles"] >= 4
    assert p["n_splits"] == -(-key_tiles // p["split_tiles"])
    assert p["grid"] == 4 * 8 * p["n_splits"]
    # stacking needs G > 1 and at most 16 query rows; then G * Nq rows per K/V head
    m = fa.attn_fwd_splitkv_plan(1, 32, 1, 3, 4096, 128, 1, 0, 1, 2)
    assert m["stacked"] == 1 and m["grid"] == -(-96 // m["block_m"]) * m["n_splits"]
    assert fa.attn_fwd_splitkv_plan(1, 8, 2, 17, 4096, 64, 1, 0, 0, 2)["stacked"] == 0
    assert fa.attn_fwd_splitkv_plan(1, 8, 8, 1, 4096, 64, 1, 0, 0, 2)["stacked"] == 0
    assert p["workspace_bytes"] == p["n_splits"] * 4 * 32 * 1 * (128 + 1) * 4
    assert fa.attn_fwd_splitkv_workspace_size(4, 32, 8, 1, 8192, 128, 1, 0, 1) == p["workspace_bytes"]
    # explicit chunk counts: ceil(tiles / ceil(tiles / P)) chunks, never more than the tiles
    for want in (1, 2, 3, 7, 64, 1000):
        q = fa.attn_fwd_splitkv_plan(1, 1, 1, 1, 1000, 64, 1, 0, 0, want)
        tiles = -(-1000 // q["block_n"])
        per = -(-tiles // min(want, tiles))
        assert q["split_tiles"] == per and q["n_splits"] == -(-tiles // per)
        assert q["workspace_bytes"] == (0 if q["n_splits"] == 1 else q["n_splits"] * (64 + 1) * 4)
    # a window: chunks cover only the 4096 keys the query sees
    wnd = fa.attn_fwd_splitkv_plan(1, 32, 1, 1, 32768, 128, 1, 4096, 1)
    vis_tiles = 4096 // wnd["block_n"]
    assert wnd["n_splits"] == -(-vis_tiles // wnd["split_tiles"]) and wnd["n_splits"] > 1
    # square prefill shapes take the plain forward's tile choice and, on grids
    # of 64 workgroups or more, one chunk
    assert fa.attn_fwd_splitkv_plan(2, 4, 4, 1024, 1024, 64, 1, 0, 0)["n_splits"] == 1
    assert fa.attn_fwd_splitkv_plan(2, 4, 4, 1024, 1024, 64, 1, 0, 0)["config_id"] == 2
    with pytest.raises(fa.AttnError) as e:                       # the C call returns -status
        fa.attn_fwd_splitkv_workspace_size(1, 3, 2, 1, 10, 64, 1, 0, 0)
    assert e.value.status == 2
    assert fa.load_library().attn_fwd_splitkv_workspace_size(1, 3, 2, 1, 10, 64, 1, 0, 0, 0, -1) == -2
    with pytest.raises(fa.AttnError):
        fa.attn_fwd_splitkv_plan(1, 1, 1, 8, 4, 64, 1, 0, 0)    # causal with Nq > Nk


# ---- paged K/V entry points (host checks, plan)
PG = dict(q=G, kp=2 * G, vp=3 * G, bt=4 * G, sl=4 * G + (1 << 20), o=5 * G, lse=6 * G, B=2, Hq=8, Hkv=2, Nq=1,
          d=128, page_size=16, num_pages=1000, max_pages=256, max_seq_len=4096, causal=1, window=0, scale=0.1,
          dtype=1, num_splits=0, config_id=-1, workspace=7 * G, workspace_bytes=1 << 20)


def validate_pg(**over):
    a = dict(PG, **over)
    return fa.attn_fwd_paged_validate(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["o"], a["lse"], a["B"],
                                      a["Hq"], a["Hkv"], a["Nq"], a["d"], a["page_size"], a["num_pages"],
                                      a["max_pages"], a["max_seq_len"], a["causal"], a["window"], a["scale"],
                                      a["dtype"], a["num_splits"], a["config_id"], a["workspace"],
                                      a["workspace_bytes"])


@pytest.mark.parametrize("over,code", [
    ({}, 0), ({"lse": None}, 0), ({"page_size": 8, "max_pages": 512}, 0), ({"page_size": 256, "max_pages": 16}, 0),
    ({"Nq": 0, "q": None, "kp": None, "vp": None, "bt": None, "sl": None, "o": None}, 0),
    ({"bt": None}, 1), ({"sl": None}, 1), ({"kp": None}, 1), ({"workspace": None}, 1),
    ({"max_seq_len": 4097}, 2), ({"max_seq_len": 0}, 2), ({"num_pages": 0}, 2), ({"max_pages": 0}, 2),
    ({"page_size": 4}, 3), ({"page_size": 24}, 3), ({"page_size": 512, "max_pages": 8}, 3), ({"d": 96}, 3),
    ({"config_id": 4}, 0), ({"config_id": 5}, 4),
    ({"num_splits": -1}, 4),
    ({"bt": 4 * G + 2}, 5), ({"sl": 4 * G + (1 << 20) + 1}, 5), ({"workspace": 7 * G + 4}, 5),
    ({"o": 2 * G + 64}, 6), ({"lse": 4 * G}, 6), ({"workspace": 3 * G}, 6), ({"workspace": 4 * G + (1 << 20)}, 6),
    ({"workspace_bytes": 16}, 9),
])
def test_paged_validate_codes(over, code):
    assert validate_pg(**over) == code


def test_paged_plan():
    p = fa.attn_fwd_paged_plan(4, 32, 8, 1, 128, 16, 3000, 512, 8192, 1, 0, 1)
    s = fa.attn_fwd_splitkv_plan(4, 32, 8, 1, 8192, 128, 1, 0, 1)
    assert p == s                       # same plan as the contiguous call of the same maximum length
    assert fa.attn_fwd_paged_workspace_size(4, 32, 8, 1, 128, 16, 3000, 512, 8192, 1, 0, 1) == p["workspace_bytes"]
    w = fa.attn_fwd_paged_plan(1, 32, 1, 1, 128, 16, 3000, 2048, 32768, 1, 4096, 1)
    assert w["n_splits"] * w["split_tiles"] >= 32768 // w["block_n"]   # lengths vary: chunks span all keys
    # causal prefill: the contiguous call pairs 64-row tiles in 128-row
    # workgroups, the paged kernel does not pair them and keeps 64-row ones
    assert fa.attn_fwd_splitkv_plan(2, 4, 4, 4096, 4096, 64, 1, 0, 0)["config_id"] == 0
    assert fa.attn_fwd_paged_plan(2, 4, 4, 4096, 64, 16, 2048, 256, 4096, 1, 0, 0)["config_id"] == 2


def test_autotune_rejects_before_touching_the_gpu():
    lib = fa.load_library()
    best = ctypes.c_int(-7)
    args = (A, 2 * A, 3 * A, 4 * A, None, 1, 1, 1, 8, 64, 0, 0, 0.1, 0)
    assert lib.attn_fwd_autotune(*args, 10, None, None, None) == 1          # NULL best_config
    assert lib.attn_fwd_autotune(*args, 0, ctypes.byref(best), None, None) == 4
    assert lib.attn_fwd_autotune(*args, 10001, ctypes.byref(best), None, None) == 4
    bad = (A, 2 * A, 3 * A, 4 * A, None, 1, 3, 2, 8, 64, 0, 0, 0.1, 0)      # Hq % Hkv != 0
    assert lib.attn_fwd_autotune(*bad, 10, ctypes.byref(best), None, None) == 2
    assert best.value == -7


# ---- backward (include/attn_bwd.h)
BG = dict(q=A, k=2 * A, v=3 * A, o=4 * A, dout=5 * A, lse=6 * A, dq=7 * A, dk=8 * A, dv=9 * A,
          B=2, Hq=4, Hkv=2, N=100, d=64, causal=1, window=0, scale=0.125, dtype=0, ws=10 * A, wsb=1 << 19)


def validate_bwd(**over):
    a = dict(BG, **over)
    return fa.attn_bwd_validate(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"], a["dv"],
                                a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"], a["window"], a["scale"],
                                a["dtype"], a["ws"], a["wsb"])


@pytest.mark.parametrize("over,code", [
    ({}, 0),
    ({"N": 0, "q": None, "k": None, "v": None, "o": None, "dout": None, "lse": None, "dq": None, "dk": None,
      "dv": None, "ws": None, "wsb": 0}, 0),
    ({"q": None}, 1), ({"o": None}, 1), ({"dout": None}, 1), ({"lse": None}, 1), ({"dq": None}, 1),
    ({"dk": None}, 1), ({"dv": None}, 1), ({"ws": None}, 1),
    ({"B": 0}, 2), ({"Hq": 3}, 2), ({"N": -1}, 2), ({"N": (1 << 24) + 1}, 2),
    ({"d": 96}, 3), ({"dtype": 2}, 3), ({"window": 8, "causal": 0}, 3), ({"window": -1}, 3),
    ({"scale": float("nan")}, 4),
    ({"q": A + 8}, 5), ({"dk": 8 * A + 4}, 5), ({"ws": 10 * A + 8}, 5), ({"lse": 6 * A + 2}, 5),
    ({"dq": A}, 6), ({"dk": 5 * A + 16}, 6), ({"dv": 8 * A}, 6), ({"ws": 6 * A}, 6), ({"ws": 9 * A + 32}, 6),
    ({"wsb": 2 * 4 * 128 * 8 + 2 * 2 * 2 * 2 * 100 * 64 * 4 - 1}, 9),
])
def test_bwd_validate_codes(over, code):
    assert validate_bwd(**over) == code


def test_bwd_workspace_size():
    # 8 bytes per query row, rows padded to a multiple of 64 per head, rounded
    # to 256 bytes; plus fp32 partial dk and dv when the heads are split
    assert fa.attn_bwd_workspace_size(2, 4, 4, 100, 64) == 2 * 4 * 128 * 8          # G = 1: no split
    assert fa.attn_bwd_workspace_size(1, 1, 1, 64, 128) == 512
    assert fa.attn_bwd_workspace_size(1, 1, 1, 0, 128) == 0
    assert fa.attn_bwd_workspace_size(4, 32, 8, 8192, 128) == 4 * 32 * 8192 * 8     # 2048 workgroups: no split
    # MQA, N = 32768: 256 workgroups of 128 keys -> the 32 query heads split 8 ways
    assert fa.attn_bwd_workspace_size(1, 32, 1, 32768, 128) == 32 * 32768 * 8 + 2 * 8 * 32768 * 128 * 4
    # G = 3 and a wish of 2048 / 1 workgroups: the largest divisor of 3, i.e. 3
    assert fa.attn_bwd_workspace_size(1, 3, 1, 100, 64) == 3 * 128 * 8 + 2 * 3 * 100 * 64 * 4
    assert fa.attn_bwd_workspace_size(1, 3, 2, 64, 64) == -1
    assert fa.attn_bwd_workspace_size(1, 1, 1, 64, 96) == -1
    # B=2, Hq=4, Hkv=2, N=100: 2 workgroups of 128 keys -> split G = 2 ways
    assert fa.attn_bwd_workspace_size(2, 4, 2, 100, 64) == 2 * 4 * 128 * 8 + 2 * 2 * 2 * 2 * 100 * 64 * 4
    assert validate_bwd(wsb=2 * 4 * 128 * 8 + 2 * 2 * 2 * 2 * 100 * 64 * 4) == 0


def test_bwd_rejects_before_touching_the_gpu():
    with pytest.raises(fa.AttnError) as e:
        fa.attn_bwd(None, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A, 7 * A, 8 * A, 9 * A, 1, 1, 1, 8, 64, 0, 0, 0.1, 0,
                    10 * A, 1 << 16, 0)
    assert e.value.status == 1


def test_flash_attn_backward_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    lse = torch.zeros(1, 2, 8, dtype=torch.float32)
    with pytest.raises(TypeError):
        fa.flash_attn_backward(q, q, q, q, lse, q)


def test_output_buffer_checks():
    """Caller-supplied out / lse / workspace tensors the kernels would write
    out of bounds or in the wrong layout are rejected before any GPU call."""
    import torch
    from flashattention_forward_05_amd._binding import _check_buffer

    cpu, gpu = torch.device("cpu"), torch.device("cuda", 0)
    o = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    _check_buffer("out", o, cpu, torch.float16, (1, 2, 8, 64))                   # well-formed
    with pytest.raises(TypeError):                                              # host tensor for a GPU call
        _check_buffer("out", o, gpu, torch.float16, (1, 2, 8, 64))
    with pytest.raises(TypeError):
        _check_buffer("out", o.numpy(), cpu)
    with pytest.raises(TypeError):                                              # wrong dtype
        _check_buffer("out", o, cpu, torch.bfloat16, (1, 2, 8, 64))
    with pytest.raises(TypeError):                                              # fp16 lse
        _check_buffer("lse", torch.zeros(1, 2, 8, dtype=torch.float16), cpu, torch.float32, (1, 2, 8))
    with pytest.raises(ValueError):                                             # too small
        _check_buffer("out", o[:, :, :4], cpu, torch.float16, (1, 2, 8, 64))
    with pytest.raises(ValueError):                                             # strided
        _check_buffer("out", torch.zeros(1, 2, 64, 8, dtype=torch.float16).transpose(2, 3), cpu, torch.float16,
                      (1, 2, 8, 64))


def test_flash_attn_forward_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    for fn in (fa.flash_attn_forward, fa.flash_attn_forward_splitkv):
        with pytest.raises(TypeError):
            fn(q, q, q)


def test_noalloc_rejects_oversized_partials_on_host():
    """attn_fwd_splitkv_noalloc refuses a split whose partials exceed its fixed
    scratch, and does so before any HIP call (this runs with no GPU)."""
    B, Hq, Hkv, Nq, Nk, d = 1, 16, 16, 512, 4096, 128
    need = fa.attn_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, True, 0, fa.ATTN_BF16, 64, -1)
    assert need > fa.ATTN_NOALLOC_SCRATCH_BYTES
    base = 1 << 40
    q, k, v, o = base, base + (1 << 30), base + (2 << 30), base + (3 << 30)
    with pytest.raises(fa.AttnError) as e:
        fa.attn_fwd_splitkv_noalloc(q, k, v, o, None, B, Hq, Hkv, Nq, Nk, d, True, 0, 0.1, fa.ATTN_BF16, 64, -1,
                                    stream=0)
    assert e.value.status == 10
    # sizes the plain split-KV entry point rejects are rejected the same way
    with pytest.raises(fa.AttnError) as e:
        fa.attn_fwd_splitkv_noalloc(q, k, v, o, None, B, Hq, 5, Nq, Nk, d, True, 0, 0.1, fa.ATTN_BF16, 64, -1,
                                    stream=0)
    assert e.value.status == 2
