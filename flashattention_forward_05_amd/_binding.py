"""ctypes marshalling for libattn_fwd.so.  No arithmetic of the method here."""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "lib", "libattn_fwd.so")

ATTN_F16 = 0
ATTN_BF16 = 1
STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_ARG", 5: "ATTN_ERR_ALIGN", 6: "ATTN_ERR_ALIAS", 7: "ATTN_ERR_LAUNCH",
    8: "ATTN_ERR_DEVICE", 9: "ATTN_ERR_WORKSPACE", 10: "ATTN_ERR_SCRATCH",
}
ATTN_NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024

_lib = None


class AttnError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({attn_status_str(status)})")


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load the built library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp, f32, cint = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    i64p = ctypes.POINTER(ctypes.c_int64)
    common = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, cint, i64, f32, cint]
    lib.attn_fwd.argtypes = common + [vp]
    lib.attn_fwd.restype = cint
    lib.attn_fwd_ex.argtypes = common + [cint, vp]
    lib.attn_fwd_ex.restype = cint
    lib.attn_fwd_validate.argtypes = common
    lib.attn_fwd_validate.restype = cint
    lib.attn_status_str.argtypes = [cint]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_fwd_plan.argtypes = [i64, i64, i64, i64, i64, cint, i64, cint, i64p]
    lib.attn_fwd_plan.restype = cint
    lib.attn_fwd_plan_ex.argtypes = [i64, i64, i64, i64, i64, cint, i64, cint, cint, i64p]
    lib.attn_fwd_plan_ex.restype = cint
    lib.attn_fwd_num_configs.argtypes = []
    lib.attn_fwd_num_configs.restype = cint
    lib.attn_fwd_config_desc.argtypes = [cint, i64, i64p]
    lib.attn_fwd_config_desc.restype = cint
    kv = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, cint, i64, f32, cint, i64]
    lib.attn_fwd_splitkv.argtypes = kv + [vp, i64, vp]
    lib.attn_fwd_splitkv.restype = cint
    lib.attn_fwd_splitkv_ex.argtypes = kv + [cint, vp, i64, vp]
    lib.attn_fwd_splitkv_ex.restype = cint
    lib.attn_fwd_splitkv_noalloc.argtypes = kv + [cint, vp]
    lib.attn_fwd_splitkv_noalloc.restype = cint
    lib.attn_fwd_splitkv_validate.argtypes = kv + [cint, vp, i64]
    lib.attn_fwd_splitkv_validate.restype = cint
    lib.attn_fwd_splitkv_plan.argtypes = [i64, i64, i64, i64, i64, i64, cint, i64, cint, i64, cint, i64p]
    lib.attn_fwd_splitkv_plan.restype = cint
    lib.attn_fwd_splitkv_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, cint, i64, cint, i64, cint]
    lib.attn_fwd_splitkv_workspace_size.restype = i64
    lib.attn_fwd_autotune.argtypes = common + [cint, ctypes.POINTER(cint), ctypes.POINTER(f32), vp]
    lib.attn_fwd_autotune.restype = cint
    pg = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i64, cint, i64, f32, cint, i64]
    lib.attn_fwd_paged.argtypes = pg + [vp, i64, vp]
    lib.attn_fwd_paged.restype = cint
    lib.attn_fwd_paged_ex.argtypes = pg + [cint, vp, i64, vp]
    lib.attn_fwd_paged_ex.restype = cint
    lib.attn_fwd_paged_validate.argtypes = pg + [cint, vp, i64]
    lib.attn_fwd_paged_validate.restype = cint
    geo = [i64, i64, i64, i64, i64, i64, i64, i64, i64, cint, i64, cint, i64, cint]
    lib.attn_fwd_paged_plan.argtypes = geo + [i64p]
    lib.attn_fwd_paged_plan.restype = cint
    lib.attn_fwd_paged_workspace_size.argtypes = geo
    lib.attn_fwd_paged_workspace_size.restype = i64
    bwd = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, cint, i64, f32, cint, vp, i64]
    lib.attn_bwd.argtypes = bwd + [vp]
    lib.attn_bwd.restype = cint
    lib.attn_bwd_validate.argtypes = bwd
    lib.attn_bwd_validate.restype = cint
    lib.attn_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64]
    lib.attn_bwd_workspace_size.restype = i64
    _lib = lib
    return lib


def _ptr(x) -> int | None:
    """Device pointer of a tensor, or an integer address, or None."""
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def attn_status_str(status: int) -> str:
    return load_library().attn_status_str(int(status)).decode()


def attn_fwd_validate(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, dtype) -> int:
    """Host-side argument checks only; returns the status code."""
    return load_library().attn_fwd_validate(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                            B, Hq, Hkv, N, d, int(causal), window, scale, dtype)


def attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, dtype,
                config_id=-1, stream=None) -> None:
    """Enqueue the forward with an explicit tile configuration; raises AttnError."""
    rc = load_library().attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                                    int(causal), window, scale, dtype, config_id, _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_ex")


def attn_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, dtype, stream=None) -> None:
    """Enqueue the forward on `stream` (default: torch's current stream)."""
    rc = load_library().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                                 int(causal), window, scale, dtype, _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd")


def attn_fwd_plan_ex(B, Hq, Hkv, N, d, causal, window, dtype, config_id=-1) -> dict:
    out = (ctypes.c_int64 * 7)()
    rc = load_library().attn_fwd_plan_ex(B, Hq, Hkv, N, d, int(causal), window, dtype, config_id, out)
    if rc != 0:
        raise AttnError(rc, "attn_fwd_plan_ex")
    keys = ("block_m", "block_n", "waves", "grid", "exact_tiles", "mask_mode", "config_id")
    return dict(zip(keys, list(out)))


def attn_fwd_plan(B, Hq, Hkv, N, d, causal, window, dtype) -> dict:
    out = (ctypes.c_int64 * 6)()
    rc = load_library().attn_fwd_plan(B, Hq, Hkv, N, d, int(causal), window, dtype, out)
    if rc != 0:
        raise AttnError(rc, "attn_fwd_plan")
    keys = ("block_m", "block_n", "waves", "grid", "exact_tiles", "mask_mode")
    return dict(zip(keys, list(out)))


def attn_fwd_num_configs() -> int:
    return int(load_library().attn_fwd_num_configs())


def attn_fwd_config_desc(config_id: int, d: int = 64) -> dict:
    out = (ctypes.c_int64 * 6)()
    rc = load_library().attn_fwd_config_desc(config_id, d, out)
    if rc != 0:
        raise AttnError(rc, "attn_fwd_config_desc")
    keys = ("query_blocks_per_wave", "waves", "block_n", "block_m", "key_groups", "stages")
    return dict(zip(keys, list(out)))


def attn_fwd_autotune(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, window, scale, dtype, reps=20,
                      stream=None) -> tuple[int, dict]:
    """Time every built tile configuration on these buffers (synchronises the
    stream); returns (fastest id, {id: ms per call})."""
    best = ctypes.c_int(-1)
    n = attn_fwd_num_configs()
    ms = (ctypes.c_float * n)()
    rc = load_library().attn_fwd_autotune(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d,
                                          int(causal), window, scale, dtype, reps, ctypes.byref(best), ms,
                                          _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_autotune")
    return best.value, {i: float(ms[i]) for i in range(n) if ms[i] >= 0.0}


# configuration picked by attn_fwd_autotune per (shape, dtype, mask, device),
# filled by flash_attn_forward(..., tune=True)
_TUNED: dict = {}


def tuned_configs() -> dict:
    """The per-shape tuning results of this process (a copy)."""
    return dict(_TUNED)


def _check_buffer(name, t, device, dtype=None, shape=None):
    """Reject a caller-supplied tensor the kernels would misuse before any GPU
    work: it must be a tensor on `device` (TypeError for a host tensor or a
    wrong dtype, ValueError for another GPU, a wrong shape or a
    non-contiguous layout: the kernels write it densely by raw pointer)."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != device.type:
        raise TypeError(f"{name} must be on {device.type}, got {t.device}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def flash_attn_forward(q, k, v, causal: bool = True, window: int = 0, scale: float | None = None,
                       config_id: int = -1, out=None, lse=None, return_lse: bool = True, tune: bool = False):
    """(B, Hq, N, d) query, (B, Hkv, N, d) key/value fp16 or bf16 CUDA tensors
    -> (o, lse).  scale defaults to 1/sqrt(d).  Inputs are made contiguous.
    With tune=True the first call of a shape times every tile configuration on
    it (attn_fwd_autotune, which synchronises) and later calls of that shape
    use the fastest."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) tensor")
        if t.dtype not in (torch.float16, torch.bfloat16):
            raise TypeError(f"{name} must be float16 or bfloat16, got {t.dtype}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D (B, H, N, d), got shape {tuple(t.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if k.shape != v.shape:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} differ")
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    Hkv = k.shape[1]
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_buffer("out", out, q.device, q.dtype, q.shape)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_buffer("lse", lse, q.device, torch.float32, (B, Hq, N))
    dtype = ATTN_F16 if q.dtype == torch.float16 else ATTN_BF16
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if tune and config_id == -1:
            key = (q.device.index, B, Hq, Hkv, N, d, dtype, bool(causal), int(window))
            if key not in _TUNED:
                _TUNED[key] = attn_fwd_autotune(q, k, v, out, lse, B, Hq, Hkv, N, d, causal, window, scale,
                                                dtype, reps=10, stream=stream)[0]
            config_id = _TUNED[key]
        attn_fwd_ex(q, k, v, out, lse, B, Hq, Hkv, N, d, causal, window, scale, dtype, config_id, stream)
    return out, lse


# ---- split-KV ("FlashDecoding"): Nq queries against Nk keys, keys cut into
# chunks over workgroups and merged by a second kernel

def attn_fwd_splitkv_validate(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, scale, dtype,
                              num_splits=0, config_id=-1, workspace=None, workspace_bytes=0) -> int:
    """Host-side argument checks of the split-KV call only; returns the status."""
    return load_library().attn_fwd_splitkv_validate(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, int(causal), window, scale,
        dtype, num_splits, config_id, _ptr(workspace), workspace_bytes)


def attn_fwd_splitkv_plan(B, Hq, Hkv, Nq, Nk, d, causal, window, dtype, num_splits=0, config_id=-1) -> dict:
    out = (ctypes.c_int64 * 9)()
    rc = load_library().attn_fwd_splitkv_plan(B, Hq, Hkv, Nq, Nk, d, int(causal), window, dtype,
                                              num_splits, config_id, out)
    if rc != 0:
        raise AttnError(rc, "attn_fwd_splitkv_plan")
    keys = ("block_m", "block_n", "waves", "grid", "n_splits", "split_tiles", "config_id", "workspace_bytes",
            "stacked")
    return dict(zip(keys, list(out)))


def attn_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal, window, dtype, num_splits=0,
                                    config_id=-1) -> int:
    n = int(load_library().attn_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, int(causal), window,
                                                           dtype, num_splits, config_id))
    if n < 0:
        raise AttnError(-n, "attn_fwd_splitkv_workspace_size")
    return n


def attn_fwd_splitkv_ex(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, scale, dtype,
                        num_splits=0, config_id=-1, workspace=None, workspace_bytes=0, stream=None) -> None:
    """Enqueue the split-KV forward; raises AttnError."""
    rc = load_library().attn_fwd_splitkv_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, int(causal), window, scale,
        dtype, num_splits, config_id, _ptr(workspace), workspace_bytes, _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_splitkv_ex")


def attn_fwd_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, scale, dtype,
                             num_splits=0, config_id=-1, stream=None) -> None:
    """Enqueue the split-KV forward with its partials in the library's fixed
    per-device scratch (no allocation); raises AttnError."""
    rc = load_library().attn_fwd_splitkv_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, int(causal), window, scale,
        dtype, num_splits, config_id, _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_splitkv_noalloc")


def attn_fwd_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, scale, dtype,
                     num_splits=0, workspace=None, workspace_bytes=0, stream=None) -> None:
    """Enqueue the split-KV forward with the automatic tile choice."""
    rc = load_library().attn_fwd_splitkv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, int(causal), window, scale,
        dtype, num_splits, _ptr(workspace), workspace_bytes, _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_splitkv")


def flash_attn_forward_splitkv(q, k, v, causal: bool = True, window: int = 0, scale: float | None = None,
                               num_splits: int = 0, config_id: int = -1, workspace=None, out=None, lse=None,
                               return_lse: bool = True):
    """(B, Hq, Nq, d) query against (B, Hkv, Nk, d) key/value fp16 or bf16
    CUDA tensors -> (o, lse), the queries being the last Nq positions.  The
    workspace (a CUDA uint8 tensor of at least attn_fwd_splitkv_workspace_size
    bytes) is allocated with torch when not given."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) tensor")
        if t.dtype not in (torch.float16, torch.bfloat16):
            raise TypeError(f"{name} must be float16 or bfloat16, got {t.dtype}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D (B, H, N, d), got shape {tuple(t.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if k.shape != v.shape:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} differ")
    B, Hq, Nq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    Hkv, Nk = k.shape[1], k.shape[2]
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dtype = ATTN_F16 if q.dtype == torch.float16 else ATTN_BF16
    need = attn_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal, window, dtype, num_splits, config_id)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check_buffer("workspace", workspace, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    _check_buffer("out", out, q.device, q.dtype, q.shape)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_buffer("lse", lse, q.device, torch.float32, (B, Hq, Nq))
    with torch.cuda.device(q.device):
        attn_fwd_splitkv_ex(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d, causal, window, scale, dtype,
                            num_splits, config_id, workspace, ws_bytes,
                            torch.cuda.current_stream(q.device).cuda_stream)
    return out, lse


# ---- paged K/V: pools (num_pages, Hkv, page_size, d), a block table per
# request and per-request lengths

_PLAN_KEYS = ("block_m", "block_n", "waves", "grid", "n_splits", "split_tiles", "config_id", "workspace_bytes",
              "stacked")


def attn_fwd_paged_plan(B, Hq, Hkv, Nq, d, page_size, num_pages, max_pages, max_seq_len, causal, window, dtype,
                        num_splits=0, config_id=-1) -> dict:
    out = (ctypes.c_int64 * 9)()
    rc = load_library().attn_fwd_paged_plan(B, Hq, Hkv, Nq, d, page_size, num_pages, max_pages, max_seq_len,
                                            int(causal), window, dtype, num_splits, config_id, out)
    if rc != 0:
        raise AttnError(rc, "attn_fwd_paged_plan")
    return dict(zip(_PLAN_KEYS, list(out)))


def attn_fwd_paged_workspace_size(B, Hq, Hkv, Nq, d, page_size, num_pages, max_pages, max_seq_len, causal,
                                  window, dtype, num_splits=0, config_id=-1) -> int:
    n = int(load_library().attn_fwd_paged_workspace_size(B, Hq, Hkv, Nq, d, page_size, num_pages, max_pages,
                                                         max_seq_len, int(causal), window, dtype, num_splits,
                                                         config_id))
    if n < 0:
        raise AttnError(-n, "attn_fwd_paged_workspace_size")
    return n


def attn_fwd_paged_validate(q, k_pool, v_pool, block_table, seq_lens, o, lse, B, Hq, Hkv, Nq, d, page_size,
                            num_pages, max_pages, max_seq_len, causal, window, scale, dtype, num_splits=0,
                            config_id=-1, workspace=None, workspace_bytes=0) -> int:
    return load_library().attn_fwd_paged_validate(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), _ptr(o), _ptr(lse), B, Hq, Hkv,
        Nq, d, page_size, num_pages, max_pages, max_seq_len, int(causal), window, scale, dtype, num_splits,
        config_id, _ptr(workspace), workspace_bytes)


def attn_fwd_paged_ex(q, k_pool, v_pool, block_table, seq_lens, o, lse, B, Hq, Hkv, Nq, d, page_size, num_pages,
                      max_pages, max_seq_len, causal, window, scale, dtype, num_splits=0, config_id=-1,
                      workspace=None, workspace_bytes=0, stream=None) -> None:
    """Enqueue the paged forward; raises AttnError."""
    rc = load_library().attn_fwd_paged_ex(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), _ptr(o), _ptr(lse), B, Hq, Hkv,
        Nq, d, page_size, num_pages, max_pages, max_seq_len, int(causal), window, scale, dtype, num_splits,
        config_id, _ptr(workspace), workspace_bytes, _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_paged_ex")


def attn_fwd_paged(q, k_pool, v_pool, block_table, seq_lens, o, lse, B, Hq, Hkv, Nq, d, page_size, num_pages,
                   max_pages, max_seq_len, causal, window, scale, dtype, num_splits=0, workspace=None,
                   workspace_bytes=0, stream=None) -> None:
    """Enqueue the paged forward with the automatic tile choice."""
    rc = load_library().attn_fwd_paged(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), _ptr(o), _ptr(lse), B, Hq, Hkv,
        Nq, d, page_size, num_pages, max_pages, max_seq_len, int(causal), window, scale, dtype, num_splits,
        _ptr(workspace), workspace_bytes, _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_fwd_paged")


def flash_attn_forward_paged(q, k_pool, v_pool, block_table, seq_lens, max_seq_len: int | None = None,
                             causal: bool = True, window: int = 0, scale: float | None = None, num_splits: int = 0,
                             config_id: int = -1, workspace=None, out=None, lse=None, return_lse: bool = True):
    """(B, Hq, Nq, d) queries against paged K/V: pools (num_pages, Hkv,
    page_size, d), block_table (B, max_pages) and seq_lens (B,) int32, all
    CUDA tensors -> (o, lse).  max_seq_len defaults to max_pages * page_size
    (it bounds every seq_lens entry); the workspace is allocated with torch
    when not given."""
    import torch

    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) tensor")
        if t.dtype not in (torch.float16, torch.bfloat16):
            raise TypeError(f"{name} must be float16 or bfloat16, got {t.dtype}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D, got shape {tuple(t.shape)}")
    for name, t in (("block_table", block_table), ("seq_lens", seq_lens)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32:
            raise TypeError(f"{name} must be an int32 CUDA tensor")
    if not (q.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("q and the pools must share one dtype")
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool differ in shape")
    B, Hq, Nq, d = q.shape
    num_pages, Hkv, page_size, dk = k_pool.shape
    if dk != d or block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("inconsistent paged shapes")
    if any(t.device != q.device for t in (k_pool, v_pool, block_table, seq_lens)):
        raise ValueError("q, the pools, block_table and seq_lens must be on one device")
    max_pages = block_table.shape[1]
    if max_seq_len is None:
        max_seq_len = max_pages * page_size
    q, k_pool, v_pool = q.contiguous(), k_pool.contiguous(), v_pool.contiguous()
    block_table, seq_lens = block_table.contiguous(), seq_lens.contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dtype = ATTN_F16 if q.dtype == torch.float16 else ATTN_BF16
    need = attn_fwd_paged_workspace_size(B, Hq, Hkv, Nq, d, page_size, num_pages, max_pages, max_seq_len, causal,
                                         window, dtype, num_splits, config_id)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check_buffer("workspace", workspace, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    _check_buffer("out", out, q.device, q.dtype, q.shape)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_buffer("lse", lse, q.device, torch.float32, (B, Hq, Nq))
    with torch.cuda.device(q.device):
        attn_fwd_paged_ex(q, k_pool, v_pool, block_table, seq_lens, out, lse, B, Hq, Hkv, Nq, d, page_size,
                          num_pages, max_pages, max_seq_len, causal, window, scale, dtype, num_splits, config_id,
                          workspace, ws_bytes, torch.cuda.current_stream(q.device).cuda_stream)
    return out, lse


# ---- backward pass (include/attn_bwd.h): gradients of sum(dO * O) from the
# forward's o and lse, scores recomputed tile by tile

def attn_bwd_workspace_size(B, Hq, Hkv, N, d) -> int:
    """Bytes of workspace attn_bwd needs (-1 for a shape it would reject)."""
    return int(load_library().attn_bwd_workspace_size(B, Hq, Hkv, N, d))


def attn_bwd_validate(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, window, scale, dtype,
                      workspace=None, workspace_bytes=0) -> int:
    """Host-side argument checks only; returns the status code."""
    return load_library().attn_bwd_validate(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                            _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d, int(causal), window, scale,
                                            dtype, _ptr(workspace), int(workspace_bytes))


def attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, window, scale, dtype,
             workspace, workspace_bytes, stream=None) -> None:
    """Enqueue the backward on `stream` (default: torch's current stream)."""
    rc = load_library().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                                 _ptr(dv), B, Hq, Hkv, N, d, int(causal), window, scale, dtype, _ptr(workspace),
                                 int(workspace_bytes), _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_bwd")


def flash_attn_backward(q, k, v, o, lse, dout, causal: bool = True, window: int = 0, scale: float | None = None,
                        workspace=None):
    """Gradients (dq, dk, dv) of sum(dout * o) for o, lse = flash_attn_forward(q,
    k, v, causal, window, scale).  Same shapes and dtype rules as the forward;
    dout is shaped like q.  The workspace is allocated with torch when not
    given."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) tensor")
        if t.dtype not in (torch.float16, torch.bfloat16) or t.dtype != q.dtype:
            raise TypeError(f"{name} must be float16 or bfloat16 like q, got {t.dtype}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D (B, H, N, d), got shape {tuple(t.shape)}")
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32:
        raise TypeError("lse must be the forward's float32 log-sum-exp tensor")
    if any(t.device != q.device for t in (k, v, o, dout, lse)):
        raise ValueError("q, k, v, o, dout and lse must be on one device")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)} disagree")
    if o.shape != q.shape or dout.shape != q.shape or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("o and dout must be shaped like q, lse (B, Hq, N)")
    Hkv = k.shape[1]
    q, k, v, o, dout, lse = (t.contiguous() for t in (q, k, v, o, dout, lse))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dtype = ATTN_F16 if q.dtype == torch.float16 else ATTN_BF16
    need = attn_bwd_workspace_size(B, Hq, Hkv, N, d)
    if need < 0:
        raise AttnError(2, "attn_bwd_workspace_size")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    with torch.cuda.device(q.device):
        attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, window, scale, dtype, workspace,
                 workspace.numel() * workspace.element_size(), torch.cuda.current_stream(q.device).cuda_stream)
    return dq, dk, dv
