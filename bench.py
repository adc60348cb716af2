#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

A step runs the whole hot path over one batch of synthetic input: every
(N, causal) variant of the workload, each one launch of the fused kernel
through the C ABI.  The pages' lab check (B=2, Hq=Hkv=4, d=64, fp16, N in
{256, 1024, 4096}, causal and not; "Lab 02 - Forward de flash attention en
Triton", "Bloque D") is --workload lab.

Metric: attention-forward TFLOP/s with 4*B*Hq*N^2*d FLOPs per variant, halved
when causal; a sliding window counts its visible (query, key) pairs instead.
Inputs are resident in HBM before the timed region starts.

Decoding workloads (``--workload decode``: one query per head against a long
K/V cache, "Optimizaciones de Atencion", section "FlashDecoding") run the
split-KV entry point (attention kernel over key chunks, then the merge kernel)
with a workspace allocated before timing; ``--splitkv`` runs any workload that
way.  Their FLOPs are 4*d per visible (query, key) pair, and since they move
far more bytes than they compute on, their roofline is HBM bandwidth.

Default workload: the largest single-GPU configuration, MQA long context
(B=1, Hq=32, Hkv=1, N=32768, d=128, bf16), causal with a 4096-token sliding
window and full causal; a step runs both.  The lab check (d=64, fp16) and the
other workloads are selectable with --workload.

Prints one JSON line.  Extra fields: "roofline" for the dominant kernel
(achieved = its FLOPs, or algorithmic bytes, per launch / its mean launch time
from HIP events on the launch stream; beside the published peak, the MFMA rate
measured on this GPU by microbench.py) and "cpu_baseline" (the fp64 oracle on a
bounded sample of the same workload, on this host's cores).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6}     # MI355X dense fp16/bf16 MFMA, 256 CU x 2.4 GHz x 4096
PEAK_HBM_GBS = 8000.0                              # MI355X HBM3E
RIDGE = PEAK_TFLOPS["f16"] * 1e12 / (PEAK_HBM_GBS * 1e9)   # FLOP per byte
WORKLOAD_SETS = {
    "lab": ["lab_n256_full", "lab_n256_causal", "lab_n1024_full", "lab_n1024_causal",
            "lab_n4096_full", "lab_n4096_causal"],
    "tiny": ["tiny"],
    "stress": ["stress_full", "stress_causal"],
    "gqa": ["gqa"],
    "mqa": ["mqa_window", "mqa_causal"],
    "mqa_window": ["mqa_window"],
    "lab4096": ["lab_n4096_full", "lab_n4096_causal"],
    "lab_n4096_full": ["lab_n4096_full"],
    "mqa_causal": ["mqa_causal"],
    "decode": ["decode_gqa", "decode_mqa", "decode_mqa_window"],
    "decode_gqa": ["decode_gqa"],
    "decode_mqa": ["decode_mqa"],
}


def metric_flops(B, Hq, N, d, causal, window=0) -> float:
    """4*B*Hq*N^2*d, halved for causal; with a window, 4*B*Hq*d per visible
    (query, key) pair."""
    if causal and window > 0 and window < N:
        pairs = window * (window + 1) / 2 + (N - window) * window
        return 4.0 * B * Hq * d * pairs
    f = 4.0 * B * Hq * N * N * d
    return f / 2 if causal else f


def page_naive_score_bytes(N, elem=4) -> float:
    """HBM bytes the unfused attention moves for the N x N score matrix of one
    head: S written, read back for the softmax, P written, read back for
    P.V ("00 - Por que la atencion domina la inferencia", section "Por que la
    attention es bandwidth-bound": 16 N^2 bytes in fp32)."""
    return 4.0 * elem * N * N


def page_tiled_bytes(N, d, block, elem=4) -> float:
    """The same page's model of the tiled kernel's traffic for one head,
    N d (3 + 2 N / block) elements (section "Lo que Flash hace de verdad, en
    un parrafo"): K and V read once per query block of `block` rows."""
    return float(N) * d * (3.0 + 2.0 * N / block) * elem


def visible_keys(i, N, causal, window, Nk=None):
    """Keys visible from query row i of N against Nk keys (row i sits at
    position Nk - N + i)."""
    Nk = N if Nk is None else Nk
    pos = Nk - N + i
    hi = min(pos, Nk - 1) if causal else Nk - 1
    lo = max(0, pos - window + 1) if window > 0 else 0
    return max(0, hi - lo + 1)


def workload_flops(w) -> float:
    """The metric's FLOPs for a workload; with Nq != Nk, 4*d per visible pair."""
    if w.nk == w.N:
        return metric_flops(w.B, w.Hq, w.N, w.d, w.causal, w.window)
    pairs = sum(visible_keys(i, w.N, w.causal, w.window, w.nk) for i in range(w.N))
    return 4.0 * w.B * w.Hq * w.d * pairs


def algorithmic_bytes(w) -> float:
    """Bytes the call must move at least: Q and the K/V rows some query sees
    (once), O and LSE written."""
    # the first query row (position nk - N) has the lowest first visible key
    lo = max(0, w.nk - w.N - w.window + 1) if (w.causal and w.window > 0) else 0
    kv_rows = (w.nk - lo) if w.N > 0 else 0
    return (2.0 * w.B * w.Hq * w.N * w.d * 2 + 2.0 * w.B * w.Hkv * kv_rows * w.d * 2
            + 4.0 * w.B * w.Hq * w.N)


def kernel_source_hash(family: str = "fwd") -> str:
    """Hash of the sources the forward kernels (family "fwd") or the backward
    kernels ("bwd") are built from: the files of csrc/ with the family's
    prefix plus the shared helpers."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "flashattention_forward_05_amd", "csrc")
    other = "attn_bwd" if family == "fwd" else "attn_fwd"
    for fn in sorted(os.listdir(csrc)):
        if fn.startswith(other) and fn != "attn_fwd_common.hpp":
            continue
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_label: str, family: str = "fwd"):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json" if family == "fwd" else "traffic_bwd.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_hash(family):
        return None
    ent = rec.get("kernels", {}).get(kernel_label)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def backward_bytes(w) -> float:
    """Bytes the backward must move at least: q, o, dO, k, v and lse read,
    dq, dk, dv written."""
    return (3 * 2.0 * w.B * w.Hq * w.N * w.d + 2 * 2.0 * w.B * w.Hkv * w.N * w.d + 4.0 * w.B * w.Hq * w.N
            + 2.0 * w.B * w.Hq * w.N * w.d + 2 * 2.0 * w.B * w.Hkv * w.N * w.d)


def cpu_baseline_backward(workloads, budget_s: float):
    """The oracle's backward, untuned, on a seeded random sample of query rows
    of each variant (its per-row entry point: scores, softmax weights, dP, D,
    dS and the row's dq), in chunks of 64 rows until that variant's share of
    the time budget is spent.  FLOPs counted per row: 6*d per visible key
    (three of the five products of the backward)."""
    import numpy as np

    import oracle
    from attn_inputs import make_dout, make_workload, to_bits

    oracle.load_library()
    flops = elapsed = 0.0
    rows_done = 0
    per_variant = budget_s / len(workloads)
    rng = np.random.default_rng(0)
    for w in workloads:
        q, k, v = (to_bits(t) for t in make_workload(w, seed=0))
        do = to_bits(make_dout(w.B, w.Hq, w.N, w.d, w.dtype, seed=0))
        ids = rng.permutation(w.B * w.Hq * w.N).astype(np.int64)
        t_var = 0.0
        for start in range(0, len(ids), 64):
            chunk = ids[start:start + 64]
            t0 = time.perf_counter()
            oracle.oracle_bwd_rows(q, k, v, do, chunk, scale=float(np.float32(w.scale)), causal=w.causal,
                                   window=w.window, dtype=w.dtype)
            t_var += time.perf_counter() - t0
            rows_done += len(chunk)
            flops += sum(6.0 * w.d * visible_keys(int(r) % w.N, w.N, w.causal, w.window) for r in chunk)
            if t_var > per_variant:
                break
        elapsed += t_var
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.max_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"fp64 oracle backward (per-row dq entry point) on random query rows of every variant, "
                   f"about {per_variant:.1f} s each ({rows_done} rows, {flops / 1e9:.2f} GFLOP in {elapsed:.1f} s)"),
    }


def cpu_baseline(workloads, budget_s: float):
    """The oracle, untuned, on a seeded random sample of query rows of each
    variant, in chunks of 64 rows until that variant's share of the time
    budget is spent; reports the achieved rate in the metric's unit (FLOPs
    counted per row: 4*d per visible key)."""
    import numpy as np

    import oracle
    from attn_inputs import make_workload, to_bits

    oracle.load_library()
    flops = 0.0
    elapsed = 0.0
    rows_done = 0
    per_variant = budget_s / len(workloads)
    rng = np.random.default_rng(0)
    for w in workloads:
        q, k, v = (to_bits(t) for t in make_workload(w, seed=0))
        ids = rng.permutation(w.B * w.Hq * w.N).astype(np.int64)
        t_var = 0.0
        for start in range(0, len(ids), 64):
            chunk = ids[start:start + 64]
            t0 = time.perf_counter()
            oracle.oracle_rows(q, k, v, chunk, scale=float(np.float32(w.scale)), causal=w.causal,
                               window=w.window, dtype=w.dtype)
            t_var += time.perf_counter() - t0
            rows_done += len(chunk)
            flops += sum(4.0 * w.d * visible_keys(int(r) % w.N, w.N, w.causal, w.window, w.nk)
                         for r in chunk)
            if t_var > per_variant:
                break
        elapsed += t_var
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.max_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"fp64 oracle on random query rows of every variant, about {per_variant:.1f} s each "
                   f"({rows_done} rows, {flops / 1e9:.2f} GFLOP in {elapsed:.1f} s)"),
    }


# ---------------------------------------------------------------------------
# rocprofv3 output -> short text summaries for profiles/ (run on any host)

def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_trace(trace_dir: str) -> str:
    """Per (kernel, grid) mean/min/max duration from a --kernel-trace CSV."""
    import glob
    import statistics
    rows = _read_csv(glob.glob(os.path.join(trace_dir, "*kernel_trace.csv"))[0])
    groups = {}
    for r in rows:
        if "attn_" not in r["Kernel_Name"]:
            continue
        key = (r["Kernel_Name"], int(r["Grid_Size"]) if "Grid_Size" in r else int(r.get("Grid_Size_X", 0)))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["kernel | grid threads | launches | mean us | min us | max us"]
    for (name, grid), d in sorted(groups.items(), key=lambda kv: -statistics.mean(kv[1])):
        out.append(f"{name} | {grid} | {len(d)} | {statistics.mean(d):.2f} | {min(d):.2f} | {max(d):.2f}")
    return "\n".join(out)


def summarize_counters(dirs: dict) -> dict:
    """Mean counter value per kernel over the dispatches of each pass."""
    import glob
    res = {}
    for tag, d in dirs.items():
        for r in _read_csv(glob.glob(os.path.join(d, "*counter_collection.csv"))[0]):
            k = (r["Kernel_Name"], r["Counter_Name"])
            res.setdefault(k, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in res.items()}


def traffic_record(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib, label):
    """HBM bytes per call of the attention library from FETCH_SIZE/WRITE_SIZE
    (KiB per dispatch, summed over the kernels of one call), each scaled by
    what the same counter reads for a plain copy of copy_mib MiB.  The counter
    runs must profile a workload with a single variant."""
    f = summarize_counters({"f": fetch_dir})
    w = summarize_counters({"w": write_dir})
    cf = summarize_counters({"cf": copy_fetch_dir})
    cw = summarize_counters({"cw": copy_write_dir})
    known = copy_mib * (1 << 20)
    cf_kib = max(v for (k, c), v in cf.items() if c == "FETCH_SIZE" and "copy" in k.lower())
    cw_kib = max(v for (k, c), v in cw.items() if c == "WRITE_SIZE" and "copy" in k.lower())
    fscale = known / (cf_kib * 1024)
    wscale = known / (cw_kib * 1024)
    # one call may launch two kernels (split-KV: attention, then the merge):
    # the per-dispatch means of every attention-library kernel are summed
    kf = sum(v for (k, c), v in f.items() if c == "FETCH_SIZE" and "attn_fwd" in k)
    kw = sum(v for (k, c), v in w.items() if c == "WRITE_SIZE" and "attn_fwd" in k)
    return {"label": label, "fetch_kib_raw": kf, "write_kib_raw": kw, "fetch_scale": fscale,
            "write_scale": wscale, "hbm_read_bytes": kf * 1024 * fscale,
            "hbm_write_bytes": kw * 1024 * wscale,
            "hbm_bytes_per_launch": kf * 1024 * fscale + kw * 1024 * wscale}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the oracle timing."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def torch_naive_time(r, reps: int):
    """Time the unfused attention the lab verifies and times the kernel against
    ("Lab 02 - Forward de flash attention en Triton", sections "Bloque C" and
    "Bloque E"): the full score matrix in the input dtype, a -inf mask,
    torch.softmax, then P V, on the GPU.  K and V are repeated to the query
    heads (GQA) and K is transposed into a contiguous copy before timing (a
    batched 16-bit product whose right operand is a transposed view is not
    safe on this platform); the mask is built before timing too.  Returns the
    mean ms per call over `reps` eager calls, and the max-abs difference from
    the kernel's output."""
    import torch
    w = r["w"]
    G = w.Hq // w.Hkv
    kk = r["k"].repeat_interleave(G, dim=1) if G > 1 else r["k"]
    vv = r["v"].repeat_interleave(G, dim=1) if G > 1 else r["v"]
    kt = kk.transpose(-1, -2).contiguous()
    vv = vv.contiguous()
    mask = None
    if w.causal:
        ones = torch.ones(w.N, w.N, dtype=torch.bool, device=r["q"].device)
        mask = ones.triu(1)
        if w.window > 0:
            mask = mask | ones.tril(-w.window)

    def naive():
        s = torch.matmul(r["q"], kt) * w.scale
        if mask is not None:
            s = s.masked_fill(mask, float("-inf"))
        return torch.matmul(torch.softmax(s, dim=-1), vv)

    out = naive()
    torch.cuda.synchronize()
    err = float((out.float() - r["o"].float()).abs().max())
    del out
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        naive()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps, err


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mqa", choices=sorted(WORKLOAD_SETS))
    ap.add_argument("--config", type=int, default=-1, help="tile configuration id (-1: automatic)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-microbench", action="store_true",
                    help="skip the measured MFMA peak (microbench.py) reported beside the published one")
    ap.add_argument("--splitkv", action="store_true",
                    help="run every variant through the split-KV entry point (decoding workloads always are)")
    ap.add_argument("--splits", type=int, default=0, help="key chunks for split-KV calls (0: automatic)")
    ap.add_argument("--tune", action="store_true",
                    help="before timing, pick each (non-split) variant's tile configuration with attn_fwd_autotune")
    ap.add_argument("--paged", type=int, default=0, metavar="PAGE_SIZE",
                    help="keep the K/V of decoding workloads in pages of this many tokens (random page order) "
                         "and run the paged entry point")
    ap.add_argument("--vs-torch", action="store_true",
                    help="also time the unfused PyTorch attention (score matrix, mask, softmax, P V) on the GPU for "
                         "variants with N <= 8192, and report the kernel's speedup over it")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (attn_bwd) of each variant instead of the forward; "
                         "FLOPs are 2.5x the forward's (the five products of the backward)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run plain device-to-device copies of MIB MiB (for scaling HBM counters)")
    ap.add_argument("--summarize-trace", metavar="DIR", help="print a summary of a rocprofv3 kernel-trace CSV dir")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="print mean counter values per kernel for rocprofv3 --pmc CSV dirs")
    ap.add_argument("--traffic", nargs=6, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR",
                                                   "COPY_MIB", "LABEL"),
                    help="compute HBM bytes per launch from counter dirs and add it to profiles/traffic.json")
    args = ap.parse_args()

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return 0
    if args.summarize_counters:
        vals = summarize_counters({d: d for d in args.summarize_counters})
        for (k, c), v in sorted(vals.items()):
            if "attn_" in k:
                print(f"{k} | {c} | {v:.6g}")
        return 0
    if args.traffic:
        fd, wd, cfd, cwd, mib, label = args.traffic
        rec = traffic_record(fd, wd, cfd, cwd, int(mib), label)
        path = os.path.join(ROOT, "profiles", "traffic.json")
        db = json.load(open(path)) if os.path.exists(path) else {}
        if db.get("kernel_source_sha") != kernel_source_hash():
            db = {"kernel_source_sha": kernel_source_hash(), "kernels": {}}
        db["kernels"][label] = rec
        with open(path, "w") as f:
            json.dump(db, f, indent=1)
        print(json.dumps(rec))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this benchmark runs on one GPU only; --gpus must be 1 "
              "(the path shards by (batch, K/V head) with no exchange between GPUs)", file=sys.stderr)
        return 2

    import torch

    import flashattention_forward_05_amd as fa
    from attn_inputs import WORKLOADS, make_paged_cache, make_workload

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                          "launches": max(1, args.steps)}), flush=True)
        return 0
    fa.load_library()
    stream = torch.cuda.current_stream(dev)
    wls = [WORKLOADS[n] for n in WORKLOAD_SETS[args.workload]]

    # inputs resident in HBM before timing
    runs = []
    for w in wls:
        qh, kh, vh = make_workload(w, seed=0)
        dt = 0 if w.dtype == "f16" else 1
        paged = None
        if args.paged and w.nk != w.N:
            # every request holds the full cache length; pages in seeded random order
            kp, vp, bt, sl = make_paged_cache(kh, vh, args.paged, [w.nk] * w.B, seed=0, spare_pages=0)
            kh, vh = kp, vp
            paged = dict(bt=bt.to(dev), sl=sl.to(dev), ps=args.paged, num_pages=kp.shape[0], max_pages=bt.shape[1])
        q, k, v = (t.to(dev) for t in (qh, kh, vh))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
        split = args.splitkv or w.nk != w.N
        ws = None
        if paged:
            plan = fa.attn_fwd_paged_plan(w.B, w.Hq, w.Hkv, w.N, w.d, paged["ps"], paged["num_pages"],
                                          paged["max_pages"], w.nk, w.causal, w.window, dt, args.splits, args.config)
            ws = torch.empty(max(16, plan["workspace_bytes"]), dtype=torch.uint8, device=dev)
        elif split:
            plan = fa.attn_fwd_splitkv_plan(w.B, w.Hq, w.Hkv, w.N, w.nk, w.d, w.causal, w.window, dt,
                                            args.splits, args.config)
            ws = torch.empty(max(16, plan["workspace_bytes"]), dtype=torch.uint8, device=dev)
        else:
            plan = fa.attn_fwd_plan_ex(w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, w.window, dt, args.config)
        flops = workload_flops(w)
        nbytes = algorithmic_bytes(w)
        cfg = args.config
        bwd = None
        if args.backward:
            if split or paged:
                print("bench.py: --backward needs square (Nq = Nk) workloads", file=sys.stderr)
                return 2
            from attn_inputs import make_dout
            fa.attn_fwd_ex(q, k, v, o, lse, w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, w.window, w.scale, dt, cfg,
                           stream.cuda_stream)
            need = fa.attn_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d)
            bwd = dict(do=make_dout(w.B, w.Hq, w.N, w.d, w.dtype, seed=0).to(dev), dq=torch.empty_like(q),
                       dk=torch.empty_like(k), dv=torch.empty_like(v),
                       ws=torch.empty(max(16, need), dtype=torch.uint8, device=dev))
            flops = 2.5 * flops
            nbytes = backward_bytes(w)
        if args.tune and not split and not paged:
            cfg, tms = fa.attn_fwd_autotune(q, k, v, o, lse, w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, w.window,
                                            w.scale, dt, reps=10)
            plan = fa.attn_fwd_plan_ex(w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, w.window, dt, cfg)
            plan["tuning_ms"] = {str(i): round(t, 5) for i, t in tms.items()}
        runs.append(dict(w=w, q=q, k=k, v=v, o=o, lse=lse, plan=plan, split=split, ws=ws, dt=dt, paged=paged, cfg=cfg,
                         flops=flops, bytes=nbytes, hbm_bound=flops / nbytes < RIDGE, bwd=bwd))

    def launch(r):
        # the current stream is torch's capture stream while a graph is recorded
        w = r["w"]
        s = torch.cuda.current_stream(dev).cuda_stream
        if r["bwd"]:
            bd = r["bwd"]
            fa.attn_bwd(r["q"], r["k"], r["v"], r["o"], bd["do"], r["lse"], bd["dq"], bd["dk"], bd["dv"], w.B, w.Hq,
                        w.Hkv, w.N, w.d, w.causal, w.window, w.scale, r["dt"], bd["ws"], bd["ws"].numel(), s)
        elif r["paged"]:
            pg = r["paged"]
            fa.attn_fwd_paged_ex(r["q"], r["k"], r["v"], pg["bt"], pg["sl"], r["o"], r["lse"], w.B, w.Hq, w.Hkv,
                                 w.N, w.d, pg["ps"], pg["num_pages"], pg["max_pages"], w.nk, w.causal, w.window,
                                 w.scale, r["dt"], args.splits, args.config, r["ws"], r["ws"].numel(), s)
        elif r["split"]:
            fa.attn_fwd_splitkv_ex(r["q"], r["k"], r["v"], r["o"], r["lse"], w.B, w.Hq, w.Hkv, w.N, w.nk, w.d,
                                   w.causal, w.window, w.scale, r["dt"], args.splits, args.config, r["ws"],
                                   r["ws"].numel(), s)
        else:
            fa.attn_fwd_ex(r["q"], r["k"], r["v"], r["o"], r["lse"], w.B, w.Hq, w.Hkv, w.N, w.d,
                           w.causal, w.window, w.scale, r["dt"], r["cfg"], s)

    for r in runs:                       # eager warm-up (also checks every launch)
        launch(r)
    torch.cuda.synchronize()

    # one step = every variant once, captured as a HIP graph so that the host
    # launch cost of the small variants does not stand in for kernel time
    step_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(step_graph):
        for r in runs:
            launch(r)
    for _ in range(args.warmup):
        step_graph.replay()
    torch.cuda.synchronize()

    # timed region: exactly K steps between synchronisations
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for _ in range(args.steps):
        step_graph.replay()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e_start.elapsed_time(e_end)

    # per-kernel launch duration: R back-to-back launches of one variant in a
    # graph, bracketed by HIP events on the launch stream
    per_kernel_ms = []
    for r in runs:
        reps = max(10, min(200, int(2e-3 / max(r["flops"] / 1e15, 1e-7))))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                launch(r)
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        per_kernel_ms.append(a.elapsed_time(b) / reps)
        del g

    # the MFMA rate this GPU reaches on a pure 32x32x16 bf16 loop (after the
    # timed region, so it does not heat the GPU before it)
    measured = None
    if not args.no_microbench:
        from flashattention_forward_05_amd import microbench
        mb = microbench.measure(quick=True)
        measured = {"tflops": round(mb["mfma_32x32x16_bf16_tflops"], 1), "clock_ghz": round(mb["clock_ghz_mfma"], 3)}

    total_flops = sum(r["flops"] for r in runs)
    ms_per_step = wall * 1e3 / args.steps
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    dom = max(range(len(runs)), key=lambda j: per_kernel_ms[j])
    dw = runs[dom]["w"]
    peak = PEAK_TFLOPS[dw.dtype]
    if runs[dom]["hbm_bound"]:
        # decoding: the call (attention over key chunks + merge) against HBM bandwidth
        roof = {"bound": "hbm", "achieved": runs[dom]["bytes"] / (per_kernel_ms[dom] * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "algorithmic_bytes": runs[dom]["bytes"]}
    else:
        roof = {"bound": "mfma", "achieved": runs[dom]["flops"] / (per_kernel_ms[dom] * 1e-3) / 1e12,
                "peak": peak, "unit": "TFLOP/s"}
    def label(r):
        return r["w"].label() + (f"_paged{r['paged']['ps']}" if r["paged"] else "")

    kernels = []
    for j, r in enumerate(runs):
        t = per_kernel_ms[j] * 1e-3
        kernels.append({"variant": label(r), "ms": round(per_kernel_ms[j], 5),
                        "tflops": round(r["flops"] / t / 1e12, 2),
                        "frac_of_peak": round(r["flops"] / t / 1e12 / peak, 4),
                        "hbm_gbs": round(r["bytes"] / t / 1e9, 1),
                        "frac_of_hbm": round(r["bytes"] / t / 1e9 / PEAK_HBM_GBS, 4),
                        "split_kv": r["split"],
                        "plan": r["plan"]})
        if args.vs_torch and not (r["split"] or r["paged"] or r["bwd"]) and r["w"].N <= 8192:
            launch(r)                    # the kernel's output, for the difference check
            torch.cuda.synchronize()
            tms, err = torch_naive_time(r, reps=max(3, min(50, int(0.5 / max(per_kernel_ms[j] * 1e-3 * 5, 1e-6)))))
            kernels[-1]["torch_naive"] = {"ms": round(tms, 5), "speedup": round(tms / per_kernel_ms[j], 2),
                                          "max_abs_diff": err}

    result = {
        "metric": ("attention bwd TFLOP/s (10*B*Hq*N^2*d, x1/2 causal) & % of MI355X MFMA peak" if args.backward
                   else "attention fwd TFLOP/s (4*B*Hq*N^2*d, x1/2 causal) & % of MI355X MFMA peak"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wls[0].dtype,
        "data": "synthetic (seeded iid N(0,1) inputs, rounded to the 16-bit dtype)",
        "config": {
            "workload": args.workload,
            "variants": [label(r) for r in runs],
            "parallelism": "single GPU",
            "tile_config": "tuned" if args.tune else args.config,
            "split_kv": any(r["split"] for r in runs),
            "paged_page_size": args.paged or None,
        },
        "roofline": {
            "bound": roof["bound"],
            "kernel": label(runs[dom]),
            "achieved": round(roof["achieved"], 2),
            "peak": roof["peak"],
            "unit": roof["unit"],
            "frac": round(roof["achieved"] / roof["peak"], 4),
            "traffic": traffic_from_profiles(label(runs[dom]), "bwd" if args.backward else "fwd"),
            **({"algorithmic_bytes": roof["algorithmic_bytes"]} if "algorithmic_bytes" in roof else {}),
            "algorithmic_intensity": round(runs[dom]["flops"] / runs[dom]["bytes"], 1),
            # the pages' byte models at this shape (16-bit elements, per head
            # times B * Hq): the unfused score-matrix traffic, and the tiled
            # kernel's with K/V read once per query tile of the plan's rows
            "page_naive_score_bytes": page_naive_score_bytes(dw.N, 2) * dw.B * dw.Hq,
            "page_tiled_model_bytes": page_tiled_bytes(dw.N, dw.d, runs[dom]["plan"].get("block_m", 64), 2)
            * dw.B * dw.Hq,
            "ridge": round(RIDGE, 1),
            **({"measured_peak": measured["tflops"], "frac_of_measured_peak":
                round(roof["achieved"] / measured["tflops"], 4), "measured_clock_ghz": measured["clock_ghz"]}
               if measured and roof["bound"] == "mfma" else {}),
        },
        "kernels": kernels,
        "frac_of_peak_whole_step": round(value / PEAK_TFLOPS[wls[0].dtype], 4),
        "gpu_event_ms_per_step": round(gpu_ms / args.steps, 5),
        "kernel_source_sha": kernel_source_hash("bwd" if args.backward else "fwd"),
    }
    if args.backward:
        result["config"]["pass"] = "backward"
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = (cpu_baseline_backward(wls, args.cpu_budget) if args.backward
                                  else cpu_baseline(wls, args.cpu_budget))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
