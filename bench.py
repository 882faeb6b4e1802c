#!/usr/bin/env python3
"""Throughput of one tensor-parallel rank's MLP shard on one MI355X.

Workload: the t = 8 shard of a Megatron MLP at hidden 8192 (ffn 32768, f =
4096 per rank) over 16384 tokens.  One step runs ALL 8 rank shards back to
back on the one GPU (Z_r = GeLU(X A_r) B_r, fp32 partials), each through the
C-ABI entry point tp_mlp_shard_fwd; inputs are resident in HBM before the
timed region.  The headline value is TFLOP/s over the step (the per-shard
rate: 8 shards of 4*M*h*f FLOP in the step's time).

Also reported:
  roofline      the dominant kernel (column GEMM + GeLU, or row GEMM), timed
                live with HIP events on the launch stream around each of its
                launches in the step's order (column and row GEMM for every
                rank), against the bf16 dense MFMA peak; ``traffic`` from
                committed rocprofv3 counter summaries when they match the
                current kernel source
  cpu_baseline  the fp64 CPU oracle on a bounded sample of rows of the same
                shard, on this host's cores
  backward      the MLP shard's backward (rank 0 of the same workload): dX_i,
                dA_i, dB_i (fp32) and the first-layer bias gradient from dZ and
                the saved pre-activation, through tp_mlp_shard_bwd
  swiglu        the SwiGLU variant of the same MLP shard (rank 0): gate and
                value projections of width f each, through tp_mlp_swiglu_shard_fwd
  sp_boundary   the sequence-parallel reduce-scatter of the step's 8 fp32
                partials into each rank's [M/8, h] shard with bias and
                residual rows (HBM-bound: GB/s against 8 TB/s)
  attention     the head-local attention shard (hidden 8192, 64 heads of 128,
                t = 8, one sequence of 4096 tokens, rank 0, non-causal): whole
                shard through tp_attn_shard_fwd, its two projection GEMMs
                through tp_column_linear / tp_row_linear at the same shapes,
                and the attention kernel's share as the difference

Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 3]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s + % bf16 MFMA peak, t=8 MLP shard (h=8192, 16384 tok), 1 GPU"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CSRC_DIR = os.path.join(ROOT, "megatron_tensor_transformer_tp_amd", "csrc")


def kernel_sources():
    """Every source the library is built from (csrc/ and the C-ABI header),
    in a fixed order: a change to any of them invalidates the committed
    counter summaries."""
    files = sorted(os.path.join("megatron_tensor_transformer_tp_amd", "csrc", f)
                   for f in os.listdir(CSRC_DIR) if f.endswith((".h", ".hip", ".cpp")))
    return files + [os.path.join("include", "tp_shard.h")]


def _code_only(text: str) -> str:
    """A C++ source without its comments and blank lines (what the compiler
    sees of it, up to formatting)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_sha() -> str:
    """Hash of the kernel sources' code (comments do not count: a comment
    edit leaves the committed counter summaries valid)."""
    h = hashlib.sha256()
    for rel in kernel_sources():
        with open(os.path.join(ROOT, rel), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(wl, target_s: float):
    """Time the fp64 oracle on a bounded sample of the same workload: rows of
    rank 0's shard if a whole shard would exceed the target time, else whole
    rank shards 0, 1, ... until the target time is reached (the MLP is
    row-independent, so tokens/s and FLOP/s are true rates).  Input
    preparation (drawing, widening to fp64) is outside the timed calls."""
    import oracle
    from megatron_tensor_transformer_tp_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1

    def weights(r):
        return (inputs.bf16_bits_to_f32(inputs.mlp_a_block(wl, r)).astype(np.float64),
                inputs.bf16_bits_to_f32(inputs.mlp_b_block(wl, r)).astype(np.float64))

    def run(x, a, b, r) -> float:
        t0 = time.perf_counter()
        h = oracle.column_linear(x, a, apply_gelu=True)
        oracle.row_linear(h, b, rank=r)
        return time.perf_counter() - t0

    a0, b0 = weights(0)
    probe_rows = 128
    t_probe = run(inputs.bf16_bits_to_f32(inputs.mlp_x_rows(wl, 0, probe_rows)).astype(np.float64), a0, b0, 0)
    rows = int(np.clip(probe_rows * target_s / max(t_probe, 1e-6), probe_rows, wl.tokens))
    rows = max(probe_rows, rows // probe_rows * probe_rows)
    x = inputs.bf16_bits_to_f32(inputs.mlp_x_rows(wl, 0, rows)).astype(np.float64)
    elapsed, shards = run(x, a0, b0, 0), 1
    while rows == wl.tokens and elapsed < target_s and shards < wl.t:
        a, b = weights(shards)
        elapsed += run(x, a, b, shards)
        shards += 1
    tokens_done = rows * shards
    flops = 4.0 * tokens_done * wl.hidden * wl.f
    what = (f"rows 0..{rows - 1} of rank 0's shard" if shards == 1 else
            f"rank shards 0..{shards - 1}, all {rows} tokens each")
    return {
        "value": round(flops / elapsed / 1e12, 4),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{what} (hidden {wl.hidden}, f {wl.f}); fp64 NumPy/OpenBLAS matmul + SciPy erfc; "
                   f"{elapsed:.2f} s wall, {tokens_done / elapsed:.1f} shard-tokens/s"),
        "seconds": round(elapsed, 3),
        "tokens_per_s": round(tokens_done / elapsed, 2),
    }


PROFILE_CMDS = {
    "trace": ("rocprofv3 --kernel-trace --stats --output-format csv -d rocprof_out/ktrace -o kt -- "
              "python3 bench.py --steps 10 --warmup 3 --no-cpu-baseline --json-out rocprof_out/ktrace/line.json"),
    "fetch": ("rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/pmc_fetch -o pmc -- "
              "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --kernel-reps 2 --calibrate-copy"),
    "write": ("rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/pmc_write -o pmc -- "
              "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --kernel-reps 2 --calibrate-copy"),
    "mfma": ("rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
             "SQ_INSTS_VALU_MFMA_MOPS_F16 GRBM_GUI_ACTIVE GRBM_COUNT --output-format csv "
             "-d rocprof_out/pmc_mfma -o pmc -- "
             "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --kernel-reps 2"),
}
# The device's SIMD count and XCD count (MI355X: 256 CUs x 4 SIMDs, 8 XCDs):
# MFMA utilisation = sum over SIMDs of SQ_VALU_MFMA_BUSY_CYCLES / (GPU-active
# cycles x SIMDs), rocprofv3's own MfmaUtil expression; the GRBM counters are
# summed over the XCDs in the per-dispatch rows, so one XCD's active cycles
# are the sum / 8, and those cycles over the dispatch's duration are its
# average shader clock.
N_SIMD, N_XCD = 1024, 8
# Profiled kernels: name pattern in the rocprofv3 output and a duration band
# in microseconds that tells the benchmark's shapes of one kernel apart (the
# GEMMs launch one round of resident workgroups whatever the shape, so their
# grids do not), with the per-launch algorithmic work (FLOP, bytes), the
# workload, and the summary's file stem.  GEMM template arguments: tile BM,
# BN, wave grid, LDS stages, A k-major, B k-major, epilogue kind, fp32 output,
# K tail (false: K % 32 == 0), paired stages (0: none, 1: B, 2: A; a
# k-contiguous operand with K % 64 == 0), MFMA (true: 16 x 16 x 32).
_M, _H, _F = 16384, 8192, 4096          # MLP shard: tokens, hidden, f = ffn / t
_M3 = 4096                              # the 4096-token rank shard
_M2, _H2, _F2 = 2048, 1024, 4096        # the t = 1 MLP: tokens, hidden, ffn
_S, _DL = 4096, 1024                    # attention shard: tokens, local width (8 heads x 128)
_GEMM = "gemm_bf16_dma_kernel<256, 256, 2, 4, 4, "   # then A k-major, B k-major, epilogue kind, fp32 out, K tail, pairs
_GEMM128 = "gemm_bf16_dma_kernel<128, 128, 2, 2, 4, "
_INF = 1e9
PROFILED = {
    "column_gemm_gelu": (_GEMM + "false, true, 1, false, false, 2, true>", (500.0, _INF),
                         2.0 * _M * _H * _F, 2 * (_M * _H + _H * _F + _M * _F),
                         "MLP rank shard, M=16384, h=8192, f=4096: X, A_i read, H_i written (bf16)",
                         "column_gemm_gelu_t8_h8192_m16384"),
    "row_gemm": (_GEMM + "false, true, 0, true, false, 2, true>", (500.0, _INF),
                 2.0 * _M * _F * _H, 2 * (_M * _F + _F * _H) + 4 * _M * _H,
                 "MLP rank shard, M=16384, h=8192, f=4096: H_i, B_i read (bf16), Z_i written (fp32)",
                 "row_gemm_t8_h8192_m16384"),
    "t8_h8192_m4096:column_gemm_gelu": (_GEMM + "false, true, 1, false, false, 2, true>", (100.0, 500.0),
                                        2.0 * _M3 * _H * _F, 2 * (_M3 * _H + _H * _F + _M3 * _F),
                                        "rank 0 of t=8, M=4096, h=8192, f=4096: X, A_0 read, H_0 written (bf16)",
                                        "column_gemm_gelu_t8_h8192_m4096"),
    "t8_h8192_m4096:row_gemm": (_GEMM + "false, true, 0, true, false, 2, true>", (140.0, 500.0),
                                2.0 * _M3 * _F * _H, 2 * (_M3 * _F + _F * _H) + 4 * _M3 * _H,
                                "rank 0 of t=8, M=4096, h=8192, f=4096: H_0, B_0 read (bf16), Z_0 written (fp32)",
                                "row_gemm_t8_h8192_m4096"),
    "t1_h1024_m2048:column_gemm_gelu": (_GEMM128 + "false, true, 1, false, false, 2, true>", (0.0, _INF),
                                        2.0 * _M2 * _H2 * _F2, 2 * (_M2 * _H2 + _H2 * _F2 + _M2 * _F2),
                                        "t=1 MLP, M=2048, h=1024, ffn=4096 (128 x 128 tiles): X, A read, "
                                        "H written (bf16)",
                                        "column_gemm_gelu_t1_h1024_m2048"),
    "t1_h1024_m2048:row_gemm": ("gemm_bf16_dma_kernel<64, 128, 1, 4, 4, false, true, 0, false, false, 2, true>", (0.0, _INF),
                                2.0 * _M2 * _F2 * _H2, 2 * (_M2 * _F2 + _F2 * _H2) + 2 * _M2 * _H2,
                                "t=1 MLP, M=2048, ffn=4096, h=1024 (64 x 128 tiles): H, B read, "
                                "Z written (bf16 final output)",
                                "row_gemm_t1_h1024_m2048"),
    "attention_core": ("attn_fwd_kernel<false, false, false>", (0.0, _INF),
                       4.0 * _S * _S * _DL, 2 * (3 * _S * _DL + _S * _DL),
                       "attention rank shard, 8 local heads of 128, seq 4096, non-causal: Q, K "
                       "(fp16) and V (bf16) read once, O written (bf16)",
                       "attention_core_t8_h8192_s4096"),
    "attn_qkv_gemm": ("gemm_bf16_dma_kernel<128, 384, 2, 4, 4, false, true, 4, false, false, 2, true>", (0.0, _INF),
                      2.0 * _S * _H * 3 * _DL, 2 * (_S * _H + _H * 3 * _DL + _S * 3 * _DL),
                      "attention rank shard packed QKV projection, M=4096, K=8192, N=3072 "
                      "(one round of 256 128 x 384 tiles), q/k written as scaled fp16, v as bf16",
                      "attn_qkv_gemm_t8_h8192_s4096"),
    "attn_out_gemm": (_GEMM + "false, true, 0, true, false, 2, true>", (0.0, 140.0),
                      2.0 * _S * _DL * _H, 2 * (_S * _DL + _DL * _H) + 4 * _S * _H,
                      "attention rank shard output projection, M=4096, K=1024, N=8192 (fp32 out)",
                      "attn_out_gemm_t8_h8192_s4096"),
    "sp_reduce_scatter": ("sp_reduce_kernel<unsigned short, unsigned short, true, true>", (0.0, _INF),
                          0.0, 8 * (_M // 8) * _H * 4 + 2 * (_M // 8) * _H * 2 + 2 * _H,
                          "sequence-parallel reduce-scatter of the 8 fp32 MLP partials into one "
                          "rank's [2048, 8192] shard with bf16 bias and residual rows, bf16 out "
                          "(HBM-bound: partial rows, residual and bias read, shard written)",
                          "sp_reduce_scatter_t8_h8192_m16384"),
    "swiglu_gemm": (_GEMM + "false, true, 3, false, false, 2, true>", (0.0, _INF),
                    2.0 * _M * _H * 2 * _F, 2 * (_M * _H + 2 * _H * _F + _M * _F),
                    "SwiGLU column layer, both projections in one product with SiLU(gate) * value "
                    "in the epilogue: X, Wg_i, Wu_i read, H_i written (bf16)",
                    "swiglu_gemm_t8_h8192_m16384"),
    "bwd_dgelu_gemm": (_GEMM + "false, false, 2, false, false, 1, true>", (0.0, _INF),
                       2.0 * _M * _H * _F, 2 * (_M * _H + _F * _H + _M * _F) + 2 * 2 * _M * _F,
                       "MLP shard backward dH = dZ B_i^T with dY_i = dH * GeLU'(Y_i) and H_i = "
                       "GeLU(Y_i) in the epilogue: dZ, B_i, Y_i read, dY_i and H_i written (bf16)",
                       "bwd_dgelu_gemm_t8_h8192_m16384"),
    "bwd_weight_grad_gemm": (_GEMM + "true, true, 0, true, false, 0, true>", (0.0, _INF),
                             2.0 * _M * _H * _F, 2 * (_M * _F + _M * _H) + 4 * _F * _H,
                             "MLP shard backward weight gradients H_i^T dZ and X^T dY_i (one "
                             "kernel, K = 16384 tokens): two bf16 operands read, fp32 [4096 x 8192] "
                             "written; both launches averaged",
                             "bwd_weight_grad_gemm_t8_h8192_m16384"),
    "bwd_dx_gemm": (_GEMM + "false, false, 0, true, false, 1, true>", (0.0, _INF),
                    2.0 * _M * _F * _H, 2 * (_M * _F + _H * _F) + 4 * _M * _H,
                    "MLP shard backward dX_i = dY_i A_i^T: dY_i, A_i read (bf16), dX_i written (fp32)",
                    "bwd_dx_gemm_t8_h8192_m16384"),
}
COPY_KEY = ("copyBuffer", 1 << 30)    # the 1 GiB calibration copy
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")


def load_counters() -> dict:
    """Per-kernel counter figures from the committed summary (profiles/
    counters.json), or {} if there is none or it was taken on a different
    kernel source."""
    try:
        with open(COUNTERS_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return {}
    if data.get("source_sha") != kernel_source_sha():
        return {}
    return data.get("kernels", {})


def summarize_profiles(trace_csv: str, fetch_csv: str, write_csv: str, mfma_csv: str,
                       line_json: str) -> None:
    """Turn the rocprofv3 CSVs of the PROFILE_CMDS runs (the per-dispatch
    kernel trace and the three counter collections) and the bench line the
    traced run printed into the committed summaries: profiles/<file stem>.md
    per profiled kernel and profiles/counters.json.
      HBM bytes = FETCH_SIZE x (1 GiB / FETCH_SIZE of the 1 GiB copy) + the
                  same for WRITE_SIZE (both counters report KiB per dispatch);
      MFMA utilisation, shader clock and MFMA FLOP from the "mfma" pass;
      the dominant kernels' trace durations over exactly the launches the
      bench line's per-kernel figures were timed on (its kernel-timing
      phase), next to those figures."""
    import csv
    import statistics

    def key_of(name, us):
        for key, (pat, band, *_rest) in PROFILED.items():
            if pat in name and band[0] <= us < band[1]:
                return key
        return "copy_1GiB" if COPY_KEY[0] in name else None

    def dur_us(row):
        return (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3

    def per_dispatch(path):
        """{dispatch id: (kernel name, duration us, {counter: value summed over rows})}"""
        out = {}
        for row in csv.DictReader(open(path)):
            d = out.setdefault(row["Dispatch_Id"], [row["Kernel_Name"], dur_us(row), {}])
            c = d[2]
            c[row["Counter_Name"]] = c.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
        return out

    def by_key(path):
        vals = {}
        for name, us, ctr in per_dispatch(path).values():
            key = key_of(name, us)
            if key is not None:
                vals.setdefault(key, []).append((us, ctr))
        return vals

    fetch, write, mfma = by_key(fetch_csv), by_key(write_csv), by_key(mfma_csv)

    def med(vals, key, fn):
        return statistics.median(fn(us, c) for us, c in vals[key]) if key in vals else None

    gib_kib = float(1 << 20)
    f_scale = gib_kib / med(fetch, "copy_1GiB", lambda us, c: c["FETCH_SIZE"])
    w_scale = gib_kib / med(write, "copy_1GiB", lambda us, c: c["WRITE_SIZE"])
    # the trace: dispatches in time order, per key
    durs = {}
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    for row in rows:
        key = key_of(row["Kernel_Name"], dur_us(row))
        if key is not None:
            durs.setdefault(key, []).append((dur_us(row), row["Kernel_Name"]))
    with open(line_json) as fh:
        line = json.load(fh)
    tm = line["timing"]
    # launches of each headline GEMM before its kernel-timing phase: warmup
    # steps, timed steps and one step in between, t launches each
    t = line["config"]["t"]
    first = (tm["warmup"] + tm["steps"] + 1) * t
    phase = slice(first, first + tm["kernel_reps"] * t)

    out = {"source_sha": kernel_source_sha(), "fetch_scale": f_scale, "write_scale": w_scale,
           "n_simd": N_SIMD, "n_xcd": N_XCD, "commands": PROFILE_CMDS, "kernels": {},
           "traced_bench_line": {k: line[k] for k in ("value", "ms_per_step", "roofline", "kernels")}}
    missing = [key for key in PROFILED if key not in durs]
    if missing:
        # a kernel renamed or no longer launched would otherwise leave its
        # old summary in profiles/ looking current
        raise SystemExit(f"no dispatch in the trace matches {missing}: update PROFILED")
    for key, (_pat, _band, flops, alg_bytes, what, stem) in PROFILED.items():
        fb = med(fetch, key, lambda us, c: c["FETCH_SIZE"]) * 1024 * f_scale
        wb = med(write, key, lambda us, c: c["WRITE_SIZE"]) * 1024 * w_scale
        util = med(mfma, key, lambda us, c: c["SQ_VALU_MFMA_BUSY_CYCLES"] /
                   (c["GRBM_GUI_ACTIVE"] / N_XCD * N_SIMD))
        # the counters' window is a few microseconds wider than the dispatch's
        # timestamps (short launches come out above the 2.4 GHz maximum), so
        # the clock is quoted for launches of 150 us and more only
        sclk = med(mfma, key, lambda us, c: c["GRBM_GUI_ACTIVE"] / N_XCD / (us * 1e3))
        if sclk is not None and med(mfma, key, lambda us, c: us) < 150.0:
            sclk = None
        mflops = med(mfma, key, lambda us, c: (c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] +
                                               c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)) * 512.0)
        us = [d for d, _ in durs[key]]
        avg_us = statistics.mean(us)
        ent = {"hbm_bytes_per_launch": int(fb + wb), "fetch_bytes": int(fb), "write_bytes": int(wb),
               "algorithmic_bytes": int(alg_bytes), "avg_us": round(avg_us, 2), "calls": len(us),
               "mfma_util": None if util is None else round(util, 4),
               "sclk_ghz": None if sclk is None else round(sclk, 3),
               "mfma_flops_per_launch": None if mflops is None else int(mflops)}
        phase_us = us[phase] if key in line.get("kernels", {}) else []
        if phase_us:
            ent["phase_avg_us"] = round(statistics.mean(phase_us), 2)
            ent["phase_calls"] = len(phase_us)
        out["kernels"][key] = ent
        md = [f"# {key} — {stem}", "",
              f"Workload: {what}.", "",
              f"kernel: `{durs[key][0][1][:120]}`", f"kernel source sha: {out['source_sha']}", "",
              "Commands (run from the repository root on the MI355X; the summary is written by "
              "`python3 bench.py --summarize-profiles` from their CSV files):", "",
              *[f"    {c}" for c in PROFILE_CMDS.values()], "",
              "| figure | value |", "|---|---|",
              f"| dispatches in the trace run | {len(us)} |",
              f"| average duration | {avg_us:.1f} us |",
              f"| median / min / max duration | {statistics.median(us):.1f} / {min(us):.1f} / {max(us):.1f} us |"]
        if flops:
            md += [f"| algorithmic FLOP per launch | {flops / 1e9:.1f} G |",
                   f"| achieved (algorithmic FLOP / avg duration) | {flops / (avg_us * 1e-6) / 1e12:.1f} TFLOP/s "
                   f"({100 * flops / (avg_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.1f}% of {PEAK_BF16_TFLOPS}) |"]
        else:
            md += [f"| achieved (algorithmic bytes / avg duration) | {alg_bytes / (avg_us * 1e-6) / 1e9:.0f} GB/s "
                   f"({100 * alg_bytes / (avg_us * 1e-6) / 1e9 / PEAK_HBM_GBS:.1f}% of {PEAK_HBM_GBS:.0f}) |"]
        if phase_us:
            live = line["kernels"][key]
            pf = flops / (ent["phase_avg_us"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS
            md += [f"| trace average over the bench's kernel-timing launches ({len(phase_us)}) | "
                   f"{ent['phase_avg_us']:.1f} us -> frac {pf:.4f} |",
                   f"| the same launches timed live by bench.py (HIP events, its JSON line in this run) | "
                   f"{live['avg_us']:.1f} us -> frac {flops / (live['avg_us'] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.4f} |"]
        if util is not None:
            md += [f"| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/8 x 1024 SIMDs), median) | "
                   f"{100 * util:.1f}% |"]
            md += [f"| shader clock (GRBM_GUI_ACTIVE / 8 / duration, median) | {sclk:.3f} GHz |"
                   if sclk is not None else
                   "| shader clock | not quoted: the counter window exceeds a launch this short |"]
            if flops:
                md += [f"| MFMA FLOP per launch ((SQ_INSTS_VALU_MFMA_MOPS_BF16 + _F16) x 512) | {mflops / 1e9:.1f} G "
                       f"({mflops / flops:.3f} x algorithmic) |"]
                if sclk is not None:
                    md += [f"| peak at that clock (2516.6 x clock / 2.4 GHz) | "
                           f"{PEAK_BF16_TFLOPS * sclk / 2.4:.1f} TFLOP/s |"]
        md += [f"| FETCH_SIZE per dispatch (median) | {fb / 1024 / f_scale:.0f} KiB (x{f_scale:.3f} from the 1 GiB copy) |",
               f"| WRITE_SIZE per dispatch (median) | {wb / 1024 / w_scale:.0f} KiB (x{w_scale:.3f}) |",
               f"| HBM bytes per launch (scaled) | {(fb + wb) / 1e6:.1f} MB (fetch {fb / 1e6:.1f}, write {wb / 1e6:.1f}) |",
               f"| algorithmic bytes per launch | {alg_bytes / 1e6:.1f} MB |", ""]
        with open(os.path.join(ROOT, "profiles", f"{stem}.md"), "w") as fh:
            fh.write("\n".join(md))
    with open(COUNTERS_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def _stats(samples):
    """median / min / max of a list of per-call times (us)."""
    return {"median": round(float(np.median(samples)), 2), "min": round(float(min(samples)), 2),
            "max": round(float(max(samples)), 2)}


def time_repeats(call, stream, reps: int, repeats: int = 3, warm: int = 3):
    """Per-call time (us) of ``call`` in ``repeats`` windows of ``reps`` calls
    each, queued back to back on ``stream`` after ``warm`` untimed calls
    (warmup, then three repeats: the fair-benchmark practice of Megatron
    Level 2, M039)."""
    import torch
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    marks = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        marks.append((e0, e1))
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e3 / reps for e0, e1 in marks]


def time_launches(calls, stream, reps: int):
    """Per-launch times (us) of each named call, the calls interleaved in the
    given order ``reps`` times, an event pair around every launch on the
    launch stream."""
    import torch
    events = {name: [] for name in calls}
    for _ in range(reps):
        for name, fn in calls.items():
            k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            k0.record(stream)
            fn()
            k1.record(stream)
            events[name].append((k0, k1))
    torch.cuda.synchronize()
    return {name: [k0.elapsed_time(k1) * 1e3 for k0, k1 in ev] for name, ev in events.items()}


def bench_mlp_config(name: str, rank: int, stream, reps: int, traffic: dict):
    """One MLP workload's shard on its own: tp_mlp_shard_fwd timed in three
    repeats, and its two GEMMs (tp_column_linear with GeLU, tp_row_linear)
    per launch, with algorithmic and (from the committed counters) measured
    HBM bytes per launch."""
    import torch
    from megatron_tensor_transformer_tp_amd import binding, inputs

    wl = inputs.MLP_WORKLOADS[name]
    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    out_dt = torch.float32 if wl.out_dtype == "f32" else torch.bfloat16
    ob = 4 if wl.out_dtype == "f32" else 2
    x, a, b = up(inputs.mlp_x_rows(wl)), up(inputs.mlp_a_block(wl, rank)), up(inputs.mlp_b_block(wl, rank))
    z = torch.empty((wl.tokens, wl.hidden), dtype=out_dt, device=dev)
    ws = torch.empty(binding.tp_mlp_shard_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t,
                                                          torch.bfloat16), dtype=torch.uint8, device=dev)
    h = ws[: wl.tokens * wl.f * 2].view(torch.bfloat16).view(wl.tokens, wl.f)
    shard = time_repeats(lambda: binding.tp_mlp_shard_fwd(x, a, b, z, ws, ffn=wl.ffn, t=wl.t, rank=rank,
                                                          stream=stream), stream, reps)
    per = time_launches({
        "column_gemm_gelu": lambda: binding.tp_column_linear(x, a, h, ffn=wl.ffn, t=wl.t, rank=rank,
                                                             apply_gelu=True, stream=stream),
        "row_gemm": lambda: binding.tp_row_linear(h, b, z, ffn=wl.ffn, t=wl.t, rank=rank, stream=stream),
    }, stream, reps)
    flops = wl.flops_per_shard()
    gemm_flops = 2.0 * wl.tokens * wl.hidden * wl.f
    alg = {"column_gemm_gelu": 2.0 * (wl.tokens * wl.hidden + wl.hidden * wl.f + wl.tokens * wl.f),
           "row_gemm": 2.0 * (wl.tokens * wl.f + wl.f * wl.hidden) + ob * wl.tokens * wl.hidden}
    med = float(np.median(shard))
    kernels = {}
    for k, us_list in per.items():
        us = float(np.mean(us_list))
        ent = {"avg_us": round(us, 2), "tflops": round(gemm_flops / (us * 1e-6) / 1e12, 2),
               "algorithmic_bytes": int(alg[k]),
               "algorithmic_gbs": round(alg[k] / (us * 1e-6) / 1e9, 1)}
        hbm = traffic.get(f"{name}:{k}")
        if hbm is not None:
            ent["hbm_bytes"] = int(hbm)
            ent["hbm_gbs"] = round(hbm / (us * 1e-6) / 1e9, 1)
            ent["frac_hbm"] = round(hbm / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        kernels[k] = ent
    res = {
        "workload": (f"{wl.name}: rank {rank} of t={wl.t}, {wl.tokens} tokens, hidden {wl.hidden}, "
                     f"ffn {wl.ffn} (f {wl.f}), {wl.out_dtype} "
                     f"{'final output' if wl.t == 1 else 'partial'}"),
        "flops": int(flops),
        "us": _stats(shard),
        "tflops": round(flops / (med * 1e-6) / 1e12, 2),
        "pct_peak": round(100.0 * flops / (med * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(wl.tokens / (med * 1e-6), 1),
        "kernels": kernels,
    }
    log(f"{name} rank {rank}: shard {med:.1f} us (min {min(shard):.1f}, max {max(shard):.1f}), "
        f"{res['tflops']} TFLOP/s; " + ", ".join(f"{k} {v['avg_us']} us" for k, v in kernels.items()))
    return res


def bench_swiglu(wl, x, b0, stream, reps: int):
    """Time tp_mlp_swiglu_shard_fwd on rank 0 of the MLP workload."""
    import torch
    from megatron_tensor_transformer_tp_amd import binding, inputs

    dev = x.device

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    wg, wu = up(inputs.mlp_wg_block(wl, 0)), up(inputs.mlp_wu_block(wl, 0))
    z = torch.empty((wl.tokens, wl.hidden), dtype=torch.float32, device=dev)
    ws = torch.empty(binding.tp_mlp_swiglu_shard_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t,
                                                                 torch.bfloat16), dtype=torch.uint8, device=dev)

    def call():
        binding.tp_mlp_swiglu_shard_fwd(x, wg, wu, b0, z, ws, ffn=wl.ffn, t=wl.t, rank=0, stream=stream)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    flops = 6.0 * wl.tokens * wl.hidden * wl.f
    res = {
        "workload": (f"{wl.name} rank 0, SwiGLU: H_i = SiLU(X Wg_i) * (X Wu_i) (one product over "
                     f"both [{wl.hidden}, {wl.f}] projections), Z_i = H_i B_i, fp32 partial"),
        "flops": int(flops),
        "us": round(us, 2),
        "tflops": round(flops / (us * 1e-6) / 1e12, 2),
        "pct_peak": round(100.0 * flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2),
    }
    log(f"swiglu shard {us:.1f} us ({res['tflops']} TFLOP/s)")
    return res


def bench_sp(wl, z, stream, reps: int):
    """Time tp_sp_reduce_scatter over the step's t partials, every rank in
    turn, bf16 bias / residual rows / output."""
    import torch
    from megatron_tensor_transformer_tp_amd import binding, inputs

    dev = z[0].device
    rows = wl.tokens // wl.t
    bias = torch.from_numpy(inputs.mlp_bias_b(wl).view(np.int16)).to(dev).view(torch.bfloat16)
    res = torch.from_numpy(inputs.mlp_residual_rows(wl, 0, rows).view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((rows, wl.hidden), dtype=torch.bfloat16, device=dev)

    def call(r):
        binding.tp_sp_reduce_scatter(z, out, t=wl.t, rank=r, bias=bias, residual_r=res, stream=stream)

    for r in range(wl.t):
        call(r)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps * wl.t):
        call(i % wl.t)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * wl.t)
    nbytes = wl.t * rows * wl.hidden * 4 + 2 * rows * wl.hidden * 2 + 2 * wl.hidden
    res_d = {
        "workload": (f"{wl.name}: one rank's sequence shard [{rows}, {wl.hidden}] of the sum of the "
                     f"{wl.t} fp32 partials, bf16 bias / residual rows / output"),
        "us": round(us, 2),
        "algorithmic_bytes": int(nbytes),
        "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
        "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
    }
    log(f"sp reduce-scatter {us:.1f} us per rank ({res_d['gbs']} GB/s)")
    return res_d


def bench_backward(wl, x, a0, b0, stream, reps: int):
    """Time tp_mlp_shard_bwd on rank 0 of the MLP workload (inputs resident)."""
    import torch
    from megatron_tensor_transformer_tp_amd import binding, inputs

    dev = x.device
    dz = torch.from_numpy(inputs.mlp_dz_rows(wl).view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((wl.tokens, wl.f), dtype=torch.bfloat16, device=dev)
    z = torch.empty((wl.tokens, wl.hidden), dtype=torch.float32, device=dev)
    fws = torch.empty(binding.tp_mlp_shard_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t,
                                                           torch.bfloat16), dtype=torch.uint8, device=dev)
    binding.tp_mlp_shard_fwd(x, a0, b0, z, fws, ffn=wl.ffn, t=wl.t, rank=0, y_save=y, stream=stream)
    del z, fws
    dx = torch.empty((wl.tokens, wl.hidden), dtype=torch.float32, device=dev)
    da = torch.empty((wl.hidden, wl.f), dtype=torch.float32, device=dev)
    db = torch.empty((wl.f, wl.hidden), dtype=torch.float32, device=dev)
    dba = torch.empty((wl.f,), dtype=torch.float32, device=dev)
    ws = torch.empty(binding.tp_mlp_shard_bwd_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t,
                                                              torch.bfloat16), dtype=torch.uint8, device=dev)

    def call():
        binding.tp_mlp_shard_bwd(x, a0, b0, y, dz, dx, da, db, ws, ffn=wl.ffn, t=wl.t, rank=0,
                                 dbias_a_i=dba, stream=stream)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    flops = 8.0 * wl.tokens * wl.hidden * wl.f
    res = {
        "workload": (f"{wl.name} rank 0: dH = dZ B_i^T with the GeLU-backward epilogue, "
                     "dB_i = H_i^T dZ, dA_i = X^T dY_i, dX_i = dY_i A_i^T (fp32 gradients), "
                     "first-layer bias gradient"),
        "flops": int(flops),
        "us": round(us, 2),
        "tflops": round(flops / (us * 1e-6) / 1e12, 2),
        "pct_peak": round(100.0 * flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(wl.tokens / (us * 1e-6), 1),
    }
    log(f"backward shard {us:.1f} us ({res['tflops']} TFLOP/s)")
    return res


def bench_attention(stream, reps: int, name: str = "attn_t8_h8192_s4096"):
    """Time one head-local attention shard (rank 0, non-causal; the causal
    form beside it) and its two projection GEMMs; the attention kernel's
    time is the difference."""
    import torch
    from megatron_tensor_transformer_tp_amd import binding, inputs

    wl = inputs.ATTN_WORKLOADS[name]
    dev = torch.device("cuda:0")
    nl = wl.heads // wl.t
    dl = nl * wl.head_dim
    tokens = wl.batch * wl.seq

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    x = up(np.stack([inputs.attn_x(wl, b) for b in range(wl.batch)]))
    wqkv, wo = up(inputs.attn_wqkv_block(wl, 0)), up(inputs.attn_wo_block(wl, 0))
    out = torch.empty((wl.batch, wl.seq, wl.hidden), dtype=torch.float32, device=dev)
    ws = torch.empty(binding.tp_attn_shard_workspace_bytes(wl.batch, wl.seq, wl.hidden, wl.heads,
                                                           wl.head_dim, wl.t, torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    qkv = torch.empty((tokens, 3 * dl), dtype=torch.bfloat16, device=dev)
    o = torch.empty((tokens, dl), dtype=torch.bfloat16, device=dev).normal_()
    x2 = x.view(tokens, wl.hidden)
    out2 = out.view(tokens, wl.hidden)
    calls = {
        "shard": lambda: binding.tp_attn_shard_fwd(x, wqkv, wo, out, ws, heads=wl.heads,
                                                   head_dim=wl.head_dim, t=wl.t, rank=0,
                                                   stream=stream),
        "shard_causal": lambda: binding.tp_attn_shard_fwd(x, wqkv, wo, out, ws, heads=wl.heads,
                                                          head_dim=wl.head_dim, t=wl.t, rank=0,
                                                          causal=True, stream=stream),
        "qkv_gemm": lambda: binding.tp_column_linear(x2, wqkv, qkv, ffn=3 * wl.hidden, t=wl.t,
                                                     rank=0, stream=stream),
        "out_gemm": lambda: binding.tp_row_linear(o, wo, out2, ffn=wl.hidden, t=wl.t, rank=0,
                                                  stream=stream),
    }
    # Sustained-state timing: the part's clock drops by up to ~20% within a
    # few milliseconds of this loop, so the shard first runs 120 times
    # (~45 ms) untimed; then the three timings interleave (order alternating by
    # round), all queued back to back on the stream with no host sync
    # between them, and each takes its median over the rounds.  The GEMMs
    # alone thus see the same clock as the shard whose share they give.
    for _ in range(120):
        calls["shard"]()
    torch.cuda.synchronize()
    per = 5
    marks = {key: [] for key in calls}
    for rnd in range(max(reps, 3)):
        for key in (list(calls) if rnd % 2 == 0 else list(calls)[::-1]):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(per):
                calls[key]()
            e1.record(stream)
            marks[key].append((e0, e1))
    torch.cuda.synchronize()
    samples = {key: [e0.elapsed_time(e1) * 1e3 / per for e0, e1 in v] for key, v in marks.items()}
    us = {key: float(np.median(v)) for key, v in samples.items()}
    f_qkv = 2.0 * tokens * wl.hidden * 3 * dl
    f_att = 4.0 * wl.batch * wl.seq * wl.seq * wl.head_dim * nl   # Q K^T and P V, non-causal
    f_out = 2.0 * tokens * dl * wl.hidden
    core_us = us["shard"] - us["qkv_gemm"] - us["out_gemm"]
    core_causal_us = us["shard_causal"] - us["qkv_gemm"] - us["out_gemm"]
    # causal: each query's keys up to itself, seq (seq + 1) / 2 pairs per head
    f_att_causal = 2.0 * wl.batch * wl.seq * (wl.seq + 1) * wl.head_dim * nl

    def tf(flops, t_us):
        return round(flops / (t_us * 1e-6) / 1e12, 2)

    res = {
        "workload": (f"{wl.name}: rank 0 of t={wl.t}, hidden {wl.hidden}, {wl.heads} heads of "
                     f"{wl.head_dim} ({nl} local), batch {wl.batch} x seq {wl.seq}, non-causal, "
                     "fp32 partial"),
        "flops": int(f_qkv + f_att + f_out),
        "shard_us": round(us["shard"], 2),
        "shard_tflops": tf(f_qkv + f_att + f_out, us["shard"]),
        "pct_peak": round(100.0 * (f_qkv + f_att + f_out) / (us["shard"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "qkv_gemm": {"avg_us": round(us["qkv_gemm"], 2), "tflops": tf(f_qkv, us["qkv_gemm"])},
        "attention_core": {"avg_us": round(core_us, 2), "tflops": tf(f_att, core_us),
                           "note": "shard time minus the two projection GEMMs timed alone, "
                                   "interleaved with the shard in the sustained clock state "
                                   "(medians over rounds)"},
        "out_gemm": {"avg_us": round(us["out_gemm"], 2), "tflops": tf(f_out, us["out_gemm"])},
        "causal": {"shard_us": round(us["shard_causal"], 2),
                   "attention_core": {"avg_us": round(core_causal_us, 2),
                                      "tflops": tf(f_att_causal, core_causal_us),
                                      "flops": int(f_att_causal)}},
    }
    log(f"attention shard {us['shard']:.1f} us ({res['shard_tflops']} TFLOP/s): qkv {us['qkv_gemm']:.1f}, "
        f"core ~{core_us:.1f} ({res['attention_core']['tflops']} TFLOP/s), out {us['out_gemm']:.1f}; "
        f"causal shard {us['shard_causal']:.1f} us, core ~{core_causal_us:.1f} "
        f"({res['causal']['attention_core']['tflops']} TFLOP/s)")
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="t8_h8192_m16384")
    ap.add_argument("--kernel-reps", type=int, default=10,
                    help="passes over the step's launches (and launches per kernel elsewhere) "
                         "for the live per-kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the attention-shard measurement")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the MLP-backward measurement")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the t=1 2048-token and the 4096-token rank-shard workloads")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the bounded oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--json-out", help="also write the JSON line to this file")
    ap.add_argument("--summarize-profiles", nargs=5,
                    metavar=("TRACE_CSV", "FETCH_CSV", "WRITE_CSV", "MFMA_CSV", "TRACED_LINE_JSON"),
                    help="write profiles/ summaries from the rocprofv3 CSVs of PROFILE_CMDS and exit")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's shard only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path: the exchange step (a SUM All-Reduce of the "
              "partials) is not implemented.", file=sys.stderr)
        return 2

    import torch
    from megatron_tensor_transformer_tp_amd import binding, inputs

    if not os.path.exists(binding.LIB_PATH):
        from megatron_tensor_transformer_tp_amd.build import build
        build()
    binding.lib()
    wl = inputs.MLP_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    counters = load_counters()

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    log(f"workload {wl.name}: tokens {wl.tokens}, hidden {wl.hidden}, ffn {wl.ffn}, t {wl.t}")
    t_gen = time.perf_counter()
    x = up(inputs.mlp_x_rows(wl))
    a = [up(inputs.mlp_a_block(wl, r)) for r in range(wl.t)]
    b = [up(inputs.mlp_b_block(wl, r)) for r in range(wl.t)]
    out_dt = torch.float32 if wl.out_dtype == "f32" else torch.bfloat16
    z = [torch.empty((wl.tokens, wl.hidden), dtype=out_dt, device=dev) for _ in range(wl.t)]
    ws = torch.empty(binding.tp_mlp_shard_workspace_bytes(wl.tokens, wl.hidden, wl.ffn, wl.t,
                                                          torch.bfloat16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"inputs generated and resident in HBM ({time.perf_counter() - t_gen:.1f} s)")

    def step():
        for r in range(wl.t):
            binding.tp_mlp_shard_fwd(x, a[r], b[r], z[r], ws, ffn=wl.ffn, t=wl.t, rank=r, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # The K timed steps, one window bracketed by synchronisations; events at
    # the thirds of the window give three repeats of the same steps (median,
    # min, max of their per-step times), without timing any step twice.
    cuts = sorted({0, args.steps // 3, (2 * args.steps) // 3, args.steps})
    evs = [torch.cuda.Event(enable_timing=True) for _ in cuts]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(args.steps + 1):
        if i in cuts:
            evs[cuts.index(i)].record(stream)
        if i < args.steps:
            step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    sub = [evs[j].elapsed_time(evs[j + 1]) / (cuts[j + 1] - cuts[j]) for j in range(len(cuts) - 1)]
    flops_step = wl.flops_per_shard() * wl.t
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (events), wall {wall * 1e3 / args.steps:.3f} ms/step; "
        f"thirds {', '.join(f'{v:.3f}' for v in sub)} ms/step")

    # ---- per-kernel live timing, in the step's context: the step's launches
    # in the step's order (column then row GEMM for every rank's operands,
    # the same kernels tp_mlp_shard_fwd runs), an event pair around each on
    # the launch stream; a kernel repeated alone runs a few percent faster
    # than between the other one's launches.
    h_view = ws[: wl.tokens * wl.f * 2].view(torch.bfloat16).view(wl.tokens, wl.f)
    kernels = {
        "column_gemm_gelu": (lambda r: binding.tp_column_linear(x, a[r], h_view, ffn=wl.ffn, t=wl.t, rank=r,
                                                                apply_gelu=True, stream=stream),
                             2.0 * wl.tokens * wl.hidden * wl.f,
                             # algorithmic bytes: X + A_i read, H written (bf16)
                             2.0 * (wl.tokens * wl.hidden + wl.hidden * wl.f + wl.tokens * wl.f)),
        "row_gemm": (lambda r: binding.tp_row_linear(h_view, b[r], z[r], ffn=wl.ffn, t=wl.t, rank=r,
                                                     stream=stream),
                     2.0 * wl.tokens * wl.f * wl.hidden,
                     # H + B_i read (bf16), Z written (fp32)
                     2.0 * (wl.tokens * wl.f + wl.f * wl.hidden) + 4.0 * wl.tokens * wl.hidden),
    }
    step()
    torch.cuda.synchronize()
    # one event between consecutive launches (chained), so that each launch's
    # interval carries one event record rather than two
    events = {name: [] for name in kernels}
    prev = torch.cuda.Event(enable_timing=True)
    prev.record(stream)
    for _ in range(args.kernel_reps):
        for r in range(wl.t):
            for name, (fn, _f, _b) in kernels.items():
                fn(r)
                nxt = torch.cuda.Event(enable_timing=True)
                nxt.record(stream)
                events[name].append((prev, nxt))
                prev = nxt
    torch.cuda.synchronize()
    per_kernel = {}
    for name, (fn, flops, nbytes) in kernels.items():
        us = sum(k0.elapsed_time(k1) for k0, k1 in events[name]) * 1e3 / len(events[name])
        per_kernel[name] = {"avg_us": round(us, 2), "tflops": round(flops / (us * 1e-6) / 1e12, 2),
                            "algorithmic_bytes": int(nbytes), "flops": int(flops),
                            "launches": len(events[name])}
        log(f"kernel {name}: {us:.1f} us/launch in the step's order, {flops / (us * 1e-6) / 1e12:.1f} TFLOP/s")
    dom = max(per_kernel, key=lambda k: per_kernel[k]["avg_us"])
    achieved = per_kernel[dom]["tflops"]
    ctr = counters.get(dom, {})
    roofline = {
        "bound": "mfma",
        "kernel": dom,
        "achieved": achieved,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": ctr.get("hbm_bytes_per_launch"),
        "algorithmic_bytes": per_kernel[dom]["algorithmic_bytes"],
        "avg_us": per_kernel[dom]["avg_us"],
    }
    if ctr.get("sclk_ghz"):
        # counter evidence from the committed profile of the same kernel
        # source: the matrix pipes' busy fraction and the shader clock the
        # part held during the kernel (it is power-limited under MFMA load),
        # and the achieved rate against the peak at that clock
        at_clk = PEAK_BF16_TFLOPS * ctr["sclk_ghz"] / 2.4
        roofline.update({"mfma_util": ctr.get("mfma_util"), "sclk_ghz": ctr["sclk_ghz"],
                         "peak_at_sclk": round(at_clk, 1), "frac_at_sclk": round(achieved / at_clk, 4)})
    for name, ent in per_kernel.items():
        c = counters.get(name, {})
        for k in ("mfma_util", "sclk_ghz", "hbm_bytes_per_launch"):
            if c.get(k) is not None:
                ent[k] = c[k]

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy of 1 GiB x3 done")

    sp_boundary = bench_sp(wl, z, stream, args.kernel_reps)
    swiglu = bench_swiglu(wl, x, b[0], stream, args.kernel_reps)
    backward = None if args.no_backward else bench_backward(wl, x, a[0], b[0], stream,
                                                            args.kernel_reps)
    del a[1:], b[1:], z[1:]
    attention = None if args.no_attention else bench_attention(stream, args.kernel_reps)
    secondary = None
    if not args.no_secondary:
        hbm = {k: v.get("hbm_bytes_per_launch") for k, v in counters.items() if ":" in k}
        secondary = {
            "t1_h1024_m2048": bench_mlp_config("t1_h1024_m2048", 0, stream, max(args.kernel_reps, 20) * 5, hbm),
            "t8_h8192_m4096": bench_mlp_config("t8_h8192_m4096", 0, stream, max(args.kernel_reps, 10), hbm),
        }

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle on a bounded sample")
        cpu = cpu_baseline(wl, args.cpu_seconds)
        log(f"cpu baseline: {cpu['sample']}")

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, rounded to bf16)",
        "config": {
            "workload": (f"{wl.name}: all {wl.t} rank shards of a t={wl.t} Megatron MLP "
                         f"(hidden {wl.hidden}, ffn {wl.ffn}, f {wl.f}) over {wl.tokens} tokens, "
                         "back to back per step; fp32 partial sums"),
            "tokens": wl.tokens, "hidden": wl.hidden, "ffn": wl.ffn, "t": wl.t,
            "shards_per_step": wl.t, "parallelism": "one rank's shard per launch, 1 GPU",
        },
        "pct_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "ms_per_shard": round(ms_step / wl.t, 4),
        "tokens_per_s_per_shard": round(wl.tokens / (ms_step / wl.t * 1e-3), 1),
        "repeats": {"windows": len(sub), "ms_per_step": [round(v, 4) for v in sub],
                    **{k: round(v / 1e3, 4) for k, v in _stats([u * 1e3 for u in sub]).items()},
                    "tflops_median": round(flops_step / (float(np.median(sub)) * 1e-3) / 1e12, 2)},
        "timing": {"warmup": args.warmup, "steps": args.steps, "kernel_reps": args.kernel_reps},
        "roofline": roofline,
        "kernels": per_kernel,
        "kernel_source_sha": kernel_source_sha(),
        "counters_valid": bool(counters),
        "cpu_baseline": cpu,
        "secondary": secondary,
        "swiglu": swiglu,
        "sp_boundary": sp_boundary,
        "backward": backward,
        "attention": attention,
    }
    line = json.dumps(result)
    print(line, flush=True)
    if args.json_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.json_out)), exist_ok=True)
        with open(args.json_out, "w") as fh:
            fh.write(line + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
