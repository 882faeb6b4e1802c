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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
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


def load_traffic(kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed counter summary, or
    None if there is none or it was taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    if data.get("source_sha") != kernel_source_sha():
        return None
    entry = data.get("kernels", {}).get(kernel)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


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
              "python3 bench.py --steps 10 --warmup 3 --no-cpu-baseline"),
    "fetch": ("rocprofv3 --pmc FETCH_SIZE --output-format csv -d rocprof_out/pmc_fetch -o pmc -- "
              "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --kernel-reps 2 --calibrate-copy"),
    "write": ("rocprofv3 --pmc WRITE_SIZE --output-format csv -d rocprof_out/pmc_write -o pmc -- "
              "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline --kernel-reps 2 --calibrate-copy"),
}
# Profiled kernels: name pattern in the rocprofv3 output and, where one
# kernel serves several of the benchmark's shapes, a selector of the dispatch
# (an int: grid size in work-items; ("us", lo, hi): duration band in
# microseconds — the GEMMs run one round of resident workgroups whatever the
# shape, so their grids do not tell shapes apart), with the per-launch
# algorithmic work (FLOP, bytes), the workload, and the summary's file stem.
# GEMM template arguments: tile BM, BN, wave grid, LDS stages, A k-major,
# B k-major, epilogue kind, fp32 output, K tail (false: K % 32 == 0), paired
# stages (0: none, 1: B, 2: A; a k-contiguous operand with K % 64 == 0).
_M, _H, _F = 16384, 8192, 4096          # MLP shard: tokens, hidden, f = ffn / t
_S, _DL = 4096, 1024                    # attention shard: tokens, local width (8 heads x 128)
_GEMM = "gemm_bf16_dma_kernel<256, 256, 2, 4, 4, "   # then A k-major, B k-major, epilogue kind, fp32 out, K tail, pairs
PROFILED = {
    "column_gemm_gelu": (_GEMM + "false, true, 1, false, false, 0>", None,
                         2.0 * _M * _H * _F, 2 * (_M * _H + _H * _F + _M * _F),
                         "MLP rank shard, M=16384, h=8192, f=4096: X, A_i read, H_i written (bf16)",
                         "column_gemm_gelu_t8_h8192_m16384"),
    "row_gemm": (_GEMM + "false, true, 0, true, false, 0>", ("us", 300.0, 1e9),
                 2.0 * _M * _F * _H, 2 * (_M * _F + _F * _H) + 4 * _M * _H,
                 "MLP rank shard, M=16384, h=8192, f=4096: H_i, B_i read (bf16), Z_i written (fp32)",
                 "row_gemm_t8_h8192_m16384"),
    "attention_core": ("attn_fwd_kernel<false>", None,
                       4.0 * _S * _S * _DL, 2 * (3 * _S * _DL + _S * _DL),
                       "attention rank shard, 8 local heads of 128, seq 4096, non-causal: Q, K "
                       "(fp16) and V (bf16) read once, O written (bf16)",
                       "attention_core_t8_h8192_s4096"),
    "attn_qkv_gemm": ("gemm_bf16_dma_kernel<128, 384, 2, 4, 4, false, true, 4, false, false, 2>", None,
                      2.0 * _S * _H * 3 * _DL, 2 * (_S * _H + _H * 3 * _DL + _S * 3 * _DL),
                      "attention rank shard packed QKV projection, M=4096, K=8192, N=3072 "
                      "(one round of 256 128 x 384 tiles), q/k written as scaled fp16, v as bf16",
                      "attn_qkv_gemm_t8_h8192_s4096"),
    "attn_out_gemm": (_GEMM + "false, true, 0, true, false, 0>", ("us", 0.0, 300.0),
                      2.0 * _S * _DL * _H, 2 * (_S * _DL + _DL * _H) + 4 * _S * _H,
                      "attention rank shard output projection, M=4096, K=1024, N=8192 (fp32 out)",
                      "attn_out_gemm_t8_h8192_s4096"),
    "sp_reduce_scatter": ("sp_reduce_kernel<unsigned short, unsigned short, true, true>", 8192 * 256,
                          0.0, 8 * (_M // 8) * _H * 4 + 2 * (_M // 8) * _H * 2 + 2 * _H,
                          "sequence-parallel reduce-scatter of the 8 fp32 MLP partials into one "
                          "rank's [2048, 8192] shard with bf16 bias and residual rows, bf16 out "
                          "(HBM-bound: partial rows, residual and bias read, shard written)",
                          "sp_reduce_scatter_t8_h8192_m16384"),
    "swiglu_gemm": (_GEMM + "false, true, 3, false, false, 0>", None,
                    2.0 * _M * _H * 2 * _F, 2 * (_M * _H + 2 * _H * _F + _M * _F),
                    "SwiGLU column layer, both projections in one product with SiLU(gate) * value "
                    "in the epilogue: X, Wg_i, Wu_i read, H_i written (bf16)",
                    "swiglu_gemm_t8_h8192_m16384"),
    "bwd_dgelu_gemm": (_GEMM + "false, false, 2, false, false, 1>", None,
                       2.0 * _M * _H * _F, 2 * (_M * _H + _F * _H + _M * _F) + 2 * 2 * _M * _F,
                       "MLP shard backward dH = dZ B_i^T with dY_i = dH * GeLU'(Y_i) and H_i = "
                       "GeLU(Y_i) in the epilogue: dZ, B_i, Y_i read, dY_i and H_i written (bf16)",
                       "bwd_dgelu_gemm_t8_h8192_m16384"),
    "bwd_weight_grad_gemm": (_GEMM + "true, true, 0, true, false, 0>", None,
                             2.0 * _M * _H * _F, 2 * (_M * _F + _M * _H) + 4 * _F * _H,
                             "MLP shard backward weight gradients H_i^T dZ and X^T dY_i (one "
                             "kernel, K = 16384 tokens): two bf16 operands read, fp32 [4096 x 8192] "
                             "written; both launches averaged",
                             "bwd_weight_grad_gemm_t8_h8192_m16384"),
    "bwd_dx_gemm": (_GEMM + "false, false, 0, true, false, 1>", None,
                    2.0 * _M * _F * _H, 2 * (_M * _F + _H * _F) + 4 * _M * _H,
                    "MLP shard backward dX_i = dY_i A_i^T: dY_i, A_i read (bf16), dX_i written (fp32)",
                    "bwd_dx_gemm_t8_h8192_m16384"),
}
COPY_KEY = ("copyBuffer", 1 << 30)    # the 1 GiB calibration copy


def summarize_profiles(trace_csv: str, fetch_csv: str, write_csv: str) -> None:
    """Turn the rocprofv3 CSVs of the three PROFILE_CMDS runs (the per-dispatch
    kernel trace and the two counter collections) into the committed
    summaries: profiles/<file stem>.md per profiled kernel and
    profiles/traffic_counters.json.  HBM bytes = FETCH_SIZE x (1 GiB / FETCH_SIZE
    of the 1 GiB copy) + the same for WRITE_SIZE (both counters report KiB per
    dispatch)."""
    import csv
    import statistics

    def key_of(name, grid, us):
        for key, (pat, sel, *_rest) in PROFILED.items():
            if pat not in name:
                continue
            if sel is None or (isinstance(sel, int) and sel == grid) or \
                    (isinstance(sel, tuple) and sel[1] <= us < sel[2]):
                return key
        return "copy_1GiB" if COPY_KEY[0] in name else None

    def dur_us(row):
        return (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3

    def per_kernel_counter(path):
        vals = {}
        for row in csv.DictReader(open(path)):
            key = key_of(row["Kernel_Name"], int(row["Grid_Size"]), dur_us(row))
            if key is not None:
                vals.setdefault(key, []).append(float(row["Counter_Value"]))
        return {k: statistics.median(v) for k, v in vals.items()}

    fetch, write = per_kernel_counter(fetch_csv), per_kernel_counter(write_csv)
    gib_kib = float(1 << 20)
    f_scale, w_scale = gib_kib / fetch["copy_1GiB"], gib_kib / write["copy_1GiB"]
    durs = {}
    for row in csv.DictReader(open(trace_csv)):
        grid = int(row["Grid_Size_X"]) * int(row["Grid_Size_Y"]) * int(row["Grid_Size_Z"])
        key = key_of(row["Kernel_Name"], grid, dur_us(row))
        if key is not None:
            durs.setdefault(key, []).append((dur_us(row), row["Kernel_Name"]))
    out = {"source_sha": kernel_source_sha(), "fetch_scale": f_scale, "write_scale": w_scale,
           "commands": PROFILE_CMDS, "kernels": {}}
    for key, (_pat, _grid, flops, alg_bytes, what, stem) in PROFILED.items():
        fb = fetch[key] * 1024 * f_scale
        wb = write[key] * 1024 * w_scale
        us = [d for d, _ in durs[key]]
        avg_us = statistics.mean(us)
        out["kernels"][key] = {"hbm_bytes_per_launch": int(fb + wb), "fetch_bytes": int(fb),
                               "write_bytes": int(wb), "algorithmic_bytes": int(alg_bytes),
                               "avg_us": round(avg_us, 2), "calls": len(us)}
        md = [f"# {key} — {stem}", "",
              f"Workload: {what}.", "",
              f"kernel: `{durs[key][0][1][:120]}`", f"kernel source sha: {out['source_sha']}", "",
              "Commands (run from the repository root on the MI355X):", "",
              *[f"    {c}" for c in PROFILE_CMDS.values()], "",
              "| figure | value |", "|---|---|",
              f"| dispatches in the trace run | {len(us)} |",
              f"| average duration | {avg_us:.1f} us |",
              f"| median / min / max duration | {statistics.median(us):.1f} / {min(us):.1f} / {max(us):.1f} us |",
              *([f"| algorithmic FLOP per launch | {flops / 1e9:.1f} G |",
                 f"| achieved (algorithmic FLOP / avg duration) | {flops / (avg_us * 1e-6) / 1e12:.1f} TFLOP/s "
                 f"({100 * flops / (avg_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.1f}% of {PEAK_BF16_TFLOPS}) |"]
                if flops else
                [f"| achieved (algorithmic bytes / avg duration) | {alg_bytes / (avg_us * 1e-6) / 1e9:.0f} GB/s "
                 f"({100 * alg_bytes / (avg_us * 1e-6) / 1e9 / PEAK_HBM_GBS:.1f}% of {PEAK_HBM_GBS:.0f}) |"]),
              f"| FETCH_SIZE per dispatch (median) | {fetch[key]:.0f} KiB (x{f_scale:.3f} from the 1 GiB copy) |",
              f"| WRITE_SIZE per dispatch (median) | {write[key]:.0f} KiB (x{w_scale:.3f}) |",
              f"| HBM bytes per launch (scaled) | {(fb + wb) / 1e6:.1f} MB (fetch {fb / 1e6:.1f}, write {wb / 1e6:.1f}) |",
              f"| algorithmic bytes per launch | {alg_bytes / 1e6:.1f} MB |", ""]
        with open(os.path.join(ROOT, "profiles", f"{stem}.md"), "w") as fh:
            fh.write("\n".join(md))
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


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
    """Time one head-local attention shard (rank 0, non-causal) and its two
    projection GEMMs; the attention kernel's time is the difference."""
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
    }
    log(f"attention shard {us['shard']:.1f} us ({res['shard_tflops']} TFLOP/s): qkv {us['qkv_gemm']:.1f}, "
        f"core ~{core_us:.1f} ({res['attention_core']['tflops']} TFLOP/s), out {us['out_gemm']:.1f}")
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
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the bounded oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_STATS_CSV", "FETCH_CSV", "WRITE_CSV"),
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

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    flops_step = wl.flops_per_shard() * wl.t
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (events), wall {wall * 1e3 / args.steps:.3f} ms/step")

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
    events = {name: [] for name in kernels}
    for _ in range(args.kernel_reps):
        for r in range(wl.t):
            for name, (fn, _f, _b) in kernels.items():
                k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                k0.record(stream)
                fn(r)
                k1.record(stream)
                events[name].append((k0, k1))
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

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy of 1 GiB x3 done")

    sp_boundary = bench_sp(wl, z, stream, args.kernel_reps)
    swiglu = bench_swiglu(wl, x, b[0], stream, args.kernel_reps)
    backward = None if args.no_backward else bench_backward(wl, x, a[0], b[0], stream,
                                                            args.kernel_reps)
    attention = None if args.no_attention else bench_attention(stream, args.kernel_reps)

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
        "roofline": {
            "bound": "mfma",
            "kernel": dom,
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": load_traffic(dom),
            "algorithmic_bytes": per_kernel[dom]["algorithmic_bytes"],
            "avg_us": per_kernel[dom]["avg_us"],
        },
        "kernels": per_kernel,
        "kernel_source_sha": kernel_source_sha(),
        "cpu_baseline": cpu,
        "swiglu": swiglu,
        "sp_boundary": sp_boundary,
        "backward": backward,
        "attention": attention,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
