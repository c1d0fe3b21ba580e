#!/usr/bin/env python3
"""Benchmark of the DF-SSM inference hot path (Mamba-2 1.3B-shaped layers) on one MI355X.

Primary workload (the JSON line's metric): 48-layer stack decode at batch 1. One step = one
dfssm_stack_decode call that decodes `--tokens` tokens (default 512) through all 48 layers with
feedback (x(t+1) = RMSNorm of the stack output), continuing from the previous step's conv/SSM
states. Inputs are seeded synthetic tensors already resident in HBM. The timed region is K steps
bracketed by torch.cuda.synchronize(); every step is also timed with HIP events on the stream the
library launches on (the persistent stack kernel is the only long-running kernel of a call),
which gives the kernel's average launch duration for the roofline.

Secondary workloads (reported under "secondary", or alone with --workload):
  prefill2048  one dfssm_stack_prefill of 2048 bf16 tokens (chunk 256) through the 48 layers from
               zero states, then 16 stack-decode steps from the handed-off states and the last
               position's output (checked, not timed); roofline: int8 MFMA ops of the scaffold
               GEMMs / step time, and / the GEMM kernels' own time from the committed trace.
  decode_b64   48-layer stack decode at batch 64 (states ~ N(0, 0.1)), 128 tokens per sequence
               per step; roofline: algorithmic HBM bytes (weights once per token step, every
               sequence's conv/SSM state read and written) / time.
  decode_sweep the same at batch 8, 32, 128 and 512 (zero states), one point per batch.
  lm_head      the tied int8 LM head alone (batch 1, HBM roofline), and a greedy decode of the whole
               model (embedding -> 48 layers -> head -> next token), 64 tokens.

Prints ONE JSON line. `roofline.achieved` = algorithmic bytes (ops) of one launch / that launch's
duration. `roofline.traffic` = HBM bytes per launch from the committed rocprofv3 FETCH_SIZE +
WRITE_SIZE counters (profiles/), or null when the kernel source differs from the one the counters
were taken on. `cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOAD = "stack48_1p3b_b1_decode512"
CPU_TOKENS = 12
COUNTERS = os.path.join(ROOT, "profiles", "stack_decode_b1_counters.json")


def bytes_per_token(d, n_layers: int) -> dict:
    """Algorithmic HBM bytes one decoded token must move (each byte once), by component."""
    H, P, N, E, D = d.nheads, d.headdim, d.d_state, d.d_inner, d.d_model
    Cd, Ninp, ri, ro = d.conv_dim, d.n_in_proj, d.rank_in, d.rank_out
    per_layer = {
        "scaffold_signs": (Ninp * D + D * E) // 8,
        "ssm_state_rw": 2 * H * P * N * 4,
        "lora_int8": ri * D + Ninp * ri + ro * E + D * ro,
        "lora_scales_fp32": 4 * (ri + Ninp + ro + D),
        "conv_state_rw": 2 * Cd * (d.d_conv - 1) * 4,
        "conv_params": Cd * d.d_conv * 4 + Cd * 4,
        "row_scales_fp16": (Ninp + D) * 2,
        "other_params": 3 * H * 4 + D * 4 + E * 4,
    }
    total = n_layers * sum(per_layer.values()) + D * 4   # + final norm weight
    return {"per_layer": per_layer, "layer_total": sum(per_layer.values()), "token_total": total}


# the files holding the device code of the persistent batch-1 stack kernel (k_flow2): counters taken
# on other device code are not reported as this kernel's traffic
STACK_SOURCES = ("bit_quantized_mamba_packed_amd/csrc/flow2.hip", "bit_quantized_mamba_packed_amd/csrc/decode_device.h")
STACK_KERNEL = "k_flow2"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in STACK_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def cpu_baseline(dims, layers_np, x0, eps) -> dict:
    """The CPU oracle (fp64 NumPy) on CPU_TOKENS tokens of the same 48-layer stack, from zero state."""
    import numpy as np
    from oracle import dfssm_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    cs = [np.zeros((dims.conv_dim, dims.d_conv - 1)) for _ in layers_np]
    ss = [np.zeros((dims.nheads, dims.headdim, dims.d_state)) for _ in layers_np]
    t0 = time.perf_counter()
    O.stack_decode(x0, layers_np, cs, ss, CPU_TOKENS, np.ones(dims.d_model), eps, keep_dense=False)
    dt = time.perf_counter() - t0
    return {"value": CPU_TOKENS / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{CPU_TOKENS} tokens through the 48-layer stack (batch 1), {dt:.1f} s on the host"}


def write_counters(fetch_csv: str, write_csv: str, tokens: int) -> dict:
    """Summarise two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
    `bench.py --steps 1 --warmup 0 --copy-calibration` into COUNTERS (KiB per dispatch, scaled by
    what the same counter reads for the 512 MiB copy that --copy-calibration performs)."""
    import csv

    def pick(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        kern = [float(r["Counter_Value"]) for r in rows if STACK_KERNEL in r["Kernel_Name"]]
        copy = [float(r["Counter_Value"]) for r in rows
                if "copyBuffer" in r["Kernel_Name"] and float(r["Counter_Value"]) > 100000]
        if len(kern) != 1 or len(copy) != 1:
            raise SystemExit(f"{path}: expected one stack kernel and one calibration copy, got {len(kern)}, {len(copy)}")
        return kern[0], copy[0]

    copy_kib = (512 << 20) / 1024
    fk, fc = pick(fetch_csv, "FETCH_SIZE")
    wk, wc = pick(write_csv, "WRITE_SIZE")
    fs, wsc = copy_kib / fc, copy_kib / wc
    out = {"source_hash": kernel_source_hash(), "tokens_per_launch": tokens,
           "fetch_kib_raw": fk, "write_kib_raw": wk,
           "calibration": {"copy_bytes": 512 << 20, "fetch_kib_raw": fc, "write_kib_raw": wc,
                           "fetch_scale": fs, "write_scale": wsc},
           "hbm_read_bytes_per_launch": fk * fs * 1024, "hbm_write_bytes_per_launch": wk * wsc * 1024,
           "hbm_bytes_per_launch": (fk * fs + wk * wsc) * 1024}
    os.makedirs(os.path.dirname(COUNTERS), exist_ok=True)
    with open(COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
    return out


def int8_ops_per_token(d) -> int:
    """Int8 MAC-pairs (2 ops per multiply-add) of the two scaffold contractions for one token."""
    return 2 * (d.n_in_proj * d.d_model + d.d_model * d.d_inner)


def decode_b64_bytes_per_step(d, n_layers: int, batch: int) -> int:
    """Algorithmic HBM bytes of one batched token step: every weight once, every sequence's conv
    and SSM state read and written once."""
    b = bytes_per_token(d, n_layers)["per_layer"]
    per_seq = b["ssm_state_rw"] + b["conv_state_rw"]
    weights = sum(v for k, v in b.items() if k not in ("ssm_state_rw", "conv_state_rw"))
    return n_layers * (weights + batch * per_seq) + d.d_model * 4


def threads_in_use() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return 1


def timed(fn, steps: int, warmup: int, torch):
    """Run fn() warmup times, then `steps` times bracketed by synchronize(); every call is also
    bracketed by HIP events on the current stream. Returns (wall seconds, per-call ms list)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(stream)
        fn()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, [a.elapsed_time(b) for a, b in evs]


def run_decode_b1(args, dims, layers_np, layers, np, torch, gen, L, Dv) -> dict:
    nL, T = args.layers, args.tokens
    states = [Dv.DeviceState(*gen.initial_states(dims, 1, l)) for l in range(nL)]
    fw = torch.ones(dims.d_model, dtype=torch.float32, device="cuda")
    x0_np = gen.token_inputs(dims, (1,), 0, tag=7)
    x0 = torch.from_numpy(x0_np).cuda()
    y = torch.empty((T, 1, dims.d_model), dtype=torch.float32, device="cuda")
    ws = Dv.workspace(dims, L.DFSSM_OP_STACK_DECODE, 1, 0, nL)
    wall, launch_ms = timed(lambda: Dv.stack_decode(dims, layers, states, fw, x0, y, T, ws, launch=LAUNCH[0]), args.steps,
                            args.warmup, torch)
    if Dv.stack_status(ws) != L.DFSSM_STATUS_OK or not torch.isfinite(y).all():
        raise SystemExit("batch-1 stack decode failed (wait timeout or non-finite output)")
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    bpt = bytes_per_token(dims, nL)
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    achieved = bpt["token_total"] * T / avg_launch_s / 1e9
    traffic = None
    if os.path.exists(COUNTERS):
        c = json.load(open(COUNTERS))
        if c.get("source_hash") == kernel_source_hash() and c.get("tokens_per_launch") == T:
            traffic = c.get("hbm_bytes_per_launch")
    out = {
        "metric": "decode tokens/s batch=1, 48-layer 1.3B shape; achieved HBM GB/s vs peak",
        "value": round(args.steps * T / wall, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 codes x 1-bit signs (int32 acc), fp32 state/epilogue",
        "data": "synthetic (seeded random weights and inputs of the pages' Mamba-2 1.3B shape)",
        "config": {"workload": WORKLOAD, "layers": nL, "batch": 1, "tokens_per_step": T,
                   "d_model": dims.d_model, "d_inner": dims.d_inner, "d_state": dims.d_state,
                   "rank": dims.rank_in},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": traffic,
                     "kernel": "k_flow2 (persistent, role-split, one launch per step)",
                     "algorithmic_bytes_per_launch": bpt["token_total"] * T,
                     "avg_launch_ms": round(avg_launch_s * 1e3, 3)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(dims, layers_np, x0_np[0].astype(np.float64), dims.eps)
    return out


def run_prefill(args, dims, layers_np, layers, np, torch, gen, L, Dv) -> dict:
    """One dfssm_stack_prefill of 2048 bf16 tokens (chunk 256) through the 48 layers from zero
    states; one step = the whole stack prefill including its final RMSNorm."""
    nL, S, Q = args.layers, 2048, 256
    # every layer's state in one allocation, reset by one fill per step
    conv_all = torch.zeros((nL, 1, dims.conv_dim, dims.d_conv - 1), dtype=torch.float32, device="cuda")
    ssm_all = torch.zeros((nL, 1, dims.nheads, dims.headdim, dims.d_state), dtype=torch.float32, device="cuda")
    states = [Dv.DeviceState.from_tensors(conv_all[l], ssm_all[l], dims, 1) for l in range(nL)]
    x_np = gen.token_inputs(dims, (1, S), 0, tag=11, bf16=True)
    xb = torch.from_numpy(x_np).cuda().to(torch.bfloat16)
    fw = torch.ones(dims.d_model, dtype=torch.float32, device="cuda")
    y = torch.empty((1, S, dims.d_model), dtype=torch.float32, device="cuda")
    ws = Dv.workspace(dims, L.DFSSM_OP_STACK_PREFILL, 1, S, nL)

    def step():
        conv_all.zero_()
        ssm_all.zero_()
        Dv.stack_prefill(dims, layers, states, fw, xb, y, Q, ws)

    wall, launch_ms = timed(step, args.steps, args.warmup, torch)
    if not torch.isfinite(y).all():
        raise SystemExit("non-finite prefill output")
    # the final states go on to 16 decode steps (not timed) from the last position's output
    x0 = y[:, -1, :].contiguous()
    yd = torch.empty((16, 1, dims.d_model), dtype=torch.float32, device="cuda")
    wsd = Dv.workspace(dims, L.DFSSM_OP_STACK_DECODE, 1, 0, nL)
    Dv.stack_decode(dims, layers, states, fw, x0, yd, 16, wsd, launch=LAUNCH[0])
    torch.cuda.synchronize()
    if Dv.stack_status(wsd) != L.DFSSM_STATUS_OK or not torch.isfinite(yd).all():
        raise SystemExit("decode after prefill failed")
    ops = int8_ops_per_token(dims) * S * nL
    avg_s = sum(launch_ms) / len(launch_ms) / 1e3
    achieved = ops / avg_s / 1e12
    out = {
        "metric": "prefill tokens/s batch=1, L=2048 bf16, 48-layer 1.3B shape; int8 MFMA TOP/s vs peak",
        "value": round(args.steps * S / wall, 2), "unit": "tokens/s", "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 3), "higher_is_better": True,
        "dtype": "int8 codes x 1-bit signs on int8 MFMA (int32 acc), fp32 SSD/epilogue",
        "config": {"workload": "stack48_1p3b_prefill2048", "layers": nL, "batch": 1, "seqlen": S, "chunk": Q,
                   "input": "bf16", "decode_after": 16},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": 5000.0, "unit": "TFLOP/s",
                     "frac": round(achieved / 5000.0, 5), "traffic": None,
                     "kernel": "whole prefill step (all kernels of 48 layers); scaffold int8 ops only",
                     "algorithmic_ops_per_launch": ops, "avg_launch_ms": round(avg_s * 1e3, 3)},
    }
    gemm = prefill_gemm_profile(dims, nL, S)
    if gemm is not None:
        out["roofline_scaffold_gemms"] = gemm
    if not args.no_cpu_baseline:
        from oracle import dfssm_oracle as O
        nl_cpu = 2
        t0 = time.perf_counter()
        xs = x_np[0].astype(np.float64)
        for l in range(nl_cpu):
            outs, _, _, _ = O.layer_tokens(xs, layers_np[l], np.zeros((dims.conv_dim, dims.d_conv - 1)),
                                           np.zeros((dims.nheads, dims.headdim, dims.d_state)))
            xs = np.asarray(outs)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(S * nl_cpu / (dt * nL), 4), "unit": "tokens/s", "cores": threads_in_use(),
                               "kind": "oracle",
                               "sample": f"all {S} tokens through the first {nl_cpu} layers ({dt:.1f} s), scaled to 48 layers"}
    return out


# how the batch-1 persistent kernel is launched (--ordinary-launch: for kernel tracers that cannot
# follow a cooperative launch)
LAUNCH = [0]

PREFILL_GEMM_PROFILE = os.path.join(ROOT, "profiles", "prefill2048_gemm_kernels.json")
PREFILL_GEMM_SOURCES = ("bit_quantized_mamba_packed_amd/csrc/gemm.hip", "bit_quantized_mamba_packed_amd/csrc/gemm_conv.h",
                        "bit_quantized_mamba_packed_amd/csrc/decode_device.h")


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def prefill_gemm_profile(d, n_layers: int, S: int):
    """The scaffold GEMM kernels' share of the int8 MFMA roofline, from the committed rocprofv3
    kernel trace of this workload (per-launch average durations of the in_proj and out_proj GEMM
    kernels); None when the GEMM sources changed since the trace was taken."""
    if not os.path.exists(PREFILL_GEMM_PROFILE):
        return None
    p = json.load(open(PREFILL_GEMM_PROFILE))
    if p.get("source_hash") != source_hash(PREFILL_GEMM_SOURCES):
        return None
    ops_in = 2 * d.n_in_proj * d.d_model * S
    ops_out = 2 * d.d_model * d.d_inner * S
    t_in, t_out = p["in_proj_avg_ns"] * 1e-9, p["out_proj_avg_ns"] * 1e-9
    tot = n_layers * (t_in + t_out)
    ach = n_layers * (ops_in + ops_out) / tot / 1e12
    return {"bound": "mfma", "peak": 5000.0, "unit": "TFLOP/s", "achieved": round(ach, 2),
            "frac": round(ach / 5000.0, 5), "gemm_ms_per_prefill": round(tot * 1e3, 3),
            "in_proj": {"kernel": p["in_proj_kernel"], "avg_us": round(t_in * 1e6, 2),
                        "frac": round(ops_in / t_in / 1e12 / 5000.0, 5)},
            "out_proj": {"kernel": p["out_proj_kernel"], "avg_us": round(t_out * 1e6, 2),
                         "frac": round(ops_out / t_out / 1e12 / 5000.0, 5)},
            "source": "profiles/prefill2048_gemm_kernels.json (rocprofv3 kernel trace of this workload)"}


def write_gemm_profile(trace_csv: str) -> dict:
    """Summarise the rocprofv3 kernel trace of `bench.py --workload prefill2048 --steps 1` into
    PREFILL_GEMM_PROFILE: the average duration of the in_proj GEMM launch (k_gemm_tile_ext, both
    of its GEMMs) and of the out_proj GEMM launch (k_gemm_tile) over the traced prefills."""
    import csv
    rows = list(csv.DictReader(open(trace_csv)))

    def avg(*tags):
        sel = [r for r in rows if any(t in r["Kernel_Name"] for t in tags)]
        if not sel:
            raise SystemExit(f"{trace_csv}: no {' / '.join(tags)} dispatch")
        d = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in sel]
        return sum(d) / len(d), len(d), sel[0]["Kernel_Name"]

    t_in, n_in, k_in = avg("k_gemm_tile_ext", "k_gemm_tile_pair")
    t_out, n_out, k_out = avg("k_gemm_tile<")
    import re

    def short(name):
        m = re.search(r"(k_\w+(?:<[^>]*>)?)", name)
        return m.group(1) if m else name

    out = {"source_hash": source_hash(PREFILL_GEMM_SOURCES), "in_proj_avg_ns": t_in, "in_proj_dispatches": n_in,
           "in_proj_kernel": short(k_in), "out_proj_avg_ns": t_out, "out_proj_dispatches": n_out,
           "out_proj_kernel": short(k_out)}
    with open(PREFILL_GEMM_PROFILE, "w") as f:
        json.dump(out, f, indent=1)
    return out


def run_decode_b64(args, dims, layers_np, layers, np, torch, gen, L, Dv) -> dict:
    nL, B, T = args.layers, 64, 128
    states = []
    for l in range(nL):
        c, s_ = gen.initial_states(dims, B, l, 0, std=0.1)
        states.append(Dv.DeviceState(c, s_))
    fw = torch.ones(dims.d_model, dtype=torch.float32, device="cuda")
    x0 = torch.from_numpy(gen.token_inputs(dims, (B,), 0, tag=8)).cuda()
    y = torch.empty((T, B, dims.d_model), dtype=torch.float32, device="cuda")
    ws = Dv.workspace(dims, L.DFSSM_OP_STACK_DECODE, B, 0, nL)
    steps = max(1, min(args.steps, 2))
    wall, launch_ms = timed(lambda: Dv.stack_decode(dims, layers, states, fw, x0, y, T, ws, launch=LAUNCH[0]), steps,
                            min(args.warmup, 1), torch)
    if Dv.stack_status(ws) != L.DFSSM_STATUS_OK or not torch.isfinite(y).all():
        raise SystemExit("batched stack decode failed")
    per_step = decode_b64_bytes_per_step(dims, nL, B)
    avg_s = sum(launch_ms) / len(launch_ms) / 1e3
    achieved = per_step * T / avg_s / 1e9
    return {
        "metric": "decode tokens/s batch=64, 48-layer 1.3B shape; achieved HBM GB/s vs peak",
        "value": round(steps * T * B / wall, 2), "unit": "tokens/s", "steps": steps,
        "ms_per_step": round(wall / steps * 1e3, 3), "higher_is_better": True,
        "dtype": "int8 codes x 1-bit signs on int8 MFMA (int32 acc), fp32 state/epilogue",
        "config": {"workload": "stack48_1p3b_b64_decode128", "layers": nL, "batch": B, "tokens_per_step": T,
                   "state_init": "N(0, 0.1)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": None,
                     "kernel": "whole step (all kernels of 128 x 48 layer steps)",
                     "algorithmic_bytes_per_launch": per_step * T, "avg_launch_ms": round(avg_s * 1e3, 3)},
    }


def run_decode_sweep(args, dims, layers_np, layers, np, torch, gen, L, Dv) -> dict:
    """48-layer stack decode at the batch sizes of the pages' batched throughput table (8, 32, 128,
    512; zero states, seeded inputs): tokens/s and algorithmic HBM bytes (weights once per token
    step, every sequence's conv/SSM state read and written) per second."""
    nL = args.layers
    out = {"metric": "decode tokens/s by batch, 48-layer 1.3B shape; achieved HBM GB/s vs peak",
           "unit": "tokens/s", "points": []}
    for B in (8, 32, 128, 512):
        T = max(16, 1024 // B)
        conv = torch.zeros((nL, B, dims.conv_dim, dims.d_conv - 1), dtype=torch.float32, device="cuda")
        ssm = torch.zeros((nL, B, dims.nheads, dims.headdim, dims.d_state), dtype=torch.float32, device="cuda")
        states = [Dv.DeviceState.from_tensors(conv[l], ssm[l], dims, B) for l in range(nL)]
        fw = torch.ones(dims.d_model, dtype=torch.float32, device="cuda")
        x0 = torch.from_numpy(gen.token_inputs(dims, (B,), 0, tag=12)).cuda()
        y = torch.empty((T, B, dims.d_model), dtype=torch.float32, device="cuda")
        ws = Dv.workspace(dims, L.DFSSM_OP_STACK_DECODE, B, 0, nL)
        steps = max(1, min(args.steps, 2))
        wall, launch_ms = timed(lambda: Dv.stack_decode(dims, layers, states, fw, x0, y, T, ws, launch=LAUNCH[0]), steps,
                                min(args.warmup, 1), torch)
        if Dv.stack_status(ws) != L.DFSSM_STATUS_OK or not torch.isfinite(y).all():
            raise SystemExit(f"batch-{B} stack decode failed")
        per_step = decode_b64_bytes_per_step(dims, nL, B)
        avg_s = sum(launch_ms) / len(launch_ms) / 1e3
        ach = per_step * T / avg_s / 1e9
        out["points"].append({"batch": B, "tokens_per_step": T, "value": round(steps * T * B / wall, 2),
                              "ms_per_step": round(wall / steps * 1e3, 3),
                              "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS,
                                           "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 5)}})
        del conv, ssm, states, y, ws
        torch.cuda.empty_cache()
    return out


def run_lm_head(args, dims, layers_np, layers, np, torch, gen, L, Dv) -> dict:
    """The tied int8 LM head alone (batch 1, 50,280 x 2,048 int8 rows, greedy token only), and a
    greedy full-model decode: token -> int8 embedding -> the 48-layer stack (one dfssm_stack_decode
    step) -> LM head -> next token, 64 tokens from zero states."""
    emb_np = gen.embedding(dims, seed=0)
    emb = Dv.DeviceEmbedding(emb_np)
    V, D = emb_np.vocab, dims.d_model
    y = torch.from_numpy(gen.token_inputs(dims, (1,), 0, tag=30)).cuda()   # any fp32 row: the head quantizes it per token
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = Dv.workspace(dims, L.DFSSM_OP_LM_HEAD, 1)
    calls = 200
    wall, launch_ms = timed(lambda: [Dv.lm_head(dims, emb, y, None, nxt, ws) for _ in range(calls)],
                            max(1, min(args.steps, 3)), 1, torch)
    avg_s = sum(launch_ms) / len(launch_ms) / 1e3 / calls
    head_bytes = V * D + 4 * V + 4 * D + 4
    ach = head_bytes / avg_s / 1e9
    out = {"metric": "LM head (tied int8, 50,280 x 2,048) batch 1: achieved HBM GB/s vs peak",
           "value": round(ach, 2), "unit": "GB/s", "us_per_call": round(avg_s * 1e6, 3),
           "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBS, 5), "traffic": None,
                        "kernel": "k_lm_head + k_argmax (one call)", "algorithmic_bytes_per_launch": head_bytes,
                        "avg_launch_us": round(avg_s * 1e6, 3)}}
    # greedy decode of the whole model
    nL, T = args.layers, 64
    conv = torch.zeros((nL, 1, dims.conv_dim, dims.d_conv - 1), dtype=torch.float32, device="cuda")
    ssm = torch.zeros((nL, 1, dims.nheads, dims.headdim, dims.d_state), dtype=torch.float32, device="cuda")
    states = [Dv.DeviceState.from_tensors(conv[l], ssm[l], dims, 1) for l in range(nL)]
    fw = torch.ones(D, dtype=torch.float32, device="cuda")
    tok = torch.from_numpy(gen.token_ids(1, V, seed=0, tag=31)).cuda()
    toks = torch.empty((T, 4), dtype=torch.int32, device="cuda")   # one 16-byte slot per token
    x = torch.empty((1, D), dtype=torch.float32, device="cuda")
    yd = torch.empty((1, 1, D), dtype=torch.float32, device="cuda")
    wsd = Dv.workspace(dims, L.DFSSM_OP_STACK_DECODE, 1, 0, nL)

    def greedy():
        conv.zero_()
        ssm.zero_()
        t = tok
        for i in range(T):
            Dv.embed(emb, t, x)
            Dv.stack_decode(dims, layers, states, fw, x, yd, 1, wsd, launch=LAUNCH[0])
            Dv.lm_head(dims, emb, yd[0], None, toks[i], ws)
            t = toks[i, :1]

    gw, g_ms = timed(greedy, max(1, min(args.steps, 2)), 1, torch)
    if Dv.stack_status(wsd) != L.DFSSM_STATUS_OK:
        raise SystemExit("greedy decode: stack status")
    per_tok = bytes_per_token(dims, nL)["token_total"] + head_bytes + 4 * D
    g_avg = sum(g_ms) / len(g_ms) / 1e3
    out["greedy_full_model"] = {"metric": "greedy decode tokens/s batch=1, embedding + 48 layers + tied LM head",
                                "value": round(T / g_avg, 2), "unit": "tokens/s", "tokens_per_step": T,
                                "bytes_per_token": per_tok,
                                "roofline": {"bound": "hbm", "achieved": round(per_tok * T / g_avg / 1e9, 2),
                                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                             "frac": round(per_tok * T / g_avg / 1e9 / HBM_PEAK_GBS, 5)},
                                "note": "one stack-decode launch per token (host loop), no host sync inside the step"}
    return out


def run_state_codec(args, dims, layers_np, layers, np, torch, gen, L, Dv) -> dict:
    """Density field codec of one 1.3B layer's SSM state at batch 64 (262,144 rows of 128 fp32 ->
    23 x 23 bit fields + mu, sigma): encode and decode timed apart, each against HBM."""
    B = 64
    _, S = gen.initial_states(dims, B, seed=0, std=0.1)
    ssm = torch.from_numpy(S).cuda()
    back = torch.empty_like(ssm)
    fields, stats = Dv.state_encode(dims, ssm, B)
    rows = B * dims.nheads * dims.headdim
    W = L.dfssm_state_field_words(dims.d_state)
    state_b, code_b = rows * dims.d_state * 4, rows * (4 * W + 8)
    calls = 20
    res = {}
    for name, fn in (("encode", lambda: Dv.state_encode(dims, ssm, B)),
                     ("decode", lambda: Dv.state_decode(dims, fields, stats, B, back))):
        wall, ms = timed(lambda: [fn() for _ in range(calls)], max(1, min(args.steps, 3)), 1, torch)
        avg_s = sum(ms) / len(ms) / 1e3 / calls
        ach = (state_b + code_b) / avg_s / 1e9
        res[name] = {"us_per_call": round(avg_s * 1e6, 3), "achieved": round(ach, 2),
                     "frac": round(ach / HBM_PEAK_GBS, 5)}
    enc = res["encode"]
    return {"metric": "density field state codec, 1.3B layer state at batch 64: encode HBM GB/s",
            "value": enc["achieved"], "unit": "GB/s", "us_per_call": enc["us_per_call"],
            "config": {"workload": "state_codec_1p3b_b64", "rows": rows, "d_state": dims.d_state,
                       "field_words": W, "state_bytes": state_b, "code_bytes": code_b},
            "roofline": {"bound": "hbm", "achieved": enc["achieved"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": enc["frac"], "traffic": None, "kernel": "k_state_encode",
                         "algorithmic_bytes_per_launch": state_b + code_b, "avg_launch_us": enc["us_per_call"]},
            "decode": res["decode"]}


def run_dfssd_prefill(args, dims, layers_np, layers, np, torch, gen, L, Dv) -> dict:
    """One 1.3B layer over 2048 bf16 tokens (chunk 256) with the density field codec on the state at
    the 7 chunk boundaries (DF-SSD), against the same prefill without it. The codec carry runs one
    wave per head sequentially over the chunks: bound by its per-row sigma-delta chain, not HBM."""
    S, Q = 2048, 256
    lay = layers[0]
    conv = torch.zeros((1, dims.conv_dim, dims.d_conv - 1), dtype=torch.float32, device="cuda")
    ssm = torch.zeros((1, dims.nheads, dims.headdim, dims.d_state), dtype=torch.float32, device="cuda")
    st = Dv.DeviceState.from_tensors(conv, ssm, dims, 1)
    xb = torch.from_numpy(gen.token_inputs(dims, (1, S), 0, tag=12, bf16=True)).cuda().to(torch.bfloat16)
    y = torch.empty((1, S, dims.d_model), dtype=torch.float32, device="cuda")
    ws = Dv.workspace(dims, L.DFSSM_OP_LAYER_PREFILL, 1, S)
    res = {}
    for name, codec in (("plain", False), ("dfssd", True)):
        def step():
            conv.zero_()
            ssm.zero_()
            Dv.layer_prefill(dims, lay, st, xb, y, Q, ws, state_codec=codec)
        _, ms = timed(step, max(3, args.steps), 1, torch)
        if not torch.isfinite(y).all():
            raise SystemExit("non-finite DF-SSD prefill output")
        res[name] = round(sum(ms) / len(ms), 4)
    extra = res["dfssd"] - res["plain"]
    # the whole stack with DF-SSD in every layer (dfssm_stack_prefill_ex)
    nL = args.layers
    conv_all = torch.zeros((nL, 1, dims.conv_dim, dims.d_conv - 1), dtype=torch.float32, device="cuda")
    ssm_all = torch.zeros((nL, 1, dims.nheads, dims.headdim, dims.d_state), dtype=torch.float32, device="cuda")
    states = [Dv.DeviceState.from_tensors(conv_all[l], ssm_all[l], dims, 1) for l in range(nL)]
    fw = torch.ones(dims.d_model, dtype=torch.float32, device="cuda")
    wss = Dv.workspace(dims, L.DFSSM_OP_STACK_PREFILL, 1, S, nL)

    def stack_step():
        conv_all.zero_()
        ssm_all.zero_()
        Dv.stack_prefill(dims, layers, states, fw, xb, y, Q, wss, state_codec=True)

    _, sms = timed(stack_step, max(1, min(args.steps, 3)), 1, torch)
    if not torch.isfinite(y).all():
        raise SystemExit("non-finite DF-SSD stack prefill output")
    stack_ms = sum(sms) / len(sms)
    return {"metric": "DF-SSD layer prefill, 1.3B layer, 2048 bf16 tokens, chunk 256: ms per layer",
            "value": res["dfssd"], "unit": "ms", "higher_is_better": False,
            "config": {"workload": "dfssd_prefill_1p3b_layer2048", "chunk": Q, "boundaries": S // Q - 1},
            "plain_ms": res["plain"], "codec_carry_ms": round(extra, 4),
            "stack": {"layers": nL, "ms_per_prefill": round(stack_ms, 3), "tokens_per_s": round(S / stack_ms * 1e3, 1)},
            "note": "codec carry = DF-SSD minus plain (the scan with 4096 state rows encoded and read back at "
                    "each of 7 boundaries, d_state / 32 lanes per row)"}


def run_dfw_proj(args, dims, layers_np, layers, np, torch, gen, L, Dv) -> dict:
    """The 17-level scaffold projection at batch 1 (decode) on the 1.3B in_proj (8,512 x 2,048) and
    out_proj (2,048 x 4,096) shapes, rank 32: quantizer + five-plane GEMV + LoRA epilogue per call."""
    res = {}
    for name, n_out, n_in in (("in_proj", dims.n_in_proj, dims.d_model), ("out_proj", dims.d_model, dims.d_inner)):
        P = gen.dfw_proj(n_out, n_in, dims.rank_in, seed=0)
        dp = Dv.DeviceDfwProj(P)
        pts = {}
        for B in (1, 4):
            x = torch.from_numpy(gen.token_inputs(gen.Dims(d_model=n_in, d_inner=n_in, d_state=16, headdim=64,
                                                           ngroups=1, d_conv=4, n_in_proj=n_in, rank_in=8,
                                                           rank_out=8), (B,), 0, tag=40)).cuda()
            y = torch.empty((B, n_out), device="cuda")
            ws = torch.empty(L.dfssm_dfw_workspace_bytes(n_in, P.rank, B), dtype=torch.uint8, device="cuda")
            calls = 200
            _, ms = timed(lambda: [Dv.dfw_project(dp, x, y, ws) for _ in range(calls)], max(1, min(args.steps, 3)), 1, torch)
            avg_s = sum(ms) / len(ms) / 1e3 / calls
            nbytes = (n_out * n_in * 5 // 8 + P.rank * n_in + n_out * P.rank + n_out * (2 + 4) + P.rank * 4
                      + B * 4 * (n_in + n_out))
            ach = nbytes / avg_s / 1e9
            pts[f"B{B}"] = {"us_per_call": round(avg_s * 1e6, 3), "algorithmic_bytes": nbytes,
                            "achieved_GBs": round(ach, 2), "frac": round(ach / HBM_PEAK_GBS, 5)}
        res[name] = pts
    top = res["in_proj"]["B1"]
    return {"metric": "17-level scaffold projection, 1.3B in_proj at batch 1: achieved HBM GB/s",
            "value": top["achieved_GBs"], "unit": "GB/s", "us_per_call": top["us_per_call"],
            "config": {"workload": "dfw_proj_1p3b", "rank": dims.rank_in, "planes": 5},
            "roofline": {"bound": "hbm", "achieved": top["achieved_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": top["frac"], "traffic": None, "kernel": "k_dfw_quant + k_dfw_gemv<1> (one call)",
                         "algorithmic_bytes_per_launch": top["algorithmic_bytes"], "avg_launch_us": top["us_per_call"]},
            "points": res}


WORKLOADS = {"decode_b1": run_decode_b1, "prefill2048": run_prefill, "decode_b64": run_decode_b64,
             "decode_sweep": run_decode_sweep, "lm_head": run_lm_head, "state_codec": run_state_codec,
             "dfw_proj": run_dfw_proj, "dfssd_prefill": run_dfssd_prefill}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--tokens", type=int, default=512, help="tokens decoded per step (batch-1 decode)")
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=None,
                    help="run one workload alone and print its line (default: batch-1 decode + secondaries)")
    ap.add_argument("--no-secondary", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, copy 512 MiB once (calibrates rocprofv3 byte counters)")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs into profiles/ and exit (no GPU)")
    ap.add_argument("--ordinary-launch", action="store_true",
                    help="launch the batch-1 persistent kernel with the ordinary launch API (same grid; for "
                         "kernel tracers that cannot follow cooperative launches)")
    ap.add_argument("--write-gemm-profile", metavar="TRACE_CSV",
                    help="summarise a rocprofv3 kernel trace of the prefill workload into profiles/ and exit (no GPU)")
    args = ap.parse_args()
    if args.write_gemm_profile:
        print(json.dumps(write_gemm_profile(args.write_gemm_profile), indent=1))
        return 0
    if args.write_counters:
        print(json.dumps(write_counters(*args.write_counters, args.tokens), indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}); "
              "the batch-1 decode does not shard usefully (its per-layer all-reduces would cost more than the layer), "
              "and batched decode and prefill would shard by sequence, which the library does not run across GPUs.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from synth import gen
    from bit_quantized_mamba_packed_amd import _lib as L, device as Dv

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    if args.ordinary_launch:
        LAUNCH[0] = L.DFSSM_LAUNCH_ORDINARY
    L.load()
    dims = gen.DIMS["1p3b"]
    layers_np = gen.stack_weights(dims, args.layers, seed=0)
    layers = [Dv.DeviceLayer(lw) for lw in layers_np]
    common = (args, dims, layers_np, layers, np, torch, gen, L, Dv)
    if args.workload is not None:
        out = WORKLOADS[args.workload](*common)
        out.setdefault("n_gpus", 1)
        print(json.dumps(out), flush=True)
        return 0
    out = run_decode_b1(*common)
    if not args.no_secondary:
        sec = {}
        for name in ("prefill2048", "decode_b64", "decode_sweep", "lm_head", "state_codec", "dfw_proj",
                     "dfssd_prefill"):
            r = WORKLOADS[name](*common)
            torch.cuda.empty_cache()
            sec[name] = {k: r[k] for k in ("metric", "value", "unit", "ms_per_step", "config", "roofline",
                                           "roofline_scaffold_gemms", "points", "us_per_call",
                                           "greedy_full_model", "cpu_baseline", "decode", "plain_ms",
                                           "codec_carry_ms", "stack") if k in r}
        out["secondary"] = sec
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
