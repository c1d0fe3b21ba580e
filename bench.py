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
  prefill2048  48 dfssm_layer_prefill calls over 2048 bf16 tokens (chunk 256) from zero states,
               then 16 stack-decode steps from the handed-off states (checked, not timed);
               roofline: int8 MFMA ops of the scaffold GEMMs / time.
  decode_b64   48-layer stack decode at batch 64 (states ~ N(0, 0.1)), 128 tokens per sequence
               per step; roofline: algorithmic HBM bytes (weights once per token step, every
               sequence's conv/SSM state read and written) / time.

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


# the sources the persistent batch-1 stack kernel (k_flow2) is compiled from
STACK_SOURCES = ("bit_quantized_mamba_packed_amd/csrc/flow2.hip", "bit_quantized_mamba_packed_amd/csrc/decode_device.h",
                 "bit_quantized_mamba_packed_amd/csrc/dfssm_internal.h", "include/dfssm.h")
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
    wall, launch_ms = timed(lambda: Dv.stack_decode(dims, layers, states, fw, x0, y, T, ws), args.steps,
                            args.warmup, torch)
    if not torch.isfinite(y).all():
        raise SystemExit("non-finite decode output")
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
    """48 layer prefills of 2048 bf16 tokens (chunk 256) from zero states; one step = the stack."""
    nL, S, Q = args.layers, 2048, 256
    # every layer's state in one allocation, reset by one fill per step
    conv_all = torch.zeros((nL, 1, dims.conv_dim, dims.d_conv - 1), dtype=torch.float32, device="cuda")
    ssm_all = torch.zeros((nL, 1, dims.nheads, dims.headdim, dims.d_state), dtype=torch.float32, device="cuda")
    states = [Dv.DeviceState.from_tensors(conv_all[l], ssm_all[l]) for l in range(nL)]
    x_np = gen.token_inputs(dims, (1, S), 0, tag=11, bf16=True)
    xb = torch.from_numpy(x_np).cuda().to(torch.bfloat16)
    h = [torch.empty((1, S, dims.d_model), dtype=torch.float32, device="cuda") for _ in range(2)]
    ws = Dv.workspace(dims, L.DFSSM_OP_LAYER_PREFILL, 1, S)

    def step():
        conv_all.zero_()
        ssm_all.zero_()
        for l in range(nL):
            src = xb if l == 0 else h[(l - 1) % 2]
            Dv.layer_prefill(dims, layers[l], states[l], src, h[l % 2], Q, ws)

    wall, launch_ms = timed(step, args.steps, args.warmup, torch)
    out_last = h[(nL - 1) % 2]
    if not torch.isfinite(out_last).all():
        raise SystemExit("non-finite prefill output")
    # hand the final states to 16 decode steps (not timed), fed the RMSNorm of the last position
    fw = torch.ones(dims.d_model, dtype=torch.float32, device="cuda")
    x_last = out_last[:, -1, :].contiguous()
    x0 = x_last * torch.rsqrt(x_last.pow(2).mean(-1, keepdim=True) + dims.eps)
    y = torch.empty((16, 1, dims.d_model), dtype=torch.float32, device="cuda")
    wsd = Dv.workspace(dims, L.DFSSM_OP_STACK_DECODE, 1, 0, nL)
    Dv.stack_decode(dims, layers, states, fw, x0, y, 16, wsd)
    torch.cuda.synchronize()
    if not torch.isfinite(y).all():
        raise SystemExit("non-finite decode after prefill")
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
    wall, launch_ms = timed(lambda: Dv.stack_decode(dims, layers, states, fw, x0, y, T, ws), steps,
                            min(args.warmup, 1), torch)
    if not torch.isfinite(y).all():
        raise SystemExit("non-finite batched decode output")
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


WORKLOADS = {"decode_b1": run_decode_b1, "prefill2048": run_prefill, "decode_b64": run_decode_b64}


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
    args = ap.parse_args()
    if args.write_counters:
        print(json.dumps(write_counters(*args.write_counters, args.tokens), indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}); "
              "the batch-1 decode does not shard usefully (its per-layer all-reduces would cost more than the layer), "
              "and batched decode and prefill would shard by sequence, which this single-GPU build does not run.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from synth import gen
    from bit_quantized_mamba_packed_amd import _lib as L, device as Dv

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
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
        for name in ("prefill2048", "decode_b64"):
            r = WORKLOADS[name](*common)
            torch.cuda.empty_cache()
            sec[name] = {k: r[k] for k in ("metric", "value", "unit", "ms_per_step", "config", "roofline",
                                           "cpu_baseline") if k in r}
        out["secondary"] = sec
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
