#!/usr/bin/env python3
"""Benchmark: 48-layer DF-SSM (Mamba-2 1.3B-shaped) stack decode at batch 1 on one MI355X.

One step = one dfssm_stack_decode call that decodes `--tokens` tokens (default 512) through all
48 layers with feedback (x(t+1) = RMSNorm of the stack output), continuing from the previous
step's conv/SSM states. Inputs are seeded synthetic tensors already resident in HBM. The timed
region is K steps bracketed by torch.cuda.synchronize(); every step is also timed with HIP events
on the stream the library launches on (the persistent stack kernel is the only long-running
kernel of a call), which gives the kernel's average launch duration for the roofline.

Prints ONE JSON line. `roofline.achieved` = algorithmic bytes of one launch (per-token bytes x
tokens, see bytes_per_token) / that launch's duration. `roofline.traffic` = HBM bytes per launch
from the committed rocprofv3 FETCH_SIZE + WRITE_SIZE counters (profiles/), or null when the
kernel source differs from the one the counters were taken on. `cpu_baseline` times the CPU
oracle on one token of the same 48-layer stack.
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
CPU_TOKENS = 4
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


# the sources the persistent stack kernel is compiled from
STACK_SOURCES = ("bit_quantized_mamba_packed_amd/csrc/stack.hip", "bit_quantized_mamba_packed_amd/csrc/decode_device.h",
                 "bit_quantized_mamba_packed_amd/csrc/dfssm_internal.h", "include/dfssm.h")


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
        kern = [float(r["Counter_Value"]) for r in rows if "k_stack_flow" in r["Kernel_Name"]]
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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--tokens", type=int, default=512, help="tokens decoded per step")
    ap.add_argument("--layers", type=int, default=48)
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
              "the batch-1 decode does not shard usefully, see DESIGN.md.", file=sys.stderr)
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
    nL, T = args.layers, args.tokens
    layers_np = gen.stack_weights(dims, nL, seed=0)
    layers = [Dv.DeviceLayer(lw) for lw in layers_np]
    states = [Dv.DeviceState(*gen.initial_states(dims, 1, l)) for l in range(nL)]
    fw = torch.ones(dims.d_model, dtype=torch.float32, device="cuda")
    x0_np = gen.token_inputs(dims, (1,), 0, tag=7)
    x0 = torch.from_numpy(x0_np).cuda()
    y = torch.empty((T, 1, dims.d_model), dtype=torch.float32, device="cuda")
    ws = Dv.workspace(dims, L.DFSSM_OP_STACK_DECODE, 1, 0, nL)

    for _ in range(args.warmup):
        Dv.stack_decode(dims, layers, states, fw, x0, y, T, ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        Dv.stack_decode(dims, layers, states, fw, x0, y, T, ws)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    if not torch.isfinite(y).all():
        print("non-finite decode output", file=sys.stderr)
        return 1
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    tokens = args.steps * T
    value = tokens / wall
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
        "value": round(value, 2),
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
                     "kernel": "k_stack_flow (persistent, one launch per step)",
                     "algorithmic_bytes_per_launch": bpt["token_total"] * T,
                     "avg_launch_ms": round(avg_launch_s * 1e3, 3)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(dims, layers_np, x0_np[0].astype(np.float64), dims.eps)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
