#!/usr/bin/env python3
"""KDA decode benchmark on one MI355X.

Workload: the 34-layer KDA stack (D=2048, 16 heads, d_k=d_v=128, all projections Q8_0,
fp32 state [16][128][128] + 3-token conv window per layer, pre-RMSNorm residual stream),
batch 1, synthetic seeded weights and inputs.  A step is one token through all 34 layers:
the fused projection GEMV, the low-rank gate kernel, the per-head delta-rule kernel and
the gated-norm + output projection GEMV per layer, replayed as one hipGraph.

Prints ONE JSON line: tokens/s over K timed steps, HBM roofline of the dominant kernel
(timed with hipEvents on the launch stream), and the CPU oracle on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM bytes per launch of the one-launch step from rocprofv3 FETCH_SIZE + WRITE_SIZE, each
# scaled by the same counter on a plain 256 MiB copy (FETCH x2.0, WRITE x1.0), valid while
# the kernel's sources hash to "sha256" (see profiles/ for the runs).
STEP_TRAFFIC = {"bytes": 752336069,
                "sha256": "f94807fba429a79eb8409f444c0f514801c66085bd7461f6071c1d5a320bbf7d",
                "sources": ("persistent.hip", "kda_device.h", "kda_internal.h")}


def step_traffic():
    """The counted traffic of the one-launch step, or None once its sources changed."""
    import hashlib
    h = hashlib.sha256()
    for f in STEP_TRAFFIC["sources"]:
        with open(os.path.join(ROOT, "linear_attention_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return STEP_TRAFFIC["bytes"] if h.hexdigest() == STEP_TRAFFIC["sha256"] else None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(w) -> dict:
    """Bytes each kernel of one layer must move at B=1 (weights incl. Q8_0 scales,
    state, conv window, activations), and the per-token total of the stack."""
    d = w.dims
    D, K, V, H = d.d_model, d.key_dim, d.value_dim, d.n_heads
    C = d.conv_channels

    def q8(rows, cols):
        return rows * cols + rows * (cols // 32) * 2

    proj_w = q8(K, D) * 2 + q8(V, D) + q8(d.rank_f, D) + q8(d.rank_g, D) + q8(H, D)
    proj = proj_w + D * 4 + C * 3 * 4 * 2 + C * 4 * 4 + (C + d.rank_f + d.rank_g + H) * 4
    state = H * d.d_k * d.d_v * 4 * 2
    gates = q8(K, d.rank_f) + q8(V, d.rank_g) + (d.rank_f + d.rank_g) * 4 + (K + V) * 4
    head = state + (C + H) * 4 + (K + V) * 4 + V * 4 * 2
    out = q8(D, V) + V * 4 * 2 + D * 4 * 2
    weights_state = proj_w + q8(K, d.rank_f) + q8(V, d.rank_g) + q8(D, V) + state
    # the one-launch step: every layer's weights, state (read + write) and conv window
    # (read + write), the input token and the output row
    step = (weights_state + C * 3 * 4 * 2 + C * 4 * 4) * w.n_layers + D * 4 * 2
    return {"proj": proj, "gates": gates, "head": head, "out": out, "step": step,
            "layer_weights_state": weights_state,
            "token_weights_state": weights_state * w.n_layers}


def cpu_baseline(run, budget_s: float = 15.0):
    """The float64 oracle, as it stands, on the first tokens of the same workload."""
    import threadpoolctl
    from oracle import kda as ok

    w = run.workload
    d = w.dims
    t0 = time.time()
    layers = [ok.prepare_layer(dr, w.wtype, d.n_heads, d.d_k, d.d_v, w.norm_eps, w.l2_eps)
              for dr in run.layers]
    log(f"[cpu] oracle weights prepared in {time.time() - t0:.1f}s")
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    n = 0
    t0 = time.time()
    S = [[run.s0[l, 0].astype(np.float64)] for l in range(w.n_layers)]
    Z = [[np.zeros((3, d.conv_channels))] for _ in range(w.n_layers)]
    while True:
        xt = run.x[n % w.steps, 0, 0].astype(np.float64)[None, :]   # inputs reused cyclically
        _, s_new, z_new = ok.stack_step(layers, xt, [S[l][0] for l in range(w.n_layers)],
                                        [Z[l][0] for l in range(w.n_layers)])
        for l in range(w.n_layers):
            S[l][0], Z[l][0] = s_new[l], z_new[l]
        n += 1
        if time.time() - t0 > budget_s:
            break
    el = time.time() - t0
    return {"value": n / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} consecutive decode tokens of the 34-layer Q8_0 stack, B=1, float64 "
                      f"numpy oracle ({el:.1f}s, BLAS threads={threads}, host nproc={os.cpu_count()})"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--per-layer", action="store_true",
                    help="time the per-layer hipGraph path instead of the one-launch step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path "
              "is measured on a single MI355X and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_calibration} MiB 5 times")
        return
    import synth
    import linear_attention_decode_amd as kda

    w = synth.WORKLOADS["stack"]
    steps_needed = max(args.steps + args.warmup, 1)
    w_run = synth.scaled(w, steps=steps_needed)
    t0 = time.time()
    run = synth.draw_run(w_run)
    log(f"[bench] drew {w.n_layers}-layer weights + inputs in {time.time() - t0:.1f}s")
    d = w.dims
    t0 = time.time()
    model = kda.KdaModel(run.layers, n_heads=d.n_heads, d_k=d.d_k, d_v=d.d_v, wtype=w.wtype,
                         prenorm_residual=True, norm_eps=w.norm_eps, l2_eps=w.l2_eps)
    log(f"[bench] packed Q8_0 weights on the device in {time.time() - t0:.1f}s")
    B = 1
    st = model.new_state(B)
    st.S.copy_(torch.from_numpy(run.s0))
    ws = model.workspace(kda.KDA_OP_DECODE, B)
    xs = torch.from_numpy(np.ascontiguousarray(run.x[:, :, 0, :])).cuda()   # [steps][B][D]
    y = torch.empty((B, d.d_model), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    model.set_option(kda.KDA_OPT_GRAPH, 1)
    model.set_option(kda.KDA_OPT_PERSISTENT, 0 if args.per_layer else 1)
    one_launch = not args.per_layer and model.persistent_blocks() > 0
    path = (f"one cooperative launch per token ({model.persistent_blocks()} blocks)" if one_launch
            else "per-layer kernels replayed as one hipGraph")
    log(f"[bench] path: {path}")
    for i in range(args.warmup):
        model.decode_step(xs[i], y, st, ws)
    torch.cuda.synchronize()
    # ---- timed region: K steps, inputs resident in HBM ----
    t0 = time.perf_counter()
    for i in range(args.steps):
        model.decode_step(xs[args.warmup + i], y, st, ws)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    tok_s = args.steps / el
    ms_step = el * 1e3 / args.steps
    log(f"[bench] {args.steps} steps in {el * 1e3:.2f} ms: {tok_s:.1f} tokens/s")

    # ---- per-kernel durations with hipEvents on the launch stream (no graph) ----
    model.set_option(kda.KDA_OPT_TIMING, 1)
    model.timing(kda.KDA_K_PROJ, reset=True)
    for i in range(args.steps):
        model.decode_step(xs[args.warmup + i], y, st, ws)
    torch.cuda.synchronize()
    kinds = {"proj": kda.KDA_K_PROJ, "gates": kda.KDA_K_GATES, "head": kda.KDA_K_HEAD,
             "out": kda.KDA_K_OUT, "step": kda.KDA_K_STEP}
    times = {k: model.timing(v) for k, v in kinds.items()}
    model.set_option(kda.KDA_OPT_TIMING, 0)
    ab = algorithmic_bytes(w)
    per = {}
    for k, (ms, n) in times.items():
        if n == 0:
            continue
        avg_us = ms * 1e3 / n
        per[k] = {"avg_us": avg_us, "launches": n, "bytes": ab[k],
                  "gbs": ab[k] / (avg_us * 1e-6) / 1e9}
        log(f"[bench] kernel {k}: {n} launches, avg {avg_us:.2f} us, "
            f"{per[k]['gbs']:.0f} GB/s algorithmic")
    dom = max(per, key=lambda k: per[k]["avg_us"] * per[k]["launches"])
    ach = per[dom]["gbs"]
    step_gbs = ab["token_weights_state"] / (ms_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(run, args.cpu_budget)
        log(f"[cpu] {cpu['sample']}: {cpu['value']:.3f} tokens/s")

    out = {
        "metric": "KDA decode tokens/s (34-layer stack, B=1)",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "kda-stack-34L-q8_0-decode", "layers": w.n_layers,
                   "d_model": d.d_model, "heads": d.n_heads, "d_k": d.d_k, "d_v": d.d_v,
                   "weights": "q8_0", "state": "f32", "batch": B, "global_batch": B,
                   "seq_len": 1, "parallelism": "none (1 GPU)",
                   "path": path,
                   "bytes_per_token": ab["token_weights_state"],
                   "step_hbm_gbs": round(step_gbs, 1),
                   "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
                   "kernels": {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv)
                                   for kk, vv in v.items()} for k, v in per.items()}},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                     "traffic": step_traffic() if dom == "step" else None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    model.close()


if __name__ == "__main__":
    main()
