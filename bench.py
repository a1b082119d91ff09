#!/usr/bin/env python3
"""KDA decode benchmark on one MI355X.

Default workload (the headline metric): the 34-layer KDA stack (D=2048, 16 heads,
d_k=d_v=128, all projections Q8_0, fp32 state [16][128][128] + 3-token conv window per
layer, pre-RMSNorm residual stream), batch 1, synthetic seeded weights and inputs.  A step
is one token through all 34 layers: one launch of the one-launch decode kernel
(or, with --per-layer, the per-layer kernels, launched directly or with --graph
replayed as one hipGraph).

Prints ONE JSON line: tokens/s over K timed steps, HBM roofline of the dominant kernel
(timed with hipEvents on the launch stream), and the CPU oracle on a bounded sample.

Other workloads (--workload, one JSON line each, for the secondary measurements):
  layer    one BF16 layer, B=1 decode (effective GB/s; the 38 MB set fits the MALL;
           --copies 8 rotates 8 weight copies so that each step streams from HBM)
  tiny     the D=256 fp32 layer (parity workload; wall time and the oracle timed multi-
           and single-threaded)
  verify   the stack, B=8 sequences x T=4 tokens a step + commit of the accepted prefix
  prefill  one BF16 layer, B=4 x L=8192 chunked prefill (MFMA-bound)

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--workload stack|layer|tiny|verify|prefill] [--per-layer] [--graph] [--copies N]
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
BF16_PEAK_TFLOPS = 2500.0      # dense MFMA, bf16

# HBM bytes per launch of the one-launch step from rocprofv3 FETCH_SIZE + WRITE_SIZE, each
# scaled by the same counter on a plain 256 MiB copy (FETCH x2.0, WRITE x1.0), valid while
# the kernel's sources hash to "sha256" (see profiles/ for the runs).
STEP_TRAFFIC = {"bytes": 744120053,
                "sha256": "f9fd605861c8b505db628d44373596d762f3aa44982023aa9e6d52a873e91c91",
                "sources": ("persistent.hip", "kda_device.h", "persist.h")}


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


def synth_default_wtype(name):
    """The weight format a decode workload is defined with."""
    import synth
    return synth.WORKLOADS[name].wtype


def algorithmic_bytes(w) -> dict:
    """Bytes each kernel of one layer must move at B=1 (weights incl. Q8_0 scales,
    state, conv window, activations), and the per-token total of the stack."""
    d = w.dims
    D, K, V, H = d.d_model, d.key_dim, d.value_dim, d.n_heads
    C = d.conv_channels

    def q8(rows, cols):   # packed bytes of one matrix in the workload's weight format
        if w.wtype == "q8_0":
            return rows * cols + rows * (cols // 32) * 2
        if w.wtype == "mxfp4":
            return rows * cols // 2 + rows * (cols // 32)
        return rows * cols * (2 if w.wtype == "bf16" else 4)

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


def cpu_baseline(run, budget_s: float = 15.0, single_thread: bool = False):
    """The float64 oracle, as it stands, on the first tokens of the same workload (with
    single_thread, also timed with its BLAS limited to one thread)."""
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
    res = _oracle_decode_rate(ok, layers, run, budget_s, threads)
    if single_thread:
        with threadpoolctl.threadpool_limits(1):
            one = _oracle_decode_rate(ok, layers, run, budget_s / 2, 1)
        res["single_thread"] = {"value": one["value"], "unit": one["unit"], "cores": 1,
                                "sample": one["sample"]}
    return res


def _oracle_decode_rate(ok, layers, run, budget_s, threads):
    w = run.workload
    d = w.dims
    n = 0
    t0 = time.time()
    S = [[run.s0[l, 0].astype(np.float64)] for l in range(w.n_layers)]
    Z = [[np.zeros((3, d.conv_channels))] for _ in range(w.n_layers)]
    while True:
        xt = run.x[n % w.steps, 0, 0].astype(np.float64)[None, :]   # inputs reused cyclically
        if w.prenorm_residual:
            _, s_new, z_new = ok.stack_step(layers, xt, [S[l][0] for l in range(w.n_layers)],
                                            [Z[l][0] for l in range(w.n_layers)])
        else:
            _, s1, z1 = ok.layer_forward(layers[0], xt, S[0][0], Z[0][0])
            s_new, z_new = [s1], [z1]
        for l in range(w.n_layers):
            S[l][0], Z[l][0] = s_new[l], z_new[l]
        n += 1
        if time.time() - t0 > budget_s:
            break
    el = time.time() - t0
    return {"value": n / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} consecutive decode tokens of the {w.n_layers}-layer {w.wtype} "
                      f"workload '{w.name}', B=1, float64 numpy oracle ({el:.1f}s, BLAS "
                      f"threads={threads}, host nproc={os.cpu_count()})"}


def timed_kinds(model, kda, kinds):
    """Per-kind (avg us, launches) of the event-timed launches since the last reset."""
    out = {}
    for k, v in kinds.items():
        ms, n = model.timing(v)
        if n:
            out[k] = (ms * 1e3 / n, n)
    return out


def roofline_entry(per, bound, peak, unit):
    dom = max(per, key=lambda k: per[k]["avg_us"] * per[k]["launches"])
    ach = per[dom]["rate"]
    return dom, {"bound": bound, "kernel": dom, "achieved": round(ach, 1), "peak": peak,
                 "unit": unit, "frac": round(ach / peak, 4)}


def bench_stack(args, torch, synth, kda, w, run, model):
    d = w.dims
    B = w.batch
    st = model.new_state(B)
    st.S.copy_(torch.from_numpy(run.s0))
    ws = model.workspace(kda.KDA_OP_DECODE, B)
    xs = torch.from_numpy(np.ascontiguousarray(run.x[:, :, 0, :])).cuda()   # [steps][B][D]
    y = torch.empty((B, d.d_model), dtype=torch.float32, device="cuda")

    model.set_option(kda.KDA_OPT_GRAPH, 1 if args.graph else 0)
    model.set_option(kda.KDA_OPT_PERSISTENT, 0 if args.per_layer else 1)
    one_launch = not args.per_layer and model.persistent_blocks() > 0 and B == 1
    models = [model]
    if args.copies > 1:
        # more weight copies than fit the 256 MB last-level cache, used in turn, so that each
        # step streams its weights from HBM (a copy per model, the state shared)
        for _ in range(args.copies - 1):
            m2 = kda.KdaModel(run.layers, n_heads=d.n_heads, d_k=d.d_k, d_v=d.d_v, wtype=w.wtype,
                              prenorm_residual=w.prenorm_residual, norm_eps=w.norm_eps,
                              l2_eps=w.l2_eps)
            m2.set_option(kda.KDA_OPT_GRAPH, 1 if args.graph else 0)
            m2.set_option(kda.KDA_OPT_PERSISTENT, 0 if args.per_layer else 1)
            models.append(m2)
        log(f"[bench] {len(models)} weight copies used in turn")
    path = (f"one launch per token ({model.persistent_blocks()} blocks)" if one_launch
            else "per-layer kernels replayed as one hipGraph" if args.graph
            else "per-layer kernels launched directly")
    log(f"[bench] path: {path}")
    # with --graph each step's input row is copied into one fixed input buffer first (as a
    # serving loop writes its next token's embedding), so that the captured graph is
    # replayed, not captured again for every new input pointer; launched directly (and the
    # one-launch kernel always is) the kernels read the step's row where it lies
    xin = torch.empty((B, d.d_model), dtype=torch.float32, device="cuda")

    def step(i):
        if not args.graph:
            models[i % len(models)].decode_step(xs[i], y, st, ws)
            return
        xin.copy_(xs[i])
        models[i % len(models)].decode_step(xin, y, st, ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # ---- timed region: K steps, inputs resident in HBM ----
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    model.status()
    for m2 in models[1:]:
        m2.close()
    tok_s = B * args.steps / el
    ms_step = el * 1e3 / args.steps
    log(f"[bench] {args.steps} steps in {el * 1e3:.2f} ms: {tok_s:.1f} tokens/s")

    # ---- per-kernel durations with hipEvents on the launch stream (no graph) ----
    model.set_option(kda.KDA_OPT_TIMING, 1)
    model.timing(kda.KDA_K_PROJ, reset=True)
    for i in range(args.steps):
        model.decode_step(xs[args.warmup + i], y, st, ws)
    torch.cuda.synchronize()
    model.status()
    times = timed_kinds(model, kda, {"proj": kda.KDA_K_PROJ, "gates": kda.KDA_K_GATES,
                                     "head": kda.KDA_K_HEAD, "out": kda.KDA_K_OUT,
                                     "step": kda.KDA_K_STEP})
    model.set_option(kda.KDA_OPT_TIMING, 0)
    ab = algorithmic_bytes(w)
    per = {}
    for k, (avg_us, n) in times.items():
        per[k] = {"avg_us": avg_us, "launches": n, "bytes": ab[k],
                  "rate": ab[k] / (avg_us * 1e-6) / 1e9}
        log(f"[bench] kernel {k}: {n} launches, avg {avg_us:.2f} us, "
            f"{per[k]['rate']:.0f} GB/s algorithmic")
    dom, roof = roofline_entry(per, "hbm", HBM_PEAK_GBS, "GB/s")
    # (the counted traffic is that of the Q8_0 step)
    roof["traffic"] = step_traffic() if dom == "step" and w.wtype == "q8_0" else None
    step_gbs = ab["token_weights_state"] / (ms_step * 1e-3) / 1e9
    # the measured sequential-read ceiling over a buffer the size of a token's bytes (the
    # byte pricing of antirez/ds4 PR #964 prices against such a ceiling); reported beside
    # the vendor peak, never in place of it
    ceil_bytes = max(ab["token_weights_state"] if w.n_layers > 1 else 8 * ab["token_weights_state"],
                     1 << 28)
    probe = torch.empty(ceil_bytes // 16 * 16, dtype=torch.uint8, device="cuda")
    ceil_ms = kda.kda_stream_read_probe(probe, 20)
    del probe
    ceiling = ceil_bytes / (ceil_ms * 1e-3) / 1e9
    roof["ceiling_gbs"] = round(ceiling, 1)
    roof["frac_of_ceiling"] = round(roof["achieved"] / ceiling, 4)
    log(f"[bench] sequential-read ceiling {ceiling:.0f} GB/s over {ceil_bytes / 1e6:.0f} MB; "
        f"the kernel reaches {roof['frac_of_ceiling']:.3f} of it")
    config = {"workload": f"kda-{w.n_layers}L-{w.wtype}-decode" if w.n_layers > 1
              else f"kda-layer-{w.wtype}-decode",
              "layers": w.n_layers, "d_model": d.d_model, "heads": d.n_heads, "d_k": d.d_k,
              "d_v": d.d_v, "weights": w.wtype, "state": "f32", "batch": B, "global_batch": B,
              "seq_len": 1, "parallelism": "none (1 GPU)", "path": path,
              "bytes_per_token": ab["token_weights_state"],
              "step_hbm_gbs": round(step_gbs, 1),
              "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
              "kernels": rounded(per)}
    if args.copies > 1:
        config["weight_copies"] = args.copies
        config["workload"] += f"-{args.copies}copies"
    if w.name == "stack":
        config["workload"] = f"kda-stack-34L-{w.wtype}-decode"
    if w.name == "tiny":
        config["workload"] = f"kda-tiny-layer-{w.wtype}-decode"
    metric = {"stack": "KDA decode tokens/s (34-layer stack, B=1)",
              "layer": "KDA decode tokens/s (one BF16 layer, B=1)",
              "tiny": "KDA decode tokens/s (tiny fp32 layer, B=1)"}[w.name]
    if w.wtype != synth_default_wtype(w.name):
        metric += f", {w.wtype} weights"
    return metric, tok_s, "tokens/s", ms_step, config, roof


def verify_bytes(w):
    """Algorithmic bytes per verify step (B sequences x T tokens): every layer's weights once
    and each sequence's state read once and written once (the previous step's commit is
    replayed inside the verify's head kernel, from the log rows of its accepted tokens)."""
    d = w.dims
    D, K, V, H = d.d_model, d.key_dim, d.value_dim, d.n_heads
    C = d.conv_channels
    N = w.batch * w.tokens

    def q8(rows, cols):
        return rows * cols + rows * (cols // 32) * 2

    rows = C + d.rank_f + d.rank_g + H
    proj_w = q8(K, D) * 2 + q8(V, D) + q8(d.rank_f, D) + q8(d.rank_g, D) + q8(H, D)
    state = H * d.d_k * d.d_v * 4
    per = {"proj": proj_w + N * (D + rows) * 4,
           "gates": q8(K, d.rank_f) + q8(V, d.rank_g) + N * (d.rank_f + d.rank_g + K + V) * 4,
           "head": w.batch * 2 * state + N * (rows + K + V + 2 * V) * 4 + N * (2 * K + V + H) * 4,
           "out": q8(D, V) + N * (2 * V + 2 * D) * 4,
           "commit": w.batch * 2 * state}
    floor = w.n_layers * (proj_w + q8(K, d.rank_f) + q8(V, d.rank_g) + q8(D, V)
                          + w.batch * 2 * 2 * state // 2)
    return per, floor


def bench_verify(args, torch, synth, kda, w, run, model):
    d = w.dims
    B, T = w.batch, w.tokens
    st = model.new_state(B)
    st.S.copy_(torch.from_numpy(run.s0))
    ws = model.workspace(kda.KDA_OP_VERIFY, B, T)
    vlog = model.verify_log(B, T)
    xs = torch.from_numpy(np.ascontiguousarray(run.x)).cuda()             # [steps][B][T][D]
    ys = torch.empty((B, T, d.d_model), dtype=torch.float32, device="cuda")
    acc = torch.from_numpy(np.ascontiguousarray(run.accept).astype(np.int32)).cuda()
    model.set_option(kda.KDA_OPT_GRAPH, 1 if args.graph else 0)
    # with --graph: fixed input and accept buffers (a serving loop's draft batch and sampler
    # output), so that the captured verify and commit graphs are replayed
    xin = torch.empty((B, T, d.d_model), dtype=torch.float32, device="cuda")
    ain = torch.empty((B,), dtype=torch.int32, device="cuda")

    def step(i):
        if args.graph:
            xin.copy_(xs[i])
            ain.copy_(acc[i])
        xi, ai = (xin, ain) if args.graph else (xs[i], acc[i])
        model.verify_steps(xi, T, ys, st, vlog, ws)
        model.verify_commit(st, vlog, T, ai)       # recorded; folded into the next verify

    for i in range(args.warmup):
        step(i)
    model.flush(st)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    model.flush(st)                                 # the last step's commit, applied
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    accepted = int(run.accept[args.warmup:args.warmup + args.steps].clip(1, T).sum())
    pos_s = B * T * args.steps / el
    log(f"[bench] verify {args.steps} steps in {el * 1e3:.2f} ms: {pos_s:.0f} positions/s, "
        f"{accepted / el:.0f} accepted tokens/s")
    model.set_option(kda.KDA_OPT_TIMING, 1)
    model.timing(kda.KDA_K_PROJ, reset=True)
    for i in range(args.steps):
        step(args.warmup + i)
    model.flush(st)
    torch.cuda.synchronize()
    times = timed_kinds(model, kda, {"proj": kda.KDA_K_PROJ, "gates": kda.KDA_K_GATES,
                                     "head": kda.KDA_K_HEAD, "out": kda.KDA_K_OUT,
                                     "commit": kda.KDA_K_COMMIT})
    model.set_option(kda.KDA_OPT_TIMING, 0)
    bper, floor = verify_bytes(w)
    per = {}
    for k, (avg_us, n) in times.items():
        per[k] = {"avg_us": avg_us, "launches": n, "bytes": bper[k],
                  "rate": bper[k] / (avg_us * 1e-6) / 1e9}
        log(f"[bench] kernel {k}: {n} launches, avg {avg_us:.2f} us, "
            f"{per[k]['rate']:.0f} GB/s algorithmic")
    dom, roof = roofline_entry(per, "hbm", HBM_PEAK_GBS, "GB/s")
    roof["traffic"] = None
    ms_step = el * 1e3 / args.steps
    gbs = floor / (ms_step * 1e-3) / 1e9
    config = {"workload": "kda-stack-34L-q8_0-verify-B8-T4", "layers": w.n_layers,
              "d_model": d.d_model, "heads": d.n_heads, "batch": B, "tokens_per_step": T,
              "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)",
              "launch": "hipGraph replays" if args.graph else "kernels launched directly",
              "accepted_tokens_per_s": round(accepted / el, 1),
              "bytes_floor_per_step": floor, "step_hbm_gbs": round(gbs, 1),
              "step_hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "kernels": rounded(per)}
    return ("KDA verify positions/s (34-layer stack, B=8, T=4)", pos_s, "positions/s", ms_step,
            config, roof)


def prefill_flops(w):
    """Algorithmic flops of one chunked prefill call per kernel kind: the two projection
    GEMMs; the chunk kernels (the forget gate's up-projection, L, A, W, U per chunk, and the
    scan's D, O, S products); the gated norm (the output gate's up-projection)."""
    d = w.dims
    M = w.batch * w.tokens
    rows = d.conv_channels + d.rank_f + d.rank_g + d.n_heads
    gemm = 2 * M * (rows * d.d_model + d.d_model * d.value_dim)
    # chunk math per (seq, head, chunk of c): L, A (2 c^2 dk), W, U (c^2 (dk + dv)),
    # D = U - W S (c dk dv), O = Q S + A D (c dk dv + c^2 dv), S += K^T D (c dk dv)
    c = w.chunk
    per_chunk = 2 * (2 * c * c * d.d_k + c * c * (d.d_k + d.d_v) + 3 * c * d.d_k * d.d_v
                     + c * c * d.d_v)
    chunk = w.batch * d.n_heads * (w.tokens // c) * per_chunk + 2 * M * d.key_dim * d.rank_f
    norm = 2 * M * d.value_dim * d.rank_g
    return {"gemm": gemm, "chunk": chunk, "norm": norm}


def bench_prefill(args, torch, synth, kda, w, run, model):
    d = w.dims
    B, L = w.batch, w.tokens
    x = torch.from_numpy(np.ascontiguousarray(run.x_bits[0]).view(np.int16)).cuda()
    y = torch.empty((B, L, d.d_model), dtype=torch.float32, device="cuda")
    ws = model.workspace(kda.KDA_OP_PREFILL, B, L)
    sts = [model.new_state(B) for _ in range(2)]

    def call(i):
        st = sts[i % 2]
        st.S.zero_()
        st.conv.zero_()
        model.prefill_chunked(x, kda.KDA_BF16, L, w.chunk, y, st, ws)

    steps, warm = max(1, min(args.steps, 10)), max(1, min(args.warmup, 2))
    for i in range(warm):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    tok_s = B * L * steps / el
    log(f"[bench] prefill {steps} calls in {el * 1e3:.2f} ms: {tok_s:.0f} tokens/s")
    model.set_option(kda.KDA_OPT_TIMING, 1)
    model.timing(kda.KDA_K_PROJ, reset=True)
    for i in range(steps):
        call(i)
    torch.cuda.synchronize()
    times = timed_kinds(model, kda, {"gemm": kda.KDA_K_GEMM, "chunk": kda.KDA_K_CHUNK,
                                     "norm": kda.KDA_K_PREFILL})
    model.set_option(kda.KDA_OPT_TIMING, 0)
    fl = prefill_flops(w)
    per = {}
    for k, (avg_us, n) in times.items():
        total = avg_us * n / steps                       # per call
        flops = fl.get(k, 0)
        per[k] = {"avg_us": avg_us, "launches": n, "us_per_call": total,
                  "flops_per_call": flops,
                  "rate": flops / (total * 1e-6) / 1e12 if flops else 0.0}
        log(f"[bench] kernel {k}: {n} launches, {total:.1f} us per call"
            + (f", {per[k]['rate']:.1f} TFLOP/s" if flops else ""))
    dom = max(per, key=lambda k: per[k]["us_per_call"])
    ach = per[dom]["rate"]
    roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2),
            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": None}
    ms_call = el * 1e3 / steps
    total_fl = sum(fl.values())
    config = {"workload": "kda-layer-bf16-prefill-B4-L8192-chunk64", "layers": 1,
              "d_model": d.d_model, "heads": d.n_heads, "batch": B, "global_batch": B,
              "seq_len": L, "chunk": w.chunk, "parallelism": "none (1 GPU)",
              "flops_per_call": total_fl,
              "call_tflops": round(total_fl / (ms_call * 1e-3) / 1e12, 2),
              "kernels": rounded(per)}
    return ("KDA chunked prefill tokens/s (one BF16 layer, B=4, L=8192)", tok_s, "tokens/s",
            ms_call, config, roof)


def rounded(per):
    return {k: {kk: (round(vv, 3) if isinstance(vv, float) else vv) for kk, vv in v.items()}
            for k, v in per.items()}


def cpu_baseline_for(name, run, budget_s):
    if name in ("stack", "layer", "tiny"):
        return cpu_baseline(run, budget_s, single_thread=name in ("layer", "tiny"))
    from oracle import kda as ok
    w = run.workload
    d = w.dims
    layers = [ok.prepare_layer(dr, w.wtype, d.n_heads, d.d_k, d.d_v, w.norm_eps, w.l2_eps)
              for dr in run.layers]
    import threadpoolctl
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    t0 = time.time()
    n = 0
    if name == "verify":
        S = [np.array(run.s0[l, 0], np.float64) for l in range(w.n_layers)]
        Z = [np.zeros((3, d.conv_channels)) for _ in range(w.n_layers)]
        k = 0
        while time.time() - t0 < budget_s:
            i = k % w.steps
            _, S, Z = ok.stack_step(layers, run.x[i, 0].astype(np.float64), S, Z,
                                    keep_after=int(np.clip(run.accept[i, 0], 1, w.tokens)))
            k += 1
            n += w.tokens
        el = time.time() - t0
        return {"value": n / el, "unit": "positions/s", "cores": threads, "kind": "oracle",
                "sample": f"{n // w.tokens} verify steps of one sequence (T={w.tokens}) through "
                          f"the 34-layer stack, float64 oracle ({el:.1f}s)"}
    # prefill: the sequential oracle over one whole sequence
    L = w.tokens
    ok.prefill_run(layers[0], run.x[0][:1, :L], run.s0[0][:1], seqs=[0])
    el = time.time() - t0
    return {"value": L / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one sequence of {L} tokens, token-by-token float64 oracle ({el:.1f}s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--workload", default="stack",
                    choices=("stack", "layer", "tiny", "verify", "prefill"))
    ap.add_argument("--wtype", default=None, choices=("f32", "bf16", "q8_0", "mxfp4"),
                    help="decode workloads (stack, layer, tiny): the same shapes with another "
                         "weight format")
    ap.add_argument("--copies", type=int, default=1,
                    help="decode workloads: weight copies used in turn (8 keeps the BF16 layer "
                         "out of the last-level cache)")
    ap.add_argument("--per-layer", action="store_true",
                    help="time the per-layer decode instead of the one-launch step")
    ap.add_argument("--graph", action="store_true",
                    help="per-layer decode and verify: replay captured hipGraphs (inputs "
                         "copied into fixed buffers) instead of launching the kernels")
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

    w = synth.WORKLOADS[args.workload]
    if args.wtype:
        if args.workload not in ("stack", "layer", "tiny"):
            print("--wtype applies to the decode workloads (stack, layer, tiny)", file=sys.stderr)
            sys.exit(2)
        w = synth.scaled(w, wtype=args.wtype)
    if args.workload != "prefill":
        w = synth.scaled(w, steps=max(args.steps + args.warmup, 1))
    t0 = time.time()
    run = synth.draw_run(w)
    log(f"[bench] drew {w.n_layers}-layer weights + inputs in {time.time() - t0:.1f}s")
    d = w.dims
    t0 = time.time()
    model = kda.KdaModel(run.layers, n_heads=d.n_heads, d_k=d.d_k, d_v=d.d_v, wtype=w.wtype,
                         prenorm_residual=w.prenorm_residual, norm_eps=w.norm_eps,
                         l2_eps=w.l2_eps)
    log(f"[bench] packed {w.wtype} weights on the device in {time.time() - t0:.1f}s")
    fn = {"stack": bench_stack, "layer": bench_stack, "tiny": bench_stack,
          "verify": bench_verify, "prefill": bench_prefill}[args.workload]
    metric, value, unit, ms_step, config, roof = fn(args, torch, synth, kda, w, run, model)
    model.close()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_for(args.workload, run, args.cpu_budget)
        log(f"[cpu] {cpu['sample']}: {cpu['value']:.3f} {cpu['unit']}")

    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
