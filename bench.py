#!/usr/bin/env python3
"""Benchmark: routed RVQ-MoE layer, batch-1 decode at K3 scale, one MI355X.

Workload: one MoE layer with d=7168, ffn=2048, E=384 experts, top-16, expert
weights as 3-stage RVQ (256-entry fp16 codebooks over 8-wide vectors, uniform
u8 codes, 16,515,072 B per expert record), router N(0, 0.02), tokens x ~ N(0,1)
with one seed per token.  A step is one token through the whole hot path:
rvq_moe_route_topk (RMS-free router GEMV + top-16 + softmax gates) then
rvq_moe_layer_forward (LUT build, gate/up gather + SiLU, down gather,
gate-weighted combine), T = 1 per call, every token distinct, all inputs
resident in HBM before the timed region.

Prints one JSON line: tokens/s (value), effective compressed-weight GB/s and
its fraction of the 8 TB/s HBM peak, the roofline record of the dominant
kernel (gate/up gather, timed with HIP events on the launch stream), and the
oracle timed on the host cores on a bounded sample (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "routed MoE-layer tokens/s + effective compressed-weight GB/s vs HBM peak"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000, help="timed tokens (one layer call each)")
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-tokens", type=int, default=2, help="tokens the oracle baseline runs (0: skip)")
    ap.add_argument("--profile-every", type=int, default=8, help="time kernels with events every n-th call")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--batch", type=int, default=1,
                    help="tokens per call; above 1 the pairs of a call are grouped by expert (batched decode)")
    ap.add_argument("--path", choices=("fused", "two-call"), default="two-call",
                    help="fused: rvq_moe_route_forward (one launch per token); "
                         "two-call: rvq_moe_route_topk then rvq_moe_layer_forward")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer is not sharded across GPUs.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from synth import gpu as G
    from synth import synth as S
    from vector_quantized_expert_amd import RvqMoe

    torch.cuda.set_device(0)
    shape = S.K3
    K, W, B = args.steps, args.warmup, args.batch
    if B < 1 or (args.path == "fused" and B * shape.top_k > 1024):
        print(f"--batch {B} outside what the chosen path takes", file=sys.stderr)
        sys.exit(2)
    print(f"[bench] staging inputs d={shape.d} ffn={shape.ffn} E={shape.n_experts} k={shape.top_k}", file=sys.stderr,
          flush=True)
    inp = G.LayerInputs(shape, seed=args.seed, layer=0)
    layer = RvqMoe(d=shape.d, ffn=shape.ffn, n_experts=shape.n_experts, top_k=shape.top_k, codebook_dtype=1,
                   router_w=inp.w_r_dev, codebooks=inp.cb_dev, codes=inp.codes_dev, max_tokens=B)
    inp.free_codes()
    torch.cuda.empty_cache()

    n_tok = (W + K) * B
    x_host = S.tokens(args.seed, 0, n_tok, shape.d)
    x = G.to_device(x_host)
    ids = torch.empty((n_tok, shape.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((n_tok, shape.top_k), dtype=torch.float32, device="cuda")
    y = torch.empty((n_tok, shape.d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step_two(t):
        r = slice(t * B, (t + 1) * B)
        layer.route_topk(x[r], B, ids[r], gates[r], stream)
        layer.layer_forward(x[r], B, ids[r], gates[r], y[r], stream)

    def step_fused(t):
        r = slice(t * B, (t + 1) * B)
        layer.route_forward(x[r], B, ids[r], gates[r], y[r], stream)

    step = step_fused if args.path == "fused" else step_two

    print(f"[bench] warmup {W} calls of {B} token(s)", file=sys.stderr, flush=True)
    for t in range(W):
        step(t)
    layer.sync(stream)
    layer.kernel_times()  # drop warmup samples
    layer.set_profiling(args.profile_every)

    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for t in range(W, W + K):
        step(t)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    layer.set_profiling(0)
    ktimes = layer.kernel_times()
    layer.sync(stream)
    print(f"[bench] timed {K} calls in {ms:.2f} ms", file=sys.stderr, flush=True)

    rec = shape.record_bytes
    cb_bytes = 3 * 3 * 256 * 8 * 2
    # Algorithmic bytes of one call: every distinct expert the call routes to,
    # read once (code record + its 3 matrices' codebooks).  At batch 1 that is
    # k experts; in a batch, experts shared by several tokens count once.
    ids_all = ids.cpu().numpy().reshape(W + K, B * shape.top_k)
    uniq = np.array([len(np.unique(ids_all[t])) for t in range(W, W + K)], dtype=np.float64)
    per_call_bytes = float(uniq.mean()) * (rec + cb_bytes)
    tok_s = K * B / (ms / 1e3)
    gbps = per_call_bytes * (K / (ms / 1e3)) / 1e9

    # Dominant kernel: the persistent LUT kernel of the layer call.
    n_l, l_ms = ktimes["route_layer_lut" if args.path == "fused" else "layer_lut"]
    l_avg_us = l_ms / max(n_l, 1) * 1e3
    l_gbps = per_call_bytes / (l_avg_us * 1e-6) / 1e9
    kernels = {k: {"launches": int(n), "avg_us": (v / n * 1e3 if n else None)} for k, (n, v) in ktimes.items()}

    # Parity on the timed tokens the oracle re-runs, and the CPU baseline.
    cpu = None
    parity = None
    if args.cpu_tokens > 0:
        from oracle import oracle as O
        ids_h = ids.cpu().numpy()
        y_h = y.cpu().numpy()
        errs, ok_ids = [], True
        t0 = time.perf_counter()
        for j in range(args.cpu_tokens):
            t = W * B + j
            ref = O.layer(x_host[t], inp.w_r, shape.top_k, inp.codebook, inp.record, shape.d, shape.ffn)
            ok_ids &= bool(np.array_equal(ids_h[t], ref.route.ids))
            errs.append(float(np.linalg.norm(y_h[t] - ref.delta) / np.linalg.norm(ref.delta)))
        cpu_s = time.perf_counter() - t0
        cpu = {"value": args.cpu_tokens / cpu_s, "unit": "tokens/s", "cores": O.threads(), "kind": "oracle",
               "sample": f"{args.cpu_tokens} timed tokens of the same workload, full layer each (route + 16 experts "
                         f"rebuilt as c1+c2+c3 in fp64); includes regenerating their code records on the host"}
        parity = {"tokens": args.cpu_tokens, "ids_bit_exact": ok_ids, "max_rel_l2": max(errs)}

    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms / K,
        "tokens_per_step": B,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"K3-scale routed RVQ-MoE layer, batch-{B} decode: d=7168 ffn=2048 E=384 top-16, "
                               f"3-stage x 256 x 8 fp16 codebooks, uniform u8 codes, T={B} per call",
                   "global_batch": B, "tokens": K * B,
                   "path": "rvq_moe_route_forward" if args.path == "fused"
                   else "rvq_moe_route_topk + rvq_moe_layer_forward"},
        "compressed_GBps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        "compressed_bytes_per_call": per_call_bytes,
        "distinct_experts_per_call": float(uniq.mean()),
        "roofline": {"bound": "hbm", "achieved": l_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": l_gbps / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "k_layer<route>" if args.path == "fused" else "k_layer",
                     "algorithmic_bytes_per_launch": per_call_bytes, "avg_us": l_avg_us, "timed_launches": int(n_l)},
        "kernels": kernels,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    layer.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
