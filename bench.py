#!/usr/bin/env python3
"""Benchmark: routed RVQ-MoE layer on one MI355X.

Default workload (the headline): one K3-scale MoE layer, batch-1 decode.
d=7168, ffn=2048, E=384 experts, top-16, expert weights as 3-stage RVQ
(256-entry fp16 codebooks over 8-wide vectors, uniform u8 codes, 16,515,072 B
per expert record), router N(0, 0.02), tokens x ~ N(0,1) with one seed per
token.  A step is one call of the whole hot path -- router GEMV, top-16,
softmax gates, LUT build, gate/up gather + SiLU, down gather, gate-weighted
combine -- by default as one rvq_moe_route_forward call (the fastest way at
batch 1; --path two-call times rvq_moe_route_topk then rvq_moe_layer_forward),
every token distinct, all inputs resident in HBM before the timed region.

Other workloads of the same layer shape:
  --batch B    B tokens per call (batched decode, pairs grouped by expert);
  --chunk      with --batch: every call takes the chunk path (prefill chunk:
               weights rebuilt as bf16 tiles feeding the matrix cores);
  --layers L   a depth chain: L layers, each with RMS normalisation before
               routing and a residual add, one token through all L per step;
  --stream-slots S   codes kept in pinned host memory and streamed through S
               HBM expert slots (copies on a side stream, overlapped); every
               record copied in has its trailer checked on the device;
  --verify     with --stream-slots: also the CRC-32 of every record's payload.
  --lookahead N  with --layers and --stream-slots: after each layer's call,
               the next layer's router runs on this layer's input and the
               first N of its predicted experts are prefetched into the next
               layer's slots (router lookahead).

Prints one JSON line: tokens/s (value), effective compressed-weight GB/s and
its fraction of the 8 TB/s HBM peak, the roofline record of the dominant
kernel (the layer kernel, timed with HIP events on its launch stream), and the
oracle timed on the host cores on a bounded sample (cpu_baseline).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "routed MoE-layer tokens/s + effective compressed-weight GB/s vs HBM peak"
CB_BYTES = 3 * 3 * 256 * 8 * 2  # one expert's fp16 codebooks (3 matrices x 3 stages)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha256() -> str:
    """Hash of the library's sources (kernels, launchers, ABI header)."""
    h = hashlib.sha256()
    files = glob.glob(os.path.join(ROOT, "vector_quantized_expert_amd", "csrc", "*.hip"))
    files += glob.glob(os.path.join(ROOT, "vector_quantized_expert_amd", "csrc", "*.hpp"))
    for f in sorted(files + [os.path.join(ROOT, "include", "rvq_moe.h")]):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(fused: bool):
    """HBM bytes per layer-kernel launch from the committed counter runs
    (FETCH_SIZE and WRITE_SIZE scaled by a reference copy), or None when the
    sources have changed since those counters were taken."""
    name = "k_layer_routed_k3_batch1_decode_traffic.md" if fused else "k_layer_k3_batch1_decode_traffic.md"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            key, sep, val = line.partition(":")
            if sep and key.strip() in ("traffic_bytes_per_launch", "source_sha256"):
                fields[key.strip()] = val.strip()
    if fields.get("source_sha256") != source_sha256():
        return None
    return int(fields["traffic_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000, help="timed steps (one call, or one token through the chain)")
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-tokens", type=int, default=2, help="tokens the oracle baseline runs (0: skip)")
    ap.add_argument("--profile-every", type=int, default=8, help="time kernels with events every n-th call")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--batch", type=int, default=1,
                    help="tokens per call; above 1 the pairs of a call are grouped by expert (batched decode)")
    ap.add_argument("--layers", type=int, default=1,
                    help="depth chain of this many layers (RMS normalisation before routing, residual add)")
    ap.add_argument("--chunk", action="store_true",
                    help="every layer_forward call takes the chunk path (bf16 matrix cores)")
    ap.add_argument("--stream-slots", type=int, default=0,
                    help="stream the codes from a pinned host bank through this many HBM slots")
    ap.add_argument("--verify", action="store_true",
                    help="with --stream-slots: check the CRC-32 of every expert record copied into a slot")
    ap.add_argument("--lut-expert-tokens", type=int, default=0,
                    help="with --chunk: experts routed fewer tokens than this take the table path (0: the "
                         "library default, 1: every expert on the matrix cores)")
    ap.add_argument("--lookahead", type=int, default=0,
                    help="with --layers and --stream-slots: after layer l's call, run layer l+1's router on layer "
                         "l's input and prefetch the first N of its predicted experts (rvq_moe_prefetch)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the run, one plain device-to-device copy of this many bytes (a reference kernel "
                         "of known traffic for scaling hardware byte counters)")
    ap.add_argument("--path", choices=("fused", "two-call"), default=None,
                    help="fused: rvq_moe_route_forward (one launch per call; the default for batch-1 decode with "
                         "resident codes); two-call: rvq_moe_route_topk then rvq_moe_layer_forward (the default "
                         "elsewhere)")
    args = ap.parse_args()
    if args.path is None:
        args.path = ("fused" if args.batch == 1 and not args.chunk and args.stream_slots == 0 and not args.lookahead
                     else "two-call")

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
    K, W, B, L = args.steps, args.warmup, args.batch, args.layers
    chain = L > 1
    streaming = args.stream_slots > 0
    if (B < 1 or L < 1 or (chain and B != 1) or
            (args.path == "fused" and (B * shape.top_k > 1024 or args.chunk or streaming)) or
            (args.verify and not streaming) or
            (args.lookahead and (not chain or not streaming or args.path == "fused" or
                                 not 1 <= args.lookahead <= shape.top_k))):
        print(f"--batch {B} / --layers {L} outside what the chosen path takes", file=sys.stderr)
        sys.exit(2)

    layers, inputs = [], []
    for li in range(L):
        log(f"staging layer {li}: d={shape.d} ffn={shape.ffn} E={shape.n_experts} k={shape.top_k}")
        inp = G.LayerInputs(shape, seed=args.seed, layer=li)
        codes, extra = inp.codes_dev, {}
        if streaming:
            codes = torch.empty(inp.codes_dev.shape, dtype=torch.uint8, pin_memory=True)
            codes.copy_(inp.codes_dev)
            extra = dict(codes_location=1, cache_slots=args.stream_slots, verify_records=args.verify)
        layers.append(RvqMoe(d=shape.d, ffn=shape.ffn, n_experts=shape.n_experts, top_k=shape.top_k,
                             codebook_dtype=1, router_w=inp.w_r_dev, codebooks=inp.cb_dev, codes=codes,
                             max_tokens=B, pre_rmsnorm=chain, residual=chain, eps=1e-6,
                             chunk_min_tokens=1 if args.chunk else B + 1,
                             lut_expert_tokens=args.lut_expert_tokens, **extra))
        del codes
        inp.free_codes()
        inputs.append(inp)
        torch.cuda.empty_cache()

    n_tok = (W + K) * B
    x_host = S.tokens(args.seed, 0, n_tok, shape.d)
    # h[l] is the input of layer l (h[0] = the tokens); h[L] the chain's output
    h = torch.empty((L + 1, n_tok, shape.d), dtype=torch.float32, device="cuda")
    h[0].copy_(G.to_device(x_host))
    ids = torch.empty((L, n_tok, shape.top_k), dtype=torch.int32, device="cuda")
    gates = torch.empty((L, n_tok, shape.top_k), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    if args.lookahead:  # predicted ids of layer l (its router on layer l-1's input), routed on a side stream
        pred = torch.full((L, n_tok, shape.top_k), -1, dtype=torch.int32, device="cuda")
        pred_g = torch.empty((n_tok, shape.top_k), dtype=torch.float32, device="cuda")
        side = torch.cuda.Stream()
        routed = torch.cuda.Event()

    def step(t):
        r = slice(t * B, (t + 1) * B)
        for li, layer in enumerate(layers):
            if args.path == "fused":
                layer.route_forward(h[li, r], B, ids[li, r], gates[li, r], h[li + 1, r], stream)
            else:
                layer.route_topk(h[li, r], B, ids[li, r], gates[li, r], stream)
                if args.lookahead and li + 1 < L:
                    routed.record(stream)  # h[li] is complete
                layer.layer_forward(h[li, r], B, ids[li, r], gates[li, r], h[li + 1, r], stream)
                if args.lookahead and li + 1 < L:
                    side.wait_event(routed)
                    layers[li + 1].route_topk(h[li, r], B, pred[li + 1, r], pred_g[r], side)
                    layers[li + 1].prefetch(pred[li + 1, r], B, args.lookahead, side)

    h2d = None
    if streaming:
        # the host -> device ceiling this box measures for pinned copies of one
        # expert record each (as the slot fills), 1 GiB in all, three rounds
        rec_b = shape.record_bytes
        n_rec = (1 << 30) // rec_b
        src = torch.empty(n_rec * rec_b, dtype=torch.uint8, pin_memory=True)
        dst = torch.empty(n_rec * rec_b, dtype=torch.uint8, device="cuda")
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            for i in range(n_rec):
                dst[i * rec_b:(i + 1) * rec_b].copy_(src[i * rec_b:(i + 1) * rec_b], non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        h2d = {"ceiling_GBps": 3 * n_rec * rec_b / (e0.elapsed_time(e1) * 1e-3) / 1e9}
        del src, dst
        torch.cuda.empty_cache()

    log(f"warmup {W} steps of {B} token(s) x {L} layer(s)")
    for t in range(W):
        step(t)
    for layer in layers:
        layer.sync(stream)
        layer.kernel_times()  # drop warmup samples
        layer.set_profiling(args.profile_every)

    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stats0 = [layer.stats() for layer in layers]
    ev0.record(stream)
    for t in range(W, W + K):
        step(t)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    n_l, l_ms = 0, 0.0
    kernels = {}
    lut_kind = "route_layer_lut" if args.path == "fused" else ("chunk" if args.chunk else "layer_lut")
    for layer in layers:
        layer.set_profiling(0)
        for kind, (n, v) in layer.kernel_times().items():
            a = kernels.setdefault(kind, [0, 0.0])
            a[0] += n
            a[1] += v
        layer.sync(stream)
    n_l, l_ms = kernels[lut_kind]
    log(f"timed {K} steps in {ms:.2f} ms")
    if streaming:
        st = [layer.stats() for layer in layers]
        moved = sum(a["h2d_bytes"] - b["h2d_bytes"] for a, b in zip(st, stats0))
        hits = sum(a["slot_hits"] - b["slot_hits"] for a, b in zip(st, stats0))
        misses = sum(a["slot_misses"] - b["slot_misses"] for a, b in zip(st, stats0))
        checked = sum(a["records_checked"] - b["records_checked"] for a, b in zip(st, stats0))
        verified = sum(a["records_verified"] - b["records_verified"] for a, b in zip(st, stats0))
        h2d.update({"slots": args.stream_slots, "h2d_bytes": moved, "GBps": moved / (ms * 1e-3) / 1e9,
                    "frac_of_ceiling": moved / (ms * 1e-3) / 1e9 / h2d["ceiling_GBps"],
                    "hit_rate": hits / max(hits + misses, 1), "records_checked": checked,
                    "records_crc_verified": verified})
        if args.lookahead:
            fills = sum(a["prefetch_fills"] - b["prefetch_fills"] for a, b in zip(st, stats0))
            phits = sum(a["prefetch_hits"] - b["prefetch_hits"] for a, b in zip(st, stats0))
            ph, ih = pred.cpu().numpy(), ids.cpu().numpy()
            right = [len(set(ph[l, t, :args.lookahead].tolist()) & set(ih[l, t].tolist()))
                     for l in range(1, L) for t in range(W, W + K)]
            h2d.update({"lookahead": args.lookahead, "prefetch_fills": fills, "prefetch_hits": phits,
                        "prefetch_used_frac": phits / max(fills, 1),
                        "prediction_precision": float(np.mean(right)) / args.lookahead})

    rec = shape.record_bytes
    # Algorithmic bytes of one layer call: every distinct expert the call routes
    # to, read once (code record + its 3 matrices' codebooks).  At batch 1 that
    # is k experts; in a batch, experts shared by several tokens count once.
    ids_h = ids.cpu().numpy()
    uniq = np.array([[len(np.unique(ids_h[li, t * B:(t + 1) * B])) for t in range(W, W + K)] for li in range(L)],
                    dtype=np.float64)
    per_call_bytes = float(uniq.mean()) * (rec + CB_BYTES)
    calls_s = K * L / (ms / 1e3)
    tok_s = K * B / (ms / 1e3)
    gbps = per_call_bytes * calls_s / 1e9
    l_avg_us = l_ms / n_l * 1e3 if n_l else float("nan")  # nan: kernel timing switched off
    l_gbps = per_call_bytes / (l_avg_us * 1e-6) / 1e9
    kernels = {k: {"launches": int(n), "avg_us": (v / n * 1e3 if n else None)} for k, (n, v) in kernels.items()}

    # Parity on timed tokens (teacher-forced through the chain: the oracle runs
    # layer l on the GPU's own input of layer l) and the CPU baseline.
    cpu = None
    parity = None
    if args.cpu_tokens > 0:
        from oracle import oracle as O
        hs = h.cpu().numpy()
        errs, ok_ids = [], True
        t0 = time.perf_counter()
        for j in range(args.cpu_tokens):
            t = W * B + j
            for li in range(L):
                inp = inputs[li]
                ref = O.layer(hs[li, t], inp.w_r, shape.top_k, inp.codebook, inp.record, shape.d, shape.ffn,
                              pre_rmsnorm=chain, eps=1e-6, residual=chain)
                ok_ids &= bool(np.array_equal(ids_h[li, t], ref.route.ids))
                delta = hs[li + 1, t].astype(np.float64) - (hs[li, t].astype(np.float64) if chain else 0.0)
                errs.append(float(np.linalg.norm(delta - ref.delta) / np.linalg.norm(ref.delta)))
        cpu_s = time.perf_counter() - t0
        what = f"{L}-layer chain, teacher-forced" if chain else "one layer"
        cpu = {"value": args.cpu_tokens / cpu_s, "unit": "tokens/s", "cores": O.threads(), "kind": "oracle",
               "sample": f"{args.cpu_tokens} timed token(s) of the same workload ({what}; route + 16 experts per "
                         f"layer rebuilt as c1+c2+c3 in fp64); includes regenerating their code records on the host"}
        parity = {"tokens": args.cpu_tokens, "layers_checked": L, "ids_bit_exact": ok_ids, "max_rel_l2": max(errs)}

    where = (f"codes streamed from pinned host memory through {args.stream_slots} HBM slots"
             + (" (each record's CRC-32 checked)" if args.verify else "") if streaming
             else "resident codes")
    if args.chunk:
        workload = (f"K3-scale prefill chunk, {where}: {B} tokens per call through d=7168 ffn=2048 E=384 "
                    f"top-16, tokens grouped by expert, RVQ tiles rebuilt as bf16 for the matrix cores "
                    f"(fp32 accumulation)")
    elif chain:
        workload = (f"K3-scale depth chain, batch-1 decode: {L} layers of d=7168 ffn=2048 E=384 top-16 "
                    f"(3-stage x 256 x 8 fp16 codebooks, uniform u8 codes), RMSNorm (w=1, eps=1e-6) before "
                    f"routing and a residual add per layer, {where}" +
                    (f", router lookahead prefetching {args.lookahead} experts of the next layer"
                     if args.lookahead else ""))
    else:
        workload = (f"K3-scale routed RVQ-MoE layer, batch-{B} decode, {where}: d=7168 ffn=2048 E=384 top-16, "
                    f"3-stage x 256 x 8 fp16 codebooks, uniform u8 codes, T={B} per call")
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
        "dtype": "bf16" if args.chunk else "f32",
        "data": "synthetic",
        "config": {"workload": workload, "global_batch": B, "layers": L, "tokens": K * B,
                   "path": "rvq_moe_route_forward" if args.path == "fused"
                   else "rvq_moe_route_topk + rvq_moe_layer_forward"},
        "layer_calls_per_s": calls_s,
        "compressed_GBps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        "compressed_bytes_per_call": per_call_bytes,
        "distinct_experts_per_call": float(uniq.mean()),
        "roofline": {"bound": "hbm", "achieved": l_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": l_gbps / HBM_PEAK_GBPS,
                     "traffic": (recorded_traffic(args.path == "fused")
                                 if (B == 1 and L == 1 and not args.chunk and not streaming) else None),
                     "kernel": "k_layer<routed> (routing and experts in one launch)" if args.path == "fused" else
                     ("k_chunk_prep + k_chunk_stage + k_chunk_gu + k_chunk_down" if args.chunk else "k_layer"),
                     "algorithmic_bytes_per_launch": per_call_bytes, "avg_us": l_avg_us, "timed_launches": int(n_l)},
        "kernels": kernels,
        "h2d": h2d,
        "mfma": ({"flops_per_call": 6.0 * B * shape.top_k * shape.d * shape.ffn,
                  "tflops": 6.0 * B * shape.top_k * shape.d * shape.ffn / (l_avg_us * 1e-6) / 1e12,
                  "frac_of_bf16_dense_peak": 6.0 * B * shape.top_k * shape.d * shape.ffn / (l_avg_us * 1e-6) / 2.5e15}
                 if args.chunk else None),
        "cpu_baseline": cpu,
        "parity": parity,
    }
    for layer in layers:
        layer.close()
    if args.copy_bytes > 0:
        torch.cuda.empty_cache()
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_reference_bytes"] = args.copy_bytes
        del src, dst
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
