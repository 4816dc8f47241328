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

The default run also reports, in the same JSON line:
  - five repetitions of the K timed steps (median and range of ms per step)
    and per-call latency percentiles from events around every call;
  - measured ceilings of this machine (HBM streaming read, the table path's
    LDS gather rate, the fixed cost of a persistent-shaped launch, pinned
    host-to-device copies of expert records);
  - sub-records for the other workloads of the same layer shape: batched
    decode (32 tokens per call), the prefill chunk (512 tokens per call,
    resident) and the 16-layer depth chain;
  - the oracle on the host cores (one thread and all threads) and a parity
    sample of the timed tokens.

Other workloads as the headline (flags):
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
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def percentile(v, q):
    s = sorted(v)
    if not s:
        return None
    i = min(len(s) - 1, max(0, int(round(q / 100.0 * (len(s) - 1)))))
    return s[i]


def measure_ceilings(torch, shape):
    """This machine's ceilings: HBM streaming read over 8 GiB, the table path's
    LDS gather rate, the fixed cost of a persistent-shaped launch, and pinned
    host-to-device copies of expert records (1 GiB in record-sized pieces)."""
    from vector_quantized_expert_amd import ceilings as C
    stream = torch.cuda.current_stream()
    out = {}
    buf = torch.empty(8 << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    rd = C.hbm_read_GBps(buf, 3, stream)
    out["hbm_read_GBps"] = rd["best"]
    out["hbm_read_frac_of_peak"] = rd["best"] / HBM_PEAK_GBPS
    out["hbm_read_bytes"] = 3 * buf.numel()
    out["hbm_read_by_kernel_shape_GBps"] = {k: v for k, v in rd.items() if k != "best"}
    del buf
    torch.cuda.empty_cache()
    out["lds"] = C.lds_rates(stream)
    out["persistent_launch_us"] = C.launch_gap_us(500, stream)
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
    out["h2d_pinned_record_GBps"] = 3 * n_rec * rec_b / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return out


def oracle_baseline(O, S, shape, tokens, w_r, cb_of, rec_of, pre, residual, layers_in=None):
    """Time the oracle on the host: one thread on a few tokens, all threads on
    more.  The code records it reads are fetched before each timed loop."""
    def run(xs):
        for x in xs:
            O.layer(x, w_r, shape.top_k, cb_of, rec_of, shape.d, shape.ffn, pre_rmsnorm=pre, eps=1e-6,
                    residual=residual)

    # records of the experts each token routes to, fetched (untimed)
    for x in tokens:
        r = O.route(x, w_r, shape.top_k, pre_rmsnorm=pre, eps=1e-6)
        for e in r.ids:
            rec_of(int(e))
    n_all = O.threads()
    one = tokens[:16]
    O.set_threads(1)
    t0 = time.perf_counter()
    run(one)
    t_one = time.perf_counter() - t0
    O.set_threads(n_all)
    t0 = time.perf_counter()
    run(tokens)
    t_all = time.perf_counter() - t0
    return {"one": len(one) / t_one, "all": len(tokens) / t_all, "n_one": len(one), "n_all": len(tokens),
            "threads": n_all, "s_one": t_one, "s_all": t_all}


class RecordCache:
    """Host copies of expert records for the oracle: from a host copy of the
    device bank when there is one, else regenerated from the seed."""

    def __init__(self, S, seed, layer, rec_bytes, bank_host=None):
        self.S, self.seed, self.layer, self.rb, self.bank = S, seed, layer, rec_bytes, bank_host
        self.cache = {}

    def __call__(self, e):
        if self.bank is not None:
            return self.bank[e]
        if e not in self.cache:
            self.cache[e] = self.S.expert_record(self.seed, self.layer, e, self.rb)
        return self.cache[e]


def sub_records(torch, np, G, S, O, RvqMoe, inp, args, bank_host):
    """Batched decode (32 tokens per call), the resident prefill chunk (512
    tokens per call) and the 16-layer depth chain, each timed briefly on the
    same layer shape with a parity sample against the oracle."""
    shape = S.K3
    stream = torch.cuda.current_stream()
    rec = shape.record_bytes
    out = {}
    rec_of = RecordCache(S, args.seed, 0, rec, bank_host)
    handle = RvqMoe(d=shape.d, ffn=shape.ffn, n_experts=shape.n_experts, top_k=shape.top_k, codebook_dtype=1,
                    router_w=inp.w_r_dev, codebooks=inp.cb_dev, codes=inp.codes_dev, max_tokens=512)
    inp.free_codes()
    torch.cuda.empty_cache()

    def timed(B, calls, warm, t0):
        x_host = S.tokens(args.seed, t0, (warm + calls) * B, shape.d)
        x = G.to_device(x_host)
        ids = torch.empty(((warm + calls) * B, shape.top_k), dtype=torch.int32, device="cuda")
        g = torch.empty(((warm + calls) * B, shape.top_k), device="cuda")
        y = torch.empty(((warm + calls) * B, shape.d), device="cuda")

        def call(c):
            r = slice(c * B, (c + 1) * B)
            handle.route_topk(x[r], B, ids[r], g[r], stream)
            handle.layer_forward(x[r], B, ids[r], g[r], y[r], stream)
        for c in range(warm):
            call(c)
        handle.sync(stream)
        handle.kernel_times()
        handle.set_profiling(1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for c in range(warm, warm + calls):
            call(c)
        e1.record(stream)
        torch.cuda.synchronize()
        handle.set_profiling(0)
        kt = handle.kernel_times()
        handle.sync(stream)
        ms = e0.elapsed_time(e1) / calls
        idh = ids.cpu().numpy()
        uniq = float(np.mean([len(np.unique(idh[c * B:(c + 1) * B])) for c in range(warm, warm + calls)]))
        t_chk = warm * B  # first timed token
        ref = O.layer(x_host[t_chk], inp.w_r, shape.top_k, inp.codebook, rec_of, shape.d, shape.ffn)
        yh = y[t_chk].cpu().numpy().astype(np.float64)
        par = {"token": t_chk, "ids_bit_exact": bool(np.array_equal(idh[t_chk], ref.route.ids)),
               "rel_l2": float(np.linalg.norm(yh - ref.delta) / np.linalg.norm(ref.delta))}
        return ms, uniq, kt, par

    log("sub-record: batched decode, 32 tokens per call")
    ms, uniq, kt, par = timed(32, 20, 3, 100000)
    byts = uniq * (rec + CB_BYTES)
    lay_n, lay_ms = kt["layer_lut"]
    out["batched_decode_32"] = {
        "workload": "32 independent tokens per call through the K3-scale layer, pairs grouped by expert, "
                    "route_topk + layer_forward (table path)",
        "ms_per_call": ms, "tokens_per_s": 32 / (ms * 1e-3), "distinct_experts_per_call": uniq,
        "compressed_bytes_per_call": byts, "compressed_GBps": byts / (ms * 1e-3) / 1e9,
        "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "layer_kernel_ms": lay_ms / lay_n if lay_n else None, "calls": 20,
        "parity": dict(par, bar="ids bit-exact, rel L2 <= 1e-4")}
    log("sub-record: prefill chunk, 512 tokens per call, resident codes")
    ms, uniq, kt, par = timed(512, 12, 2, 200000)
    byts = uniq * (rec + CB_BYTES)
    flops = 6.0 * 512 * shape.top_k * shape.d * shape.ffn
    ck_n, ck_ms = kt["chunk"]
    out["prefill_chunk_512"] = {
        "workload": "512 tokens per call through the K3-scale layer on the chunk path (tokens grouped by expert, "
                    "RVQ tiles rebuilt as bf16 for the matrix cores, experts with fewer than 4 tokens on the "
                    "table path), codes resident",
        "ms_per_call": ms, "tokens_per_s": 512 / (ms * 1e-3), "distinct_experts_per_call": uniq,
        "compressed_bytes_per_call": byts, "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "flops_per_call": flops, "tflops": flops / (ms * 1e-3) / 1e12,
        "bf16_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "chunk_kernels_ms": ck_ms / ck_n if ck_n else None,
        "chunk_kernels_note": "HIP events around layer_forward's launches: grouping, staging, the two "
                              "contraction kernels and the table-path launch for the listed experts",
        "calls": 12,
        "parity": dict(par, bar="ids bit-exact, rel L2 <= 2e-2")}
    handle.close()
    del handle
    torch.cuda.empty_cache()

    L = 16
    log(f"sub-record: depth chain of {L} layers, staging")
    chain, chain_inp = [], []
    for li in range(L):
        ci = G.LayerInputs(shape, seed=args.seed, layer=100 + li)
        chain.append(RvqMoe(d=shape.d, ffn=shape.ffn, n_experts=shape.n_experts, top_k=shape.top_k,
                            codebook_dtype=1, router_w=ci.w_r_dev, codebooks=ci.cb_dev, codes=ci.codes_dev,
                            max_tokens=1, pre_rmsnorm=True, residual=True, eps=1e-6))
        ci.free_codes()
        torch.cuda.empty_cache()
        chain_inp.append(ci)
    n_tok, warm = 20, 2
    h = torch.empty((L + 1, warm + n_tok, shape.d), device="cuda")
    h[0].copy_(G.to_device(S.tokens(args.seed, 300000, warm + n_tok, shape.d)))
    ids = torch.empty((L, warm + n_tok, shape.top_k), dtype=torch.int32, device="cuda")
    g = torch.empty((L, warm + n_tok, shape.top_k), device="cuda")

    def tok(t):
        for li, lay in enumerate(chain):
            lay.route_forward(h[li, t:t + 1], 1, ids[li, t:t + 1], g[li, t:t + 1], h[li + 1, t:t + 1], stream)
    for t in range(warm):
        tok(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in range(warm, warm + n_tok):
        tok(t)
    e1.record(stream)
    torch.cuda.synchronize()
    for lay in chain:
        lay.sync(stream)
    ms = e0.elapsed_time(e1) / n_tok
    hs, idh = h.cpu().numpy(), ids.cpu().numpy()
    errs, ok = [], True
    for li in (0, L - 1):  # teacher-forced: the oracle's layer li on the GPU's input of layer li
        ci = chain_inp[li]
        ref = O.layer(hs[li, warm], ci.w_r, shape.top_k, ci.codebook,
                      RecordCache(S, args.seed, 100 + li, rec), shape.d, shape.ffn, pre_rmsnorm=True, eps=1e-6,
                      residual=True)
        ok &= bool(np.array_equal(idh[li, warm], ref.route.ids))
        delta = hs[li + 1, warm].astype(np.float64) - hs[li, warm].astype(np.float64)
        errs.append(float(np.linalg.norm(delta - ref.delta) / np.linalg.norm(ref.delta)))
    byts = L * shape.top_k * (rec + CB_BYTES)
    out["depth_chain_16"] = {
        "workload": f"one token through {L} resident K3-scale layers (RMSNorm before routing, residual add), "
                    "one rvq_moe_route_forward call per layer",
        "ms_per_token": ms, "tokens_per_s": 1e3 / ms, "layer_tokens_per_s": L * 1e3 / ms,
        "compressed_bytes_per_token": byts, "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "tokens": n_tok,
        "parity": {"token": warm, "layers_checked": [0, L - 1], "ids_bit_exact": ok, "max_rel_l2": max(errs),
                   "bar": "teacher-forced, ids bit-exact, rel L2 <= 1e-4"}}
    for lay in chain:
        lay.close()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000, help="timed steps (one call, or one token through the chain)")
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--repeats", type=int, default=5, help="blocks of --steps timed steps (median and range)")
    ap.add_argument("--latency-calls", type=int, default=200, help="calls timed one by one for p50/p99")
    ap.add_argument("--cpu-tokens", type=int, default=160,
                    help="tokens the oracle baseline runs on all host threads (the first 16 also on one; 0: skip)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the machine-ceiling measurements")
    ap.add_argument("--no-sub", action="store_true",
                    help="skip the sub-records (batched decode, prefill chunk, depth chain) of the default run")
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
    ap.add_argument("--deterministic", action="store_true",
                    help="fixed-order combine (bitwise reproducible outputs) instead of fp32 atomics")
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
    headline = (B == 1 and L == 1 and not args.chunk and not streaming and args.path == "fused"
                and not args.deterministic)
    want_sub = headline and not args.no_sub

    ceil = None
    if not args.no_ceilings:
        log("ceilings: HBM read, LDS gather, launch cost, pinned H2D")
        ceil = measure_ceilings(torch, shape)

    layers, inputs = [], []
    bank_host = None
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
                             lut_expert_tokens=args.lut_expert_tokens, deterministic=int(args.deterministic),
                             **extra))
        del codes
        if L == 1 and args.cpu_tokens > 0:
            bank_host = inp.codes_dev.cpu().numpy()  # the oracle's records (host copy of the bank)
        if not want_sub:
            inp.free_codes()
        inputs.append(inp)
        torch.cuda.empty_cache()

    n_tok = (W + K * max(1, args.repeats) + args.latency_calls) * B
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
                    # a streaming handle's router needs no co-resident grid, so
                    # it may overlap the layer kernel on the main stream
                    side.wait_event(routed)
                    layers[li + 1].route_topk(h[li, r], B, pred[li + 1, r], pred_g[r], side)
                    layers[li + 1].prefetch(pred[li + 1, r], B, args.lookahead, side)

    log(f"warmup {W} steps of {B} token(s) x {L} layer(s)")
    for t in range(W):
        step(t)
    for layer in layers:
        layer.sync(stream)
        layer.kernel_times()  # drop warmup samples
        layer.set_profiling(args.profile_every)

    # ---- the timed region: exactly K steps
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stats0 = [layer.stats() for layer in layers]
    ev0.record(stream)
    for t in range(W, W + K):
        step(t)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
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
    st_end = [layer.stats() for layer in layers]

    # ---- repetitions of the K steps (the timed block above is the first)
    rep_ms = [ms / K]
    t_next = W + K
    for _ in range(max(1, args.repeats) - 1):
        torch.cuda.synchronize()
        ev0.record(stream)
        for t in range(t_next, t_next + K):
            step(t)
        ev1.record(stream)
        torch.cuda.synchronize()
        rep_ms.append(ev0.elapsed_time(ev1) / K)
        t_next += K
    # ---- per-call latency: events around every call
    lat = []
    if args.latency_calls > 0:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.latency_calls)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            step(t_next + i)
            b.record(stream)
        torch.cuda.synchronize()
        lat = [a.elapsed_time(b) * 1e3 for a, b in evs]
    for layer in layers:
        layer.sync(stream)

    h2d = None
    if streaming:
        moved = sum(a["h2d_bytes"] - b["h2d_bytes"] for a, b in zip(st_end, stats0))
        hits = sum(a["slot_hits"] - b["slot_hits"] for a, b in zip(st_end, stats0))
        misses = sum(a["slot_misses"] - b["slot_misses"] for a, b in zip(st_end, stats0))
        checked = sum(a["records_checked"] - b["records_checked"] for a, b in zip(st_end, stats0))
        verified = sum(a["records_verified"] - b["records_verified"] for a, b in zip(st_end, stats0))
        h2d = {"slots": args.stream_slots, "h2d_bytes": moved, "GBps": moved / (ms * 1e-3) / 1e9,
               "hit_rate": hits / max(hits + misses, 1), "records_checked": checked,
               "records_crc_verified": verified}
        if ceil:
            h2d["ceiling_GBps"] = ceil["h2d_pinned_record_GBps"]
            h2d["frac_of_ceiling"] = h2d["GBps"] / ceil["h2d_pinned_record_GBps"]
        if args.lookahead:
            fills = sum(a["prefetch_fills"] - b["prefetch_fills"] for a, b in zip(st_end, stats0))
            phits = sum(a["prefetch_hits"] - b["prefetch_hits"] for a, b in zip(st_end, stats0))
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
    # The dominant kernel's time per launch.  With the one-launch path a step
    # is exactly one launch per layer, so the step time bounds it; event pairs
    # around single launches also count the dispatch before the kernel and
    # read a little longer (reported beside it).
    ev_us = l_ms / n_l * 1e3 if n_l else float("nan")
    step_us = ms / K * 1e3 / L
    if args.path == "fused":
        l_us, src = step_us, "timed steps (one launch per layer and step)"
    else:
        l_us, src = min(ev_us, step_us), "HIP events around the layer kernel on its launch stream"
    l_gbps = per_call_bytes / (l_us * 1e-6) / 1e9
    kernels = {k: {"launches": int(n), "avg_us": (v / n * 1e3 if n else None)} for k, (n, v) in kernels.items()}

    # Parity on timed tokens (teacher-forced through the chain: the oracle runs
    # layer l on the GPU's own input of layer l) and the CPU baseline.
    cpu = None
    parity = None
    if args.cpu_tokens > 0:
        from oracle import oracle as O
        hs = h.cpu().numpy()
        rec_of = [RecordCache(S, args.seed, li, rec, bank_host if L == 1 else None) for li in range(L)]
        errs, ok_ids = [], True
        n_par = min(2, args.cpu_tokens)
        for j in range(n_par):
            t = W * B + j
            for li in range(L):
                inp = inputs[li]
                ref = O.layer(hs[li, t], inp.w_r, shape.top_k, inp.codebook, rec_of[li], shape.d, shape.ffn,
                              pre_rmsnorm=chain, eps=1e-6, residual=chain)
                ok_ids &= bool(np.array_equal(ids_h[li, t], ref.route.ids))
                delta = hs[li + 1, t].astype(np.float64) - (hs[li, t].astype(np.float64) if chain else 0.0)
                errs.append(float(np.linalg.norm(delta - ref.delta) / np.linalg.norm(ref.delta)))
        parity = {"tokens": n_par, "layers_checked": L, "ids_bit_exact": ok_ids, "max_rel_l2": max(errs),
                  "bar": "ids bit-exact, rel L2 <= 1e-4" if not args.chunk else "ids bit-exact, rel L2 <= 2e-2"}
        # the oracle's own time on the first layer of this workload
        toks = [hs[0, W * B + j] for j in range(min(args.cpu_tokens, hs.shape[1] - W * B))]
        base = oracle_baseline(O, S, shape, toks, inputs[0].w_r, inputs[0].codebook, rec_of[0], chain, chain)
        cpu = {"value": base["all"], "unit": "tokens/s", "cores": base["threads"], "kind": "oracle",
               "sample": f"{base['n_all']} tokens of the same workload through one layer (router, top-16 and 16 "
                         f"experts with every weight rebuilt as c1+c2+c3, fp64) on {base['threads']} OpenMP "
                         f"threads, {base['s_all']:.1f} s; the first {base['n_one']} also on one thread "
                         f"({base['s_one']:.1f} s); code records fetched before each timed loop",
               "single_thread_tokens_per_s": base["one"],
               "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}

    subs = None
    if want_sub:
        for layer in layers:
            layer.close()
        layers = []
        torch.cuda.empty_cache()
        from oracle import oracle as O
        subs = sub_records(torch, np, G, S, O, RvqMoe, inputs[0], args, bank_host)

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
    traffic = (recorded_traffic(args.path == "fused")
               if (B == 1 and L == 1 and not args.chunk and not streaming and not args.deterministic) else None)
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
                   else "rvq_moe_route_topk + rvq_moe_layer_forward",
                   "combine": "fixed order" if args.deterministic else "fp32 atomics"},
        "layer_calls_per_s": calls_s,
        "compressed_GBps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        "compressed_bytes_per_call": per_call_bytes,
        "distinct_experts_per_call": float(uniq.mean()),
        "repeats": {"n": len(rep_ms), "steps_each": K, "ms_per_step_median": statistics.median(rep_ms),
                    "ms_per_step_min": min(rep_ms), "ms_per_step_max": max(rep_ms),
                    "tokens_per_s_median": B / (statistics.median(rep_ms) * 1e-3)},
        "latency_us": ({"calls": len(lat), "p50": percentile(lat, 50), "p99": percentile(lat, 99),
                        "min": min(lat), "max": max(lat),
                        "note": "HIP events recorded on the stream around each call (includes the dispatch "
                                "before the kernel)"} if lat else None),
        "roofline": {"bound": "hbm", "achieved": l_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": l_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     "traffic_source": ("recorded: FETCH_SIZE + WRITE_SIZE counter runs of this source version "
                                        "(profiles/), scaled by a reference copy" if traffic else None),
                     "kernel": "k_layer<routed> (routing and experts in one launch)" if args.path == "fused" else
                     ("k_chunk_prep + k_chunk_stage + k_chunk_gu + k_chunk_down" if args.chunk else "k_layer"),
                     "algorithmic_bytes_per_launch": per_call_bytes, "avg_us": l_us, "time_source": src,
                     "event_avg_us": ev_us, "timed_launches": int(n_l)},
        "ceilings": ceil,
        "kernels": kernels,
        "h2d": h2d,
        "mfma": ({"flops_per_call": 6.0 * B * shape.top_k * shape.d * shape.ffn,
                  "tflops": 6.0 * B * shape.top_k * shape.d * shape.ffn / (l_us * 1e-6) / 1e12,
                  "frac_of_bf16_dense_peak": 6.0 * B * shape.top_k * shape.d * shape.ffn / (l_us * 1e-6) / 2.5e15}
                 if args.chunk else None),
        "sub_records": subs,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    if ceil:
        out["roofline"]["frac_of_measured_read_ceiling"] = l_gbps / ceil["hbm_read_GBps"]
    for layer in layers:
        layer.close()
    if args.copy_bytes > 0:
        torch.cuda.empty_cache()
        src_t = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src_t)
        torch.cuda.synchronize()
        dst.copy_(src_t)
        torch.cuda.synchronize()
        out["copy_reference_bytes"] = args.copy_bytes
        del src_t, dst
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
