"""Benchmark of the routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

Headline (one JSON line on stdout): MoE decode tokens/s for batch 1 through
48 stacked layers shaped like the pages' model (512 experts per layer, top-10
plus one shared expert, d_model 2048, d_ff 768, every expert resident,
2-bit scale+min blocks at 3.0 bits per weight).  A step is one token through
all 48 layers in one moe_decode_stack call: per layer router top-k, cache
lookup, the decode FFN and its routing-weighted combine, whose output plus a
per-layer addend is the next layer's input (x_{l+1} = y_l + a_{l+1}; the
addends stand in for the rest of the model between two MoE layers and are
chosen so that each layer's input stays near its own seeded draw).  Router
logits are fresh for every token and layer.  Inputs are seeded synthetic
tensors, resident in HBM before timing starts.  Steps are replayed from HIP
graphs.

Extra objects on the same line: the decode kernel's roofline (HBM), the
expert-cache workload (94 of 512 experts resident, about 72% hits; whole
layers with the misses read from a pinned host copy, with the host link as
their roofline), the 1+3-token verify step, the router projection, the
8,192-token prefill chunk with its GEMMs' MFMA roofline, and the CPU oracle
timed on a bounded sample of the decode workload on this host.

For profiling, --cache-only, --tiers-only, --prefill-only and --router-only
run one part alone and print its object, and --decode-only prints the
headline line with only the verify object beside it; --counters and
--counters-verify run the short passes the HBM counter summaries are taken
from.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
N_LAYERS = 48
COPY_BYTES = 512 << 20         # calibration copy of the counter pass
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_layer_e512_k10_d2048_f768_q2sm_traffic.txt")
DECODE_SOURCES = ["bit_expert_ffn_top_amd/csrc/ffn_decode.hip",
                  "bit_expert_ffn_top_amd/csrc/decode_stack.hip",
                  "bit_expert_ffn_top_amd/csrc/moe_common.h",
                  "bit_expert_ffn_top_amd/csrc/route_device.h"]
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles",
                                    "prefill_e512_k10_d2048_f768_q2sm_t8192_traffic.txt")
PREFILL_SOURCES = ["bit_expert_ffn_top_amd/csrc/ffn_prefill.hip",
                   "bit_expert_ffn_top_amd/csrc/cache_lookup.hip",
                   "bit_expert_ffn_top_amd/csrc/moe_common.h",
                   "bit_expert_ffn_top_amd/csrc/route_device.h"]
VERIFY_TRAFFIC_FILE = os.path.join(ROOT, "profiles",
                                   "verify_t4_e512_k10_d2048_f768_q2sm_q3g_kernel_stats_and_traffic.txt")
PREFILL_MFMA_FILE = os.path.join(ROOT, "profiles",
                                 "prefill_e512_k10_d2048_f768_q2sm_t8192_mfma_counters.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--graphs", type=int, default=16, help="distinct token graphs replayed in turn")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=2)
    ap.add_argument("--decode-only", action="store_true",
                    help="the decode headline and the verify step only (no other workloads, "
                         "no CPU baseline)")
    ap.add_argument("--cache-only", action="store_true",
                    help="run only the expert-cache workloads (host tier, staged prefill, "
                         "adaptive cache; for profiling); prints their object")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the prefill workload (for profiling); prints its object")
    ap.add_argument("--tiers-only", action="store_true",
                    help="run only whole expert-cache layers with every miss read from the "
                         "host tier in the same launch (for profiling); prints its object")
    ap.add_argument("--router-only", action="store_true",
                    help="run only the router projection (for profiling); prints its object")
    ap.add_argument("--counters", action="store_true",
                    help="counter pass for rocprofv3 --pmc: two eager decode steps plus one "
                         "device copy of COPY_BYTES for calibration; prints no result line "
                         "(with --prefill-only: the prefill workload, then the copy)")
    ap.add_argument("--counters-verify", action="store_true",
                    help="counter pass of the verify step (T = 4): two eager steps, then the "
                         "calibration copy; prints no result line")
    return ap.parse_args()


def build_pools(torch, synth, cfg, fmt_of_layer, dev, n_layers=N_LAYERS, resident=None):
    """Packed pools of n_layers layers on the device; returns list of
    (pool, slot_of_expert (device int32), shared_slot)."""
    shape = synth.config_shape(cfg)
    E = shape.n_experts
    out = []
    for l in range(n_layers):
        fmt = fmt_of_layer(l)
        table, shared_slot, slot_expert = synth.make_slot_table(cfg, l)
        pool = synth.make_layer_pool(cfg, l, slot_expert, device=dev, fmt=fmt, batch=64)
        out.append((pool, torch.tensor(table, dtype=torch.int32, device=dev), shared_slot, fmt))
    return out


class StackStep:
    """Steps of T tokens through a stack of layers, one moe_decode_stack call
    each, with preallocated buffers so that a step can be captured in a
    graph.  Step g uses logit set g and addend set g; only the last layer's y
    is written (with routing=True every layer's routing outputs and miss
    lists are written too)."""

    def __init__(self, torch, bf, shape, pools, T, dev, x0, logit_sets, routing=False):
        self.torch, self.bf = torch, bf
        self.T = T
        self.layers = [bf.MoeLayer(shape.d_model, shape.d_ff, shape.n_experts, shape.top_k, fmt,
                                   pool, shared_slot) for pool, _, shared_slot, fmt in pools]
        self.tables = [t for _, t, _, _ in pools]
        self.x0 = x0
        self.logit_sets = logit_sets
        self.add_sets = None
        self.routing = routing
        self.ws = bf.new_stack_workspace(self.layers, T)
        self.y = torch.empty((T, shape.d_model), dtype=torch.float32, device=dev)

    def set_addends(self, xs):
        """Addends that keep layer l's input near xs[l] for every logit set:
        a_l = xs[l] - y_{l-1}, y_{l-1} the output of layer l-1 run alone on
        xs[l-1] (one-layer moe_decode_stack calls)."""
        torch, bf = self.torch, self.bf
        self.add_sets = []
        for lg in self.logit_sets:
            adds = [torch.zeros_like(self.x0)]
            for l in range(1, len(self.layers)):
                y = bf.decode_stack([self.layers[l - 1]], xs[l - 1], [lg[l - 1]],
                                    [self.tables[l - 1]], ys=torch.empty_like(self.x0),
                                    ws=self.ws)["y"]
                adds.append((xs[l] - y).contiguous())
            self.add_sets.append(torch.stack(adds))
        torch.cuda.synchronize()

    def step(self, g):
        out = self.bf.decode_stack(self.layers, self.x0, self.logit_sets[g], self.tables,
                                   addends=self.add_sets[g], ys=self.y, ws=self.ws,
                                   routing=self.routing)
        if self.routing:
            self.routing_out = out
        return self.y


class DecodeChain:
    """48 layers of decode for T tokens, one moe_decode_layer call per layer
    (plus moe_decode_misses from a host tier and cache counting when given;
    with one_launch, one moe_decode_layer_tiers call instead of the two),
    with preallocated buffers, so that a whole step can be captured in a
    graph.  Each layer reads its own seeded input x_l and writes its y to a
    scratch buffer."""

    def __init__(self, torch, bf, shape, pools, T, dev, xs, logit_sets, tiers=None,
                 host_table=None, max_rank=None, counts=None, overlap=False, misses_only=False,
                 one_launch=False):
        self.torch, self.bf = torch, bf
        self.one_launch = one_launch   # hits and misses in one moe_decode_layer_tiers call
        self.T = T
        self.tiers, self.host_table, self.max_rank = tiers, host_table, max_rank
        self.overlap = overlap
        self.misses_only = misses_only   # overlapped step without the GPU part (timing)
        self.counts = counts
        self.logit_sets = logit_sets
        self.layers = [bf.MoeLayer(shape.d_model, shape.d_ff, shape.n_experts, shape.top_k, fmt,
                                   pool, shared_slot) for pool, _, shared_slot, fmt in pools]
        self.tables = [t for _, t, _, _ in pools]
        k, E, d = shape.top_k, shape.n_experts, shape.d_model
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.slot = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.miss_e = torch.empty((T * k,), dtype=torch.int32, device=dev)
        self.miss_p = torch.empty((T * k,), dtype=torch.int32, device=dev)
        self.n_miss = torch.empty((4,), dtype=torch.int32, device=dev)
        ws = max(bf.decode_workspace_bytes(L, T) for L in self.layers)
        self.ws = torch.empty((ws,), dtype=torch.uint8, device=dev)
        if overlap:   # the host-tier read runs on its own stream, with its own workspace
            self.ws_miss = torch.empty((ws,), dtype=torch.uint8, device=dev)
            self.side = torch.cuda.Stream()
        self.xs = xs
        self.y = torch.empty((T, d), dtype=torch.float32, device=dev)

    def step(self, g):
        """One moe_decode_layer call per layer (route, look up, expert FFN,
        combine) on logit set g; with host tiers, then one moe_decode_misses
        call that adds the missed experts."""
        bf = self.bf
        logits = self.logit_sets[g]
        if self.overlap:
            return self._step_overlapped(logits)
        for l, L in enumerate(self.layers):
            if self.one_launch:
                bf.decode_layer_tiers(L, self.tiers[l], self.xs[l], logits[l], self.tables[l],
                                      self.host_table, max_rank=self.max_rank, idx=self.idx,
                                      w=self.w, slot=self.slot, miss_expert=self.miss_e,
                                      miss_pair=self.miss_p, n_miss=self.n_miss, y=self.y,
                                      ws=self.ws)
            else:
                bf.decode_layer(L, self.xs[l], logits[l], self.tables[l], idx=self.idx, w=self.w,
                                slot=self.slot, miss_expert=self.miss_e, miss_pair=self.miss_p,
                                n_miss=self.n_miss, y=self.y, ws=self.ws)
            if self.tiers is not None and not self.one_launch:
                bf.decode_misses(self.tiers[l], self.xs[l], self.idx, self.slot, self.w,
                                 self.host_table, self.y, max_rank=self.max_rank, ws=self.ws)
            if self.counts is not None:
                bf.cache_count(self.idx, self.counts[l])
        return self.y

    def _step_overlapped(self, logits):
        """Per layer: routing and lookup; then the missed experts' host-tier
        read (moe_decode_misses_phases, READ) on the side stream while the GPU
        part (moe_expert_ffn_decode) runs; then the join (JOIN) once both
        are done, before the next layer."""
        torch, bf = self.torch, self.bf
        main = torch.cuda.current_stream()
        k = self.layers[0].top_k
        for l, L in enumerate(self.layers):
            bf.route_topk(logits[l], k, idx=self.idx, w=self.w)
            bf.cache_lookup(self.idx, self.tables[l], slot=self.slot, miss_expert=self.miss_e,
                            miss_pair=self.miss_p, n_miss=self.n_miss)
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                bf.decode_misses(self.tiers[l], self.xs[l], self.idx, self.slot, None,
                                 self.host_table, None, max_rank=self.max_rank, ws=self.ws_miss,
                                 phases=bf.MISSES_READ)
            if not self.misses_only:
                bf.expert_ffn_decode(L, self.xs[l], self.idx, self.slot, self.w, y=self.y,
                                     ws=self.ws)
            main.wait_stream(self.side)
            bf.decode_misses(self.tiers[l], None, self.idx, self.slot, self.w, self.host_table,
                             self.y, max_rank=self.max_rank, ws=self.ws_miss,
                             phases=bf.MISSES_JOIN)
        return self.y


def time_graph_steps(torch, chain, steps, warmup, n_graphs):
    """Capture n_graphs token steps (chain.step(g), each its own inputs) and
    replay them in turn.
    Returns (wall seconds, event milliseconds) over the timed replays; the
    events are recorded on the stream the graphs run on."""
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for g in range(min(3, n_graphs)):       # warm the allocator and the code paths
            chain.step(g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for g in range(n_graphs):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            chain.step(g)
        graphs.append(graph)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % n_graphs].replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        graphs[i % n_graphs].replay()
    ev1.record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    return dt, ev0.elapsed_time(ev1), graphs


def sources_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def summary_keys(path, sources):
    """The key: value lines of a committed counter summary, or None when the
    file is missing or the kernels' sources changed since it was taken."""
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    key, val = line.split(":", 1)
                    kv[key.strip()] = val.strip()
        if kv.get("sources_sha256_16") != sources_digest(sources):
            return None
        return kv
    except OSError:
        return None


def measured_traffic(path=TRAFFIC_FILE, sources=DECODE_SOURCES):
    """HBM bytes per unit from a committed counter summary (FETCH_SIZE +
    WRITE_SIZE per dispatch, scaled by what the counters read for a plain
    copy of known size); None when the file is missing or the kernels'
    sources changed since it was taken.  Defaults: one layer of the decode
    step (its route+FFN kernel and its combine kernel)."""
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    key, val = line.split(":", 1)
                    kv[key.strip()] = val.strip()
        if kv.get("sources_sha256_16") != sources_digest(sources):
            return None
        return int(float(kv["bytes_per_call"]))
    except (OSError, KeyError, ValueError):
        return None


def counter_pass(torch, bf, synth, chain, dev):
    """Two eager decode steps, then one device copy of COPY_BYTES (the
    counters' calibration); run under rocprofv3 --pmc."""
    for g in range(2):
        chain.step(g)
    torch.cuda.synchronize()
    calibration_copy(torch, dev)
    log(f"counter pass: {2 * len(chain.layers)} decode layers, copy of {COPY_BYTES} bytes")


def calibration_copy(torch, dev):
    """One device-to-device copy of COPY_BYTES: the known traffic that HBM
    counters are scaled by."""
    src = torch.empty((COPY_BYTES // 4,), dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def stack_layer_bytes(synth, shape, fmt, T, n_union):
    """Algorithmic HBM bytes of one layer of a decode step: the packed bytes
    of every distinct resident expert chosen (plus the shared one) read once;
    the layer's input x, the addend, the router logits and the slot table
    read; the next input written."""
    sb = synth.slot_bytes(fmt, shape.d_model, shape.d_ff)
    return (n_union * sb + 3 * T * shape.d_model * 4 + T * shape.n_experts * 4
            + shape.n_experts * 4)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import bit_expert_ffn_top_amd as bf
    import synth

    bf.lib()
    dev = torch.device("cuda:0")
    shape = synth.config_shape(1)
    E, k, d, f = shape.n_experts, shape.top_k, shape.d_model, shape.d_ff
    if args.cache_only:
        print(json.dumps(run_extras(torch, np, bf, synth, None, dev, args, cache_only=True)),
              flush=True)
        return

    if args.router_only:
        print(json.dumps({"router": run_router(torch, bf, synth, dev)}), flush=True)
        return

    if args.tiers_only:
        print(json.dumps({"host_tier_one_launch": run_tiers_only(torch, bf, synth, dev, args)}),
              flush=True)
        return

    t_gen = time.perf_counter()
    pools = build_pools(torch, synth, 1, lambda l: synth.FMT_Q2SM, dev)
    torch.cuda.synchronize()
    log(f"decode pools: {N_LAYERS} layers x {E + 1} experts in {time.perf_counter() - t_gen:.1f} s")

    if args.prefill_only:
        print(json.dumps({"prefill": run_prefill(torch, np, bf, synth, pools, dev, args)}), flush=True)
        if args.counters:
            calibration_copy(torch, dev)
        return

    if args.counters_verify:
        chain3, _, _ = verify_chain(torch, bf, synth, shape, pools, dev, 2)
        counter_pass(torch, bf, synth, chain3, dev)
        return

    # ---------------- decode (headline) ----------------
    n_graphs = args.graphs
    xs = [synth.make_x(1, l, 1, d, device=dev) for l in range(N_LAYERS)]
    logit_sets = [torch.stack([synth.make_logits(1, l, 1, E, 1.5, device=dev, step=g)
                               for l in range(N_LAYERS)]) for g in range(n_graphs)]
    chain = StackStep(torch, bf, shape, pools, 1, dev, xs[0], logit_sets)
    chain.set_addends(xs)
    if args.counters:
        counter_pass(torch, bf, synth, chain, dev)
        return
    dt, ev_ms, graphs = time_graph_steps(torch, chain, args.steps, args.warmup, n_graphs)
    if not bool(torch.isfinite(chain.y).all()):
        raise RuntimeError("decode step: non-finite output")
    tok_s = args.steps / dt
    ms_step = dt * 1e3 / args.steps
    log(f"decode: {tok_s:.1f} tok/s, {ms_step * 1e3:.1f} us/token ({ms_step * 1e3 / N_LAYERS:.2f} us/layer)")
    del graphs
    layer_us = ev_ms * 1e3 / (args.steps * N_LAYERS)
    bytes_layer = stack_layer_bytes(synth, shape, synth.FMT_Q2SM, 1, k + 1)
    ach = bytes_layer / (layer_us * 1e-6) / 1e9
    log(f"decode layer: {layer_us:.2f} us avg (events), {ach:.0f} GB/s algorithmic")
    token_bytes = N_LAYERS * bytes_layer
    result = {
        "metric": "MoE decode tok/s (48 layers, bs=1)",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (2-bit scale+min weight blocks)",
        "data": "synthetic (seeded; weights ~N(0,0.02) block-quantized, x ~N(0,1), logits ~N(0,1.5) fresh per token and layer)",
        "config": {
            "workload": "decode, batch 1, 48 stacked MoE layers chained through their outputs: "
                        "E=512 routed (top-10) + 1 shared expert, d_model=2048, d_ff=768, all "
                        "experts resident under a seeded slot permutation, Q2SM blocks "
                        "(3.0 bits/weight)",
            "tokens_per_step": 1, "layers": N_LAYERS, "experts_per_layer": E, "top_k": k,
            "shared_experts": 1, "d_model": d, "d_ff": f, "format": "Q2SM",
        },
        "token_hbm_bytes_algorithmic": token_bytes,
        "token_hbm_GBps_algorithmic": round(token_bytes * tok_s / 1e9, 1),
        "token_frac_of_hbm_peak": round(token_bytes * tok_s / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {
            "kernel": "one layer of moe_decode_stack: decode_ffn_kernel (routing + gate/up + "
                      "SiLU + down partials) then decode_combine_kernel (fixed-order sum, "
                      "y + addend into the next layer's input); the unit is the layer, timed "
                      "over the graph replays",
            "bound": "hbm",
            "achieved": round(ach, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "avg_layer_us": round(layer_us, 3),
            "bytes_per_layer": bytes_layer,
        },
    }

    extra = {}
    if not args.no_extra:
        extra.update(run_extras(torch, np, bf, synth, pools, dev, args))
    result.update(extra)

    if not args.no_cpu and not args.decode_only:
        result["cpu_baseline"] = cpu_baseline(np, synth, pools, shape)
    print(json.dumps(result), flush=True)


def run_extras(torch, np, bf, synth, pools, dev, args, cache_only=False):
    out = {}
    shape = synth.config_shape(1)
    E, k, d, f = shape.n_experts, shape.top_k, shape.d_model, shape.d_ff
    n_graphs = min(args.graphs, 8)
    if getattr(args, "decode_only", False):
        return run_verify(torch, np, bf, synth, shape, pools, dev, args, n_graphs, out)

    # ---------------- expert-cache workload ----------------
    t0 = time.perf_counter()
    c2 = synth.WORKLOADS[2]
    pools2 = build_pools(torch, synth, 2, lambda l: synth.FMT_Q2SM, dev)
    n_graphs = min(args.graphs, 8)
    logits2 = [torch.stack([synth.zipf_gumbel_logits(2, l, 1, E, c2["zipf_s"], device=dev, step=g)
                            for l in range(N_LAYERS)]) for g in range(n_graphs)]
    xs2 = [synth.make_x(2, l, 1, d, device=dev) for l in range(N_LAYERS)]
    chain2 = StackStep(torch, bf, shape, pools2, 1, dev, xs2[0], logits2, routing=True)
    chain2.set_addends(xs2)
    steps2 = max(20, args.steps // 2)
    dt, _, graphs = time_graph_steps(torch, chain2, steps2, 5, n_graphs)
    del graphs
    hits = tot = 0
    for g in range(n_graphs):
        for l in range(N_LAYERS):
            idx = np.argsort(-logits2[g][l].cpu().numpy(), axis=1, kind="stable")[:, :k]
            tab = pools2[l][1].cpu().numpy()
            hits += int((tab[idx] >= 0).sum())
            tot += idx.size
    out["expert_cache"] = {
        "workload": "decode batch 1, 48 stacked layers, 94 of 512 experts + shared resident per layer, "
                    "Zipf(1.1) routing; GPU computes the resident part and writes every layer's "
                    "routing outputs and miss list (one moe_decode_stack call per token)",
        "tok_s": round(steps2 / dt, 2), "ms_per_step": round(dt * 1e3 / steps2, 5),
        "hit_rate": round(hits / tot, 4),
    }
    log(f"expert cache: {steps2 / dt:.1f} tok/s, hit rate {hits / tot:.3f} ({time.perf_counter() - t0:.1f} s)")
    del chain2
    tiers, host_table = build_host_tiers(torch, bf, synth, shape, dev)
    out["expert_cache"].update(run_host_tier(torch, np, bf, synth, shape, pools2, logits2, dev,
                                             steps2, n_graphs, tot - hits, tiers, host_table,
                                             xs2))
    out["prefill_streamed"] = run_prefill_streamed(torch, np, bf, synth, pools2, tiers, dev)
    torch.cuda.empty_cache()
    out["expert_cache"]["adaptive"] = run_adaptive_cache(torch, np, bf, synth, shape, pools2,
                                                         tiers, host_table, xs2, dev)
    del pools2, logits2, tiers
    torch.cuda.empty_cache()
    if cache_only:
        return out
    run_verify(torch, np, bf, synth, shape, pools, dev, args, n_graphs, out)

    # ---------------- router projection ----------------
    out["router"] = run_router(torch, bf, synth, dev)

    # ---------------- prefill chunk ----------------
    out["prefill"] = run_prefill(torch, np, bf, synth, pools, dev, args)
    return out


def run_verify(torch, np, bf, synth, shape, pools, dev, args, n_graphs, out):
    """The verify step (workload 3) timed into out["verify"]."""
    k, d, f = shape.top_k, shape.d_model, shape.d_ff
    t0 = time.perf_counter()
    chain3, pools3, logits3 = verify_chain(torch, bf, synth, shape, pools, dev, n_graphs)
    steps3 = max(20, args.steps // 2)
    dt, ev_ms3, graphs = time_graph_steps(torch, chain3, steps3, 5, n_graphs)
    del graphs
    union = []
    for g in range(n_graphs):
        for l in range(N_LAYERS):
            idx = np.argsort(-logits3[g][l].cpu().numpy(), axis=1, kind="stable")[:, :k]
            union.append(len(set(idx.reshape(-1).tolist())) + 1)
    sb2 = synth.slot_bytes(synth.FMT_Q2SM, d, f)
    sb3 = synth.slot_bytes(synth.FMT_Q3G, d, f)
    mean_u = float(np.mean(union))
    step_bytes = sum(mean_u * (sb2 if l % 2 == 0 else sb3) for l in range(N_LAYERS))
    sps = steps3 / dt
    out["verify"] = {
        "workload": "verify step: 1 real + 3 draft tokens routed independently through 48 layers "
                    "alternating Q2SM / Q3G, chained through their outputs; each distinct chosen "
                    "expert read once per layer (one moe_decode_stack call per step)",
        "steps_per_s": round(sps, 2), "token_positions_per_s": round(4 * sps, 2),
        "ms_per_step": round(dt * 1e3 / steps3, 5), "mean_union_experts": round(mean_u, 2),
        "hbm_GBps_algorithmic": round(step_bytes * sps / 1e9, 1),
        "frac_of_hbm_peak": round(step_bytes * sps / 1e9 / HBM_PEAK_GBS, 4),
        "avg_layer_us": round(ev_ms3 * 1e3 / (steps3 * N_LAYERS), 3),
        "bytes_per_layer_algorithmic": round(step_bytes / N_LAYERS),
        "traffic": measured_traffic(VERIFY_TRAFFIC_FILE, DECODE_SOURCES),
    }
    log(f"verify: {sps:.1f} steps/s, union {mean_u:.2f} ({time.perf_counter() - t0:.1f} s)")
    del pools3, chain3, logits3
    torch.cuda.empty_cache()
    return out


class RouterChain:
    """48 router projections (one per layer) of one token step; step g takes
    the weights of matrices 48g .. 48g+47 (mod the count), so that a replay
    reads weights no recent replay has left in the caches."""

    def __init__(self, torch, bf, ws, x, out):
        self.bf, self.ws, self.x, self.out = bf, ws, x, out

    def step(self, g):
        n = len(self.ws)
        for l in range(N_LAYERS):
            self.bf.router_logits(self.x, self.ws[(N_LAYERS * g + l) % n], logits=self.out[l])


def run_router(torch, bf, synth, dev):
    """The router projection at the model's size (E = 512, d_model = 2048, bf16
    weights: 2 MiB per layer), T = 1 and the verify step's T = 4, timed as 48
    launches per graph.  160 distinct weight matrices (320 MiB, more than the
    last-level cache) are cycled through."""
    shape = synth.config_shape(1)
    E, d = shape.n_experts, shape.d_model
    n_w = 160
    ws = [synth.make_router_weights(1, l, E, d, device=dev) for l in range(n_w)]
    res = {"workload": "router projection: logits [T, 512] = x [T, 2048] (fp32) times bf16 weights "
                       "[512, 2048] (2 MiB), 48 layers per step, weights cycled over 320 MiB",
           "bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    for T in (1, 4):
        x = synth.make_x(1, 0, T, d, device=dev)
        out = torch.empty((N_LAYERS, T, E), dtype=torch.float32, device=dev)
        chain = RouterChain(torch, bf, ws, x, out)
        steps = 60
        _, ev_ms, graphs = time_graph_steps(torch, chain, steps, 5, 6)
        del graphs
        us = ev_ms * 1e3 / (steps * N_LAYERS)
        nbytes = E * d * 2 + T * d * 4 + T * E * 4
        res[f"T{T}"] = {"us_per_call": round(us, 3), "achieved": round(nbytes / us / 1e3, 1),
                        "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4), "bytes_per_call": nbytes}
        log(f"router T={T}: {us:.2f} us per call, {nbytes / us / 1e3:.0f} GB/s")
    del ws
    torch.cuda.empty_cache()
    return res


def verify_chain(torch, bf, synth, shape, pools, dev, n_graphs):
    """The verify workload: 1 + 3 tokens through 48 layers alternating Q2SM
    (the decode workload's pools) and Q3G; a StackStep over n_graphs logit
    sets, its addends set."""
    E, d = shape.n_experts, shape.d_model
    pools3 = []
    for l in range(N_LAYERS):
        if l % 2 == 0:
            pools3.append(pools[l])       # Q2SM layers shared with the decode workload
        else:
            table, shared_slot, slot_expert = synth.make_slot_table(3, l)
            pool = synth.make_layer_pool(3, l, slot_expert, device=dev, fmt=synth.FMT_Q3G, batch=64)
            pools3.append((pool, torch.tensor(table, dtype=torch.int32, device=dev), shared_slot,
                           synth.FMT_Q3G))
    logits3 = [torch.stack([synth.make_logits(3, l, 4, E, 1.5, device=dev, step=g)
                            for l in range(N_LAYERS)]) for g in range(n_graphs)]
    xs3 = [synth.make_x(3, l, 4, d, device=dev) for l in range(N_LAYERS)]
    chain3 = StackStep(torch, bf, shape, pools3, 4, dev, xs3[0], logits3)
    chain3.set_addends(xs3)
    return chain3, pools3, logits3


def build_host_tiers(torch, bf, synth, shape, dev):
    """A pinned host copy of all 512 experts of each expert-cache layer, host
    slot = expert id."""
    E, k, d, f = shape.n_experts, shape.top_k, shape.d_model, shape.d_ff
    t0 = time.perf_counter()
    sb = synth.slot_bytes(synth.FMT_Q2SM, d, f)
    tiers = []
    for l in range(N_LAYERS):
        hp = torch.empty((E, sb), dtype=torch.uint8, pin_memory=True)
        for e0 in range(0, E, 128):
            ids = list(range(e0, min(E, e0 + 128)))
            hp[e0:e0 + len(ids)].copy_(synth.make_layer_pool(2, l, ids, device=dev,
                                                             fmt=synth.FMT_Q2SM, batch=64))
        tiers.append(bf.HostTier(d, f, E, k, synth.FMT_Q2SM, hp))
    host_table = torch.arange(E, dtype=torch.int32, device=dev)   # host slot = expert id
    torch.cuda.synchronize()
    log(f"host tiers: {N_LAYERS} x {E} experts pinned ({N_LAYERS * E * sb / 1e9:.1f} GB) "
        f"in {time.perf_counter() - t0:.1f} s")
    return tiers, host_table


def run_tiers_only(torch, bf, synth, dev, args):
    """The expert-cache workload's whole layers with every miss read from
    the host tier by moe_decode_layer_tiers, and nothing else (so that a
    profile of this command shows that layer's kernels alone)."""
    shape = synth.config_shape(2)
    E, d = shape.n_experts, shape.d_model
    c2 = synth.WORKLOADS[2]
    pools2 = build_pools(torch, synth, 2, lambda l: synth.FMT_Q2SM, dev)
    n_graphs = min(args.graphs, 8)
    logits2 = [torch.stack([synth.zipf_gumbel_logits(2, l, 1, E, c2["zipf_s"], device=dev, step=g)
                            for l in range(N_LAYERS)]) for g in range(n_graphs)]
    xs2 = [synth.make_x(2, l, 1, d, device=dev) for l in range(N_LAYERS)]
    tiers, host_table = build_host_tiers(torch, bf, synth, shape, dev)
    chain = DecodeChain(torch, bf, shape, pools2, 1, dev, xs2, logits2, tiers=tiers,
                        host_table=host_table, one_launch=True)
    steps = max(20, args.steps // 2)
    dt, _, graphs = time_graph_steps(torch, chain, steps, 5, n_graphs)
    del graphs
    res = {"tok_s": round(steps / dt, 2), "ms_per_step": round(dt * 1e3 / steps, 5),
           "avg_layer_us": round(dt * 1e6 / (steps * N_LAYERS), 3), "steps": steps}
    log(f"one-launch host-tier layers: {res}")
    return res


HOST_LINK_GBPS = 63.0   # PCIe 5.0 x16: 64 GB/s per direction less 128b/130b coding


def run_host_tier(torch, np, bf, synth, shape, pools2, logits2, dev, steps, n_graphs, n_missed,
                  tiers, host_table, xs):
    """The expert-cache workload as whole layers: after each layer's GPU
    part, moe_decode_misses reads the missed experts from a pinned host copy
    of that layer (all 512 experts) and joins them into y.  Timed with every
    miss run and with misses of rank >= 5 left out; the change that leaving
    them out makes to the layers' updates is reported too."""
    E, k, d, f = shape.n_experts, shape.top_k, shape.d_model, shape.d_ff
    t0 = time.perf_counter()
    sb = synth.slot_bytes(synth.FMT_Q2SM, d, f)
    res = {}
    misses_per_token = n_missed / n_graphs
    for name, r, ov, mo, one in (("full_layer", None, False, False, False),
                                 ("rank_limit_5", 5, False, False, False),
                                 ("full_layer_two_streams", None, True, False, False),
                                 ("host_part_only", None, True, True, False),
                                 ("full_layer_one_launch", None, False, False, True),
                                 ("rank_limit_5_one_launch", 5, False, False, True)):
        chain = DecodeChain(torch, bf, shape, pools2, 1, dev, xs, logits2, tiers=tiers,
                            host_table=host_table, max_rank=r, overlap=ov, misses_only=mo,
                            one_launch=one)
        dt, _, graphs = time_graph_steps(torch, chain, steps, 5, n_graphs)
        del graphs
        res[name + "_tok_s"] = round(steps / dt, 2)
        res[name + "_ms_per_step"] = round(dt * 1e3 / steps, 5)
        log(f"expert cache, {name}: {steps / dt:.1f} tok/s")
    # at batch 1 every missed pair is a distinct expert read from the host tier
    res["missed_experts_per_token"] = round(misses_per_token, 2)
    res["host_read_MB_per_token"] = round(misses_per_token * sb / 1e6, 1)
    # misses of k-slot < 5 (the ones the rank limit keeps), same routings
    kept = 0
    for g in range(n_graphs):
        for l in range(N_LAYERS):
            idx = np.argsort(-logits2[g][l].cpu().numpy(), axis=1, kind="stable")[:, :k]
            kept += int((pools2[l][1].cpu().numpy()[idx[:, :5]] < 0).sum())
    kept_per_token = kept / n_graphs
    res["rank_limit_5_host_read_MB_per_token"] = round(kept_per_token * sb / 1e6, 1)
    # the host link as the roofline of the one-launch layers: host bytes per token
    # over the token time, against PCIe 5.0 x16's 63 GB/s of payload per direction
    link = {}
    for name, per_tok in (("full_layer_one_launch", misses_per_token),
                          ("rank_limit_5_one_launch", kept_per_token)):
        gbps = per_tok * sb / (res[name + "_ms_per_step"] * 1e-3) / 1e9
        link[name] = {"achieved": round(gbps, 1), "frac": round(gbps / HOST_LINK_GBPS, 3)}
    res["host_link_roofline"] = dict(bound="host link", peak=HOST_LINK_GBPS, unit="GB/s", **link)
    # effect of the rank limit on each layer's update y - x (graph 0's routing)
    chain_full = DecodeChain(torch, bf, shape, pools2, 1, dev, xs, logits2, tiers=tiers,
                             host_table=host_table)
    rel = []
    for l in range(N_LAYERS):
        L = chain_full.layers[l]
        args = dict(idx=chain_full.idx, w=chain_full.w, slot=chain_full.slot,
                    miss_expert=chain_full.miss_e, miss_pair=chain_full.miss_p,
                    n_miss=chain_full.n_miss, ws=chain_full.ws)
        y_full, *_ = bf.decode_layer(L, xs[l], logits2[0][l], chain_full.tables[l], **args)
        y_lim = y_full.clone()
        bf.decode_misses(tiers[l], xs[l], chain_full.idx, chain_full.slot, chain_full.w,
                         host_table, y_full, ws=chain_full.ws)
        bf.decode_misses(tiers[l], xs[l], chain_full.idx, chain_full.slot, chain_full.w,
                         host_table, y_lim, max_rank=5, ws=chain_full.ws)
        upd = (y_full - xs[l]).norm().item()
        rel.append((y_full - y_lim).norm().item() / upd if upd > 0 else 0.0)
    res["rank_limit_5_rel_change_of_update"] = round(float(np.mean(rel)), 4)
    res["host_tier"] = ("all 512 experts of each layer in pinned host memory, read by the decode "
                        "kernel over the host link (no copy engine); full_layer, rank_limit_5: "
                        "moe_decode_layer then moe_decode_misses on one stream, in one graph; "
                        "full_layer_two_streams: per layer routing and lookup, then the host-tier "
                        "read (moe_decode_misses_phases READ) on a second stream while the GPU "
                        "part runs, the join (JOIN) after both; host_part_only: that step "
                        "without the GPU part; *_one_launch: moe_decode_layer_tiers, the hits "
                        "and the misses in the same two kernels per layer")
    log(f"host tier: {res} ({time.perf_counter() - t0:.1f} s)")
    del chain, chain_full
    return res


def run_prefill_streamed(torch, np, bf, synth, pools2, tiers, dev):
    """Prefill chunks of 8,192 tokens through 48 layers whose GPU cache
    holds 94 of 512 experts: each layer is staged (moe_stage_layer: resident
    experts copied device to device, the other 418 host to device) into one
    of two staging pools on a copy stream, while the previous layer's
    prefill runs on the compute stream."""
    shape = synth.config_shape(4)
    E, k, d, f = shape.n_experts, shape.top_k, shape.d_model, shape.d_ff
    T = synth.WORKLOADS[4]["T"]
    sb = synth.slot_bytes(synth.FMT_Q2SM, d, f)
    t0 = time.perf_counter()
    caches = [bf.MoeLayer(d, f, E, k, fmt, pool, shared_slot) for pool, _, shared_slot, fmt in pools2]
    tabs = [t.cpu().numpy() for _, t, _, _ in pools2]
    host_slot = np.arange(E, dtype=np.int32)
    n_res = [int((t >= 0).sum()) for t in tabs]
    h2d = sum((E - r) * sb for r in n_res)
    xs = [synth.make_x(4, l, T, d, device=dev, dtype=torch.bfloat16) for l in range(N_LAYERS)]
    logits = [synth.make_logits(4, l, T, E, 1.5, device=dev) for l in range(N_LAYERS)]
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    slot = torch.empty((T, k), dtype=torch.int32, device=dev)
    me = torch.empty((T * k,), dtype=torch.int32, device=dev)
    n_miss = torch.empty((4,), dtype=torch.int32, device=dev)
    lws = torch.empty((max(bf.lookup_workspace_bytes(T, k, E), 256),), dtype=torch.uint8, device=dev)
    out_pairs = torch.empty((T * k, d), dtype=torch.float32, device=dev)
    pair_pos = torch.empty((T, k), dtype=torch.int32, device=dev)
    offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    out_sh = torch.empty((T, d), dtype=torch.float32, device=dev)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    staging = [torch.empty((E + 1, sb), dtype=torch.uint8, device=dev) for _ in range(2)]
    staged = [bf.MoeLayer(d, f, E, k, synth.FMT_Q2SM, st, E) for st in staging]
    pws = torch.empty((bf.prefill_workspace_bytes(staged[0], T),), dtype=torch.uint8, device=dev)
    ident = torch.arange(E, dtype=torch.int32, device=dev)
    up = torch.cuda.Stream()
    comp = torch.cuda.current_stream()

    def one_step(stage=True, compute=True):
        ev_up = [torch.cuda.Event() for _ in range(N_LAYERS)]
        ev_done = [torch.cuda.Event() for _ in range(N_LAYERS)]
        up.wait_stream(comp)
        for l in range(N_LAYERS):
            if stage:
                with torch.cuda.stream(up):
                    if l >= 2 and compute:
                        up.wait_event(ev_done[l - 2])
                    bf.stage_layer(caches[l], tabs[l], tiers[l], host_slot, staging[l % 2],
                                   stream=up)
                    ev_up[l].record(up)
                if compute:
                    comp.wait_event(ev_up[l])
            if compute:
                bf.route_topk(logits[l], k, idx=idx, w=w)
                bf.cache_lookup(idx, ident, slot=slot, miss_expert=me, n_miss=n_miss, ws=lws,
                                want_pairs=False)
                bf.expert_ffn_prefill(staged[l % 2], xs[l], idx, slot, out_pairs=out_pairs,
                                      pair_pos=pair_pos, expert_offsets=offs, out_shared=out_sh,
                                      ws=pws)
                bf.combine(xs[l], out_pairs, pair_pos, w, out_sh, y=y)
                ev_done[l].record(comp)
        comp.wait_stream(up)

    def timed(**kw):
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        one_step(**kw)
        torch.cuda.synchronize()
        return time.perf_counter() - t1

    one_step()                                    # warm-up
    dt = timed()
    dt_stage = timed(compute=False)
    dt_compute = timed(stage=False)               # on whatever the staging pools hold
    res = {
        "workload": "prefill chunk: 8,192 bf16 tokens through 48 layers of the expert-cache "
                    "shape (94 of 512 experts + shared resident per layer, the rest in pinned "
                    "host memory); each layer staged into one of two pools on a copy stream "
                    "while the previous layer computes",
        "tok_s": round(T / dt, 1),
        "ms_per_layer": round(dt * 1e3 / N_LAYERS, 3),
        "staging_only_ms_per_layer": round(dt_stage * 1e3 / N_LAYERS, 3),
        "compute_only_ms_per_layer": round(dt_compute * 1e3 / N_LAYERS, 3),
        "host_to_device_GB_per_layer": round(h2d / N_LAYERS / 1e9, 3),
        "host_to_device_GBps": round(h2d / dt / 1e9, 1),
        "overlap": round(max(dt_stage, dt_compute) / dt, 3),
    }
    log(f"prefill streamed: {res} ({time.perf_counter() - t0:.1f} s)")
    return res


def run_adaptive_cache(torch, np, bf, synth, shape, pools2, tiers, host_table, xs, dev,
                       period=16, max_swaps=8, warm_steps=128, steps=64):
    """Routing drifts to another conversation (a new popularity order per
    layer), and the cache follows it: every token counts its experts, every
    `period` tokens each layer plans up to `max_swaps` swaps (counts halve),
    copies the newcomers from the host tier and commits them.  Whole layers:
    the resident experts and the misses from the host tier in one
    moe_decode_layer_tiers call per layer.  Reported: the hit rate of the
    original cache on the new routing, the hit rate after adapting (on
    held-out tokens of the new routing), and tok/s of the timed steps with
    the maintenance included."""
    E, k, d = shape.n_experts, shape.top_k, shape.d_model
    c2 = synth.WORKLOADS[2]
    t0 = time.perf_counter()
    drift = 1000                     # layer offset of the new popularity order

    def logits_of(step):             # [48, 1, E], a fresh token per step
        return torch.stack([synth.zipf_gumbel_logits(2, l + drift, 1, E, c2["zipf_s"],
                                                     device=dev, step=step)
                            for l in range(N_LAYERS)])

    def hit_rate(tables, first_step, n):
        hits = tot = 0
        for st in range(first_step, first_step + n):
            lg = logits_of(st).cpu().numpy()
            for l in range(N_LAYERS):
                idx = np.argsort(-lg[l], axis=1, kind="stable")[:, :k]
                hits += int((tables[l][idx] >= 0).sum())
                tot += idx.size
        return hits / tot

    tables = [t for _, t, _, _ in pools2]
    held_out = 10_000
    static_hit = hit_rate([t.cpu().numpy() for t in tables], held_out, 16)
    eos = []
    shared = []
    for l in range(N_LAYERS):
        _, shared_slot, slot_expert = synth.make_slot_table(2, l)
        eos.append(torch.tensor(slot_expert, dtype=torch.int32, device=dev))
        shared.append(shared_slot)
    counts = [torch.zeros(E, dtype=torch.int32, device=dev) for _ in range(N_LAYERS)]
    lg_buf = logits_of(0)
    chain = DecodeChain(torch, bf, shape, pools2, 1, dev, xs, [lg_buf], tiers=tiers,
                        host_table=host_table, counts=counts, one_launch=True)
    swaps = [torch.full((max_swaps, 4), -1, dtype=torch.int32, device=dev) for _ in range(N_LAYERS)]
    n_sw = [torch.zeros(4, dtype=torch.int32, device=dev) for _ in range(N_LAYERS)]

    def maintain():
        for l in range(N_LAYERS):
            bf.cache_plan(counts[l], tables[l], eos[l], shared[l], host_table, E, max_swaps, 1,
                          swaps=swaps[l], n_swaps=n_sw[l])
            bf.cache_fill(chain.layers[l], tiers[l], swaps[l], n_sw[l])
            bf.cache_commit(tables[l], swaps[l], n_sw[l])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain.step(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g_step, g_maint = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step):
        chain.step(0)
    with torch.cuda.graph(g_maint):
        maintain()
    for c in counts:
        c.zero_()
    torch.cuda.synchronize()
    # inputs of every step resident in HBM before timing
    all_lg = torch.stack([logits_of(st) for st in range(warm_steps + steps)])
    swaps_done = 0

    def run(first, n, count_swaps=False):
        nonlocal swaps_done
        for i in range(first, first + n):
            lg_buf.copy_(all_lg[i])
            g_step.replay()
            if (i + 1) % period == 0:
                g_maint.replay()
                if count_swaps:
                    torch.cuda.synchronize()
                    swaps_done += sum(int(t[0]) for t in n_sw)

    # the original cache on the new routing, no maintenance (same timed tokens)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(warm_steps, warm_steps + steps):
        lg_buf.copy_(all_lg[i])
        g_step.replay()
    torch.cuda.synchronize()
    dt_static = time.perf_counter() - t1
    for c in counts:
        c.zero_()
    run(0, warm_steps, count_swaps=True)
    warm_swaps = swaps_done
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    run(warm_steps, steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t1
    adapted_hit = hit_rate([t.cpu().numpy() for t in tables], held_out, 16)
    # reference point: a cache holding the 94 most popular experts of the new order
    top_tabs = []
    for l in range(N_LAYERS):
        tab = np.full(E, -1, np.int32)
        tab[synth.zipf_popularity(2, l + drift, E)[:94]] = 0
        top_tabs.append(tab)
    top_hit = hit_rate(top_tabs, held_out, 16)
    res = {
        "workload": f"routing moves to another popularity order; count every token, every "
                    f"{period} tokens up to {max_swaps} swaps per layer (counts halve), newcomers "
                    f"copied from the host tier by a kernel; whole layers with misses from the "
                    f"host tier (moe_decode_layer_tiers); timed after {warm_steps} adapting "
                    f"tokens",
        "hit_rate_before": round(static_hit, 4),
        "hit_rate_after": round(adapted_hit, 4),
        "hit_rate_of_the_new_top_94": round(top_hit, 4),
        "swaps_while_adapting": warm_swaps,
        "tok_s": round(steps / dt, 2),
        "ms_per_step": round(dt * 1e3 / steps, 5),
        "tok_s_without_adapting": round(steps / dt_static, 2),
    }
    log(f"adaptive cache: {res} ({time.perf_counter() - t0:.1f} s)")
    del g_step, g_maint, chain
    return res


def run_prefill(torch, np, bf, synth, pools, dev, args):
    shape = synth.config_shape(4)
    E, k, d, f = shape.n_experts, shape.top_k, shape.d_model, shape.d_ff
    T = synth.WORKLOADS[4]["T"]
    layers = [bf.MoeLayer(d, f, E, k, fmt, pool, shared_slot)
              for pool, _, shared_slot, fmt in pools]
    tables = [t for _, t, _, _ in pools]
    xs = [synth.make_x(4, l, T, d, device=dev, dtype=torch.bfloat16) for l in range(N_LAYERS)]
    logits = [synth.make_logits(4, l, T, E, 1.5, device=dev) for l in range(N_LAYERS)]
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    slot = torch.empty((T, k), dtype=torch.int32, device=dev)
    me = torch.empty((T * k,), dtype=torch.int32, device=dev)
    n_miss = torch.empty((4,), dtype=torch.int32, device=dev)
    lws = torch.empty((max(bf.lookup_workspace_bytes(T, k, E), 256),), dtype=torch.uint8, device=dev)
    out_pairs = torch.empty((T * k, d), dtype=torch.float32, device=dev)
    pair_pos = torch.empty((T, k), dtype=torch.int32, device=dev)
    offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    out_sh = torch.empty((T, d), dtype=torch.float32, device=dev)
    y = torch.empty((T, d), dtype=torch.float32, device=dev)
    pws = torch.empty((bf.prefill_workspace_bytes(layers[0], T),), dtype=torch.uint8, device=dev)

    def one_step(events=None):
        for l, L in enumerate(layers):
            bf.route_topk(logits[l], k, idx=idx, w=w)
            bf.cache_lookup(idx, tables[l], slot=slot, miss_expert=me, n_miss=n_miss, ws=lws,
                            want_pairs=False)
            if events is not None:
                events[l][0].record()
            bf.expert_ffn_prefill(L, xs[l], idx, slot, out_pairs=out_pairs, pair_pos=pair_pos,
                                  expert_offsets=offs, out_shared=out_sh, ws=pws)
            if events is not None:
                events[l][1].record()
            bf.combine(xs[l], out_pairs, pair_pos, w, out_sh, y=y)

    one_step()
    torch.cuda.synchronize()
    steps = args.prefill_steps
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(N_LAYERS)]
    one_step(evs)
    torch.cuda.synchronize()
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    flops = 2 * 3 * d * f * T * (k + 1)
    tflops = flops / (call_ms * 1e-3) / 1e12
    toks = steps * T / dt
    log(f"prefill: {toks:.0f} tok/s (48 layers), prefill call {call_ms:.3f} ms, {tflops:.1f} TFLOP/s")
    return {
        "workload": "prefill chunk: 8,192 bf16 tokens, top-10 + shared, 48 independent layers of the decode shape (Q2SM)",
        "tok_s": round(toks, 1),
        "ms_per_layer": round(dt * 1e3 / steps / N_LAYERS, 4),
        "roofline": {
            "kernel": "moe_expert_ffn_prefill (grouping + gate/up + down GEMMs)",
            "bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(PREFILL_TRAFFIC_FILE, PREFILL_SOURCES),
            "avg_call_ms": round(call_ms, 4), "flops_per_call": flops,
        },
        "mfma_busy_counters": mfma_busy_counters(),
    }


def mfma_busy_counters():
    """MFMA utilisation of the two prefill GEMMs from the committed rocprofv3
    counter summary (SQ_VALU_MFMA_BUSY_CYCLES over the active cycles of all
    SIMDs), or None when the prefill sources changed since it was taken."""
    kv = summary_keys(PREFILL_MFMA_FILE, PREFILL_SOURCES)
    if kv is None:
        return None
    try:
        return {"gate_up": float(kv["mfma_busy_gate_up"]), "down": float(kv["mfma_busy_down"]),
                "source": os.path.basename(PREFILL_MFMA_FILE)}
    except (KeyError, ValueError):
        return None


def cpu_baseline(np, synth, pools, shape):
    """The oracle on this host's cores: one token through all 48 decode layers
    (route, lookup, unpack of the chosen slots, expert FFNs, combine)."""
    import oracle
    avail = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        blas = 1
    cores = min(blas, avail)        # NumPy's BLAS threads, bounded by the CPUs this process may use
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    E, k, d, f = shape.n_experts, shape.top_k, shape.d_model, shape.d_ff
    n_tok = 2
    inputs = []
    for step in range(n_tok):          # device -> host copies stay outside the timing
        for l in range(N_LAYERS):
            pool, table_dev, shared_slot, fmt = pools[l]
            table = table_dev.cpu().numpy()
            logits = synth.make_logits(1, l, 1, E, 1.5, step=step).numpy()
            chosen = set(table[np.argsort(-logits[0], kind="stable")[:k]].tolist())
            host = {s: pool[s].cpu().numpy() for s in chosen | {shared_slot}}
            x = synth.make_x(1, l, 1, d).double().numpy()
            inputs.append((x, logits, table, host, shared_slot, fmt))
    t0 = time.perf_counter()
    for x, logits, table, host, shared_slot, fmt in inputs:
        idx, w = oracle.route_topk(logits, k)
        slot, _, _, _ = oracle.cache_lookup(idx, table)
        oracle.layer_decode(x, idx, slot, w,
                            lambda s: oracle.unpack_expert(host[s], fmt, d, f), shared_slot)
    dt = time.perf_counter() - t0
    return {"value": round(n_tok / dt, 5), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 NumPy oracle, {n_tok} tokens (two logit draws) through all {N_LAYERS} "
                      f"decode layers over the same packed pools as the timed workload, logits "
                      f"drawn on the host (route, lookup, unpack of the 11 chosen slots, FFNs, "
                      f"combine)",
            "seconds": round(dt, 2), "cpus_available": avail, "cpu_model": cpu_model}


if __name__ == "__main__":
    main()
