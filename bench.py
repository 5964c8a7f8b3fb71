#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

Workload: the Llama-3-70B-shaped decode batch over all 80 layers -- 20
sequences of 8,000 tokens, 64 query / 8 KV heads of 128, bf16 KV cache in
blocks of 16 tokens with shuffled block tables (10,000 blocks and 655 MB of
K+V per layer, 52.4 GB in HBM).  One step is the whole decode path of one
token per sequence: for each of the 80 layers, the write of the new token's
K/V into its slot (found through the block table) and the paged attention
over all 8,000 tokens -- by default in one fused pa_decode call per layer,
with --unfused as pa_slot_mapping + pa_reshape_and_cache + pa_decode.

Prints one JSON line.  ``value`` is KV GB/s over the whole step (K and V
bytes of all 8,000 tokens x 80 layers, counted once, / step time), with
tokens/s beside it; ``roofline`` prices the decode launch against the
8 TB/s HBM peak; ``cpu_baseline`` times the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD's published figure


# --------------------------------------------------------------------------
# byte accounting (host arithmetic)
# --------------------------------------------------------------------------

def kv_bytes(context_lens, num_kv_heads: int, head_dim: int, elem_bytes: int, layers: int = 1) -> int:
    """2 (K and V) x layers x kv heads x head_dim x tokens x bytes: the
    KV-size formula of the ia-vox article ("Pourquoi le KV cache domine"),
    summed over the batch's real context lengths."""
    return 2 * layers * num_kv_heads * head_dim * int(sum(int(n) for n in context_lens)) * elem_bytes


def decode_algorithmic_bytes(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                             kv_elem: int, q_elem: int, int8_scales: bool = False, token_scales: bool = False,
                             query_rows: int = 0) -> int:
    """Bytes one decode call must move at least: K and V of every token
    (not padded to the block), the scales of quantised caches (per (block,
    head), or per token), the table entries in use, the context lengths, q
    and the fp32 output (query_rows rows when several per sequence)."""
    S = len(context_lens)
    rows = query_rows or S
    blocks = sum(-(-int(n) // block_size) for n in context_lens)
    b = kv_bytes(context_lens, num_kv_heads, head_dim, kv_elem)
    if token_scales:
        b += sum(int(n) for n in context_lens) * num_kv_heads * 2 * 4
    elif int8_scales:
        b += blocks * num_kv_heads * 2 * 4
    b += blocks * 4 + S * 4 + rows * num_q_heads * head_dim * (q_elem + 4)
    return b


def waste_report(context_lens, block_size: int, reserved: int):
    """Reserved-but-empty KV slots: one contiguous region of `reserved`
    tokens per request versus pages of `block_size` (forum thread, ia-vox and
    deeplearn.tn articles; glossary figure)."""
    used = sum(int(n) for n in context_lens)
    paged = sum(-(-int(n) // block_size) * block_size for n in context_lens)
    contig = reserved * len(context_lens)
    return {"contiguous_waste": 1.0 - used / contig if contig else 0.0,
            "paged_waste": 1.0 - used / paged if paged else 0.0}


# --------------------------------------------------------------------------
# benchmark
# --------------------------------------------------------------------------

def pctl(sorted_vals, p: float) -> float:
    """p-th percentile of an ascending list, linear between closest ranks."""
    n = len(sorted_vals)
    if n == 1:
        return float(sorted_vals[0])
    x = (n - 1) * p / 100.0
    i = int(math.floor(x))
    j = min(i + 1, n - 1)
    return float(sorted_vals[i] + (sorted_vals[j] - sorted_vals[i]) * (x - i))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


# HBM bytes of one pa_decode call on the 70B-shaped layer (decode + merge
# kernels, fused cache write), from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE runs: FETCH_SIZE scaled by 1.99226 and WRITE_SIZE by 1.0, the
# ratios of a plain copy's known bytes to what the same counters read for it
# (profiles/decode_mfma_llama3-70b_pmc_traffic.md).  Valid only for the
# sources the counters were taken on: a changed kernel or plan reports null.
PMC_TRAFFIC = {
    "sources_sha256": "3771626bdf6aa622e106d3a8103b10ed1f21a78f57d35395baf912066c20be1f",
    "fetch_kib": 320854.71875 + 1386.5,
    "write_kib": 2680.0625 + 640.0,
    "fetch_factor": 1.99226,
    "write_factor": 1.0,
}
PMC_SOURCES = ("paged_kv_cache_192_amd/csrc/pa_decode.hip", "paged_kv_cache_192_amd/csrc/pa_api.cpp",
               "paged_kv_cache_192_amd/csrc/pa_internal.h")


def sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in PMC_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(fused: bool):
    t = PMC_TRAFFIC
    if not fused or t["sources_sha256"] != sources_sha256():
        return None
    return int(round((t["fetch_kib"] * t["fetch_factor"] + t["write_kib"] * t["write_factor"]) * 1024))


def llama70b_prepare(stream, Q, K, V, KN, VN, bt, cl, outs, ws, slots, total_context_len: int, scale: float,
                     context_len: int, block_size: int, fused: bool = True, partition_tokens: int = 0):
    """One step of the 70B-shaped workload, arguments packed once, on
    `stream`: per layer the write of the new token's K/V into its slot and
    the decode over all tokens -- one fused pa_decode call per layer (the
    timed form), or with fused=False a slot-mapping launch per step and a
    cache-write launch per layer before each decode.  Returns (calls before
    the layers, [(write calls, decode call)] per layer)."""
    import paged_kv_cache_192_amd as pa

    pre = [pa.prepare_slot_mapping(bt, block_size, slots, context_lens=cl, stream=stream)] if not fused else []
    layers = []
    for layer in range(len(Q)):
        writes = [] if fused else [pa.prepare_reshape_and_cache(KN[layer], VN[layer], K[layer], V[layer], slots,
                                                                 stream=stream)]
        d = pa.PreparedDecode(Q[layer], K[layer], V[layer], bt, cl, scale, context_len, outs[layer], workspace=ws,
                              stream=stream, new_key=KN[layer] if fused else None,
                              new_value=VN[layer] if fused else None, partition_tokens=partition_tokens,
                              total_context_len=total_context_len)
        layers.append((writes, d))
    return pre, layers


def run(args) -> dict:
    import numpy as np
    import torch

    import paged_kv_cache_192_amd as pa
    import synth

    pa.library()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    c = synth.CFG3
    L = args.layers
    st = synth.config3_structure()
    S, Hq, Hkv, D, BS, ctx = c["num_seqs"], c["num_q_heads"], c["num_kv_heads"], c["head_dim"], c["block_size"], \
        c["context_len"]
    scale = float(st["scale"])
    print("bench: generating %d layers of %d x %d tokens on the device" % (L, S, ctx), file=sys.stderr, flush=True)
    K, V, Q, KN, VN = [], [], [], [], []
    for layer in range(L):
        q, k, v, kn, vn = synth.config3_layer_values(layer, dev)
        K.append(k)
        V.append(v)
        Q.append(q)
        KN.append(kn)
        VN.append(vn)
    bt = torch.from_numpy(st["block_tables"]).to(dev)
    cl = torch.from_numpy(st["context_lens"]).to(dev)
    outs = [torch.empty(S, Hq, D, dtype=torch.float32, device=dev) for _ in range(L)]
    slots = torch.empty(S, dtype=torch.int64, device=dev)
    probe = pa.make_decode_args(Q[0], K[0], V[0], bt, cl, scale, ctx, out=outs[0],
                                partition_tokens=args.partition_tokens)
    ws_bytes = pa.decode_workspace_size(probe)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    fused = not args.unfused

    def prepare(stream):
        return llama70b_prepare(stream, Q, K, V, KN, VN, bt, cl, outs, ws, slots, int(st["context_lens"].sum()),
                                scale, ctx, BS, fused, args.partition_tokens)

    main_stream = torch.cuda.current_stream()
    eager_pre, eager_layers = prepare(main_stream)

    def eager_step():
        for f in eager_pre:
            f()
        for writes, d in eager_layers:
            for f in writes:
                f()
            d()

    # the same step captured once as a HIP graph (no memsets in it: every
    # node is one of the library's kernels)
    graph = None
    if args.graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(main_stream)
        g_pre, g_layers = prepare(cap)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            for f in g_pre:
                f()
            for writes, d in g_layers:
                for f in writes:
                    f()
                d()
        torch.cuda.synchronize()

    def step():
        if graph is not None:
            graph.replay()
        else:
            eager_step()

    # replays must reproduce the eager result bit for bit (checked before the
    # warmup, so that the warmup runs straight into the timed region)
    eager_step()
    torch.cuda.synchronize()
    ref = torch.stack(outs).clone()
    step()
    torch.cuda.synchronize()
    if not torch.equal(torch.stack(outs), ref):
        raise RuntimeError("graph replay differs from the eager step")
    warm_run = warm_up(step, args.warmup, args.warmup_ms)

    # timed region: exactly `steps` steps between two synchronisations; an
    # event pair around each step gives the per-step distribution (events
    # are recorded on the stream the step runs on, no synchronisation)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step_ev[i].record()
        step()
    step_ev[args.steps].record()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    step_ms = sorted(step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(args.steps))

    # per-launch duration of the decode call: events around each eager call
    launch_ms = []
    for _ in range(max(1, min(args.steps, 5))):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(L)]
        for f in eager_pre:
            f()
        for layer, (writes, d) in enumerate(eager_layers):
            for f in writes:
                f()
            evs[layer][0].record()
            d()
            evs[layer][1].record()
        torch.cuda.synchronize()
        launch_ms += [a.elapsed_time(b) for a, b in evs]
    launch_ms = sorted(launch_ms)
    # average launch duration of pa_decode: with the write fused, the timed
    # region holds exactly steps x L decode calls and nothing else; else the
    # events around each eager call
    launch_avg = ms_per_step / L if fused else sum(launch_ms) / len(launch_ms)
    if not torch.equal(torch.stack(outs), ref):
        raise RuntimeError("timed steps changed the result")

    cls = st["context_lens"]
    kv_step = kv_bytes(cls, Hkv, D, 2, layers=L)
    alg_launch = decode_algorithmic_bytes(cls, Hq, Hkv, D, BS, 2, 2)
    gbs = kv_step / (ms_per_step * 1e-3) / 1e9
    achieved = alg_launch / (launch_avg * 1e-3) / 1e9
    res = {
        "metric": "paged decode KV GB/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_run,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3-70b-shaped gqa decode, 80 layers", "layers": L, "num_seqs": S,
                   "context_len": ctx, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "block_size": BS,
                   "kv_dtype": "bf16", "global_batch": S, "seq_len": ctx},
        "tokens_per_s": round(S / (ms_per_step * 1e-3), 1),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "step_ms": {"p10": round(pctl(step_ms, 10), 4), "p50": round(pctl(step_ms, 50), 4),
                    "p90": round(pctl(step_ms, 90), 4), "min": round(step_ms[0], 4), "max": round(step_ms[-1], 4),
                    "source": "event pair around each step of the timed region"},
        "kv_bytes_per_step": kv_step,
        "wall_s_timed_region": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(fused),
                     "kernel": "pa_decode = decode_mfma_kernel + decode_merge_kernel", "launch_ms_avg": round(launch_avg, 5),
                     "launch_ms_source": ("timed region / (steps x layers)" if fused else
                                          "events around each eager call"),
                     "eager_call_ms_p10": round(launch_ms[len(launch_ms) // 10], 5),
                     "eager_call_ms_p50": round(launch_ms[len(launch_ms) // 2], 5),
                     "eager_call_ms_p90": round(launch_ms[(9 * len(launch_ms)) // 10], 5),
                     "algorithmic_bytes_per_launch": alg_launch, "workspace_bytes": ws_bytes},
        "waste": waste_report(cls, BS, 8192),
        "step_mode": ("hip graph replay" if graph is not None else "eager prepared calls") +
                     (", cache write fused into pa_decode" if fused else ", separate slot-mapping and cache-write launches"),
    }
    if args.cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args, K, V, Q, st, L)
    return res


WORKLOADS = {
    "int8-token": "int8 KV with per-token scales: each new token quantised and written, then decode, in one "
                  "pa_decode call (--unfused: pa_quantize_and_cache first) (64 seqs, log-normal lengths, 32/8 heads)",
    "fp8": "E4M3 fp8 KV with per-token scales: each new token quantised and written, then decode, in one pa_decode "
           "call (--unfused: pa_quantize_and_cache first) (64 seqs, log-normal lengths, 32/8 heads)",
    "spec-decode": "70B-shaped layer (20 x 8,000 tokens, 64/8 heads, bf16) with 4 causal query rows per sequence "
                   "(checking 3 drafted tokens)",
    "chunked-prefill": "70B-shaped layer (20 x 8,000 tokens, 64/8 heads, bf16) with a 64-row causal prefill chunk "
                       "per sequence",
    "chunked-prefill-int8": "the chunked-prefill layer over an int8 cache (per-(block, head) scales, seeded codes)",
    "llama3-70b": "70B-shaped GQA decode, 80 layers (20 x 8,000 tokens, 64/8 heads, bf16, block 16)",
    "tiny": "tiny fp32 decode (4 seqs of 17/33/100/200 tokens, 8 heads of 64, block 16)",
    "llama13b": "13B-shaped MHA decode, one layer (32 seqs, U[200,2048] tokens, 40 heads of 128, bf16)",
    "prefix": "prefix sharing + copy-on-write, one layer (50 seqs, 2,000 shared + U[50,500], 32/8 heads, block 32)",
    "int8": "int8 KV decode, one layer (64 seqs, log-normal lengths, 32/8 heads, per-(block, head) scales)",
    "gqa-d64": "70B-shaped batch at head_dim 64 (20 x 8,000 tokens, 64/8 heads, bf16, block 16, fused write)",
    "int8-d64": "70B-shaped batch at head_dim 64 with an int8 cache (per-(block, head) scales)",
}


def run_single_layer(args) -> dict:
    """The four one-layer workloads.  A step is one decode layer per replica:
    the pool is replicated R times (R such that >= 1 GB is touched between
    reuses of the same bytes, so MALL/L2 cannot serve it) and each step
    walks all replicas; per-layer time = step time / R.  The new token's
    cache write is fused into pa_decode (not for int8: no quantising
    write); the prefix workload also copies the shared partial block to 50
    scratch blocks per layer (pa_copy_blocks) before decoding, and passes
    the 62 shared full blocks as the decode's shared prefix (unless
    --no-shared-prefix)."""
    import numpy as np
    import torch

    import paged_kv_cache_192_amd as pa
    import synth

    pa.library()
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    w = args.workload
    case = {"tiny": synth.config1, "llama13b": synth.config2, "prefix": synth.config4,
            "int8": synth.config5}[w]()
    if w == "int8":
        synth.random_int8_cache(case, seed=55)

    def put(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    S, Hq, Hkv, D, BS = case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    e = {"f32": 4, "bf16": 2, "i8": 1}[case.kv_dtype]
    eq = {"f32": 4, "bf16": 2}[case.q_dtype]
    layer_bytes = 2 * case.k_cache.nbytes
    R = max(1, -(-(1 << 30) // layer_bytes)) if w != "tiny" else 1
    q, bt, cl = put(case.q), put(case.block_tables), put(case.context_lens)
    k0, v0 = put(case.k_cache), put(case.v_cache)
    ks = put(case.k_scales) if case.k_scales is not None else None
    vs = put(case.v_scales) if case.v_scales is not None else None
    K = [k0] + [k0.clone() for _ in range(R - 1)]
    V = [v0] + [v0.clone() for _ in range(R - 1)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    tdt = torch.float32 if case.kv_dtype == "f32" else torch.bfloat16
    newk = torch.randn(S, Hkv, D, generator=gen, device=dev).to(tdt) if w != "int8" else None
    newv = torch.randn(S, Hkv, D, generator=gen, device=dev).to(tdt) if w != "int8" else None
    pairs = None
    shared, shared_len = None, 0
    if w == "prefix":
        pr = np.stack([np.full(S, case.extra["partial"]), case.extra["scratch"]], axis=1).astype(np.int64)
        pairs = put(pr)
        if args.shared_prefix:
            # the 62 full blocks every table starts with, read once per layer
            shared = put(case.extra["shared"].astype(np.int32))
            shared_len = len(case.extra["shared"]) * BS
    outs = [torch.empty(S, Hq, D, dtype=torch.float32, device=dev) for _ in range(R)]
    ws = torch.zeros(1 << 26, dtype=torch.uint8, device=dev)
    mcl = case.max_context_len

    def prepare(stream):
        calls = []
        for r in range(R):
            if pairs is not None:
                calls.append(pa.prepare_copy_blocks(K[r], V[r], pairs, stream=stream))
            calls.append(pa.PreparedDecode(q, K[r], V[r], bt, cl, float(case.scale), mcl, outs[r], k_scales=ks,
                                           v_scales=vs, workspace=ws, stream=stream, new_key=newk, new_value=newv,
                                           partition_tokens=args.partition_tokens, kernel=args.kernel,
                                           total_context_len=int(np.sum(case.context_lens, dtype=np.int64)),
                                           shared_prefix_table=shared, shared_prefix_len=shared_len))
        return calls

    main = torch.cuda.current_stream()
    eager = prepare(main)
    for f in eager:
        f()
    torch.cuda.synchronize()
    ref = torch.stack(outs).clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(main)
    gcalls = prepare(cap)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for f in gcalls:
            f()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    if not torch.equal(torch.stack(outs), ref):
        raise RuntimeError("graph replay differs from the eager step")
    warm_run = warm_up(graph.replay, args.warmup, args.warmup_ms)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_layer = e0.elapsed_time(e1) / args.steps / R
    cls = case.context_lens
    kvb = kv_bytes(cls, Hkv, D, e)
    alg = decode_algorithmic_bytes(cls, Hq, Hkv, D, BS, e, eq, int8_scales=(w == "int8"))
    res = {"workload": w, "description": WORKLOADS[w], "replicas": R, "partition_tokens": args.partition_tokens,
           "kernel": args.kernel, "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": warm_run,
           "ms_per_layer": round(ms_layer, 5), "tokens_per_s": round(S / (ms_layer * 1e-3), 1),
           "kv_gbs": round(kvb / (ms_layer * 1e-3) / 1e9, 1),
           "pct_hbm_peak": round(100.0 * alg / (ms_layer * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
           "algorithmic_bytes_per_layer": alg, "kv_bytes_per_layer": kvb, "sum_ctx": int(sum(int(x) for x in cls)),
           "step": ("copy_blocks + " if pairs is not None else "") + "pa_decode" +
                   (" with fused cache write" if newk is not None else "") +
                   (" and the shared prefix's %d blocks passed" % (shared_len // BS) if shared_len else "")}
    if w == "prefix":
        # unique bytes: every physical block's valid tokens once
        valid = synth.valid_slots_per_block(case)
        uniq = 2 * Hkv * D * e * int(valid.sum())
        copy = 2 * 2 * len(case.extra["scratch"]) * Hkv * BS * D * e
        # the HBM lower bound of the step: unique K/V, tables, q, out, and the
        # copy's reads and writes; the logical rate is reported as effective
        unique_alg = alg - kvb + uniq + copy
        res["unique_kv_bytes_per_layer"] = uniq
        res["copy_bytes_per_layer"] = copy
        res["unique_kv_gbs"] = round(uniq / (ms_layer * 1e-3) / 1e9, 1)
        res["effective_pct_hbm_peak"] = res["pct_hbm_peak"]
        res["pct_hbm_peak"] = round(100.0 * unique_alg / (ms_layer * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)
        res["effective_kv_gbs_note"] = ("kv_gbs and effective_pct_hbm_peak count each sequence's prefix (logical "
                                        "bytes); pct_hbm_peak counts each physical block once plus the copy")
    res["waste"] = waste_report(cls, BS, 2048 if w != "int8" else 32768)
    return res


def warm_up(step, warmup: int, min_ms: float) -> int:
    """Untimed steps before a timed region: at least `warmup` of them and at
    least `min_ms` of wall time, synchronising every few steps so that the
    host does not run ahead of the device.  Returns the steps run.

    The floor is there because the device's clocks settle under load: after
    an idle gap of a few milliseconds the first ~30 ms of matrix-core work
    run up to a quarter slower (replay times rise, then fall back), and a
    handful of short steps ends inside that transient."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t0) * 1e3 < min_ms:
        step()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def _timed_graph(prepare, steps: int, warmup: int, outs, warmup_ms: float = 0.0):
    """Capture prepare()'s calls once as a graph, check one replay against
    the eager result bit for bit, warm up, and return the mean replay time
    in ms and the warmup replays run."""
    import torch

    main = torch.cuda.current_stream()
    for f in prepare(main):
        f()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    cap = torch.cuda.Stream()
    cap.wait_stream(main)
    gcalls = prepare(cap)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for f in gcalls:
            f()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip(outs, ref)):
        raise RuntimeError("graph replay differs from the eager step")
    warm_run = warm_up(graph.replay, warmup, warmup_ms)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, warm_run


def run_next_workload(args) -> dict:
    """Workloads of the quantised and multi-query paths, one layer per
    replica (R replicas so that >= 1 GB is touched between reuses):
      int8-token / fp8: the int8 workload's batch with per-token scales; a
        step quantises and writes every sequence's new token and decodes,
        in one pa_decode call with new_key/new_value (with --unfused:
        pa_quantize_and_cache, then pa_decode);
      spec-decode / chunked-prefill: the 70B-shaped layer with L causal
        query rows per sequence (the last L tokens of each context);
        chunked-prefill-int8 the same 64-row chunks over seeded int8 codes
        with per-(block, head) scales;
      gqa-d64 / int8-d64: the 70B-shaped batch (tables and lengths) at
        head_dim 64, bf16 with the fused write or int8 codes with
        per-(block, head) scales, seeded device values."""
    import numpy as np
    import torch

    import paged_kv_cache_192_amd as pa
    import synth

    pa.library()
    dev = torch.device("cuda:0")
    w = args.workload
    res = {"workload": w, "description": WORKLOADS[w], "steps": args.steps, "warmup": args.warmup,
           "partition_tokens": args.partition_tokens}
    gen = torch.Generator(device=dev)
    gen.manual_seed(91)
    if w in ("int8-token", "fp8"):
        case = synth.config5()
        if w == "fp8":
            synth.random_fp8_cache(case, seed=56, per_token=True)
        else:
            synth.random_int8_cache(case, seed=56, per_token=True)
        S, Hq, Hkv, D, BS = case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
        layer_bytes = 2 * case.k_cache.nbytes
        R = max(1, -(-(1 << 30) // layer_bytes))

        def put(a):
            t = torch.from_numpy(np.ascontiguousarray(a))
            if a.dtype == np.uint16:
                t = t.view(torch.int16).view(torch.bfloat16)
            t = t.to(dev)
            return t.view(torch.float8_e4m3fn) if a.dtype == np.uint8 else t

        q, bt, cl = put(case.q), put(case.block_tables), put(case.context_lens)
        K = [put(case.k_cache) for _ in range(R)]
        V = [put(case.v_cache) for _ in range(R)]
        KS = [put(case.k_scales) for _ in range(R)]
        VS = [put(case.v_scales) for _ in range(R)]
        newk = torch.randn(S, Hkv, D, generator=gen, device=dev).to(torch.bfloat16)
        newv = torch.randn(S, Hkv, D, generator=gen, device=dev).to(torch.bfloat16)
        slots = pa.slot_mapping(bt, BS, context_lens=cl)
        outs = [torch.empty(S, Hq, D, dtype=torch.float32, device=dev) for _ in range(R)]
        ws = torch.empty(1 << 27, dtype=torch.uint8, device=dev)
        total = int(np.sum(case.context_lens, dtype=np.int64))

        fused = not args.unfused

        def prepare(stream):
            calls = []
            for r in range(R):
                if not fused:
                    calls.append(pa.prepare_quantize_and_cache(newk, newv, K[r], V[r], KS[r], VS[r], slots,
                                                               stream=stream))
                calls.append(pa.PreparedDecode(q, K[r], V[r], bt, cl, float(case.scale), case.max_context_len,
                                               outs[r], k_scales=KS[r], v_scales=VS[r], workspace=ws, stream=stream,
                                               partition_tokens=args.partition_tokens, total_context_len=total,
                                               new_key=newk if fused else None, new_value=newv if fused else None))
            return calls

        ms, warm_run = _timed_graph(prepare, args.steps, args.warmup, outs, args.warmup_ms)
        ms /= R
        cls = case.context_lens
        alg = decode_algorithmic_bytes(cls, Hq, Hkv, D, BS, 1, 2, token_scales=True)
        kvb = kv_bytes(cls, Hkv, D, 1)
        res.update({"replicas": R, "warmup_steps_run": warm_run, "ms_per_layer": round(ms, 5),
                    "tokens_per_s": round(S / (ms * 1e-3), 1),
                    "kv_gbs": round(kvb / (ms * 1e-3) / 1e9, 1),
                    "pct_hbm_peak": round(100.0 * alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                    "algorithmic_bytes_per_layer": alg, "sum_ctx": int(np.sum(cls)),
                    "step": ("pa_decode quantising and writing each new token (per-token scales) as it attends"
                             if fused else "pa_quantize_and_cache (new token, per-token scales) + pa_decode")})
        return res
    if w in ("gqa-d64", "int8-d64"):
        st = synth.config3_structure()
        c = synth.CFG3
        S, Hq, Hkv, BS, D = c["num_seqs"], c["num_q_heads"], c["num_kv_heads"], c["block_size"], 64
        NB = st["num_blocks"]
        i8 = w == "int8-d64"
        e = 1 if i8 else 2
        R = max(1, -(-(1 << 30) // (2 * NB * Hkv * BS * D * e)))
        bt = torch.from_numpy(st["block_tables"]).to(dev)
        cl = torch.from_numpy(st["context_lens"]).to(dev)
        shape = (NB, Hkv, BS, D)
        if i8:
            K = [torch.randint(-127, 128, shape, generator=gen, dtype=torch.int8, device=dev) for _ in range(R)]
            V = [torch.randint(-127, 128, shape, generator=gen, dtype=torch.int8, device=dev) for _ in range(R)]
            KS = [torch.rand(NB, Hkv, generator=gen, device=dev) * 0.03 + 0.01 for _ in range(R)]
            VS = [torch.rand(NB, Hkv, generator=gen, device=dev) * 0.03 + 0.01 for _ in range(R)]
            newk = newv = None
        else:
            K = [torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
            V = [torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
            KS = VS = [None] * R
            newk = torch.randn(S, Hkv, D, generator=gen, device=dev).to(torch.bfloat16)
            newv = torch.randn(S, Hkv, D, generator=gen, device=dev).to(torch.bfloat16)
        q = torch.randn(S, Hq, D, generator=gen, device=dev).to(torch.bfloat16)
        outs = [torch.empty(S, Hq, D, dtype=torch.float32, device=dev) for _ in range(R)]
        ws = torch.empty(1 << 26, dtype=torch.uint8, device=dev)
        ctx = int(st["context_lens"][0])
        total = int(np.sum(st["context_lens"], dtype=np.int64))

        def prepare(stream):
            return [pa.PreparedDecode(q, K[r], V[r], bt, cl, float(1.0 / math.sqrt(D)), ctx, outs[r],
                                      k_scales=KS[r], v_scales=VS[r], workspace=ws, stream=stream,
                                      new_key=newk, new_value=newv, partition_tokens=args.partition_tokens,
                                      kernel=args.kernel, total_context_len=total) for r in range(R)]

        ms, warm_run = _timed_graph(prepare, args.steps, args.warmup, outs, args.warmup_ms)
        ms /= R
        cls = st["context_lens"]
        alg = decode_algorithmic_bytes(cls, Hq, Hkv, D, BS, e, 2, int8_scales=i8)
        res.update({"replicas": R, "warmup_steps_run": warm_run, "ms_per_layer": round(ms, 5),
                    "tokens_per_s": round(S / (ms * 1e-3), 1),
                    "kv_gbs": round(kv_bytes(cls, Hkv, D, e) / (ms * 1e-3) / 1e9, 1),
                    "pct_hbm_peak": round(100.0 * alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                    "algorithmic_bytes_per_layer": alg,
                    "step": "pa_decode" + (" (int8 codes, per-(block, head) scales)" if i8 else " with fused write")})
        return res
    # multi-query rows on the 70B-shaped layer
    L = 4 if w == "spec-decode" else 64
    i8 = w == "chunked-prefill-int8"
    e = 1 if i8 else 2
    st = synth.config3_structure()
    c = synth.CFG3
    S, Hq, Hkv, D, BS = c["num_seqs"], c["num_q_heads"], c["num_kv_heads"], c["head_dim"], c["block_size"]
    R = 2
    bt = torch.from_numpy(st["block_tables"]).to(dev)
    cl = torch.from_numpy(st["context_lens"]).to(dev)
    KS = VS = [None] * R
    if i8:
        NB = st["num_blocks"]
        shape = (NB, Hkv, BS, D)
        layers = [(None, torch.randint(-127, 128, shape, generator=gen, dtype=torch.int8, device=dev),
                   torch.randint(-127, 128, shape, generator=gen, dtype=torch.int8, device=dev)) for _ in range(R)]
        KS = [torch.rand(NB, Hkv, generator=gen, device=dev) * 0.03 + 0.01 for _ in range(R)]
        VS = [torch.rand(NB, Hkv, generator=gen, device=dev) * 0.03 + 0.01 for _ in range(R)]
    else:
        layers = [synth.config3_layer_values(r, dev) for r in range(R)]
    qsl = torch.arange(0, S * L + 1, L, dtype=torch.int32, device=dev)
    qs = [torch.randn(S * L, Hq, D, generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    outs = [torch.empty(S * L, Hq, D, dtype=torch.float32, device=dev) for _ in range(R)]
    ws = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    ctx = int(st["context_lens"][0])

    def prepare(stream):
        return [pa.PreparedDecode(qs[r], layers[r][1], layers[r][2], bt, cl, float(st["scale"]), ctx, outs[r],
                                  k_scales=KS[r], v_scales=VS[r], workspace=ws, stream=stream,
                                  partition_tokens=args.partition_tokens, query_start_loc=qsl, max_query_len=L)
                for r in range(R)]

    ms, warm_run = _timed_graph(prepare, args.steps, args.warmup, outs, args.warmup_ms)
    ms /= R
    cls = st["context_lens"]
    alg = decode_algorithmic_bytes(cls, Hq, Hkv, D, BS, e, 2, int8_scales=i8, query_rows=S * L)
    visible = sum(sum(int(n) - L + i + 1 for i in range(L)) for n in cls)
    flops = 4 * Hq * D * visible
    res.update({"replicas": R, "warmup_steps_run": warm_run, "query_rows_per_seq": L, "ms_per_layer": round(ms, 5),
                "query_tokens_per_s": round(S * L / (ms * 1e-3), 1),
                "kv_gbs": round(kv_bytes(cls, Hkv, D, e) / (ms * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100.0 * alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "algorithmic_bytes_per_layer": alg,
                "step": "pa_decode with query_start_loc (%d causal rows per sequence)" % L})
    return res


def run_swap(args) -> dict:
    """pa_swap_blocks bandwidth: --swap-blocks blocks of the 70B-shaped
    layer's shape (8 heads x 16 slots x 128 bf16 = 32 KB per K or V block)
    out to a pinned host pool and back in, as separate timed calls."""
    import torch

    import paged_kv_cache_192_amd as pa

    pa.library()
    dev = torch.device("cuda:0")
    n = args.swap_blocks
    shape = (n, 8, 16, 128)
    dk = torch.randn(shape, device=dev).to(torch.bfloat16)
    dv = torch.randn(shape, device=dev).to(torch.bfloat16)
    hk = torch.empty(shape, dtype=torch.bfloat16).pin_memory()
    hv = torch.empty(shape, dtype=torch.bfloat16).pin_memory()
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(5))
    pairs = torch.stack([torch.arange(n), perm], dim=1).to(torch.int64).to(dev)
    back = torch.stack([perm, torch.arange(n)], dim=1).to(torch.int64).to(dev)
    out_call = pa.prepare_swap_blocks(dk, dv, hk, hv, pairs)
    in_call = pa.prepare_swap_blocks(hk, hv, dk, dv, back)
    res = {"mode": "swap", "blocks": n, "bytes_per_direction": 2 * dk.numel() * 2}
    for name, f in (("device_to_host", out_call), ("host_to_device", in_call)):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        res[name] = {"ms": round(ms, 4), "gbs": round(res["bytes_per_direction"] / (ms * 1e-3) / 1e9, 1)}
    ref = torch.randn(shape, device=dev).to(torch.bfloat16)
    dk.copy_(ref)
    out_call()
    dk.zero_()
    in_call()
    torch.cuda.synchronize()
    res["round_trip_exact"] = bool(torch.equal(dk, ref))
    return res


def cpu_baseline(args, K, V, Q, st, L) -> dict:
    """The CPU oracle (fp64, OpenMP over (sequence, head) rows) on a bounded
    sample of the same workload: whole layers, all 20 sequences, copied back
    from the device; layers are added until about `cpu_seconds` of wall time
    have been spent in the oracle.  Reported in the metric's unit."""
    import numpy as np
    import torch

    import oracle
    import synth

    c = synth.CFG3

    def host(t):
        return t.cpu().view(torch.int16).numpy().view(np.uint16)

    done, spent = 0, 0.0
    for layer in range(L):
        k, v, q = host(K[layer]), host(V[layer]), host(Q[layer])
        t0 = time.perf_counter()
        oracle.paged_decode(q, k, v, st["block_tables"], st["context_lens"], float(st["scale"]))
        spent += time.perf_counter() - t0
        done += 1
        del k, v
        if spent >= args.cpu_seconds:
            break
    kvb = kv_bytes(st["context_lens"], c["num_kv_heads"], c["head_dim"], 2, layers=done)
    return {"value": round(kvb / spent / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d of %d layers, all %d sequences x %d tokens, fp64 oracle, %.1f s (device-to-host copies "
                      "excluded); tokens/s over 80 layers = %.4f" % (done, L, c["num_seqs"], c["context_len"],
                                                                    spent, c["num_seqs"] / (spent / done * 80)),
            "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0))}


def read_ceiling(args) -> dict:
    """The memory system's read ceiling for decode's access pattern, on the
    70B-shaped layer's bytes (K and V caches of 10,000 blocks, 655 MB, one
    allocation): pa_read_probe reading every 4 KiB (block, kv head) chunk
    once, in address order (plain streaming) and in the decode's table
    order (the shuffled blocks of 20 sequences x 500 blocks x 8 kv heads,
    K then V), over a sweep of wave counts; then pa_decode on the same
    layer (no fused write, the library's plan), timed the same way, as a
    fraction of both ceilings.  Each figure is the mean over `steps`
    launches between two events."""
    import numpy as np
    import torch

    import paged_kv_cache_192_amd as pa
    import synth

    pa.library()
    dev = torch.device("cuda:0")
    c = synth.CFG3
    st = synth.config3_structure()
    NB, Hkv, BS, D = st["num_blocks"], c["num_kv_heads"], c["block_size"], c["head_dim"]
    q, k, v, _, _ = synth.config3_layer_values(0, dev)
    kv = torch.empty((2, NB, Hkv, BS, D), dtype=torch.bfloat16, device=dev)
    kv[0].copy_(k)
    kv[1].copy_(v)
    del k, v
    chunk = BS * D * 2
    assert chunk == 4096
    n = 2 * NB * Hkv
    tab = st["block_tables"]
    order = (tab[:, :, None].astype(np.int64) * Hkv + np.arange(Hkv)[None, None, :]).reshape(-1)
    ids = torch.from_numpy(np.concatenate([order, order + NB * Hkv]).astype(np.int32)).to(dev)
    assert ids.numel() == n
    total = n * chunk
    sink = torch.empty(16384 * 64, dtype=torch.int32, device=dev)

    def timed(f):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    res = {"mode": "read-ceiling", "bytes_per_launch": total, "chunk_bytes": chunk, "chunks": n,
           "steps": args.steps, "sequential_gbs": {}, "table_order_gbs": {}}
    waves_sweep = (256, 512, 1024, 2048, 4096, 8192, 16384)
    for waves in waves_sweep:
        for name, cid in (("sequential_gbs", None), ("table_order_gbs", ids)):
            ms = timed(pa.prepare_read_probe(kv, n, sink, chunk_ids=cid, num_waves=waves))
            res[name][str(waves)] = round(total / (ms * 1e-3) / 1e9, 1)
    res["best_sequential_gbs"] = max(res["sequential_gbs"].values())
    res["best_table_order_gbs"] = max(res["table_order_gbs"].values())
    # smaller chunks over the same 655 MB (a 1-byte cache's (block, kv head)
    # is 2 KiB): address order, and a seeded random order of all chunks
    res["by_chunk_gbs"] = {}
    rng = np.random.default_rng(17)
    for cb in (1024, 2048, 4096):
        nc = total // cb
        perm = torch.from_numpy(rng.permutation(nc).astype(np.int32)).to(dev)
        for order, cid in (("sequential", None), ("random", perm)):
            best = 0.0
            for waves in waves_sweep:
                ms = timed(pa.prepare_read_probe(kv, nc, sink, chunk_ids=cid, num_waves=waves, chunk_bytes=cb))
                gbs = total / (ms * 1e-3) / 1e9
                res["by_chunk_gbs"]["%d_%s_%d" % (cb, order, waves)] = round(gbs, 1)
                best = max(best, gbs)
            res["by_chunk_gbs"]["%d_%s_best" % (cb, order)] = round(best, 1)
    bt = torch.from_numpy(tab).to(dev)
    cl = torch.from_numpy(st["context_lens"]).to(dev)
    out = torch.empty(c["num_seqs"], c["num_q_heads"], D, dtype=torch.float32, device=dev)
    d = pa.PreparedDecode(q, kv[0], kv[1], bt, cl, float(st["scale"]), c["context_len"], out,
                          total_context_len=int(st["context_lens"].sum()))
    ms = timed(d)
    kvb = kv_bytes(st["context_lens"], Hkv, D, 2)
    assert kvb == total
    gbs = kvb / (ms * 1e-3) / 1e9
    res["decode_call_ms"] = round(ms, 5)
    res["decode_kv_gbs"] = round(gbs, 1)
    res["decode_frac_of_sequential"] = round(gbs / res["best_sequential_gbs"], 4)
    res["decode_frac_of_table_order"] = round(gbs / res["best_table_order_gbs"], 4)
    res["note"] = ("decode_* = one pa_decode call (decode + merge kernels, launched eagerly) on the same bytes; "
                   "KV bytes only, the same bytes the probe reads")
    return res


def copy_calibration(args) -> dict:
    """A plain copy of known size through pa_copy_blocks, for scaling HBM
    byte counters: `pairs` whole blocks of K and of V (8 kv heads x 32 slots
    x 128 bf16 = 64 KiB each) read once and written once."""
    import torch

    import paged_kv_cache_192_amd as pa

    pa.library()
    dev = torch.device("cuda:0")
    pairs = args.copy_pairs
    NB = 2 * pairs
    k = torch.zeros(NB, 8, 32, 128, dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    pr = torch.stack([torch.arange(pairs), torch.arange(pairs, 2 * pairs)], dim=1).to(torch.int64).to(dev)
    for _ in range(args.steps):
        pa.copy_blocks(k, v, pr)
    torch.cuda.synchronize()
    per = 2 * pairs * 8 * 32 * 128 * 2
    return {"mode": "copy-calibration", "kernel": "copy_blocks_kernel", "launches": args.steps,
            "bytes_read_per_launch": per, "bytes_written_per_launch": per,
            "kib_read_per_launch": per / 1024, "kib_written_per_launch": per / 1024}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-ms", type=float, default=200.0,
                    help="keep warming up until this much wall time has passed (the clocks settle under load)")
    ap.add_argument("--layers", type=int, default=80, help="layers of the 70B-shaped model (80 is the workload)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--unfused", action="store_true",
                    help="separate slot-mapping and reshape_and_cache (or pa_quantize_and_cache) launches instead "
                         "of the fused cache write")
    ap.add_argument("--eager", dest="graph", action="store_false",
                    help="launch each call from Python instead of replaying the captured step")
    ap.add_argument("--mode", choices=["decode", "copy-calibration", "swap", "read-ceiling"], default="decode",
                    help="copy-calibration: a known-size block copy for scaling HBM byte counters; swap: "
                         "pa_swap_blocks bandwidth between the device and a pinned host pool; read-ceiling: "
                         "plain and table-order reads of the 70B-shaped layer's bytes, and pa_decode beside them")
    ap.add_argument("--swap-blocks", type=int, default=4096, help="blocks per swap call (--mode swap)")
    ap.add_argument("--copy-pairs", type=int, default=4096)
    ap.add_argument("--partition-tokens", type=int, default=0,
                    help="override the library's automatic split-K partition length (tuning only)")
    ap.add_argument("--kernel", type=int, default=0, choices=[0, 1, 2],
                    help="decode kernel of the one-layer workloads: 0 library's choice, 1 vector-ALU, 2 matrix-core")
    ap.add_argument("--no-shared-prefix", dest="shared_prefix", action="store_false",
                    help="prefix workload: do not pass the shared prefix's blocks to pa_decode")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="llama3-70b",
                    help="the 70B-shaped 80-layer step (default; the JSON metric line) or one of the single-layer "
                         "workloads, reported as a per-layer record")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path (asked for --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.layers != 80:
        print("note: --layers %d is not the 80-layer workload; the result is for tuning only" % args.layers,
              file=sys.stderr)
    if args.mode == "copy-calibration":
        res = copy_calibration(args)
    elif args.mode == "swap":
        res = run_swap(args)
    elif args.mode == "read-ceiling":
        res = read_ceiling(args)
    elif args.workload in ("int8-token", "fp8", "spec-decode", "chunked-prefill", "chunked-prefill-int8", "gqa-d64",
                           "int8-d64"):
        res = run_next_workload(args)
    elif args.workload != "llama3-70b":
        res = run_single_layer(args)
    else:
        res = run(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
