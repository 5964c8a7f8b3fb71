"""The one-layer workloads of configurations 2, 4 and 5 in the call form the
benchmark times, against the CPU oracle on every sequence.

* llama13b: 32 sequences of U[200, 2048] tokens, 40/40 heads; pa_decode
  writes each newest token (bf16 rows) and attends (grouped launch).
* int8: 64 sequences of log-normal lengths, 32/8 heads, the benchmark's
  random int8 codes with per-(block, head) scales near 1/73 (its own scales,
  up to 0.035, give values of spread ~1.5 and rows dominated by a few
  tokens, where the weights' ~16-bit error grows with the output and the
  absolute guard is not pinned); balanced split.
* prefix: 50 sequences of 2,000 shared + U[50, 500] tokens, 32/8 heads,
  blocks of 32; pa_copy_blocks of the shared partial block to each
  sequence's scratch block, then pa_decode with the fused write and the 62
  shared full blocks passed as the shared prefix.

Each step is prepared once with the batch's total length as the split hint,
run eagerly, then captured as a HIP graph on a side stream and replayed.
Gates: the caches after the step equal the oracle's copy and write bit for
bit; every output is within 2e-3 of the oracle's decode, rows of sequences
of at least 2,048 tokens within the 2e-5 regression guard; the eager step
and every replay give the same bytes (the step is idempotent)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import GUARD_BF16, TOL_BF16, case_on_device, guard_err, max_err, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w", ["llama13b", "int8", "prefix"])
def test_one_layer_workload_in_the_benchmark_call_form(w):
    case = {"llama13b": synth.config2, "int8": synth.config5, "prefix": synth.config4}[w]()
    if w == "int8":
        synth.random_int8_cache(case, seed=55)
        rng = np.random.default_rng(56)
        # unit spread: uniform codes in [-127, 127] have standard deviation ~73
        case.k_scales = (rng.uniform(0.8, 1.2, case.k_scales.shape) / 73.0).astype(np.float32)
        case.v_scales = (rng.uniform(0.8, 1.2, case.v_scales.shape) / 73.0).astype(np.float32)
    S, Hq, Hkv, D, BS = case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    dev = torch.device("cuda:0")
    d = case_on_device(case)
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    newk = newv = None
    if w != "int8":
        newk = torch.randn(S, Hkv, D, generator=gen, device=dev).to(torch.bfloat16)
        newv = torch.randn(S, Hkv, D, generator=gen, device=dev).to(torch.bfloat16)
    pairs_h = pairs = shared = None
    shared_len = 0
    if w == "prefix":
        e = case.extra
        pairs_h = np.stack([np.full(S, e["partial"]), e["scratch"]], axis=1).astype(np.int64)
        pairs = to_dev(pairs_h)
        shared = to_dev(e["shared"].astype(np.int32))
        shared_len = len(e["shared"]) * BS
        assert np.all(case.block_tables[:, :len(e["shared"])] == e["shared"][None, :])
    total = int(np.sum(case.context_lens, dtype=np.int64))
    out = torch.empty(S, Hq, D, dtype=torch.float32, device=dev)
    ws = torch.zeros(1 << 26, dtype=torch.uint8, device=dev)

    # the oracle: the step's copy, its write of each newest token, its decode
    say("workload", w, "oracle")
    kh, vh = case.k_cache.copy(), case.v_cache.copy()
    if pairs_h is not None:
        oracle.copy_blocks(kh, vh, pairs_h)
    if newk is not None:
        slots = oracle.slot_mapping(case.block_tables, case.context_lens - 1, BS)
        oracle.reshape_and_cache(to_host(newk), to_host(newv), kh, vh, slots)
    expect = oracle.paged_decode(case.q, kh, vh, case.block_tables, case.context_lens, float(case.scale),
                                 case.k_scales, case.v_scales)

    def prepare(stream):
        calls = []
        if pairs is not None:
            calls.append(pa.prepare_copy_blocks(d["k"], d["v"], pairs, stream=stream))
        calls.append(pa.PreparedDecode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale),
                                       case.max_context_len, out, k_scales=d["ks"], v_scales=d["vs"], workspace=ws,
                                       stream=stream, new_key=newk, new_value=newv, total_context_len=total,
                                       shared_prefix_table=shared, shared_prefix_len=shared_len))
        return calls

    def check(tag):
        assert np.array_equal(to_host(d["k"]), kh) and np.array_equal(to_host(d["v"]), vh), (tag, w, "cache")
        got = out.cpu().numpy().astype(np.float64)
        err = max_err(got, expect)
        gerr = guard_err(got, expect, case.context_lens)
        say(tag, w, "max |gpu - oracle| = %.3e, on long rows %.3e" % (err, gerr))
        assert err <= TOL_BF16, (tag, w, err)
        assert gerr <= GUARD_BF16, (tag, w, gerr)

    main = torch.cuda.current_stream()
    say("workload", w, "eager")
    for f in prepare(main):
        f()
    torch.cuda.synchronize()
    check("eager")
    eager = out.clone()

    cap = torch.cuda.Stream()
    cap.wait_stream(main)
    calls = prepare(cap)
    graph = torch.cuda.CUDAGraph()
    say("workload", w, "graph capture")
    with torch.cuda.graph(graph, stream=cap):
        for f in calls:
            f()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        say("workload", w, "replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), ("replay", rep)
    check("replayed")
