"""The 70B-shaped batch at head_dim 64 at full size and in the call form the
benchmark times (its gqa-d64 and int8-d64 workloads), against the CPU
oracle.

20 sequences x 8,000 tokens, 64 query / 8 KV heads, blocks of 16, a pool
of 10,000 blocks; one prepared pa_decode call with the batch's total length
as the split hint -- over a bf16 cache with the newest token's K/V written
by the call itself, or over int8 codes with per-(block, head) scales --
captured once as a HIP graph on a side stream and replayed.

Gates: all 20 sequences' outputs within 2e-3 of the oracle and within the
2e-5 regression guard (every row sees 8,000 tokens); for bf16 the cache
after the call equals the oracle's write bit for bit; the eager call and
every replay give the same bytes.  Values have unit spread (bf16 N(0, 1);
int8 codes times scales near 1/73), the spread the guard is pinned for."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import GUARD_BF16, TOL_BF16, max_err, say, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["bf16", "i8"])
def test_head_dim64_batch_in_the_benchmark_call_form(kv):
    st = synth.config3_structure()
    c = synth.CFG3
    S, Hq, Hkv, BS, D = c["num_seqs"], c["num_q_heads"], c["num_kv_heads"], c["block_size"], 64
    NB = st["num_blocks"]
    ctx = int(st["context_lens"][0])
    total = int(np.sum(st["context_lens"], dtype=np.int64))
    scale = 1.0 / math.sqrt(D)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(6400 + (kv == "i8"))
    shape = (NB, Hkv, BS, D)
    say("head_dim 64 batch", kv, "generation")
    ks = vs = newk = newv = None
    if kv == "i8":
        k = torch.randint(-127, 128, shape, generator=gen, dtype=torch.int8, device=dev)
        v = torch.randint(-127, 128, shape, generator=gen, dtype=torch.int8, device=dev)
        ks = (torch.rand(NB, Hkv, generator=gen, device=dev) * 0.4 + 0.8) / 73.0
        vs = (torch.rand(NB, Hkv, generator=gen, device=dev) * 0.4 + 0.8) / 73.0
    else:
        k = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
        newk = torch.randn(S, Hkv, D, generator=gen, device=dev).to(torch.bfloat16)
        newv = torch.randn(S, Hkv, D, generator=gen, device=dev).to(torch.bfloat16)
    q = torch.randn(S, Hq, D, generator=gen, device=dev).to(torch.bfloat16)
    bt = torch.from_numpy(st["block_tables"]).to(dev)
    cl = torch.from_numpy(st["context_lens"]).to(dev)
    out = torch.empty(S, Hq, D, dtype=torch.float32, device=dev)
    ws = torch.empty(1 << 26, dtype=torch.uint8, device=dev)

    # the oracle on the device bytes, after its own write of each newest token
    kh, vh, qh = to_host(k), to_host(v), to_host(q)
    ksh = None if ks is None else to_host(ks)
    vsh = None if vs is None else to_host(vs)
    if newk is not None:
        slots = oracle.slot_mapping(st["block_tables"], st["context_lens"] - 1, BS)
        oracle.reshape_and_cache(to_host(newk), to_host(newv), kh, vh, slots)
    say("head_dim 64 batch", kv, "oracle")
    expect = oracle.paged_decode(qh, kh, vh, st["block_tables"], st["context_lens"], scale, ksh, vsh)

    def prepare(stream):
        return pa.PreparedDecode(q, k, v, bt, cl, scale, ctx, out, k_scales=ks, v_scales=vs, workspace=ws,
                                 stream=stream, new_key=newk, new_value=newv, total_context_len=total)

    def check(tag):
        got = out.cpu().numpy().astype(np.float64)
        err = max_err(got, expect)
        say(tag, kv, "max |gpu - oracle| = %.3e" % err)
        assert err <= TOL_BF16, (tag, kv, err)
        assert err <= GUARD_BF16, (tag, kv, err)
        if newk is not None:
            assert np.array_equal(to_host(k), kh) and np.array_equal(to_host(v), vh), (tag, "cache")

    main = torch.cuda.current_stream()
    say("head_dim 64 batch", kv, "eager")
    prepare(main)()
    torch.cuda.synchronize()
    check("eager")
    eager = out.clone()

    cap = torch.cuda.Stream()
    cap.wait_stream(main)
    call = prepare(cap)
    graph = torch.cuda.CUDAGraph()
    say("head_dim 64 batch", kv, "graph capture")
    with torch.cuda.graph(graph, stream=cap):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        say("head_dim 64 batch", kv, "replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), ("replay", rep)
    check("replayed")
