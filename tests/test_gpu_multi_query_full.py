"""Several query rows per sequence at the full 70B-shaped size, in the call
form the benchmark times (one prepared pa_decode call per layer with
query offsets, the library's own split, captured once as a HIP graph on a
side stream and replayed), against the CPU oracle on sampled sequences.

Workloads: 4 causal rows per sequence over a bf16 cache (checking drafted
tokens: two column groups per wave), 64 rows (a prefill chunk: the
shared-tile kernel) over a bf16 cache and over int8 codes with
per-(block, head) scales.  The 20 sequences x 8,000 tokens share one pool;
the oracle recomputes the first and the last sequence, every row and
head, from the same bytes.  Gates: 2e-3 (parity) and the long-context
regression guard 2e-5 (every row sees at least 7,937 tokens, so a dropped
tile or partial would breach it); the eager call and every replay give
the same bytes.  Values have unit spread (bf16 N(0, 1); int8 codes times
scales near 1/73), the spread the guard is pinned for: it bounds an
absolute error, which grows with the values' magnitude."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import GUARD_BF16, TOL_BF16, max_err, say, to_host

pytestmark = pytest.mark.gpu

SAMPLED = (0, 19)


@pytest.mark.parametrize("rows,kv", [(4, "bf16"), (64, "bf16"), (64, "i8")])
def test_full_size_query_rows_in_the_benchmark_call_form(rows, kv):
    c = synth.CFG3
    st = synth.config3_structure()
    S, Hq, Hkv, D, BS = c["num_seqs"], c["num_q_heads"], c["num_kv_heads"], c["head_dim"], c["block_size"]
    NB = st["num_blocks"]
    ctx = int(st["context_lens"][0])
    scale = float(st["scale"])
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 + rows)
    say("full-size query rows", rows, kv, "generation")
    ks = vs = None
    if kv == "i8":
        shape = (NB, Hkv, BS, D)
        k = torch.randint(-127, 128, shape, generator=gen, dtype=torch.int8, device=dev)
        v = torch.randint(-127, 128, shape, generator=gen, dtype=torch.int8, device=dev)
        # scales around 1/73 give the values unit spread (uniform codes in
        # [-127, 127] have standard deviation ~73), the spread the guard is
        # pinned for
        ks = (torch.rand(NB, Hkv, generator=gen, device=dev) * 0.4 + 0.8) / 73.0
        vs = (torch.rand(NB, Hkv, generator=gen, device=dev) * 0.4 + 0.8) / 73.0
    else:
        _, k, v, _, _ = synth.config3_layer_values(rows, dev)
    q = torch.randn(S * rows, Hq, D, generator=gen, device=dev).to(torch.bfloat16)
    qsl = torch.arange(0, S * rows + 1, rows, dtype=torch.int32, device=dev)
    bt = torch.from_numpy(st["block_tables"]).to(dev)
    cl = torch.from_numpy(st["context_lens"]).to(dev)
    out = torch.empty(S * rows, Hq, D, dtype=torch.float32, device=dev)
    ws = torch.empty(1 << 28, dtype=torch.uint8, device=dev)

    def prepare(stream):
        return pa.PreparedDecode(q, k, v, bt, cl, scale, ctx, out, k_scales=ks, v_scales=vs, workspace=ws,
                                 stream=stream, query_start_loc=qsl, max_query_len=rows)

    # the oracle on the sampled sequences, from the device bytes
    kh, vh, qh = to_host(k), to_host(v), to_host(q)
    ksh = None if ks is None else to_host(ks)
    vsh = None if vs is None else to_host(vs)
    sel = np.concatenate([np.arange(s * rows, (s + 1) * rows) for s in SAMPLED])
    sub_qsl = np.arange(0, len(SAMPLED) * rows + 1, rows, dtype=np.int32)
    say("full-size query rows", rows, kv, "oracle")
    expect = oracle.paged_attention(qh[sel], kh, vh, st["block_tables"][list(SAMPLED)],
                                    st["context_lens"][list(SAMPLED)], sub_qsl, scale, ksh, vsh)

    def check(tag):
        got = out.cpu().numpy().astype(np.float64)[sel]
        err = max_err(got, expect)
        say(tag, "max |gpu - oracle| = %.3e" % err)
        assert err <= TOL_BF16, (tag, rows, kv, err)
        assert err <= GUARD_BF16, (tag, rows, kv, err)

    main = torch.cuda.current_stream()
    say("full-size query rows", rows, kv, "eager")
    prepare(main)()
    torch.cuda.synchronize()
    check("eager")
    eager = out.clone()

    cap = torch.cuda.Stream()
    cap.wait_stream(main)
    call = prepare(cap)
    graph = torch.cuda.CUDAGraph()
    say("full-size query rows", rows, kv, "graph capture")
    with torch.cuda.graph(graph, stream=cap):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        say("full-size query rows", rows, kv, "replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), ("replay", rep)
    check("replayed")
