"""The 70B-shaped workload in the exact form the benchmark times, against
the CPU oracle.

Two of the 80 layers (the first and the last) are built with the
benchmark's own step function (`bench.llama70b_prepare`): per layer one
pa_decode call that writes each sequence's newest token into its slot and
attends over all 8,000 tokens, with the batch's total length as the
partition hint, captured once as a HIP graph on a side stream and
replayed.  Checked on all 20 sequences x 64 query heads x 128 values:

* the cache after the step equals, bit for bit over the whole pool, the
  original cache with the oracle's slot mapping and cache write applied;
* the eager step and every graph replay give the same bytes, each within
  2e-3 of the fp64 oracle run on the written cache (parity), and within
  the long-context regression guard (a dropped tile would breach it).

Replays are separated by the program's own eager work and synchronisations
(a graph must give the eager result on every replay, not just the first)."""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from gpu_helpers import GUARD_BF16, TOL_BF16, max_err, say, to_host

pytestmark = pytest.mark.gpu

LAYERS = (0, 79)


def test_config3_benchmark_call_all_sequences():
    c = synth.CFG3
    st = synth.config3_structure()
    S, Hq, Hkv, D, BS, ctx = c["num_seqs"], c["num_q_heads"], c["num_kv_heads"], c["head_dim"], c["block_size"], \
        c["context_len"]
    scale = float(st["scale"])
    dev = torch.device("cuda:0")
    Q, K, V, KN, VN, K0, V0 = [], [], [], [], [], [], []
    for layer in LAYERS:
        say("config3 layer", layer, "generation")
        q, k, v, kn, vn = synth.config3_layer_values(layer, dev)
        Q.append(q)
        K.append(k)
        V.append(v)
        KN.append(kn)
        VN.append(vn)
        K0.append(to_host(k))
        V0.append(to_host(v))
    bt = torch.from_numpy(st["block_tables"]).to(dev)
    cl = torch.from_numpy(st["context_lens"]).to(dev)
    outs = [torch.empty(S, Hq, D, dtype=torch.float32, device=dev) for _ in LAYERS]
    slots = torch.empty(S, dtype=torch.int64, device=dev)
    ws = torch.empty(1 << 24, dtype=torch.uint8, device=dev)
    total = int(st["context_lens"].sum())

    def prepare(stream):
        return bench.llama70b_prepare(stream, Q, K, V, KN, VN, bt, cl, outs, ws, slots, total, scale, ctx, BS,
                                      fused=True, partition_tokens=0)

    # the oracle's write on the original bytes, then its attention
    exp_slots = oracle.slot_mapping(st["block_tables"], st["context_lens"] - 1, BS)
    expect, k_after, v_after = [], [], []
    for i, layer in enumerate(LAYERS):
        kh, vh = K0[i].copy(), V0[i].copy()
        oracle.reshape_and_cache(to_host(KN[i]), to_host(VN[i]), kh, vh, exp_slots)
        k_after.append(kh)
        v_after.append(vh)
        say("config3 layer", layer, "oracle")
        expect.append(oracle.paged_decode(to_host(Q[i]), kh, vh, st["block_tables"], st["context_lens"], scale))

    def check(tag):
        for i, layer in enumerate(LAYERS):
            got = outs[i].cpu().numpy().astype(np.float64)
            err = max_err(got, expect[i])
            say(tag, "layer", layer, "max |gpu - oracle| = %.3e" % err)
            assert err <= TOL_BF16, (tag, layer, err)
            assert err <= GUARD_BF16, (tag, layer, err)

    main = torch.cuda.current_stream()
    pre, layers = prepare(main)
    assert not pre and all(not w for w, _ in layers)          # the fused form: one call per layer
    say("config3 eager step")
    for _, d in layers:
        d()
    torch.cuda.synchronize()
    for i, layer in enumerate(LAYERS):
        assert np.array_equal(to_host(K[i]), k_after[i]), ("K cache after the write", layer)
        assert np.array_equal(to_host(V[i]), v_after[i]), ("V cache after the write", layer)
    check("eager")
    eager = [o.clone() for o in outs]

    cap = torch.cuda.Stream()
    cap.wait_stream(main)
    _, glayers = prepare(cap)
    graph = torch.cuda.CUDAGraph()
    say("config3 graph capture")
    with torch.cuda.graph(graph, stream=cap):
        for _, d in glayers:
            d()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))                               # eager work between replays
        torch.cuda.synchronize()
        say("config3 graph replay", rep)
        graph.replay()
        torch.cuda.synchronize()
        for i in range(len(LAYERS)):
            assert torch.equal(outs[i], eager[i]), ("replay differs from the eager step", rep, LAYERS[i])
        check("replay %d" % rep)
    for i, layer in enumerate(LAYERS):
        assert np.array_equal(to_host(K[i]), k_after[i]), ("K cache after the replays", layer)
        assert np.array_equal(to_host(V[i]), v_after[i]), ("V cache after the replays", layer)
