"""GPU parity of paged attention with several causal query rows per
sequence (chunked prefill, checking drafted tokens) against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import TOL_BF16, case_on_device, max_err, quantize_case_by_token, say, to_dev

pytestmark = pytest.mark.gpu

MQ_SHAPES = [
    # (Hq, Hkv, BS, kv dtype, scale mode)
    (64, 8, 16, synth.BF16, None),
    (32, 8, 32, synth.BF16, None),
    (40, 40, 16, synth.BF16, None),
    (12, 4, 16, synth.BF16, None),
    (32, 8, 16, synth.I8, pa.PA_SCALE_TOKEN),
    (64, 8, 16, synth.FP8, pa.PA_SCALE_TOKEN),
    (32, 8, 32, synth.FP8, pa.PA_SCALE_BLOCK),
    (64, 8, 32, synth.I8, pa.PA_SCALE_BLOCK),
]
# (context length, query rows): decode rows, drafted tokens, prefill chunks,
# a whole-sequence prefill, and rows that see nothing (more rows than tokens)
BATCH = [(1, 1), (17, 2), (100, 4), (257, 7), (1000, 16), (33, 33), (600, 64), (0, 0), (5, 0), (3, 5)]


def _mq_case(shape, seed):
    Hq, Hkv, BS, kvd, mode = shape
    lens = [n for n, _ in BATCH]
    qlens = [L for _, L in BATCH]
    case = synth.make_case("mq", seed, lens, Hq, Hkv, 128, BS, kv_dtype=kvd, free_frac=0.2)
    if kvd in (synth.I8, synth.FP8):
        quantize_case_by_token(case, mode)
    rng = np.random.default_rng(seed + 1)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = synth.bf16_bits(rng.standard_normal((int(qsl[-1]), Hq, 128)).astype(np.float32))
    return case, q, qsl, max(qlens)


@pytest.mark.parametrize("shape", MQ_SHAPES, ids=lambda s: "Hq%d-Hkv%d-BS%d-%s-%s" % s)
def test_multi_query_parity(shape):
    case, q, qsl, maxq = _mq_case(shape, 500 + MQ_SHAPES.index(shape))
    mode = shape[4] if shape[4] is not None else pa.PA_SCALE_BLOCK
    expect = oracle.paged_attention(q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, qsl,
                                    float(case.scale), case.k_scales, case.v_scales, scale_mode=mode)
    d = case_on_device(case)
    dq, dqsl = to_dev(q), to_dev(qsl)
    for P in (0, 16, 256, 2048):
        say("multi-query", shape, "partition", P)
        out = pa.decode(dq, d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                        k_scales=d["ks"], v_scales=d["vs"], partition_tokens=P, query_start_loc=dqsl,
                        max_query_len=maxq)
        torch.cuda.synchronize()
        err = max_err(out.cpu().numpy().astype(np.float64), expect)
        assert err <= TOL_BF16, (shape, P, err)


def test_single_row_queries_match_decode():
    """query_start_loc = 0, 1, ..., S gives exactly the decode path's result."""
    case = synth.config4()
    d = case_on_device(case)
    qsl = np.arange(case.num_seqs + 1, dtype=np.int32)
    for P in (0, 256):
        say("single-row multi-query vs decode, partition", P)
        a = pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                      partition_tokens=P)
        b = pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                      partition_tokens=P, query_start_loc=to_dev(qsl), max_query_len=1)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_offsets_past_num_queries_touch_nothing_outside():
    """query_start_loc ending past num_queries (a caller error): rows beyond
    num_queries are skipped, so memory after q and out is never touched
    (both are views into larger buffers holding sentinels), and the rows
    inside still equal the oracle's."""
    case, q, qsl, maxq = _mq_case(MQ_SHAPES[0], 520)
    R = int(qsl[-1])
    keep = R - 5                                  # the call is told only keep rows exist
    d = case_on_device(case)
    q_big = to_dev(q)
    out_big = torch.full((R, case.num_q_heads, 128), 7.0, dtype=torch.float32, device="cuda:0")
    say("multi-query offsets past num_queries")
    pa.decode(q_big[:keep], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
              out=out_big[:keep], partition_tokens=256, query_start_loc=to_dev(qsl), max_query_len=maxq)
    torch.cuda.synchronize()
    got = out_big.cpu().numpy().astype(np.float64)
    assert np.all(got[keep:] == 7.0)
    expect = oracle.paged_attention(q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, qsl,
                                    float(case.scale))
    assert max_err(got[:keep], expect[:keep]) <= TOL_BF16
