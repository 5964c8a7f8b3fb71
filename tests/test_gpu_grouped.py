"""Grouped launches of the matrix-core kernel on the GPU against the CPU
oracle.  With one column group per (sequence, kv head) item, 2 to 8
partitions and at least 256 items, the plan runs the partitions of an item
as the waves of one workgroup (2, 4 or 8 waves) and combines them through
LDS: no partials, no merge launch, no workspace.  Lengths around tile and
partition edges leave some waves of a workgroup with nothing to attend
to; they still take part in the combination with no weight.

The oracle knows nothing of partitions: the result must be the attention
over each sequence's table.  Tolerance max |gpu - oracle| <= 2e-3 (bf16,
int8 or E4M3 cache, fp32 accumulation); fused cache writes bit-exact;
single-row query offsets give the decode result bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import (TOL_BF16, case_on_device, max_err, quantize_case, quantize_case_by_token, run_oracle, say,
                         to_dev, to_host)

pytestmark = pytest.mark.gpu

# 16 edge lengths (empty, one token, tile and partition edges) and 16 seeded
# ones up to 1,200; with 8 or 16 kv heads, 256 (sequence, kv head) items
EDGES = [0, 1, 15, 16, 17, 127, 128, 129, 255, 256, 257, 511, 512, 513, 1023, 1024]


def _lens(seed, S):
    rng = np.random.default_rng(seed)
    extra = [int(x) for x in rng.integers(1, 1201, size=S - len(EDGES))]
    return EDGES + extra[:-1] + [1200]


# partition sizes for max length 1,200: 0 = automatic (re-cut into 4 for
# the bf16 wave target), 160 -> 8 partitions, 256 -> 5 of 8 waves, 512 -> 3
# of 4, 608 -> 2 of 2
PARTS = (0, 160, 256, 512, 608)


def _grouped(case, d, P, **kw):
    """The plan for this call is grouped: no workspace needed."""
    a = pa.make_decode_args(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                            k_scales=d["ks"], v_scales=d["vs"], partition_tokens=P, **kw)
    return pa.decode_workspace_size(a) == 0


SHAPES = [
    # (S, Hq, Hkv, BS)
    (32, 64, 8, 16),    # 8 query heads per kv head
    (32, 32, 8, 32),    # 4, blocks of 32
    (32, 8, 8, 16),     # 1 (MHA)
    (16, 256, 16, 16),  # 16: every MFMA column
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "S%d-Hq%d-Hkv%d-BS%d" % s)
def test_grouped_decode_matches_oracle(shape):
    S, Hq, Hkv, BS = shape
    case = synth.make_case("grouped", 900 + SHAPES.index(shape), _lens(31 + S, S), Hq, Hkv, 128, BS, free_frac=0.1)
    expect = run_oracle(case)
    d = case_on_device(case)
    for P in PARTS:
        assert _grouped(case, d, P), (shape, P)
        say("grouped decode", shape, "partition", P)
        out = pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                        partition_tokens=P)
        torch.cuda.synchronize()
        err = max_err(out.cpu().numpy().astype(np.float64), expect)
        assert err <= TOL_BF16, (shape, P, err)
    # the same batch with more partitions than a workgroup takes (partials
    # and the merge) agrees with the grouped result to the same tolerance
    assert not _grouped(case, d, 64)
    out = pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                    partition_tokens=64)
    torch.cuda.synchronize()
    assert max_err(out.cpu().numpy().astype(np.float64), expect) <= TOL_BF16


@pytest.mark.parametrize("kv", [synth.BF16, synth.I8])
def test_short_ragged_batch_regrouped(kv):
    """A short ragged batch with the length hint: the automatic split asks
    for more than 8 short partitions, and the plan re-cuts it into 4-wave
    groups (no workspace) when the longest sequence has at most 128 tiles."""
    S, Hq, Hkv, BS = 32, 32, 8, 16
    rng = np.random.default_rng(17)
    lens = [0, 1, 15, 16, 17, 63, 64, 65] + [int(x) for x in rng.integers(50, 1001, size=S - 9)] + [1000]
    case = synth.make_case("grouped-short", 950, lens, Hq, Hkv, 128, BS, kv_dtype=kv, free_frac=0.1)
    if kv == synth.I8:
        quantize_case(case)
    expect = oracle.paged_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                 float(case.scale), case.k_scales, case.v_scales)
    d = case_on_device(case)
    total = int(np.sum(case.context_lens, dtype=np.int64))
    assert _grouped(case, d, 0, total_context_len=total)
    assert not _grouped(case, d, 64, total_context_len=total)
    for P in (0, 64):
        say("short ragged batch", kv, "partition", P)
        out = pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                        k_scales=d["ks"], v_scales=d["vs"], partition_tokens=P, total_context_len=total)
        torch.cuda.synchronize()
        err = max_err(out.cpu().numpy().astype(np.float64), expect)
        assert err <= TOL_BF16, (kv, P, err)


def test_fewer_items_than_compute_units_are_not_grouped():
    """160 items (20 sequences x 8 kv heads, the 70B-shaped batch) keep the
    partials and the merge: a workgroup per item would leave compute units
    idle."""
    case = synth.make_case("ungrouped", 77, [1200] * 20, 64, 8, 128, 16)
    d = case_on_device(case)
    assert not _grouped(case, d, 0)


def test_grouped_fused_cache_write():
    """The newest token's K/V written by the wave whose partition holds it
    (in any of a workgroup's waves): caches bit-identical to the oracle's
    write, outputs bit-identical to the separate write + decode and within
    tolerance of the oracle."""
    S, Hq, Hkv, BS = 32, 64, 8, 16
    lens = _lens(5, S)
    case = synth.make_case("grouped-fused", 910, lens, Hq, Hkv, 128, BS, free_frac=0.1)
    rng = np.random.default_rng(11)
    nk = synth.bf16_bits(rng.standard_normal((S, Hkv, 128), dtype=np.float32))
    nv = synth.bf16_bits(rng.standard_normal((S, Hkv, 128), dtype=np.float32))
    slots = oracle.slot_mapping(case.block_tables, case.context_lens - 1, BS)
    exp_k, exp_v = case.k_cache.copy(), case.v_cache.copy()
    oracle.reshape_and_cache(nk, nv, exp_k, exp_v, slots)
    updated = synth.make_case("grouped-fused", 910, lens, Hq, Hkv, 128, BS, free_frac=0.1)
    updated.k_cache, updated.v_cache = exp_k, exp_v
    expect = run_oracle(updated)
    dnk, dnv = to_dev(nk), to_dev(nv)
    for P in (0, 160, 512):
        say("grouped fused write, partition", P)
        a = case_on_device(case)
        assert _grouped(case, a, P, new_key=dnk, new_value=dnv)
        sl = pa.slot_mapping(a["bt"], BS, context_lens=a["cl"])
        pa.reshape_and_cache(dnk, dnv, a["k"], a["v"], sl)
        out_a = pa.decode(a["q"], a["k"], a["v"], a["bt"], a["cl"], float(case.scale), case.max_context_len,
                          partition_tokens=P)
        b = case_on_device(case)
        out_b = pa.decode(b["q"], b["k"], b["v"], b["bt"], b["cl"], float(case.scale), case.max_context_len,
                          partition_tokens=P, new_key=dnk, new_value=dnv)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(b["k"]), exp_k)
        assert np.array_equal(to_host(b["v"]), exp_v)
        ob = out_b.cpu().numpy().astype(np.float64)
        assert np.array_equal(out_a.cpu().numpy().astype(np.float64), ob), P
        err = max_err(ob, expect)
        assert err <= TOL_BF16, (P, err)


@pytest.mark.parametrize("kv,mode", [(synth.I8, pa.PA_SCALE_BLOCK), (synth.I8, pa.PA_SCALE_TOKEN),
                                     (synth.FP8, pa.PA_SCALE_TOKEN), (synth.FP8, pa.PA_SCALE_BLOCK)])
def test_grouped_quantised(kv, mode):
    """1-byte caches in a grouped launch (given partition sizes: the
    automatic split of a 1-byte cache targets more waves than a workgroup
    holds)."""
    S, Hq, Hkv, BS = 32, 32, 8, 16
    case = synth.make_case("grouped-q", 920, _lens(9, S), Hq, Hkv, 128, BS, kv_dtype=kv, free_frac=0.1)
    if kv == synth.I8 and mode == pa.PA_SCALE_BLOCK:
        quantize_case(case)
    else:
        quantize_case_by_token(case, mode)
    expect = oracle.paged_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                 float(case.scale), case.k_scales, case.v_scales, scale_mode=mode)
    d = case_on_device(case)
    for P in (160, 256, 608):
        assert _grouped(case, d, P), (kv, mode, P)
        say("grouped quantised", kv, mode, "partition", P)
        out = pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                        k_scales=d["ks"], v_scales=d["vs"], partition_tokens=P)
        torch.cuda.synchronize()
        err = max_err(out.cpu().numpy().astype(np.float64), expect)
        assert err <= TOL_BF16, (kv, mode, P, err)


def test_grouped_multi_query():
    """Query offsets with one column group per item (one row: bit for bit
    the decode result; two rows of 8 heads: against the oracle's causal
    attention) run grouped too."""
    S, Hq, Hkv, BS = 32, 64, 8, 16
    case = synth.make_case("grouped-mq", 930, _lens(13, S), Hq, Hkv, 128, BS, free_frac=0.1)
    d = case_on_device(case)
    one = to_dev(np.arange(S + 1, dtype=np.int32))
    for P in (0, 256):
        say("grouped single-row query offsets, partition", P)
        assert _grouped(case, d, P, query_start_loc=one, max_query_len=1)
        a = pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                      partition_tokens=P)
        b = pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                      partition_tokens=P, query_start_loc=one, max_query_len=1)
        torch.cuda.synchronize()
        assert torch.equal(a, b), P
    # two rows per sequence (one for the empty and one-token sequences)
    qlens = [min(2, int(n)) for n in case.context_lens]
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    rng = np.random.default_rng(14)
    q = synth.bf16_bits(rng.standard_normal((int(qsl[-1]), Hq, 128)).astype(np.float32))
    expect = oracle.paged_attention(q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, qsl,
                                    float(case.scale))
    dq, dqsl = to_dev(q), to_dev(qsl)
    for P in (0, 160, 512):
        say("grouped two-row queries, partition", P)
        assert _grouped(case, dict(d, q=dq), P, query_start_loc=dqsl, max_query_len=2)
        out = pa.decode(dq, d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                        partition_tokens=P, query_start_loc=dqsl, max_query_len=2)
        torch.cuda.synchronize()
        err = max_err(out.cpu().numpy().astype(np.float64), expect)
        assert err <= TOL_BF16, (P, err)


def test_grouped_deterministic_and_permutation_invariant():
    """Two runs give the same bits; renaming the physical blocks (the same
    tokens in other blocks of a larger pool) gives the same bits."""
    S, Hq, Hkv, BS = 32, 64, 8, 16
    case = synth.make_case("grouped-det", 940, _lens(21, S), Hq, Hkv, 128, BS, free_frac=0.3)
    d = case_on_device(case)
    outs = []
    for _ in range(2):
        outs.append(pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len))
    # move every used block to a new id
    NB = case.k_cache.shape[0]
    rng = np.random.default_rng(3)
    perm = rng.permutation(NB)
    k2, v2 = np.empty_like(case.k_cache), np.empty_like(case.v_cache)
    k2[perm] = case.k_cache
    v2[perm] = case.v_cache
    bt2 = np.where(case.block_tables >= 0, perm[np.maximum(case.block_tables, 0)], case.block_tables).astype(np.int32)
    out2 = pa.decode(d["q"], to_dev(k2), to_dev(v2), to_dev(bt2), d["cl"], float(case.scale), case.max_context_len)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(outs[0], out2)
