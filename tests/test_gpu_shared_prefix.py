"""Paged decode with a shared prefix (the cascade path: the prefix's blocks
read once for the whole batch, every sequence's own tokens after them) on
the GPU against the CPU oracle, which knows nothing of the prefix: the
result must be the attention over each sequence's table.

Tolerance: max |gpu - oracle| <= 2e-3 (bf16, int8 or E4M3 inputs, fp32
accumulation); the fused cache write bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import TOL_BF16, case_on_device, max_err, quantize_case_by_token, run_oracle, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _shared_case(name, seed, lens, Hq, Hkv, BS, prefix_blocks, kv_dtype=synth.BF16):
    """A seeded batch whose table rows all start with the first
    prefix_blocks blocks of row 0 (lens[0] covers them)."""
    assert lens[0] >= prefix_blocks * BS
    case = synth.make_case(name, seed, lens, Hq, Hkv, 128, BS, kv_dtype=kv_dtype, free_frac=0.1)
    case.block_tables[:, :prefix_blocks] = case.block_tables[0, :prefix_blocks]
    return case


def _run(case, dev, prefix_blocks, partition_tokens=0, hint=False, new=None, kernel=0):
    BS = case.block_size
    table = to_dev(np.ascontiguousarray(case.block_tables[0, :prefix_blocks]))
    total = int(np.sum(case.context_lens, dtype=np.int64)) if hint else 0
    nk, nv = (None, None) if new is None else new
    out = pa.decode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale), case.max_context_len,
                    k_scales=dev["ks"], v_scales=dev["vs"], partition_tokens=partition_tokens,
                    total_context_len=total, shared_prefix_table=table, shared_prefix_len=prefix_blocks * BS,
                    new_key=nk, new_value=nv, kernel=kernel)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


# (Hq, Hkv, BS, prefix blocks): GQA groups of 4 and 8, MHA-like 1, blocks of 16 and 32
SHAPES = [(32, 8, 32, 5), (16, 2, 16, 9), (64, 8, 16, 4), (8, 8, 16, 3)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "hq%d_hkv%d_bs%d_pb%d" % s)
def test_shared_prefix_matches_oracle(shape):
    """Lengths around the prefix's end (shorter than it, equal, one past,
    a block past) and long ones, with automatic and given partitions (the
    prefix and the rest split alike: one tile, a few tiles, one block)."""
    Hq, Hkv, BS, pb = shape
    L = pb * BS
    lens = [L + 700, 0, 1, L - 1, L, L + 1, L + BS, L + 3 * BS + 5, L + 250, 2, L + 61, L + 999, L // 2]
    case = _shared_case("prefix_%d_%d_%d" % (Hq, Hkv, BS), 17 + Hq + BS, lens, Hq, Hkv, BS, pb)
    expect = run_oracle(case)
    dev = case_on_device(case)
    for P in (0, 16, 64, BS * 4):
        for hint in ((False, True) if P == 0 else (False,)):
            say("shared prefix", shape, "partition", P, "hint", hint)
            err = max_err(_run(case, dev, pb, P, hint), expect)
            assert err <= TOL_BF16, (shape, P, hint, err)


def test_shared_prefix_many_sequences():
    """200 sequences x 8 heads per kv head: 100 column groups over the
    prefix, ragged lengths after it."""
    rng = np.random.default_rng(5)
    pb, BS = 6, 16
    lens = [pb * BS + 400] + [int(x) for x in rng.integers(pb * BS - 20, pb * BS + 300, size=199)]
    case = _shared_case("prefix_many", 23, lens, 64, 8, BS, pb)
    expect = run_oracle(case)
    dev = case_on_device(case)
    for hint in (False, True):
        say("shared prefix many sequences, hint", hint)
        err = max_err(_run(case, dev, pb, 0, hint), expect)
        assert err <= TOL_BF16, (hint, err)


def test_whole_context_shared():
    """Every sequence is the prefix (nothing after it): prefix partials only,
    or with one partition the prefix items write the output directly."""
    pb, BS = 8, 16
    case = _shared_case("prefix_only", 31, [pb * BS] * 6, 32, 8, BS, pb)
    expect = run_oracle(case)
    dev = case_on_device(case)
    for P in (0, 32, pb * BS):
        say("whole context shared, partition", P)
        err = max_err(_run(case, dev, pb, P), expect)
        assert err <= TOL_BF16, (P, err)


@pytest.mark.parametrize("kv,mode", [(synth.I8, pa.PA_SCALE_TOKEN), (synth.FP8, pa.PA_SCALE_BLOCK),
                                     (synth.I8, pa.PA_SCALE_BLOCK)])
def test_shared_prefix_quantised(kv, mode):
    pb, BS = 4, 32
    L = pb * BS
    lens = [L + 300, L - 7, L, L + 1, L + 40, 0, L + 129]
    case = _shared_case("prefix_q", 41, lens, 32, 8, BS, pb, kv_dtype=kv)
    quantize_case_by_token(case, mode)
    expect = oracle.paged_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                 float(case.scale), case.k_scales, case.v_scales, scale_mode=mode)
    dev = case_on_device(case)
    for P in (0, 64):
        say("shared prefix quantised", kv, mode, "partition", P)
        err = max_err(_run(case, dev, pb, P), expect)
        assert err <= TOL_BF16, (kv, mode, P, err)


def test_config4_with_shared_prefix_and_fused_write():
    """The prefix-sharing workload's step with the prefix passed: the 62
    shared full blocks as the prefix, each newest token written by the
    fused cache write (bit-exact over the pool) and attended."""
    case = synth.config4()
    e = case.extra
    dev = case_on_device(case)
    n_full = len(e["shared"])
    assert np.all(case.block_tables[:, :n_full] == e["shared"][None, :])
    say("config4 shared prefix + fused write")
    got = _run(case, dev, n_full, new=(to_dev(e["k_new"]), to_dev(e["v_new"])))
    slots = oracle.slot_mapping(case.block_tables, case.context_lens - 1, case.block_size)
    oracle.reshape_and_cache(e["k_new"], e["v_new"], case.k_cache, case.v_cache, slots)
    assert np.array_equal(to_host(dev["k"]), case.k_cache)
    assert np.array_equal(to_host(dev["v"]), case.v_cache)
    err = max_err(got, run_oracle(case))
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("kernel", [0, pa.KERNEL_VALU, pa.KERNEL_MFMA])
def test_fused_write_inside_the_prefix_is_skipped(kernel):
    """A sequence whose newest token lies inside the shared prefix: its row
    is neither stored (a shared block is never written) nor attended; the
    others are written and attended as usual -- on either kernel (the
    vector-ALU kernel reads the prefix through each table row, but must
    skip the same writes)."""
    pb, BS = 4, 16
    L = pb * BS
    lens = [L + 50, L, L - 3, L + 1]
    case = _shared_case("prefix_write", 53, lens, 16, 4, BS, pb)
    rng = np.random.default_rng(9)
    k_new = synth.bf16_bits(rng.standard_normal((4, 4, 128), dtype=np.float32))
    v_new = synth.bf16_bits(rng.standard_normal((4, 4, 128), dtype=np.float32))
    dev = case_on_device(case)
    say("fused write inside the prefix, kernel", kernel)
    got = _run(case, dev, pb, new=(to_dev(k_new), to_dev(v_new)), kernel=kernel)
    written = [0, 3]                                  # sequences past the prefix
    slots = oracle.slot_mapping(case.block_tables[written], case.context_lens[written] - 1, BS)
    oracle.reshape_and_cache(k_new[written], v_new[written], case.k_cache, case.v_cache, slots)
    assert np.array_equal(to_host(dev["k"]), case.k_cache)
    assert np.array_equal(to_host(dev["v"]), case.v_cache)
    err = max_err(got, run_oracle(case))
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("kv", [synth.I8, synth.FP8])
def test_fused_quantising_write_with_a_shared_prefix(kv):
    """The fused write into a per-token-scaled 1-byte cache with a shared
    prefix: sequences whose newest token lies past the prefix get its codes
    and scales (bit for bit the oracle's quantising write) and attend with
    them; a newest token inside the prefix is neither stored nor taken from
    the new rows."""
    pb, BS = 4, 32
    L = pb * BS
    lens = [L + 300, L - 7, L, L + 1, L + 40, L + 129, 1 + L + 31]
    case = _shared_case("prefix_qwrite", 61, lens, 32, 8, BS, pb, kv_dtype=kv)
    quantize_case_by_token(case, pa.PA_SCALE_TOKEN)
    S, Hkv = case.num_seqs, case.num_kv_heads
    rng = np.random.default_rng(10)
    k_new = synth.bf16_bits(rng.standard_normal((S, Hkv, 128), dtype=np.float32))
    v_new = synth.bf16_bits(rng.standard_normal((S, Hkv, 128), dtype=np.float32))
    written = [i for i, n in enumerate(lens) if n > L]
    slots = oracle.slot_mapping(case.block_tables[written], case.context_lens[written] - 1, BS)
    exp = [a.copy() for a in (case.k_cache, case.v_cache, case.k_scales, case.v_scales)]
    oracle.quantize_and_cache(k_new[written], v_new[written], *exp, slots, pa.PA_SCALE_TOKEN, 0.0, 0.0)
    expect = oracle.paged_decode(case.q, exp[0], exp[1], case.block_tables, case.context_lens, float(case.scale),
                                 exp[2], exp[3], scale_mode=pa.PA_SCALE_TOKEN)
    for P in (0, 64):
        dev = case_on_device(case)
        say("fused quantising write with a shared prefix", kv, "partition", P)
        got = _run(case, dev, pb, P, new=(to_dev(k_new), to_dev(v_new)))
        for key, want in zip(("k", "v", "ks", "vs"), exp):
            assert np.array_equal(to_host(dev[key]), want), (kv, P, key)
        err = max_err(got, expect)
        assert err <= TOL_BF16, (kv, P, err)
