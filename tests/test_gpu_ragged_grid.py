"""Ragged decode batches (log-normal lengths, a few empty sequences, one
long one) under the plans the length hint selects -- the balanced split
(each kv head's tiles cut into equal ranges over the sequences, up to 1,024
sequences: four register chunks of lengths up to 256, sixteen past that),
short partitions, long ones: the result must not depend on the
hint's value, which only shapes the split.  Checked
against the CPU oracle, max |gpu - oracle| <= 2e-3 (bf16, int8 or E4M3
inputs), and the rows of sequences of 2,048 tokens or more within the
regression guard (a lost tile or partial breaches it); the fused cache
write bit-exact."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import GUARD_BF16, TOL_BF16, case_on_device, guard_err, max_err, quantize_case_by_token, run_oracle, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _lognormal(seed, n, median, lo=0, hi=6000):
    rng = np.random.default_rng(seed)
    x = np.rint(rng.lognormal(math.log(median), 1.0, size=n)).astype(np.int64)
    x[rng.random(n) < 0.05] = 0                      # a few empty sequences
    return np.clip(x, lo, hi).astype(np.int32)


def _decode(case, dev, total, P=0, new=None):
    nk, nv = (None, None) if new is None else new
    out = pa.decode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale), case.max_context_len,
                    k_scales=dev["ks"], v_scales=dev["vs"], partition_tokens=P, total_context_len=int(total),
                    new_key=nk, new_value=nv)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("S", [7, 64, 200, 256, 257, 640, 1024, 1025])
def test_ragged_grid_any_hint(S):
    """The exact total (the balanced split, wide past 256 sequences; short
    partitions past 1,024), a quarter of it (a hint below the truth: longer ranges than
    the hint suggests) and the near-uniform bound (long partitions)."""
    lens = _lognormal(S, S, 300)
    lens[0] = max(int(lens.max()), 1500)             # one long sequence: most of its partitions' peers empty
    case = synth.make_case("ragged_%d" % S, 100 + S, lens, 32, 8, 128, 16, free_frac=0.05)
    expect = run_oracle(case)
    dev = case_on_device(case)
    total = int(lens.sum())
    for hint in (total, max(1, total // 4), S * case.max_context_len):
        for P in (0, 64):
            say("ragged grid S", S, "hint", hint, "partition", P)
            got = _decode(case, dev, hint, P)
            err, gerr = max_err(got, expect), guard_err(got, expect, lens)
            say("max |gpu - oracle| = %.3e, on long rows %.3e" % (err, gerr))
            assert err <= TOL_BF16, (S, hint, P, err)
            assert gerr <= GUARD_BF16, (S, hint, P, gerr)


def test_ragged_grid_block32_and_fused_write():
    S = 48
    lens = _lognormal(3, S, 200, lo=1)
    lens[5] = 3000
    case = synth.make_case("ragged_write", 61, lens, 16, 2, 128, 32, free_frac=0.05)
    rng = np.random.default_rng(4)
    k_new = synth.bf16_bits(rng.standard_normal((S, 2, 128), dtype=np.float32))
    v_new = synth.bf16_bits(rng.standard_normal((S, 2, 128), dtype=np.float32))
    dev = case_on_device(case)
    say("ragged grid fused write")
    got = _decode(case, dev, int(lens.sum()), new=(to_dev(k_new), to_dev(v_new)))
    slots = oracle.slot_mapping(case.block_tables, case.context_lens - 1, case.block_size)
    oracle.reshape_and_cache(k_new, v_new, case.k_cache, case.v_cache, slots)
    assert np.array_equal(to_host(dev["k"]), case.k_cache)
    assert np.array_equal(to_host(dev["v"]), case.v_cache)
    expect = run_oracle(case)
    err, gerr = max_err(got, expect), guard_err(got, expect, lens)
    say("max |gpu - oracle| = %.3e, on long rows %.3e" % (err, gerr))
    assert err <= TOL_BF16, err
    assert gerr <= GUARD_BF16, gerr


@pytest.mark.parametrize("kv,mode,S", [(synth.I8, pa.PA_SCALE_BLOCK, 96), (synth.FP8, pa.PA_SCALE_TOKEN, 96),
                                       (synth.I8, pa.PA_SCALE_BLOCK, 700), (synth.I8, pa.PA_SCALE_TOKEN, 700)])
def test_ragged_grid_quantised(kv, mode, S):
    lens = _lognormal(7, S, 400)
    lens[1] = 4000
    case = synth.make_case("ragged_q", 71, lens, 32, 8, 128, 16, kv_dtype=kv, free_frac=0.05)
    quantize_case_by_token(case, mode)
    expect = oracle.paged_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                 float(case.scale), case.k_scales, case.v_scales, scale_mode=mode)
    dev = case_on_device(case)
    for hint in (int(lens.sum()), int(lens.sum()) // 3):
        say("ragged grid quantised", kv, mode, "S", S, "hint", hint)
        got = _decode(case, dev, hint)
        err, gerr = max_err(got, expect), guard_err(got, expect, lens)
        say("max |gpu - oracle| = %.3e, on long rows %.3e" % (err, gerr))
        assert err <= TOL_BF16, (kv, mode, hint, err)
        assert gerr <= GUARD_BF16, (kv, mode, hint, gerr)


def test_ragged_hint_with_every_sequence_empty():
    """A hint that claims tokens for a batch of empty sequences (max length
    64 passed): nothing to attend to, every output row zero."""
    case = synth.make_case("ragged_empty", 81, [64] + [0] * 11, 16, 4, 128, 16)
    case.context_lens[:] = 0
    dev = case_on_device(case)
    say("ragged hint, all sequences empty")
    out = pa.decode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale), 64,
                    total_context_len=100)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 0.0)
