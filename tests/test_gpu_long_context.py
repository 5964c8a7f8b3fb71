"""Long contexts on the GPU against the CPU oracle: the partition plans at
their limits.

* One sequence of 131,072 tokens: a partition holds at most 128 blocks, so
  the near-equal plan cuts it into 64 partitions of 2,048 tokens (and the
  vector-ALU kernel likewise), and the merge reads 64 partials per row with
  several waves.
* A skewed batch, one 100,000-token sequence among short ones, with the
  length hint: the balanced split cuts the long sequence into dozens of
  ranges, each leaving its own partial, while the short sequences share
  ranges with each other.

Attention over the sequence's table is the only thing the oracle knows;
max |gpu - oracle| <= 2e-3 (bf16 or int8 cache, fp32 accumulation), and
the rows of long sequences within the regression guard (a lost tile or
partial breaches it while staying under 2e-3)."""
import pytest

import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import GUARD_BF16, TOL_BF16, case_on_device, guard_err, max_err, quantize_case, run_decode, run_oracle, say

pytestmark = pytest.mark.gpu

VALU, MFMA = pa.KERNEL_VALU, pa.KERNEL_MFMA


def _case(name, seed, lens, kv):
    case = synth.make_case(name, seed, lens, 8, 1, 128, 16, kv_dtype=kv, free_frac=0.05)
    if kv == synth.I8:
        quantize_case(case)
    return case


@pytest.mark.parametrize("kv", [synth.BF16, synth.I8])
def test_one_sequence_of_131072_tokens(kv):
    case = _case("long-131072", 41, [131072], kv)
    expect = run_oracle(case)
    dev = case_on_device(case)
    for kern in (0, VALU, MFMA):
        for P in (0, 2048):
            say(case.name, kv, "kernel", kern, "partition", P)
            got = run_decode(case, dev, partition_tokens=P, kernel=kern)
            err, gerr = max_err(got, expect), guard_err(got, expect, case.context_lens)
            say("max |gpu - oracle| = %.3e, on long rows %.3e" % (err, gerr))
            assert err <= TOL_BF16, (kv, kern, P, err)
            assert gerr <= GUARD_BF16, (kv, kern, P, gerr)


@pytest.mark.parametrize("kv", [synth.BF16, synth.I8])
def test_skewed_batch_with_a_100000_token_sequence(kv):
    lens = [100000] + [17, 1, 0, 300, 2049, 64, 5, 1000, 33] * 3
    case = _case("skewed-100000", 42, lens, kv)
    expect = run_oracle(case)
    dev = case_on_device(case)
    for kern in (0, MFMA):
        for hint in (True, False):
            say(case.name, kv, "kernel", kern, "hint", hint)
            got = run_decode(case, dev, kernel=kern, length_hint=hint)
            err, gerr = max_err(got, expect), guard_err(got, expect, case.context_lens)
            say("max |gpu - oracle| = %.3e, on long rows %.3e" % (err, gerr))
            assert err <= TOL_BF16, (kv, kern, hint, err)
            assert gerr <= GUARD_BF16, (kv, kern, hint, gerr)
