"""The long-context regression guard (GUARD_BF16 = 2e-5 on the rows of
sequences of at least GUARD_MIN_LEN = 2,048 tokens, beside the 2e-3 parity
gate of the GPU tests) catches lost work that the gate alone lets through.
Pinned on the CPU with the oracle only: the same attention with one
16-token tile, or one whole split-K partition, left out of a sequence's
table moves the outputs by more than the guard -- at the 70B-shaped
layer's 8,000 tokens and at 131,072 tokens, where the gate alone would not
notice a dropped tile -- and below 2,048 tokens by more than the gate.

Dropping a tile is done through the table: with blocks of 16 tokens a tile
is one block, so removing one entry from the row (and 16 tokens from the
length) is the attention the kernel would compute had it skipped that
tile."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import GUARD_BF16, GUARD_MIN_LEN, TOL_BF16


def _drop_blocks(case, s, first, count):
    """Attention of sequence s with blocks [first, first + count) of its
    table left out."""
    row = case.block_tables[s]
    n = int(case.context_lens[s])
    nb = -(-n // case.block_size)
    assert first + count <= nb - 1 or (first + count == nb and n % case.block_size == 0)
    kept = np.concatenate([row[:first], row[first + count:nb]]).astype(np.int32)
    tab = np.full((1, row.shape[0]), -1, np.int32)
    tab[0, :kept.shape[0]] = kept
    lens = np.array([n - count * case.block_size], np.int32)
    return oracle.paged_decode(case.q[s:s + 1], case.k_cache, case.v_cache, tab, lens, float(case.scale))


def _full(case, s):
    return oracle.paged_decode(case.q[s:s + 1], case.k_cache, case.v_cache, case.block_tables[s:s + 1],
                               case.context_lens[s:s + 1], float(case.scale))


def test_dropped_tile_at_8000_tokens_breaks_the_guard():
    """70B-shaped heads (64 query / 8 kv heads of 128, bf16 N(0, 1) values,
    blocks of 16): leaving out any one of the first, a middle or the last
    full tile moves some output by more than the guard (over the 8,192
    outputs of one sequence, by a few 1e-3); for a single query head, the
    largest move is mostly under the 2e-3 gate."""
    case = synth.make_case("guard-8000", 5, [8000], 64, 8, 128, 16, free_frac=0.0)
    full = _full(case, 0)
    per_head = []
    for first in (0, 1, 250, 498):
        diff = np.abs(_drop_blocks(case, 0, first, 1) - full)[0]
        assert float(diff.max()) > 20 * GUARD_BF16, (first, float(diff.max()))
        per_head += list(diff.max(axis=1))
        assert float(diff.max(axis=1).min()) > GUARD_BF16, first   # every head moves past the guard
    assert np.median(per_head) < TOL_BF16, np.median(per_head)


def test_dropped_tile_or_partition_at_131072_tokens_breaks_the_guard():
    """One sequence of 131,072 tokens, 8 query heads on one kv head (the
    long-context GPU test's shape): a dropped tile moves the outputs by
    well over the guard and under the gate; a dropped 2,048-token partition
    (one of the 64 partials the merge combines) by more than the guard."""
    case = synth.make_case("guard-131072", 41, [131072], 8, 1, 128, 16, free_frac=0.0)
    full = _full(case, 0)
    for first in (3, 4000, 8190):
        d = float(np.max(np.abs(_drop_blocks(case, 0, first, 1) - full)))
        assert GUARD_BF16 < d < TOL_BF16, (first, d)
    d = float(np.max(np.abs(_drop_blocks(case, 0, 128 * 17, 128) - full)))
    assert d > GUARD_BF16, d


def test_double_counted_tile_breaks_the_guard():
    """The opposite mistake, a tile taken twice (one table entry repeated,
    16 tokens more), at 8,000 tokens."""
    case = synth.make_case("guard-dup", 6, [8000], 64, 8, 128, 16, free_frac=0.0)
    full = _full(case, 0)
    row = case.block_tables[0]
    nb = 500
    tab = np.full((1, row.shape[0] + 1), -1, np.int32)
    tab[0, :nb + 1] = np.concatenate([row[:nb], row[100:101]])
    got = oracle.paged_decode(case.q, case.k_cache, case.v_cache, tab, np.array([8016], np.int32),
                              float(case.scale))
    d = float(np.max(np.abs(got - full)))
    assert d > 5 * GUARD_BF16, d


@pytest.mark.parametrize("n,hq,hkv", [(17, 8, 1), (300, 32, 8), (1000, 8, 1), (2047, 8, 1), (2047, 32, 8)])
def test_dropped_tile_below_the_guard_length_breaks_the_gate(n, hq, hkv):
    """Rows the guard leaves out (sequences under GUARD_MIN_LEN tokens, in
    the GPU tests' head shapes): leaving out any one of their full tiles
    moves some output of the sequence by more than the 2e-3 gate."""
    assert n < GUARD_MIN_LEN
    case = synth.make_case("gate-%d" % n, 11 + n, [n], hq, hkv, 128, 16, free_frac=0.0)
    full = _full(case, 0)
    nb = -(-n // 16)
    for first in range(0, nb - 1, max(1, (nb - 1) // 12)):
        d = float(np.max(np.abs(_drop_blocks(case, 0, first, 1) - full)))
        assert d > TOL_BF16, (n, first, d)
