"""Seeded input generators: determinism and the workload shapes."""
import numpy as np

import synth


def _same(a, b):
    return np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_generators_are_deterministic():
    a, b = synth.config1(), synth.config1()
    for f in ("q", "k_cache", "v_cache", "block_tables", "context_lens"):
        assert _same(getattr(a, f), getattr(b, f))
    c, d = synth.config4(), synth.config4()
    assert _same(c.k_cache, d.k_cache) and _same(c.block_tables, d.block_tables)


def test_config1_shape():
    c = synth.config1()
    assert list(c.context_lens) == [17, 33, 100, 200]
    assert c.num_blocks == 64 and c.k_cache.shape == (64, 8, 16, 64) and c.q.dtype == np.float32
    assert c.scale == np.float32(0.125)
    used = c.block_tables[c.block_tables >= 0]
    assert len(used) == 2 + 3 + 7 + 13 == len(set(used.tolist()))
    assert sorted(used.tolist() + c.free_blocks.tolist()) == list(range(64))
    # free blocks and tails are poisoned
    assert np.all(np.isnan(c.k_cache[c.free_blocks]))
    assert np.all(np.isnan(c.k_cache[c.block_tables[0, 1], :, 1:, :]))
    assert not np.any(np.isnan(c.k_cache[c.block_tables[0, 1], :, :1, :]))


def test_config2_shape():
    c = synth.config2()
    assert c.num_seqs == 32 and c.num_q_heads == c.num_kv_heads == 40 and c.head_dim == 128
    assert c.context_lens.min() >= 200 and c.context_lens.max() <= 2048
    used = int(np.sum(-(-c.context_lens // 16)))
    assert c.num_blocks == int(np.ceil(used * 1.1))
    assert c.q.dtype == np.uint16 and c.k_cache.dtype == np.uint16


def test_config3_structure_and_bytes(golden):
    st = synth.config3_structure()
    g = golden("kv_size_formula.json")
    c = synth.CFG3
    assert st["num_blocks"] == 10000 and st["block_tables"].shape == (20, 500)
    assert sorted(st["block_tables"].ravel().tolist()) == list(range(10000))
    per_layer = st["num_blocks"] * c["num_kv_heads"] * c["block_size"] * c["head_dim"] * 2 * 2
    assert per_layer * c["layers"] == g["kv_bytes"]


def test_config4_structure():
    c = synth.config4()
    e = c.extra
    assert c.block_size == 32 and c.num_seqs == 50
    assert len(e["shared"]) == 62
    for s in range(50):
        assert np.array_equal(c.block_tables[s, :62], e["shared"])
        assert c.block_tables[s, 62] == e["private"][s][0]
        # the private copy holds the prefix's last 16 tokens
        assert _same(c.k_cache[e["private"][s][0], :, :16], c.k_cache[e["partial"], :, :16])
    assert np.all(c.context_lens == 2000 + e["suffix"])
    assert e["suffix"].min() >= 50 and e["suffix"].max() <= 500
    ids = set(e["shared"].tolist()) | {e["partial"]} | set(e["scratch"].tolist())
    for p in e["private"]:
        ids |= set(p.tolist())
    assert len(ids) == 62 + 1 + 50 + sum(len(p) for p in e["private"])


def test_config5_lengths():
    c = synth.config5()
    assert c.kv_dtype == "i8" and c.num_seqs == 64
    assert c.context_lens.min() >= 16 and c.context_lens.max() <= 32768
    assert c.num_blocks == int(np.sum(-(-c.context_lens // 16)))
    big = synth.config5_lengths(np.random.default_rng(123), 200000)
    assert abs(np.median(big) - 1500) < 30
