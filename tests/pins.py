"""Pins of the CPU oracle to facts other than itself.

Each ``pin_*`` function raises AssertionError when the oracle (whichever
build ``oracle`` currently routes to) disagrees with a value fixed by the
pages or by mathematics: closed forms, hand-built cases, an independent
unpaged implementation, invariances, the worked block table of the
architecture figure.  ``test_oracle.py`` runs them on the real oracle and
``test_oracle_mutants.py`` checks that each planted mistake trips at least
one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
from synth import bf16_bits, bits_to_f32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# building paged caches from logical (per-sequence) arrays
# --------------------------------------------------------------------------

def paginate(seq_arrays, block_size, num_blocks, rng=None, tables=None, fill=np.nan, dtype=None):
    """Scatter per-sequence logical arrays ``[n_s][H][D]`` into a paged cache
    ``[NB][H][BS][D]``.  Physical ids come from ``tables`` when given, else
    from a seeded permutation.  Unused memory is filled with ``fill``."""
    H, D = seq_arrays[0].shape[1:]
    dtype = dtype or seq_arrays[0].dtype
    nbs = [-(-a.shape[0] // block_size) for a in seq_arrays]
    if tables is None:
        perm = (rng or np.random.default_rng(0)).permutation(num_blocks)
        tables = np.full((len(seq_arrays), max(max(nbs), 1)), -1, np.int32)
        k = 0
        for s, nb in enumerate(nbs):
            tables[s, :nb] = perm[k:k + nb]
            k += nb
    cache = np.empty((num_blocks, H, block_size, D), dtype=dtype)
    cache[...] = fill
    for s, a in enumerate(seq_arrays):
        for t in range(a.shape[0]):
            cache[tables[s][t // block_size], :, t % block_size, :] = a[t]
    return cache, np.asarray(tables, np.int32)


def unit(D, i, scale=1.0, dtype=np.float32):
    v = np.zeros(D, dtype)
    v[i] = scale
    return v


# --------------------------------------------------------------------------
# decode-attention pins
# --------------------------------------------------------------------------

def pin_ctx1_returns_v0():
    """One token: its weight is exp(0)/exp(0) = 1, so out = v0 exactly."""
    rng = np.random.default_rng(11)
    S, Hq, Hkv, D, BS = 3, 8, 2, 128, 16
    K = [bf16_bits(rng.standard_normal((1, Hkv, D), dtype=np.float32)) for _ in range(S)]
    V = [bf16_bits(rng.standard_normal((1, Hkv, D), dtype=np.float32)) for _ in range(S)]
    kc, bt = paginate(K, BS, 7, rng, fill=0x7FC0)
    vc, _ = paginate(V, BS, 7, tables=bt, fill=0x7FC0)
    q = bf16_bits(rng.standard_normal((S, Hq, D), dtype=np.float32))
    out = oracle.paged_decode(q, kc, vc, bt, np.ones(S, np.int32), 0.0883883461356163)
    for s in range(S):
        for h in range(Hq):
            assert np.array_equal(out[s, h], bits_to_f32(V[s][0, h // (Hq // Hkv)]).astype(np.float64))


def _hand_case(ctx, q, ks, vs, scale, block_size=16, table=None, num_blocks=4):
    D = q.shape[-1]
    K = np.stack([k[None, :] for k in ks]).astype(np.float32)  # [n][1][D]
    V = np.stack([v[None, :] for v in vs]).astype(np.float32)
    tables = None if table is None else np.asarray([table], np.int32)
    kc, bt = paginate([K], block_size, num_blocks, tables=tables)
    vc, _ = paginate([V], block_size, num_blocks, tables=bt)
    return oracle.paged_decode(q.reshape(1, 1, D).astype(np.float32), kc, vc, bt,
                               np.array([ctx], np.int32), scale)[0, 0]


def pin_ctx2_closed_form():
    g = golden("attention_closed_forms.json")["ctx2"]
    D = 64
    for qscale, scale in ((1.0, 1.0), (2.0, 0.5), (8.0, 0.125)):
        out = _hand_case(2, unit(D, 0, qscale), [np.zeros(D), unit(D, 0)], [unit(D, 0), unit(D, 1)],
                         scale, table=[2])
        assert abs(out[0] - g["out_d0"]) < 1e-15 and abs(out[1] - g["out_d1"]) < 1e-15, out[:2]
        assert np.all(out[2:] == 0.0)


def pin_ctx3_closed_form_across_blocks():
    """Three tokens over two blocks of 2 slots, table [3, 1]: token 2 lives in
    physical block 1, slot 0."""
    g = golden("attention_closed_forms.json")["ctx3"]
    D = 64
    out = _hand_case(3, unit(D, 0), [t * unit(D, 0) for t in range(3)], [unit(D, t) for t in range(3)],
                     1.0, block_size=2, table=[3, 1], num_blocks=4)
    assert np.max(np.abs(out[:3] - np.array(g["out"]))) < 1e-15, out[:3]
    assert np.all(out[3:] == 0.0)


def pin_head_mapping():
    """Query head h reads KV head h // (Hq / Hkv): with KV head 0 holding
    values e0 and KV head 1 values e1, heads 0-1 see e0 and heads 2-3 e1."""
    rng = np.random.default_rng(5)
    n, D, BS = 37, 64, 16
    K = rng.standard_normal((n, 2, D), dtype=np.float32)
    V = np.zeros((n, 2, D), np.float32)
    V[:, 0, 0] = 1.0
    V[:, 1, 1] = 1.0
    kc, bt = paginate([K], BS, 5, rng)
    vc, _ = paginate([V], BS, 5, tables=bt)
    q = rng.standard_normal((1, 4, D), dtype=np.float32)
    out = oracle.paged_decode(q, kc, vc, bt, np.array([n], np.int32), 0.125)[0]
    for h in range(4):
        expect = unit(D, h // 2, dtype=np.float64)
        assert np.max(np.abs(out[h] - expect)) < 1e-14, (h, out[h][:3])


def pin_equal_keys_give_mean():
    rng = np.random.default_rng(6)
    n, D = 45, 128
    k = rng.standard_normal(D, dtype=np.float32)
    K = np.broadcast_to(k, (n, 1, D)).copy()
    V = rng.standard_normal((n, 1, D), dtype=np.float32)
    kc, bt = paginate([K], 16, 6, rng)
    vc, _ = paginate([V], 16, 6, tables=bt)
    q = rng.standard_normal((1, 1, D), dtype=np.float32)
    out = oracle.paged_decode(q, kc, vc, bt, np.array([n], np.int32), 0.3)[0, 0]
    assert np.max(np.abs(out - V[:, 0, :].astype(np.float64).mean(axis=0))) < 1e-14


def pin_dominant_score_is_one_hot():
    rng = np.random.default_rng(7)
    n, D, star = 50, 64, 29
    K = np.zeros((n, 1, D), np.float32)
    K[star, 0, 0] = 200.0
    V = rng.standard_normal((n, 1, D), dtype=np.float32)
    kc, bt = paginate([K], 16, 4, rng)
    vc, _ = paginate([V], 16, 4, tables=bt)
    out = oracle.paged_decode(unit(64, 0).reshape(1, 1, D), kc, vc, bt, np.array([n], np.int32), 1.0)
    assert np.max(np.abs(out[0, 0] - V[star, 0].astype(np.float64))) < 1e-14


def pin_ctx0_is_zero():
    rng = np.random.default_rng(8)
    K = [rng.standard_normal((5, 2, 64), dtype=np.float32), np.zeros((0, 2, 64), np.float32)]
    kc, bt = paginate(K, 16, 3, rng)
    vc, _ = paginate(K, 16, 3, tables=bt)
    q = rng.standard_normal((2, 2, 64), dtype=np.float32)
    out = oracle.paged_decode(q, kc, vc, bt, np.array([5, 0], np.int32), 0.125)
    assert np.all(out[1] == 0.0) and np.all(np.isfinite(out[0]))


def _random_case(seed, lens, Hq, Hkv, D, BS, kind):
    rng = np.random.default_rng(seed)
    nbs = sum(-(-n // BS) for n in lens)
    NB = nbs + 3
    if kind == "i8":
        Kc = [rng.integers(-127, 128, (n, Hkv, D)).astype(np.int8) for n in lens]
        Vc = [rng.integers(-127, 128, (n, Hkv, D)).astype(np.int8) for n in lens]
        kc, bt = paginate(Kc, BS, NB, rng, fill=127)
        vc, _ = paginate(Vc, BS, NB, tables=bt, fill=-127)
        ks = (rng.random((NB, Hkv)) * 0.05 + 0.001).astype(np.float32)
        vs = (rng.random((NB, Hkv)) * 0.05 + 0.001).astype(np.float32)
        q = bf16_bits(rng.standard_normal((len(lens), Hq, D), dtype=np.float32))
        return q, kc, vc, bt, ks, vs
    mk = (lambda x: bf16_bits(x)) if kind == "bf16" else (lambda x: x)
    fill = 0x7FC0 if kind == "bf16" else np.nan
    K = [mk(rng.standard_normal((n, Hkv, D), dtype=np.float32)) for n in lens]
    V = [mk(rng.standard_normal((n, Hkv, D), dtype=np.float32)) for n in lens]
    kc, bt = paginate(K, BS, NB, rng, fill=fill)
    vc, _ = paginate(V, BS, NB, tables=bt, fill=fill)
    q = mk(rng.standard_normal((len(lens), Hq, D), dtype=np.float32))
    return q, kc, vc, bt, None, None


CONTIG_CASES = [
    (21, [17, 33, 100, 200], 8, 8, 64, 16, "f32"),
    (22, [1, 31, 32, 33, 64, 250], 32, 8, 128, 32, "bf16"),
    (23, [16, 90, 300], 64, 8, 128, 16, "bf16"),
    (24, [5, 47, 129], 32, 8, 128, 16, "i8"),
]


def pin_matches_contiguous_attention():
    """Paged oracle vs an independent NumPy attention over contiguous
    per-sequence arrays read back through the tables: within 1e-12."""
    for seed, lens, Hq, Hkv, D, BS, kind in CONTIG_CASES:
        q, kc, vc, bt, ks, vs = _random_case(seed, lens, Hq, Hkv, D, BS, kind)
        cl = np.asarray(lens, np.int32)
        scale = float(np.float32(1 / math.sqrt(D)))
        got = oracle.paged_decode(q, kc, vc, bt, cl, scale, ks, vs)
        keys = oracle.gather_logical(kc, bt, cl, ks)
        vals = oracle.gather_logical(vc, bt, cl, vs)
        ref = oracle.contiguous_attention(oracle.as_float64(q), keys, vals, scale)
        err = np.max(np.abs(got - ref))
        assert err < 1e-12, (seed, kind, err)


def pin_permutation_invariance():
    """Moving every physical block elsewhere (and remapping the tables)
    leaves the output bit-identical."""
    q, kc, vc, bt, _, _ = _random_case(31, [40, 77, 16, 3], 32, 8, 128, 16, "bf16")
    cl = np.array([40, 77, 16, 3], np.int32)
    base = oracle.paged_decode(q, kc, vc, bt, cl, 0.0883883461356163)
    rng = np.random.default_rng(32)
    NB = kc.shape[0]
    pi = rng.permutation(NB)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    bt2 = np.where(bt >= 0, pi[np.maximum(bt, 0)], -1).astype(np.int32)
    got = oracle.paged_decode(q, kc2, vc2, bt2, cl, 0.0883883461356163)
    assert np.array_equal(base, got)


def pin_prefix_sharing_identical():
    """Two sequences with the same query and the same logical K/V give
    bit-identical outputs whether their tables point at the same physical
    blocks or at private copies."""
    rng = np.random.default_rng(33)
    n, Hkv, D, BS = 70, 2, 64, 16
    K = rng.standard_normal((n, Hkv, D), dtype=np.float32)
    V = rng.standard_normal((n, Hkv, D), dtype=np.float32)
    kc, bt = paginate([K, K], BS, 12, rng)        # private copies
    vc, _ = paginate([V, V], BS, 12, tables=bt)
    shared = bt.copy()
    shared[1] = shared[0]                          # both point at seq 0's blocks
    q1 = rng.standard_normal((1, 4, D), dtype=np.float32)
    q = np.concatenate([q1, q1])
    cl = np.array([n, n], np.int32)
    a = oracle.paged_decode(q, kc, vc, bt, cl, 0.125)
    b = oracle.paged_decode(q, kc, vc, shared, cl, 0.125)
    assert np.array_equal(a[0], a[1]) and np.array_equal(a, b)


def pin_gqa_equals_replicated_mha():
    q, kc, vc, bt, _, _ = _random_case(34, [23, 50], 16, 4, 64, 16, "f32")
    cl = np.array([23, 50], np.int32)
    gqa = oracle.paged_decode(q, kc, vc, bt, cl, 0.125)
    kr = np.repeat(kc, 4, axis=1)
    vr = np.repeat(vc, 4, axis=1)
    mha = oracle.paged_decode(q, kr, vr, bt, cl, 0.125)
    assert np.array_equal(gqa, mha)


def pin_block_size_invariance():
    rng = np.random.default_rng(35)
    lens = [33, 64, 95]
    K = [rng.standard_normal((n, 2, 64), dtype=np.float32) for n in lens]
    V = [rng.standard_normal((n, 2, 64), dtype=np.float32) for n in lens]
    q = rng.standard_normal((3, 4, 64), dtype=np.float32)
    cl = np.array(lens, np.int32)
    outs = []
    for BS in (16, 32):
        kc, bt = paginate(K, BS, 20, rng)
        vc, _ = paginate(V, BS, 20, tables=bt)
        outs.append(oracle.paged_decode(q, kc, vc, bt, cl, 0.125))
    assert np.array_equal(outs[0], outs[1])


def pin_convex_hull():
    q, kc, vc, bt, _, _ = _random_case(36, [19, 64, 101], 8, 8, 64, 16, "f32")
    cl = np.array([19, 64, 101], np.int32)
    out = oracle.paged_decode(q, kc, vc, bt, cl, 0.125)
    vals = oracle.gather_logical(vc, bt, cl)
    for s in range(3):
        for h in range(8):
            lo = vals[s][:, h, :].min(axis=0)
            hi = vals[s][:, h, :].max(axis=0)
            assert np.all(out[s, h] >= lo - 1e-12) and np.all(out[s, h] <= hi + 1e-12)


def pin_poison_is_never_read():
    """NaN in free blocks and in slots past each context leaves the output
    finite and bit-identical to a run with zeros there."""
    rng = np.random.default_rng(37)
    lens = [7, 16, 30]
    K = [rng.standard_normal((n, 2, 64), dtype=np.float32) for n in lens]
    V = [rng.standard_normal((n, 2, 64), dtype=np.float32) for n in lens]
    q = rng.standard_normal((3, 2, 64), dtype=np.float32)
    cl = np.array(lens, np.int32)
    kn, bt = paginate(K, 16, 9, np.random.default_rng(1), fill=np.nan)
    vn, _ = paginate(V, 16, 9, tables=bt, fill=np.nan)
    kz, _ = paginate(K, 16, 9, tables=bt, fill=0.0)
    vz, _ = paginate(V, 16, 9, tables=bt, fill=0.0)
    a = oracle.paged_decode(q, kn, vn, bt, cl, 0.125)
    b = oracle.paged_decode(q, kz, vz, bt, cl, 0.125)
    assert np.all(np.isfinite(a)) and np.array_equal(a, b)


def pin_int8_dequant_closed_form():
    """int8 codes times the per-(block, head) scale: K codes 2 with k-scale
    0.5 make the logits (0, 1); V codes 4 and 6 with v-scale 0.25 make the
    values e0 and 1.5*e1."""
    g = golden("attention_closed_forms.json")["ctx2"]
    D, BS = 64, 16
    K = np.zeros((2, 1, D), np.int8)
    K[1, 0, 0] = 2
    V = np.zeros((2, 1, D), np.int8)
    V[0, 0, 0] = 4
    V[1, 0, 1] = 6
    kc, bt = paginate([K], BS, 3, tables=np.array([[1]]), fill=99)
    vc, _ = paginate([V], BS, 3, tables=bt, fill=-99)
    ks = np.full((3, 1), 7.0, np.float32)
    vs = np.full((3, 1), 9.0, np.float32)
    ks[1, 0] = 0.5
    vs[1, 0] = 0.25
    q = bf16_bits(unit(D, 0).reshape(1, 1, D))
    out = oracle.paged_decode(q, kc, vc, bt, np.array([2], np.int32), 1.0, ks, vs)[0, 0]
    assert abs(out[0] - g["out_d0"]) < 1e-15 and abs(out[1] - 1.5 * g["out_d1"]) < 1e-15, out[:2]


DECODE_PINS = [pin_ctx1_returns_v0, pin_ctx2_closed_form, pin_ctx3_closed_form_across_blocks,
               pin_head_mapping, pin_equal_keys_give_mean, pin_dominant_score_is_one_hot,
               pin_ctx0_is_zero, pin_matches_contiguous_attention, pin_permutation_invariance,
               pin_prefix_sharing_identical, pin_gqa_equals_replicated_mha, pin_block_size_invariance,
               pin_convex_hull, pin_poison_is_never_read, pin_int8_dequant_closed_form]


# --------------------------------------------------------------------------
# slot mapping, cache writes, copies, quantiser
# --------------------------------------------------------------------------

def pin_slot_mapping_figure():
    g = golden("block_table_figure.json")
    bt = np.array([g["table"]], np.int32)
    pos = np.arange(g["tokens"], dtype=np.int32)
    slots = oracle.slot_mapping(bt, pos, g["block_size"], seq_idx=np.zeros(g["tokens"], np.int32))
    assert slots[g["probe"]["token"]] == g["probe"]["slot"]
    assert list(slots[::g["block_size"]]) == g["first_slot_of_each_logical_block"]
    # every slot lies in a block of the request, never in the free or foreign one
    blocks = set((slots // g["block_size"]).tolist())
    assert blocks == set(g["table"])
    assert not blocks & set(g["free_blocks"] + g["other_request_blocks"])
    # consecutive tokens inside a block are consecutive slots
    assert np.all(np.diff(slots.reshape(3, 16), axis=1) == 1)


def pin_slot_mapping_edges():
    bt = np.array([[5, -1], [3, 0]], np.int32)
    slots = oracle.slot_mapping(bt, np.array([0, 17, -1, 31, 32, 15], np.int32), 16,
                                seq_idx=np.array([0, 0, 1, 1, 1, 1], np.int32))
    assert list(slots) == [80, -1, -1, 15, -1, 63]
    # seq_idx omitted: token t belongs to sequence t
    assert list(oracle.slot_mapping(bt, np.array([3, 20], np.int32), 16)) == [83, 4]


def pin_reshape_writes_exactly_one_slot_per_token():
    rng = np.random.default_rng(41)
    NB, H, BS, D, T = 6, 2, 16, 64, 5
    for dt in (np.float32, np.uint16, np.int8):
        base = rng.integers(0, 100, (NB, H, BS, D)).astype(dt)
        kc, vc = base.copy(), (base + 1).copy()
        key = rng.integers(100, 120, (T, H, D)).astype(dt)
        val = rng.integers(120, 127, (T, H, D)).astype(dt)
        slots = np.array([17, -1, 95, 0, 40], np.int64)
        oracle.reshape_and_cache(key, val, kc, vc, slots)
        expect_k, expect_v = base.copy(), (base + 1).copy()
        for t, sl in enumerate(slots):
            if sl >= 0:
                expect_k[sl // BS, :, sl % BS, :] = key[t]
                expect_v[sl // BS, :, sl % BS, :] = val[t]
        assert np.array_equal(kc, expect_k) and np.array_equal(vc, expect_v)
        changed = np.any(kc != base, axis=(1, 3))  # [NB][BS]
        assert changed.sum() <= 4


def pin_copy_blocks_exact():
    rng = np.random.default_rng(42)
    NB, H, BS, D = 8, 2, 32, 64
    kc = rng.integers(-128, 128, (NB, H, BS, D)).astype(np.int8)
    vc = rng.integers(-128, 128, (NB, H, BS, D)).astype(np.int8)
    ks = rng.random((NB, H)).astype(np.float32)
    vs = rng.random((NB, H)).astype(np.float32)
    k0, v0, ks0, vs0 = kc.copy(), vc.copy(), ks.copy(), vs.copy()
    pairs = np.array([[1, 4], [1, 6], [3, 0]], np.int64)
    oracle.copy_blocks(kc, vc, pairs, ks, vs)
    for src, dst in pairs:
        assert np.array_equal(kc[dst], k0[src]) and np.array_equal(vc[dst], v0[src])
        assert np.array_equal(ks[dst], ks0[src]) and np.array_equal(vs[dst], vs0[src])
    for b in (1, 2, 3, 5, 7):
        assert np.array_equal(kc[b], k0[b]) and np.array_equal(vc[b], v0[b])
        assert np.array_equal(ks[b], ks0[b]) and np.array_equal(vs[b], vs0[b])


def pin_quantiser_hand_values():
    """amax 127 gives scale exactly 1; -63.5 and 0.5 are ties that round to
    the even codes -64 and 0, 1.5 rounds to 2; an all-zero (block, head)
    gets scale 1 and zero codes; slots past the valid count get 0."""
    x = np.zeros((2, 1, 4, 4), np.float32)
    x[0, 0, 0, :] = [127.0, -63.5, 0.5, 1.5]
    x[0, 0, 1, :] = [2.49, -2.5, 3.5, -126.6]
    x[0, 0, 3, :] = 1000.0                  # past the valid count
    codes, scales = oracle.quantize_int8(x, np.array([2, 4], np.int32))
    assert scales[0, 0] == np.float32(1.0) and scales[1, 0] == np.float32(1.0)
    assert list(codes[0, 0, 0]) == [127, -64, 0, 2]
    assert list(codes[0, 0, 1]) == [2, -2, 4, -127]
    assert np.all(codes[0, 0, 2:] == 0) and np.all(codes[1] == 0)


def pin_quantiser_invariants():
    rng = np.random.default_rng(43)
    NB, H, BS, D = 12, 4, 16, 128
    x = rng.standard_normal((NB, H, BS, D), dtype=np.float32) * rng.random((NB, H, 1, 1)).astype(np.float32)
    valid = rng.integers(1, BS + 1, NB).astype(np.int32)
    codes, scales = oracle.quantize_int8(x, valid)
    assert codes.min() >= -127 and codes.max() <= 127
    for b in range(NB):
        n = valid[b]
        for h in range(H):
            blk = x[b, h, :n]
            amax = np.float32(np.abs(blk).max())
            assert scales[b, h] == np.float32(amax / np.float32(127.0))
            assert np.abs(codes[b, h, :n]).max() == 127
            err = np.abs(blk.astype(np.float64) - scales[b, h] * codes[b, h, :n].astype(np.float64))
            assert err.max() <= 0.5 * scales[b, h] * (1 + 1e-6)
            assert np.all(codes[b, h, n:] == 0)


# --------------------------------------------------------------------------
# quantised caches: E4M3 format, per-token scales, quantising write, swap
# --------------------------------------------------------------------------

def _torch_e4m3_values():
    """float64[256] from torch's own float8_e4m3fn decoding (a library
    routine independent of the oracle), or None if torch lacks the type."""
    import torch
    if not hasattr(torch, "float8_e4m3fn"):
        return None
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def pin_fp8_format_values():
    """The E4M3 format's closed forms: 0x38 = 1, 0x7E = 448 (largest),
    0x01 = 2^-9 (smallest subnormal), 0x08 = 2^-6 (smallest normal),
    0x07 = 7 * 2^-9, 0x7F and 0xFF NaN, sign bit = negation; every code
    agrees with torch's float8_e4m3fn decoding."""
    t = oracle.fp8_table()
    assert t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6
    assert t[0x07] == 7 * 2.0 ** -9 and t[0x3F] == 1.875 and t[0x40] == 2.0
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF]) and np.isfinite(t).sum() == 254
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F]) and math.copysign(1.0, t[0x80]) == -1.0
    finite = t[:0x7F]
    assert np.all(np.diff(finite) > 0)           # codes 0..0x7E are increasing
    ref = _torch_e4m3_values()
    if ref is not None:
        ok = ~np.isnan(ref)
        assert np.array_equal(np.isnan(t), ~ok) and np.array_equal(t[ok], ref[ok])


def pin_fp8_encode():
    """Round to the nearest code, ties to the even mantissa, saturating at
    +-448: every finite code is a fixed point; midpoints go to the even
    neighbour; beyond 448 gives 0x7E; NaN gives 0x7F; torch's fp32 ->
    float8_e4m3fn conversion agrees inside the finite range."""
    t = oracle.fp8_table()
    for c in list(range(0, 0x7F)) + list(range(0x80, 0xFF)):
        assert oracle.fp8_e4m3_encode(t[c]) == c, hex(c)
    for c in range(0, 0x7E):
        mid = (t[c] + t[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.fp8_e4m3_encode(mid) == even, hex(c)
        assert oracle.fp8_e4m3_encode(-mid) == even | 0x80
    assert oracle.fp8_e4m3_encode(449.0) == 0x7E and oracle.fp8_e4m3_encode(1e30) == 0x7E
    assert oracle.fp8_e4m3_encode(-500.0) == 0xFE and oracle.fp8_e4m3_encode(float("nan")) == 0x7F
    import torch
    if hasattr(torch, "float8_e4m3fn"):
        x = np.random.default_rng(44).uniform(-440, 440, 4000).astype(np.float32)
        x[:1000] *= np.float32(1e-3)
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = np.array([oracle.fp8_e4m3_encode(v) for v in x], np.uint8)
        assert np.array_equal(got, ref)


def pin_per_token_scales_closed_form():
    """Per-token scales: slot 1's K code 2 with its own scale 0.5 gives the
    logits (0, 1); V codes 4 and 6 with slot scales 0.25 and 1/3 give the
    values e0 and 2 e1.  The other slots' scales (7, 9) must not be read.
    The same with E4M3 codes (0x48 = 4, 0x4C = 6, 0x40 = 2)."""
    g = golden("attention_closed_forms.json")["ctx2"]
    D, BS = 64, 16
    for dt, two, four, six in ((np.int8, 2, 4, 6), (np.uint8, 0x40, 0x48, 0x4C)):
        K = np.zeros((2, 1, D), dt)
        K[1, 0, 0] = two
        V = np.zeros((2, 1, D), dt)
        V[0, 0, 0] = four
        V[1, 0, 1] = six
        kc, bt = paginate([K], BS, 3, tables=np.array([[1]]), fill=0)
        vc, _ = paginate([V], BS, 3, tables=bt, fill=0)
        ks = np.full((3, 1, BS), 7.0, np.float32)
        vs = np.full((3, 1, BS), 9.0, np.float32)
        ks[1, 0, 1] = 0.5
        vs[1, 0, 0] = 0.25
        vs[1, 0, 1] = np.float32(1.0 / 3.0)
        q = bf16_bits(unit(D, 0).reshape(1, 1, D))
        out = oracle.paged_decode(q, kc, vc, bt, np.array([2], np.int32), 1.0, ks, vs,
                                  scale_mode=oracle.SCALE_TOKEN)[0, 0]
        v1 = 6.0 * float(np.float32(1.0 / 3.0))
        assert abs(out[0] - g["out_d0"]) < 1e-15 and abs(out[1] - v1 * g["out_d1"]) < 1e-15, out[:2]


def pin_quantised_decode_matches_contiguous():
    """int8 and E4M3 caches, both scale layouts: the paged oracle equals
    unpaged NumPy attention over the dequantised logical rows."""
    rng = np.random.default_rng(45)
    lens = [1, 17, 40]
    Hq, Hkv, D, BS, NB = 4, 2, 64, 16, 12
    for dt in (np.int8, np.uint8):
        for mode in (oracle.SCALE_BLOCK, oracle.SCALE_TOKEN):
            seqs_k = [rng.integers(-127, 128, (n, Hkv, D)).astype(np.int8) for n in lens]
            seqs_v = [rng.integers(-127, 128, (n, Hkv, D)).astype(np.int8) for n in lens]
            if dt == np.uint8:   # random finite E4M3 codes
                seqs_k = [(a.view(np.uint8) & 0x77) | (a.view(np.uint8) & 0x80) for a in seqs_k]
                seqs_v = [(a.view(np.uint8) & 0x77) | (a.view(np.uint8) & 0x80) for a in seqs_v]
            kc, bt = paginate(seqs_k, BS, NB, rng=rng, fill=0)
            vc, _ = paginate(seqs_v, BS, NB, tables=bt, fill=0)
            shp = oracle.scale_shape(NB, Hkv, BS, mode)
            ks = (rng.random(shp) * 0.05).astype(np.float32)
            vs = (rng.random(shp) * 0.05).astype(np.float32)
            q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
            cl = np.array(lens, np.int32)
            got = oracle.paged_decode(q, kc, vc, bt, cl, 0.125, ks, vs, scale_mode=mode)
            K64 = oracle.gather_logical(kc, bt, cl, ks)
            V64 = oracle.gather_logical(vc, bt, cl, vs)
            ref = oracle.contiguous_attention(q.astype(np.float64), K64, V64, 0.125)
            assert np.max(np.abs(got - ref)) < 1e-12


def pin_quantising_write_hand_values():
    """int8, per token: a row with amax 127 gets scale 1 and rint codes
    (ties to even); an all-zero row scale 1 and codes 0.  Static: the given
    scale (different for K and V) is stamped in the (block, head) and codes
    saturate at +-127.  E4M3 per token: a row with amax 448 gets scale 1 and
    the nearest codes.  Skipped slots and other slots stay untouched."""
    NB, H, BS, D = 3, 2, 4, 4
    key = np.zeros((3, H, D), np.float32)
    key[0, 0] = [127.0, -63.5, 0.5, 1.5]
    key[0, 1] = [2.49, -2.5, 3.5, -127.0]
    val = -key
    val[0, 1] = [0.0, 0.0, 0.0, 0.0]
    key[1] = 5.0
    slots = np.array([6, -1, 11], np.int64)     # block 1 slot 2, skipped, block 2 slot 3
    kc = np.full((NB, H, BS, D), 55, np.int8)
    vc = kc.copy()
    ks = np.full((NB, H, BS), -1.0, np.float32)
    vs = ks.copy()
    oracle.quantize_and_cache(key, val, kc, vc, ks, vs, slots, oracle.SCALE_TOKEN)
    assert list(kc[1, 0, 2]) == [127, -64, 0, 2] and ks[1, 0, 2] == 1.0
    assert list(kc[1, 1, 2]) == [2, -2, 4, -127] and ks[1, 1, 2] == 1.0
    assert list(vc[1, 0, 2]) == [-127, 64, 0, -2] and list(vc[1, 1, 2]) == [0, 0, 0, 0] and vs[1, 1, 2] == 1.0
    assert np.all(kc[2, :, 3] == 0) and np.all(ks[2, :, 3] == 1.0)        # token 2 is all zeros
    touched = np.zeros((NB, H, BS), bool)
    touched[1, :, 2] = touched[2, :, 3] = True
    assert np.all(kc[~touched] == 55) and np.all(ks[~touched] == -1.0)
    # static scales per layer, stamped per (block, head)
    kc2 = np.full((NB, H, BS, D), 55, np.int8)
    vc2 = kc2.copy()
    ks2 = np.full((NB, H), -1.0, np.float32)
    vs2 = ks2.copy()
    oracle.quantize_and_cache(key, val, kc2, vc2, ks2, vs2, slots, oracle.SCALE_BLOCK, 0.5, 2.0)
    assert list(kc2[1, 0, 2]) == [127, -127, 1, 3] and ks2[1, 0] == 0.5 and vs2[1, 0] == 2.0
    assert list(vc2[1, 0, 2]) == [-64, 32, 0, -1] and ks2[0, 0] == -1.0
    # E4M3, per token: amax 448 -> scale 1
    key3 = np.zeros((1, 1, 4), np.float32)
    key3[0, 0] = [448.0, -1.0625, 0.3, 2.0 ** -9]
    kc3 = np.zeros((1, 1, BS, 4), np.uint8)
    vc3 = kc3.copy()
    ks3 = np.zeros((1, 1, BS), np.float32)
    vs3 = ks3.copy()
    oracle.quantize_and_cache(key3, key3, kc3, vc3, ks3, vs3, np.array([1], np.int64), oracle.SCALE_TOKEN)
    assert ks3[0, 0, 1] == 1.0 and list(kc3[0, 0, 1]) == [0x7E, 0xB8, oracle.fp8_e4m3_encode(0.3), 0x01]


def pin_quantising_write_round_trip():
    """Per-token int8: |code * s - x| <= s / 2 and the largest |x| of a row
    maps to +-127; per-token E4M3: the largest |x| maps to +-448 and every
    element is within half a code spacing (relative 2^-4 for normals)."""
    rng = np.random.default_rng(46)
    T, H, D, BS, NB = 9, 2, 32, 16, 4
    x = (rng.standard_normal((T, H, D)) * rng.random((T, H, 1)) * 10).astype(np.float32)
    slots = rng.permutation(NB * BS)[:T].astype(np.int64)
    for dt, qmax in ((np.int8, 127), (np.uint8, 448)):
        kc = np.zeros((NB, H, BS, D), dt)
        vc = kc.copy()
        ks = np.zeros((NB, H, BS), np.float32)
        vs = ks.copy()
        oracle.quantize_and_cache(x, x, kc, vc, ks, vs, slots, oracle.SCALE_TOKEN)
        for t, sl in enumerate(slots):
            for h in range(H):
                row = x[t, h].astype(np.float64)
                s = float(ks[sl // BS, h, sl % BS])
                assert s == float(np.float32(np.float32(np.abs(x[t, h]).max()) / np.float32(qmax)))
                codes = oracle.as_float64(kc[sl // BS, h, sl % BS])
                assert np.max(np.abs(codes)) == qmax
                deq = codes * s
                if dt == np.int8:
                    assert np.max(np.abs(deq - row)) <= 0.5 * s * (1 + 1e-6)
                else:
                    big = np.abs(row) >= 2.0 ** -6 * s
                    assert np.all(np.abs(deq - row)[big] <= np.abs(row)[big] * 2.0 ** -4 * (1 + 1e-6))


def pin_swap_blocks_exact():
    """Swap between pools of different sizes copies whole blocks (K, V and
    their scales in either layout) and nothing else."""
    rng = np.random.default_rng(47)
    H, BS, D = 2, 16, 32
    for mode in (oracle.SCALE_BLOCK, oracle.SCALE_TOKEN):
        sk = rng.integers(-128, 128, (6, H, BS, D)).astype(np.int8)
        sv = rng.integers(-128, 128, (6, H, BS, D)).astype(np.int8)
        dk = rng.integers(-128, 128, (9, H, BS, D)).astype(np.int8)
        dv = rng.integers(-128, 128, (9, H, BS, D)).astype(np.int8)
        sks = rng.random(oracle.scale_shape(6, H, BS, mode)).astype(np.float32)
        svs = rng.random(oracle.scale_shape(6, H, BS, mode)).astype(np.float32)
        dks = rng.random(oracle.scale_shape(9, H, BS, mode)).astype(np.float32)
        dvs = rng.random(oracle.scale_shape(9, H, BS, mode)).astype(np.float32)
        d0 = (dk.copy(), dv.copy(), dks.copy(), dvs.copy())
        pairs = np.array([[5, 0], [2, 8], [5, 3]], np.int64)
        oracle.swap_blocks(sk, sv, dk, dv, pairs, sks, svs, dks, dvs, scale_mode=mode)
        for src, dst in pairs:
            assert np.array_equal(dk[dst], sk[src]) and np.array_equal(dv[dst], sv[src])
            assert np.array_equal(dks[dst], sks[src]) and np.array_equal(dvs[dst], svs[src])
        for b in (1, 2, 4, 5, 6, 7):
            assert np.array_equal(dk[b], d0[0][b]) and np.array_equal(dv[b], d0[1][b])
            assert np.array_equal(dks[b], d0[2][b]) and np.array_equal(dvs[b], d0[3][b])
    # copy_blocks moves per-token scales whole as well
    kc = rng.integers(-128, 128, (4, H, BS, D)).astype(np.int8)
    vc = kc.copy()
    ks = rng.random((4, H, BS)).astype(np.float32)
    vs = rng.random((4, H, BS)).astype(np.float32)
    ks0 = ks.copy()
    oracle.copy_blocks(kc, vc, np.array([[1, 3]], np.int64), ks, vs, scale_mode=oracle.SCALE_TOKEN)
    assert np.array_equal(ks[3], ks0[1]) and np.array_equal(ks[:3], ks0[:3])


# --------------------------------------------------------------------------
# several causal query rows per sequence
# --------------------------------------------------------------------------

def pin_multi_query_closed_forms():
    """Three cached tokens, the last two of them queries (k_t = t e0, v_t =
    e_t, q = e0, scale 1): the first query row sits at position 1 and sees
    logits (0, 1); the second sees (0, 1, 2).  A one-token sequence before
    it (one query row, context 1) returns its v0."""
    g = golden("attention_closed_forms.json")
    D, BS = 64, 2
    K = np.stack([t * unit(D, 0) for t in range(3)])[:, None, :]
    V = np.stack([unit(D, t) for t in range(3)])[:, None, :]
    K0 = np.zeros((1, 1, D), np.float32)
    V0 = (3.0 * unit(D, 5))[None, None, :]
    kc, bt = paginate([K0, K], BS, 5, tables=np.array([[4, -1], [3, 1]]), fill=np.nan)
    vc, _ = paginate([V0, V], BS, 5, tables=bt, fill=np.nan)
    q = np.stack([unit(D, 0), unit(D, 0), unit(D, 0)])[:, None, :]
    out = oracle.paged_attention(q, kc, vc, bt, np.array([1, 3], np.int32), np.array([0, 1, 3], np.int32), 1.0)
    assert out[0, 0, 5] == 3.0 and np.count_nonzero(out[0, 0]) == 1
    assert abs(out[1, 0, 0] - g["ctx2"]["out_d0"]) < 1e-15 and abs(out[1, 0, 1] - g["ctx2"]["out_d1"]) < 1e-15
    assert np.all(out[1, 0, 2:] == 0.0)
    assert np.max(np.abs(out[2, 0, :3] - np.array(g["ctx3"]["out"]))) < 1e-15


def pin_multi_query_rows_are_prefix_decodes():
    """Row i of a sequence with L query rows and context n is the one-query
    decode of the same sequence cut to n - L + i + 1 tokens (rows that see
    nothing are zero), for every row of a random batch."""
    rng = np.random.default_rng(48)
    lens = [5, 17, 33, 3]
    qlens = [1, 4, 16, 5]            # the last sequence has more rows than tokens
    Hq, Hkv, D, BS, NB = 4, 2, 32, 16, 12
    ks = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    vs = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    kc, bt = paginate(ks, BS, NB, rng=rng)
    vc, _ = paginate(vs, BS, NB, tables=bt)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32)
    out = oracle.paged_attention(q, kc, vc, bt, np.array(lens, np.int32), qsl, 0.25)
    for s, (n, L) in enumerate(zip(lens, qlens)):
        for i in range(L):
            r = int(qsl[s]) + i
            m = max(0, n - L + i + 1)
            one = oracle.paged_decode(q[r:r + 1], kc, vc, bt[s:s + 1], np.array([m], np.int32), 0.25)
            assert np.array_equal(out[r], one[0]), (s, i)


def pin_multi_query_matches_library_attention():
    """Several causal query rows against a library routine: torch's
    scaled_dot_product_attention in float64 on the CPU over each sequence's
    contiguous K/V (each kv head repeated for its query heads), with an
    explicit mask in which query row i of L sees the first n - L + i + 1
    tokens (the rows are the sequence's last L tokens); within 1e-12."""
    import torch  # noqa: PLC0415

    rng = np.random.default_rng(49)
    lens = [40, 100, 7, 64, 1]
    qlens = [8, 33, 7, 1, 1]          # every row sees at least one token
    Hq, Hkv, D, BS, NB = 8, 2, 64, 16, 20
    K = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    V = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in lens]
    kc, bt = paginate(K, BS, NB, rng=rng)
    vc, _ = paginate(V, BS, NB, tables=bt)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32)
    scale = 0.125
    out = oracle.paged_attention(q, kc, vc, bt, np.array(lens, np.int32), qsl, scale)
    for s, (n, L) in enumerate(zip(lens, qlens)):
        qs = torch.from_numpy(q[qsl[s]:qsl[s + 1]].astype(np.float64)).permute(1, 0, 2)
        ks = torch.from_numpy(K[s].astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        vs = torch.from_numpy(V[s].astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
        mask = torch.arange(n)[None, :] <= (n - L + torch.arange(L))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask, scale=scale)
        err = np.max(np.abs(out[qsl[s]:qsl[s + 1]] - ref.permute(1, 0, 2).numpy()))
        assert err < 1e-12, (s, err)


QUANT_PINS = [pin_fp8_format_values, pin_fp8_encode, pin_per_token_scales_closed_form,
              pin_quantised_decode_matches_contiguous, pin_quantising_write_hand_values,
              pin_quantising_write_round_trip, pin_swap_blocks_exact]

CACHE_PINS = [pin_slot_mapping_figure, pin_slot_mapping_edges,
              pin_reshape_writes_exactly_one_slot_per_token, pin_copy_blocks_exact,
              pin_quantiser_hand_values, pin_quantiser_invariants]

MULTI_QUERY_PINS = [pin_multi_query_closed_forms, pin_multi_query_rows_are_prefix_decodes,
                    pin_multi_query_matches_library_attention]

ALL_PINS = DECODE_PINS + CACHE_PINS + QUANT_PINS + MULTI_QUERY_PINS
