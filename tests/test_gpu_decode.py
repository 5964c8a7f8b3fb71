"""Paged decode on the GPU against the CPU oracle.

Tolerance: max |gpu - oracle| over every output element, 2e-3 for bf16 or
int8 inputs (fp32 accumulation) and 1e-5 for fp32 inputs.  Every case runs
through the C ABI; unused cache memory is NaN-poisoned (int8: +127)."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import (GUARD_BF16, TOL_BF16, TOL_F32, case_on_device, max_err, quantize_case, run_decode, run_oracle, say,
                         to_dev, to_host, tolerance)

pytestmark = pytest.mark.gpu

VALU, MFMA = pa.KERNEL_VALU, pa.KERNEL_MFMA


def _kernels(case):
    ks = [0, VALU]
    if case.q_dtype == synth.BF16 and case.kv_dtype in (synth.BF16, synth.I8):
        ks.append(MFMA)
    return ks


def _check_all_kernels(case, partitions=(0,), expect=None):
    expect = run_oracle(case) if expect is None else expect
    dev = case_on_device(case)
    tol = tolerance(case)
    for kern in _kernels(case):
        for P in partitions:
            # the library's own split is taken with and without the length hint
            for hint in ((False, True) if P == 0 else (False,)):
                say(case.name, "kernel", kern, "partition", P, "hint", hint)
                got = run_decode(case, dev, partition_tokens=P, kernel=kern, length_hint=hint)
                err = max_err(got, expect)
                assert err <= tol, (case.name, kern, P, hint, err)
    return expect


# --------------------------------------------------------------------------
# the five workload configurations
# --------------------------------------------------------------------------

def test_config1_tiny_fp32():
    case = synth.config1()
    _check_all_kernels(case, partitions=(0, 16, 64, 208))


def test_config2_llama13b_mha():
    case = synth.config2()
    _check_all_kernels(case, partitions=(0, 256))


def test_config4_prefix_share_cow_step():
    """One timed step of the prefix-sharing workload: copy the shared partial
    block to every sequence's scratch block, write each newest token, decode;
    copies and writes bit-exact over the whole pool, attention within
    tolerance."""
    case = synth.config4()
    e = case.extra
    dev = case_on_device(case)
    pairs = np.stack([np.full(50, e["partial"]), e["scratch"]], axis=1).astype(np.int64)
    say("config4 copy + slot mapping + reshape")
    pa.copy_blocks(dev["k"], dev["v"], to_dev(pairs))
    slots = pa.slot_mapping(dev["bt"], case.block_size, context_lens=dev["cl"])
    pa.reshape_and_cache(to_dev(e["k_new"]), to_dev(e["v_new"]), dev["k"], dev["v"], slots)
    torch.cuda.synchronize()
    oracle.copy_blocks(case.k_cache, case.v_cache, pairs)
    exp_slots = oracle.slot_mapping(case.block_tables, case.context_lens - 1, case.block_size)
    assert np.array_equal(to_host(slots), exp_slots)
    oracle.reshape_and_cache(e["k_new"], e["v_new"], case.k_cache, case.v_cache, exp_slots)
    assert np.array_equal(to_host(dev["k"]), case.k_cache)
    assert np.array_equal(to_host(dev["v"]), case.v_cache)
    expect = run_oracle(case)
    for kern in _kernels(case):
        say("config4 decode kernel", kern)
        err = max_err(run_decode(case, dev, kernel=kern), expect)
        assert err <= TOL_BF16, (kern, err)


def test_config5_int8():
    case = synth.config5()
    quantize_case(case)
    expect = _check_all_kernels(case, partitions=(0, 512))
    # quantisation error against unquantised attention is reported, not gated
    ref = oracle.paged_decode(synth.bits_to_f32(case.q), case.extra["k_f32"], case.extra["v_f32"],
                              case.block_tables, case.context_lens, float(case.scale))
    print("config5 quantisation error vs fp32 KV: %.3e" % np.max(np.abs(expect - ref)))


def _seq_slice(k, v, bt_row, n, BS):
    """One sequence's blocks as a stand-alone pool with an identity table."""
    nb = -(-n // BS)
    ids = torch.as_tensor(bt_row[:nb].astype(np.int64), device=k.device)
    return to_host(k.index_select(0, ids)), to_host(v.index_select(0, ids)), np.arange(nb, dtype=np.int32)[None]


def test_config3_full_size_sampled():
    """One 70B-shaped layer at full size (20 x 8,000 tokens, 10,000 blocks)
    through the plain pa.decode call (no fused write, no length hint), on
    both kernels; four sequences checked in full against the oracle on
    bytes read back from the device.  The benchmark's own call form (fused
    write, hint, graph replay) is checked on every sequence in
    test_gpu_headline.py."""
    st = synth.config3_structure()
    say("config3 layer 0 generation")
    q, k, v, _, _ = synth.config3_layer_values(0, "cuda:0")
    bt, cl = to_dev(st["block_tables"]), to_dev(st["context_lens"])
    for kern in (0, VALU):
        say("config3 decode kernel", kern)
        out = pa.decode(q, k, v, bt, cl, float(st["scale"]), 8000, kernel=kern)
        torch.cuda.synchronize()
        out = out.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(out))
        for s in (0, 7, 13, 19):
            kc, vc, tab = _seq_slice(k, v, st["block_tables"][s], 8000, 16)
            qs = to_host(q[s:s + 1])
            exp = oracle.paged_decode(qs, kc, vc, tab, np.array([8000], np.int32), float(st["scale"]))
            err = max_err(out[s:s + 1], exp)
            say("sequence", s, "max |gpu - oracle| = %.3e" % err)
            assert err <= TOL_BF16, (kern, s, err)
            assert err <= GUARD_BF16, (kern, s, err)


# --------------------------------------------------------------------------
# shapes, lengths, kernels, partitions
# --------------------------------------------------------------------------

EDGE_LENS = [0, 1, 2, 3, 15, 16, 17, 31, 32, 33, 100, 255, 256, 257, 1000, 1023, 1025]

SHAPES = [
    # (Hq, Hkv, D, BS, q dtype, kv dtype)
    (8, 8, 64, 16, synth.F32, synth.F32),
    (8, 2, 64, 32, synth.F32, synth.F32),
    (4, 4, 128, 16, synth.F32, synth.BF16),
    (40, 40, 128, 16, synth.BF16, synth.BF16),
    (16, 8, 128, 16, synth.BF16, synth.BF16),
    (32, 8, 128, 16, synth.BF16, synth.BF16),
    (32, 8, 128, 32, synth.BF16, synth.BF16),
    (64, 8, 128, 16, synth.BF16, synth.BF16),
    (64, 4, 128, 16, synth.BF16, synth.BF16),
    (12, 4, 128, 32, synth.BF16, synth.BF16),
    (16, 16, 64, 16, synth.BF16, synth.BF16),
    (64, 8, 64, 16, synth.BF16, synth.BF16),
    (32, 8, 64, 32, synth.BF16, synth.BF16),
    (32, 8, 128, 16, synth.BF16, synth.I8),
    (32, 8, 128, 32, synth.BF16, synth.I8),
    (32, 8, 64, 16, synth.BF16, synth.I8),
    (16, 16, 64, 32, synth.BF16, synth.I8),
    (8, 8, 64, 16, synth.F32, synth.I8),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "Hq%d-Hkv%d-D%d-BS%d-%s-%s" % s)
def test_edge_lengths_all_kernels(shape):
    Hq, Hkv, D, BS, qd, kvd = shape
    seed = 100 + SHAPES.index(shape)
    case = synth.make_case("edge", seed, EDGE_LENS, Hq, Hkv, D, BS, q_dtype=qd, kv_dtype=kvd, free_frac=0.2)
    if kvd == synth.I8:
        quantize_case(case)
    _check_all_kernels(case, partitions=(0, 16, 48, 256, 1024))


def test_closed_forms_on_gpu(golden):
    """The hand cases of the oracle's pins: logits (0, 1) and (0, 1, 2) with
    one-hot values, in fp32 and in bf16 (all values exact in bf16)."""
    g = golden("attention_closed_forms.json")
    for qd, kvd, D, Hq, Hkv in ((synth.F32, synth.F32, 64, 1, 1), (synth.BF16, synth.BF16, 128, 8, 1)):
        for ctx in (2, 3):
            K = np.zeros((ctx, Hkv, D), np.float32)
            V = np.zeros((ctx, Hkv, D), np.float32)
            for t in range(ctx):
                K[t, :, 0] = t
                V[t, :, t] = 1.0
            case = synth.make_case("hand", 1, [ctx], Hq, Hkv, D, 16, num_blocks=3, q_dtype=qd, kv_dtype=kvd,
                                   scale=1.0)
            b = case.block_tables[0, 0]
            conv = synth.bf16_bits if kvd == synth.BF16 else (lambda x: x)
            case.k_cache[b, :, :ctx, :] = conv(K.transpose(1, 0, 2))
            case.v_cache[b, :, :ctx, :] = conv(V.transpose(1, 0, 2))
            qv = np.zeros((1, Hq, D), np.float32)
            qv[:, :, 0] = 1.0
            case.q = synth.bf16_bits(qv) if qd == synth.BF16 else qv
            want = [g["ctx2"]["out_d0"], g["ctx2"]["out_d1"]] if ctx == 2 else g["ctx3"]["out"]
            for kern in _kernels(case):
                say("closed form ctx", ctx, qd, kern)
                out = run_decode(case, kernel=kern)
                tol = TOL_F32 if kvd == synth.F32 else TOL_BF16
                assert np.max(np.abs(out[0, :, :ctx] - np.array(want))) <= tol
                assert np.all(out[0, :, ctx:] == 0.0)


def test_ctx1_is_exactly_v0():
    case = synth.make_case("ctx1", 3, [1, 1, 1], 32, 8, 128, 16)
    for kern in _kernels(case):
        say("ctx1 kernel", kern)
        out = run_decode(case, kernel=kern)
        for s in range(3):
            v0 = synth.bits_to_f32(case.v_cache[case.block_tables[s, 0], :, 0, :]).astype(np.float64)
            assert np.array_equal(out[s], np.repeat(v0, 4, axis=0)), kern


def test_block_table_figure(golden):
    """The figure's request: table [7, 2, 11], 48 tokens in a pool of 12
    blocks whose free block 1 and foreign block 0 hold NaN."""
    g = golden("block_table_figure.json")
    rng = np.random.default_rng(12)
    NB, H, D, BS = g["pool_blocks"], 8, 128, g["block_size"]
    k = synth.bf16_bits(rng.standard_normal((NB, H, BS, D), dtype=np.float32))
    v = synth.bf16_bits(rng.standard_normal((NB, H, BS, D), dtype=np.float32))
    for b in g["free_blocks"] + g["other_request_blocks"]:
        k[b] = synth.BF16_NAN
        v[b] = synth.BF16_NAN
    case = synth.make_case("figure", 12, [g["tokens"]], 32, H, D, BS, num_blocks=NB)
    case.k_cache, case.v_cache = k, v
    case.block_tables = np.array([g["table"]], np.int32)
    _check_all_kernels(case, partitions=(0, 16))


# --------------------------------------------------------------------------
# invariances
# --------------------------------------------------------------------------

def test_permutation_invariance_bit_identical():
    case = synth.make_case("perm", 41, [300, 77, 1000, 5], 32, 8, 128, 16, free_frac=0.3)
    rng = np.random.default_rng(42)
    pi = rng.permutation(case.num_blocks)
    moved = synth.make_case("perm", 41, [300, 77, 1000, 5], 32, 8, 128, 16, free_frac=0.3)
    moved.k_cache = np.empty_like(case.k_cache)
    moved.v_cache = np.empty_like(case.v_cache)
    moved.k_cache[pi] = case.k_cache
    moved.v_cache[pi] = case.v_cache
    moved.block_tables = np.where(case.block_tables >= 0, pi[np.maximum(case.block_tables, 0)], -1).astype(np.int32)
    for kern in _kernels(case):
        say("permutation kernel", kern)
        a = run_decode(case, kernel=kern)
        b = run_decode(moved, kernel=kern)
        assert np.array_equal(a, b), kern


def test_prefix_sharing_bit_identical():
    """Sequences 0 and 1 hold identical queries and logical K/V: sharing the
    physical blocks or holding private copies gives the same bits."""
    case = synth.make_case("share", 43, [700, 700, 90], 32, 8, 128, 32, free_frac=0.2)
    case.q[1] = case.q[0]
    n0 = -(-700 // 32)
    for j in range(n0):
        case.k_cache[case.block_tables[1, j]] = case.k_cache[case.block_tables[0, j]]
        case.v_cache[case.block_tables[1, j]] = case.v_cache[case.block_tables[0, j]]
    shared = synth.make_case("share", 43, [700, 700, 90], 32, 8, 128, 32, free_frac=0.2)
    shared.q, shared.k_cache, shared.v_cache = case.q, case.k_cache, case.v_cache
    shared.block_tables = case.block_tables.copy()
    shared.block_tables[1] = case.block_tables[0]
    for kern in _kernels(case):
        say("prefix sharing kernel", kern)
        a = run_decode(case, kernel=kern)
        b = run_decode(shared, kernel=kern)
        assert np.array_equal(a[0], a[1]) and np.array_equal(a, b), kern


def test_deterministic_across_runs():
    case = synth.make_case("det", 44, [4000, 17, 2500], 64, 8, 128, 16)
    dev = case_on_device(case)
    for kern in _kernels(case):
        say("determinism kernel", kern)
        a = run_decode(case, dev, kernel=kern)
        b = run_decode(case, dev, kernel=kern)
        assert np.array_equal(a, b)


def test_explicit_workspace_and_stream():
    """Caller-owned workspace on a side stream gives the same bits."""
    case = synth.make_case("ws", 45, [3000, 1200], 32, 8, 128, 16)
    dev = case_on_device(case)
    a = run_decode(case, dev, partition_tokens=256)
    args = pa.make_decode_args(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale), 3000,
                               out=torch.empty(2, 32, 128, device="cuda:0"), partition_tokens=256)
    need = pa.decode_workspace_size(args)
    assert need > 0
    ws = torch.zeros(need + 64, dtype=torch.uint8, device="cuda:0")
    side = torch.cuda.Stream()
    say("explicit workspace, side stream")
    with torch.cuda.stream(side):
        out = pa.decode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale), 3000,
                        workspace=ws, partition_tokens=256)
    side.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.float64), a)


def test_workspace_reused_across_shapes():
    """One workspace (filled with garbage first) serves calls of different
    shapes and partition sizes back to back."""
    big = synth.make_case("ws-big", 46, [5000, 3000, 700], 64, 8, 128, 16)
    small = synth.make_case("ws-small", 47, [900, 33], 32, 8, 128, 32)
    db, ds = case_on_device(big), case_on_device(small)
    ws = torch.full((64 << 20,), 0xA5, dtype=torch.uint8, device="cuda:0")
    for case, dev, P in ((big, db, 256), (small, ds, 64), (big, db, 0), (small, ds, 0), (big, db, 256)):
        say("workspace reuse", case.name, P)
        for kern in _kernels(case):
            out = pa.decode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale),
                            case.max_context_len, workspace=ws, partition_tokens=P, kernel=kern)
            torch.cuda.synchronize()
            err = max_err(out.cpu().numpy().astype(np.float64), run_oracle(case))
            assert err <= TOL_BF16, (case.name, P, kern, err)


def test_graph_replay_matches_eager():
    """A captured step (slot mapping, cache write, decode) replayed several
    times, with eager work and synchronisations between replays, gives the
    eager result every time."""
    case = synth.make_case("graph", 48, [4000, 1234, 64, 8000], 64, 8, 128, 16)
    dev = case_on_device(case)
    kn = to_dev(synth.bf16_bits(np.random.default_rng(5).standard_normal((4, 8, 128), dtype=np.float32)))
    out = torch.zeros(4, 64, 128, device="cuda:0")
    slots = torch.empty(4, dtype=torch.int64, device="cuda:0")
    main = torch.cuda.current_stream()

    def calls(stream):
        return [pa.prepare_slot_mapping(dev["bt"], 16, slots, context_lens=dev["cl"], stream=stream),
                pa.prepare_reshape_and_cache(kn, kn, dev["k"], dev["v"], slots, stream=stream),
                pa.PreparedDecode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale), 8000, out,
                                  stream=stream)]

    say("graph eager reference")
    for f in calls(main):
        f()
    torch.cuda.synchronize()
    ref = out.clone()
    cap = torch.cuda.Stream()
    cap.wait_stream(main)
    gcalls = calls(cap)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for f in gcalls:
            f()
    torch.cuda.synchronize()
    for i in range(4):
        say("graph replay", i)
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i
        for f in calls(main):  # eager work between replays
            f()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i


# --------------------------------------------------------------------------
# fused cache write (new_key / new_value)
# --------------------------------------------------------------------------

FUSED_SHAPES = [
    (64, 8, 128, 16, synth.BF16, synth.BF16),
    (32, 8, 128, 32, synth.BF16, synth.BF16),
    (40, 40, 128, 16, synth.BF16, synth.BF16),
    (16, 16, 64, 16, synth.BF16, synth.BF16),
    (32, 8, 64, 16, synth.BF16, synth.BF16),
    (8, 8, 64, 16, synth.F32, synth.F32),
    (8, 2, 64, 32, synth.F32, synth.F32),
]


@pytest.mark.parametrize("shape", FUSED_SHAPES, ids=lambda s: "Hq%d-Hkv%d-D%d-BS%d-%s-%s" % s)
def test_fused_cache_write(shape):
    """pa_decode with new_key/new_value == slot mapping + reshape_and_cache +
    pa_decode: caches bit-identical (and equal to the oracle's write),
    outputs bit-identical, and within tolerance of the oracle."""
    Hq, Hkv, D, BS, qd, kvd = shape
    lens = [0, 1, 16, 17, 31, 32, 33, 500, 1000, 2049]
    case = synth.make_case("fused", 200 + FUSED_SHAPES.index(shape), lens, Hq, Hkv, D, BS, q_dtype=qd,
                           kv_dtype=kvd, free_frac=0.1)
    rng = np.random.default_rng(7)
    nk = rng.standard_normal((len(lens), Hkv, D), dtype=np.float32)
    nv = rng.standard_normal((len(lens), Hkv, D), dtype=np.float32)
    if kvd == synth.BF16:
        nk, nv = synth.bf16_bits(nk), synth.bf16_bits(nv)
    # oracle: write the newest tokens, then attend
    slots = oracle.slot_mapping(case.block_tables, case.context_lens - 1, BS)
    exp_k, exp_v = case.k_cache.copy(), case.v_cache.copy()
    oracle.reshape_and_cache(nk, nv, exp_k, exp_v, slots)
    updated = synth.make_case("fused", 200 + FUSED_SHAPES.index(shape), lens, Hq, Hkv, D, BS, q_dtype=qd,
                              kv_dtype=kvd, free_frac=0.1)
    updated.k_cache, updated.v_cache = exp_k, exp_v
    expect = run_oracle(updated)
    dnk, dnv = to_dev(nk), to_dev(nv)
    for kern in _kernels(case):
        for P in (0, 16, 256):
            say("fused write", shape, "kernel", kern, "partition", P)
            a = case_on_device(case)
            sl = pa.slot_mapping(a["bt"], BS, context_lens=a["cl"])
            pa.reshape_and_cache(dnk, dnv, a["k"], a["v"], sl)
            out_a = pa.decode(a["q"], a["k"], a["v"], a["bt"], a["cl"], float(case.scale), case.max_context_len,
                              partition_tokens=P, kernel=kern)
            b = case_on_device(case)
            out_b = pa.decode(b["q"], b["k"], b["v"], b["bt"], b["cl"], float(case.scale), case.max_context_len,
                              partition_tokens=P, kernel=kern, new_key=dnk, new_value=dnv)
            torch.cuda.synchronize()
            kb, vb = to_host(b["k"]), to_host(b["v"])
            assert np.array_equal(kb.view(np.uint8), exp_k.view(np.uint8))
            assert np.array_equal(vb.view(np.uint8), exp_v.view(np.uint8))
            assert np.array_equal(to_host(a["k"]).view(np.uint8), kb.view(np.uint8))
            oa = out_a.cpu().numpy().astype(np.float64)
            ob = out_b.cpu().numpy().astype(np.float64)
            assert np.array_equal(oa, ob), (kern, P)
            err = max_err(ob, expect)
            assert err <= tolerance(case), (kern, P, err)


@pytest.mark.parametrize("kvd", [synth.BF16, synth.I8])
def test_block_outside_the_pool_contributes_nothing(kvd):
    """An in-use table entry outside [0, num_blocks) -- a caller error that
    PA_DEBUG reports -- is never read: its tokens drop out of the sequence,
    so the result equals the oracle's attention over the sequence with that
    block removed (attention does not depend on token order).  Library
    partitions (short: the masked tile body) and 1,024-token partitions (the
    bad block deep inside a run of fully visible tiles: the mask-free
    body)."""
    case = synth.make_case("bad-block", 91, [1000, 700, 33], 32, 8, 128, 16, kv_dtype=kvd)
    if kvd == synth.I8:
        quantize_case(case)
    NB = case.k_cache.shape[0]
    ref_tables = case.block_tables.copy()
    ref_lens = case.context_lens.copy()
    for s, k in ((0, 20), (1, 3)):                 # full blocks, inside the sequence
        row = list(case.block_tables[s])
        ref_tables[s] = row[:k] + row[k + 1:] + [-1]
        ref_lens[s] -= 16
    case.block_tables[0, 20] = NB + 7
    case.block_tables[1, 3] = -5
    expect = oracle.paged_decode(case.q, case.k_cache, case.v_cache, ref_tables, ref_lens, float(case.scale),
                                 case.k_scales, case.v_scales)
    dev = case_on_device(case)
    kernels = (0, VALU, MFMA) if kvd == synth.BF16 else (MFMA,)
    for kern in kernels:
        for P in (0, 1024):
            say("block outside the pool", kvd, "kernel", kern, "partition", P)
            err = max_err(run_decode(case, dev, partition_tokens=P, kernel=kern), expect)
            assert err <= TOL_BF16, (kvd, kern, P, err)
