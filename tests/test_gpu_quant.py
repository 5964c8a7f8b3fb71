"""GPU tests of the quantised-cache paths against the CPU oracle: the
quantising cache write (int8 / E4M3, static and per-token scales) bit for
bit, decode over quantised caches in both scale layouts, the hardware E4M3
decoding of every code, and block swaps to and from pinned host memory."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import TOL_BF16, case_on_device, max_err, quantize_case_by_token, run_decode, say, to_dev, to_host

pytestmark = pytest.mark.gpu

MFMA, VALU = pa.KERNEL_MFMA, pa.KERNEL_VALU
KV_DTYPES = {synth.I8: np.int8, synth.FP8: np.uint8}


def _rows(rng, T, Hkv, D, src):
    """Key/value rows with the awkward values: ties, zeros, huge, tiny."""
    x = (rng.standard_normal((T, Hkv, D)) * rng.uniform(0.01, 30.0, (T, Hkv, 1))).astype(np.float32)
    x[0, 0] = 0.0                                  # all-zero row: scale 1, codes 0
    if T > 1:
        x[1, 0, :8] = [127.0, -63.5, 0.5, 1.5, 2.5, -2.5, 3.5, 1e-30]
        x[1, 0, 8:] = 0.25
    if T > 2:
        x[2, -1, :4] = [1e6, -1e6, 448.0, -448.0]  # saturation under static scales
    if src == "bf16":
        return synth.bf16_bits(x)
    return x


@pytest.mark.parametrize("kv", [synth.I8, synth.FP8])
@pytest.mark.parametrize("mode", [pa.PA_SCALE_BLOCK, pa.PA_SCALE_TOKEN], ids=["static", "per-token"])
@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("D,BS", [(128, 16), (64, 32)])
def test_quantize_and_cache_bit_exact(kv, mode, src, D, BS):
    rng = np.random.default_rng(7 + D + BS + 2 * mode + 5 * (kv == synth.FP8) + 11 * (src == "bf16"))
    NB, Hkv, T = 40, 4, 37
    say("quantize_and_cache", kv, "mode", mode, src, "D", D, "BS", BS)
    key = _rows(rng, T, Hkv, D, src)
    val = _rows(rng, T, Hkv, D, src)
    slots = rng.permutation(NB * BS)[:T].astype(np.int64)
    slots[5] = -1                                   # skipped token
    dt = KV_DTYPES[kv]
    kc = rng.integers(0, 256, (NB, Hkv, BS, D)).astype(np.uint8).view(dt)
    vc = rng.integers(0, 256, (NB, Hkv, BS, D)).astype(np.uint8).view(dt)
    sshape = oracle.scale_shape(NB, Hkv, BS, mode)
    ks = rng.random(sshape).astype(np.float32)
    vs = rng.random(sshape).astype(np.float32)
    st_k, st_v = (0.0, 0.0) if mode == pa.PA_SCALE_TOKEN else (0.05, 0.125)
    dk, dv, dks, dvs = to_dev(kc), to_dev(vc), to_dev(ks), to_dev(vs)
    pa.quantize_and_cache(to_dev(key), to_dev(val), dk, dv, dks, dvs, to_dev(slots), st_k, st_v)
    torch.cuda.synchronize()
    oracle.quantize_and_cache(key, val, kc, vc, ks, vs, slots, mode, st_k, st_v)
    assert np.array_equal(to_host(dk).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(to_host(dv).view(np.uint8), vc.view(np.uint8))
    assert np.array_equal(to_host(dks).view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(to_host(dvs).view(np.uint32), vs.view(np.uint32))


def test_e4m3_codes_decode_exactly():
    """Context length 1 with value scale 1: out = V of the one token, so
    every finite E4M3 code read by the decode kernels must come out as the
    format's exact value (matrix-core and vector-ALU kernels)."""
    table = oracle.fp8_table()
    codes = np.array([c for c in range(256) if not np.isnan(table[c])], np.uint8)   # 254 codes
    D, BS, Hkv = 128, 16, 1
    S = -(-codes.size // D)
    vrows = np.zeros((S, D), np.uint8)
    vrows.flat[:codes.size] = codes
    NB = S
    kc = np.zeros((NB, Hkv, BS, D), np.uint8)
    vc = np.full((NB, Hkv, BS, D), 0x7F, np.uint8)     # NaN past the one token
    vc[:, 0, 0, :] = vrows
    bt = np.arange(NB, dtype=np.int32).reshape(S, 1)
    cl = np.ones(S, np.int32)
    ones = np.ones((NB, Hkv), np.float32)
    expect = table[vrows].reshape(S, 1, D)
    for kern, qd, Hq in ((MFMA, synth.BF16, 4), (MFMA, synth.BF16, 1), (VALU, synth.F32, 1), (VALU, synth.BF16, 2)):
        say("e4m3 exact decode, kernel", kern, qd, Hq)
        q = np.zeros((S, Hq, D), np.float32)
        q = synth.bf16_bits(q) if qd == synth.BF16 else q
        out = pa.decode(to_dev(q), to_dev(kc), to_dev(vc), to_dev(bt), to_dev(cl), 0.1, 1, k_scales=to_dev(ones),
                        v_scales=to_dev(ones), kernel=kern)
        got = out.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, np.repeat(expect, Hq, axis=1)), (kern, Hq)


QUANT_SHAPES = [
    # (Hq, Hkv, D, BS, q dtype, kv dtype, scale mode)
    (32, 8, 128, 16, synth.BF16, synth.I8, pa.PA_SCALE_TOKEN),
    (32, 8, 128, 32, synth.BF16, synth.FP8, pa.PA_SCALE_TOKEN),
    (32, 8, 128, 16, synth.BF16, synth.FP8, pa.PA_SCALE_BLOCK),
    (64, 8, 128, 16, synth.BF16, synth.FP8, pa.PA_SCALE_TOKEN),
    (40, 40, 128, 16, synth.BF16, synth.I8, pa.PA_SCALE_TOKEN),
    (8, 8, 64, 16, synth.F32, synth.FP8, pa.PA_SCALE_TOKEN),
    (8, 2, 64, 32, synth.F32, synth.I8, pa.PA_SCALE_BLOCK),
    (32, 8, 64, 16, synth.BF16, synth.FP8, pa.PA_SCALE_TOKEN),
    (64, 8, 64, 32, synth.BF16, synth.I8, pa.PA_SCALE_BLOCK),
    (16, 4, 64, 16, synth.BF16, synth.I8, pa.PA_SCALE_TOKEN),
]
EDGE_LENS = [0, 1, 2, 15, 16, 17, 33, 255, 256, 257, 1000, 1025]


def _kernels(case):
    ks = [VALU]
    if case.q_dtype == synth.BF16:
        ks.append(MFMA)
    return ks


@pytest.mark.parametrize("shape", QUANT_SHAPES, ids=lambda s: "Hq%d-Hkv%d-D%d-BS%d-%s-%s-mode%d" % s)
def test_quantised_decode_parity(shape):
    Hq, Hkv, D, BS, qd, kvd, mode = shape
    case = synth.make_case("quant", 300 + QUANT_SHAPES.index(shape), EDGE_LENS, Hq, Hkv, D, BS, q_dtype=qd,
                           kv_dtype=kvd, free_frac=0.2)
    quantize_case_by_token(case, mode)
    expect = oracle.paged_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                 float(case.scale), case.k_scales, case.v_scales, scale_mode=mode)
    dev = case_on_device(case)
    for kern in _kernels(case):
        for P in (0, 16, 256):
            for hint in ((False, True) if P == 0 else (False,)):
                say(case.name, shape, "kernel", kern, "partition", P, "hint", hint)
                got = run_decode(case, dev, partition_tokens=P, kernel=kern, length_hint=hint)
                err = max_err(got, expect)
                assert err <= TOL_BF16, (shape, kern, P, err)


@pytest.mark.parametrize("kvd,mode,D", [(synth.I8, pa.PA_SCALE_TOKEN, 128), (synth.FP8, pa.PA_SCALE_TOKEN, 64),
                                        (synth.FP8, pa.PA_SCALE_BLOCK, 128)])
def test_nan_scales_outside_the_context_are_never_used(kvd, mode, D):
    """Scales of slots past a sequence's length (and of free blocks) set to
    NaN: a masked token's weight must stay zero, not 0 x NaN, in the
    single-row decode (both kernels) and with several query rows (the
    shared-tile kernel for 64 rows of 8 heads, the per-wave one for 2)."""
    lens = [1, 15, 17, 100, 257, 1000, 0, 33]
    case = synth.make_case("nan-scales", 380 + D + mode, lens, 64, 8, D, 16, kv_dtype=kvd, free_frac=0.2)
    quantize_case_by_token(case, mode, poison=np.nan)
    expect = oracle.paged_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                 float(case.scale), case.k_scales, case.v_scales, scale_mode=mode)
    assert np.isfinite(expect).all()
    dev = case_on_device(case)
    for kern in (MFMA, VALU):
        for P in (0, 16, 256):
            say("NaN scales", kvd, mode, D, "kernel", kern, "partition", P)
            err = max_err(run_decode(case, dev, partition_tokens=P, kernel=kern), expect)
            assert err <= TOL_BF16, (kvd, mode, D, kern, P, err)
    rng = np.random.default_rng(7)
    for rows in (2, 64):
        qlens = [min(rows, n) for n in lens]
        qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        q = synth.bf16_bits(rng.standard_normal((int(qsl[-1]), 64, D)).astype(np.float32))
        exp_mq = oracle.paged_attention(q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, qsl,
                                        float(case.scale), case.k_scales, case.v_scales, scale_mode=mode)
        for P in (0, 256):
            say("NaN scales, query rows", rows, "partition", P)
            out = pa.decode(to_dev(q), dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale),
                            case.max_context_len, k_scales=dev["ks"], v_scales=dev["vs"], partition_tokens=P,
                            query_start_loc=to_dev(qsl), max_query_len=rows)
            torch.cuda.synchronize()
            err = max_err(out.cpu().numpy().astype(np.float64), exp_mq)
            assert err <= TOL_BF16, (kvd, mode, D, rows, P, err)


def _fused_cases(kvd):
    """A skewed batch (the balanced split with the length hint) and a short
    one of 32 sequences x 8 kv heads (grouped launches)."""
    rng = np.random.default_rng(21)
    skewed = [1, 2, 15, 16, 17, 31, 32, 33, 255, 256, 257] + [int(x) for x in rng.integers(1, 1500, size=28)] + [12000]
    short = [1, 16, 17, 64, 65, 127, 128, 129] + [int(x) for x in rng.integers(1, 1200, size=23)] + [1200]
    for name, lens in (("skewed", skewed), ("short", short)):
        case = synth.make_case("fused-q-" + name, 390 + len(lens), lens, 32, 8, 128, 16, kv_dtype=kvd, free_frac=0.1)
        quantize_case_by_token(case, pa.PA_SCALE_TOKEN)
        yield name, case


@pytest.mark.parametrize("kvd", [synth.I8, synth.FP8])
def test_fused_quantising_write(kvd):
    """pa_decode with new_key/new_value (bf16 rows) on a 1-byte cache with
    per-token scales quantises and stores every sequence's newest token
    and attends with it: codes and scales bit for bit those of the oracle's
    quantising write (and of pa_quantize_and_cache), outputs bit for bit
    those of pa_quantize_and_cache + pa_decode and within tolerance of the
    oracle after its write.  Rows include all-zero ones (scale 1) and a key
    outlier; plain, many-partition, balanced and grouped launches."""
    for name, case in _fused_cases(kvd):
        S, Hkv, D, BS = case.num_seqs, case.num_kv_heads, case.head_dim, case.block_size
        rng = np.random.default_rng(31)
        # rows of unit-order spread (the 2e-3 gate is absolute), one all
        # zero, one key row with an outlier that sets its scale
        kf = (rng.standard_normal((S, Hkv, D)) * rng.uniform(0.05, 4.0, (S, Hkv, 1))).astype(np.float32)
        vf = (rng.standard_normal((S, Hkv, D)) * rng.uniform(0.05, 2.0, (S, Hkv, 1))).astype(np.float32)
        kf[0, 0] = 0.0
        vf[2, 1] = 0.0
        kf[1, -1, :3] = [300.0, -300.0, 0.5]
        nk, nv = synth.bf16_bits(kf), synth.bf16_bits(vf)
        slots = oracle.slot_mapping(case.block_tables, case.context_lens - 1, BS)
        exp_k, exp_v = case.k_cache.copy(), case.v_cache.copy()
        exp_ks, exp_vs = case.k_scales.copy(), case.v_scales.copy()
        oracle.quantize_and_cache(nk, nv, exp_k, exp_v, exp_ks, exp_vs, slots, pa.PA_SCALE_TOKEN, 0.0, 0.0)
        expect = oracle.paged_decode(case.q, exp_k, exp_v, case.block_tables, case.context_lens, float(case.scale),
                                     exp_ks, exp_vs, scale_mode=pa.PA_SCALE_TOKEN)
        dnk, dnv = to_dev(nk), to_dev(nv)
        total = int(np.sum(case.context_lens, dtype=np.int64))
        for P, hint in ((0, False), (16, False), (0, True), (256, False)):
            say("fused quantising write", kvd, name, "partition", P, "hint", hint)
            kw = dict(partition_tokens=P, total_context_len=total if hint else 0)
            a = case_on_device(case)
            sl = pa.slot_mapping(a["bt"], BS, context_lens=a["cl"])
            pa.quantize_and_cache(dnk, dnv, a["k"], a["v"], a["ks"], a["vs"], sl)
            out_a = pa.decode(a["q"], a["k"], a["v"], a["bt"], a["cl"], float(case.scale), case.max_context_len,
                              k_scales=a["ks"], v_scales=a["vs"], **kw)
            b = case_on_device(case)
            out_b = pa.decode(b["q"], b["k"], b["v"], b["bt"], b["cl"], float(case.scale), case.max_context_len,
                              k_scales=b["ks"], v_scales=b["vs"], new_key=dnk, new_value=dnv, **kw)
            torch.cuda.synchronize()
            for key in ("k", "v", "ks", "vs"):
                assert np.array_equal(to_host(b[key]), to_host(a[key])), (name, P, hint, key)
            assert np.array_equal(to_host(b["k"]), exp_k) and np.array_equal(to_host(b["v"]), exp_v)
            assert np.array_equal(to_host(b["ks"]), exp_ks) and np.array_equal(to_host(b["vs"]), exp_vs)
            ob = out_b.cpu().numpy().astype(np.float64)
            assert np.array_equal(out_a.cpu().numpy().astype(np.float64), ob), (name, P, hint)
            err = max_err(ob, expect)
            assert err <= TOL_BF16, (kvd, name, P, hint, err)


@pytest.mark.parametrize("kvd", [synth.I8, synth.FP8])
def test_config5_per_token_scales(kvd):
    """The int8 workload's batch (64 sequences, log-normal lengths) with
    per-token scales, as int8 and as E4M3."""
    case = synth.config5()
    if kvd == synth.FP8:
        case.kv_dtype = synth.FP8
        case.k_cache = case.k_cache.view(np.uint8)
        case.v_cache = case.v_cache.view(np.uint8)
    quantize_case_by_token(case, pa.PA_SCALE_TOKEN)
    expect = oracle.paged_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                 float(case.scale), case.k_scales, case.v_scales, scale_mode=pa.PA_SCALE_TOKEN)
    dev = case_on_device(case)
    for kern in (MFMA, VALU):
        say("config5 per-token", kvd, "kernel", kern)
        err = max_err(run_decode(case, dev, kernel=kern, length_hint=True), expect)
        assert err <= TOL_BF16, (kvd, kern, err)


def test_decode_step_with_quantising_write():
    """One decode step on a per-token E4M3 cache: write each newest token
    with pa_quantize_and_cache, then decode; caches, scales and outputs
    against the oracle doing the same two steps."""
    lens = [1, 16, 17, 100, 513]
    case = synth.make_case("qstep", 77, lens, 32, 8, 128, 16, kv_dtype=synth.FP8, free_frac=0.1)
    mode = pa.PA_SCALE_TOKEN
    quantize_case_by_token(case, mode)
    rng = np.random.default_rng(78)
    kn = synth.bf16_bits(rng.standard_normal((len(lens), 8, 128)).astype(np.float32))
    vn = synth.bf16_bits(rng.standard_normal((len(lens), 8, 128)).astype(np.float32))
    dev = case_on_device(case)
    slots = pa.slot_mapping(dev["bt"], 16, context_lens=dev["cl"])
    pa.quantize_and_cache(to_dev(kn), to_dev(vn), dev["k"], dev["v"], dev["ks"], dev["vs"], slots)
    torch.cuda.synchronize()
    exp_slots = oracle.slot_mapping(case.block_tables, case.context_lens - 1, 16)
    oracle.quantize_and_cache(kn, vn, case.k_cache, case.v_cache, case.k_scales, case.v_scales, exp_slots, mode)
    assert np.array_equal(to_host(dev["k"]), case.k_cache) and np.array_equal(to_host(dev["v"]), case.v_cache)
    assert np.array_equal(to_host(dev["ks"]), case.k_scales) and np.array_equal(to_host(dev["vs"]), case.v_scales)
    expect = oracle.paged_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                 float(case.scale), case.k_scales, case.v_scales, scale_mode=mode)
    err = max_err(run_decode(case, dev), expect)
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("where", ["device-to-host", "host-to-device", "device-to-device"])
@pytest.mark.parametrize("quant", [False, True], ids=["bf16", "int8-per-token"])
def test_swap_blocks_bit_exact(where, quant):
    rng = np.random.default_rng(90 + quant)
    Hkv, BS, D, sNB, dNB = 8, 16, 128, 50, 70
    dt = np.int8 if quant else np.uint16
    isz = np.dtype(dt).itemsize

    def pool(nb):
        return rng.integers(0, 256, (nb, Hkv, BS, D * isz), dtype=np.uint8).view(dt)

    src_k, src_v, dst_k, dst_v = pool(sNB), pool(sNB), pool(dNB), pool(dNB)
    scl = [rng.random(s).astype(np.float32) for s in ((sNB, Hkv, BS), (sNB, Hkv, BS), (dNB, Hkv, BS),
                                                       (dNB, Hkv, BS))] if quant else [None] * 4
    pairs = np.stack([rng.permutation(sNB)[:30], rng.permutation(dNB)[:30]], axis=1).astype(np.int64)
    pairs[3] = [-1, 5]                                  # skipped pair

    def place(a, host):
        if a is None:
            return None
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        return t.pin_memory() if host else t.to("cuda:0")

    def bits(t):
        t = t.detach().cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    src_host, dst_host = where == "host-to-device", where == "device-to-host"
    S = [place(a, src_host) for a in (src_k, src_v, scl[0], scl[1])]
    Dd = [place(a, dst_host) for a in (dst_k, dst_v, scl[2], scl[3])]
    say("swap", where, "quant", quant)
    pa.swap_blocks(S[0], S[1], Dd[0], Dd[1], to_dev(pairs), S[2], S[3], Dd[2], Dd[3])
    torch.cuda.synchronize()
    # the library skips a pair with an id outside its pool; the oracle takes the others
    keep = pairs[:, 0] >= 0
    oracle.swap_blocks(src_k, src_v, dst_k, dst_v, pairs[keep], scl[0], scl[1], scl[2], scl[3],
                       scale_mode=oracle.SCALE_TOKEN)
    assert np.array_equal(bits(Dd[0]), dst_k) and np.array_equal(bits(Dd[1]), dst_v)
    if quant:
        assert np.array_equal(bits(Dd[2]), scl[2]) and np.array_equal(bits(Dd[3]), scl[3])


def test_swap_refuses_pageable_host_memory():
    k = torch.zeros(4, 1, 16, 64, dtype=torch.bfloat16)          # not pinned
    d = torch.zeros(4, 1, 16, 64, dtype=torch.bfloat16, device="cuda:0")
    pairs = torch.tensor([[0, 1]], dtype=torch.int64, device="cuda:0")
    lib = pa.library()
    st = lib.pa_swap_blocks(k.data_ptr(), k.data_ptr(), None, None, d.data_ptr(), d.data_ptr(), None, None,
                            pa.PA_BF16, 0, pairs.data_ptr(), 1, 1, 64, 16, 4, 4, None)
    assert st == pa.PA_ERR_INVALID and "pinned" in lib.pa_last_error().decode()
