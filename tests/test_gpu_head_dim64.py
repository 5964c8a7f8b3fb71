"""head_dim 64 on the matrix-core kernel (bf16 queries; bf16, int8 or E4M3
cache) against the CPU oracle, in every launch form the plan can pick: one wave per
partition with the merge, a grouped launch (at least 256 (sequence, kv
head) items), the balanced split of a skewed batch, a shared prefix read
once, several query rows per sequence (one and two column groups per wave),
and the fused cache write.  A bf16 row (128 bytes) is loaded like a 1-byte
cache's row at head_dim 128 (two 16-byte chunks per lane for K, an 8-byte
sixteenth of each V row); a 1-byte row (64 bytes) in one 16-byte K chunk
per lane and a 4-byte sixteenth of each V row; either way two score
products and four accumulator blocks per tile.

Tolerance max |gpu - oracle| <= 2e-3; the fused write bit-exact; a forced
vector-ALU run of the same call within the same tolerance."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import (TOL_BF16, case_on_device, max_err, quantize_case, quantize_case_by_token, run_decode,
                         run_oracle, say, to_dev, to_host)

pytestmark = pytest.mark.gpu

D = 64


def _ws_bytes(case, dev, P=0, hint=0, **kw):
    a = pa.make_decode_args(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale),
                            case.max_context_len, partition_tokens=P, total_context_len=hint, **kw)
    return pa.decode_workspace_size(a)


@pytest.mark.parametrize("Hq,Hkv,BS", [(64, 8, 16), (32, 8, 32), (16, 16, 16), (32, 2, 16)])
def test_decode_head_dim64(Hq, Hkv, BS):
    lens = [0, 1, 15, 16, 17, 33, 100, 255, 256, 257, 1000, 2049, 3000]
    case = synth.make_case("d64", 300 + Hq + BS, lens, Hq, Hkv, D, BS, free_frac=0.1)
    expect = run_oracle(case)
    dev = case_on_device(case)
    for kern in (0, pa.KERNEL_MFMA, pa.KERNEL_VALU):
        for P in (0, 16, 256, 2048):
            say("head_dim 64", (Hq, Hkv, BS), "kernel", kern, "partition", P)
            err = max_err(run_decode(case, dev, partition_tokens=P, kernel=kern), expect)
            assert err <= TOL_BF16, (Hq, Hkv, BS, kern, P, err)


def test_grouped_head_dim64():
    """32 sequences x 8 kv heads = 256 items: one workgroup per item."""
    rng = np.random.default_rng(3)
    lens = [0, 1, 16, 17, 511, 512, 513] + [int(x) for x in rng.integers(1, 1201, size=24)] + [1200]
    case = synth.make_case("d64-grouped", 310, lens, 64, 8, D, 16, free_frac=0.1)
    expect = run_oracle(case)
    dev = case_on_device(case)
    for P in (0, 160, 512):
        assert _ws_bytes(case, dev, P) == 0, P           # grouped: no partials
        say("head_dim 64 grouped, partition", P)
        err = max_err(run_decode(case, dev, partition_tokens=P), expect)
        assert err <= TOL_BF16, (P, err)


def test_balanced_head_dim64():
    """A skewed batch with the length hint: the balanced split."""
    rng = np.random.default_rng(4)
    lens = np.clip(np.rint(rng.lognormal(np.log(200), 1.0, size=40)), 0, 5000).astype(np.int32)
    lens[0] = 5000
    case = synth.make_case("d64-balanced", 320, lens, 32, 8, D, 16, free_frac=0.05)
    expect = run_oracle(case)
    dev = case_on_device(case)
    say("head_dim 64 balanced split")
    err = max_err(run_decode(case, dev, length_hint=True), expect)
    assert err <= TOL_BF16, err


def test_shared_prefix_head_dim64():
    pb, BS = 5, 32
    L = pb * BS
    lens = [L + 300, L - 7, L, L + 1, L + 40, 0, L + 129, L + 999]
    case = synth.make_case("d64-prefix", 330, lens, 32, 8, D, BS, free_frac=0.1)
    case.block_tables[:, :pb] = case.block_tables[0, :pb]
    expect = run_oracle(case)
    dev = case_on_device(case)
    table = to_dev(np.ascontiguousarray(case.block_tables[0, :pb]))
    for P in (0, 64):
        say("head_dim 64 shared prefix, partition", P)
        out = pa.decode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale), case.max_context_len,
                        partition_tokens=P, shared_prefix_table=table, shared_prefix_len=L)
        torch.cuda.synchronize()
        err = max_err(out.cpu().numpy().astype(np.float64), expect)
        assert err <= TOL_BF16, (P, err)


@pytest.mark.parametrize("Hq,Hkv,rows", [(32, 8, 4), (64, 8, 4), (16, 16, 3)])
def test_multi_query_head_dim64(Hq, Hkv, rows):
    """rows causal query rows per sequence: G x rows columns, one column
    group (32/8 x 4 = 16) or two (64/8 x 4 = 32) per item."""
    lens = [1, 17, 100, 257, 1000, 2, 3]
    qlens = [min(rows, n) for n in lens]
    case = synth.make_case("d64-mq", 340 + Hq + rows, lens, Hq, Hkv, D, 16, free_frac=0.2)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    rng = np.random.default_rng(5)
    q = synth.bf16_bits(rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32))
    expect = oracle.paged_attention(q, case.k_cache, case.v_cache, case.block_tables, case.context_lens, qsl,
                                    float(case.scale))
    dev = case_on_device(case)
    dq, dqsl = to_dev(q), to_dev(qsl)
    for P in (0, 16, 256):
        say("head_dim 64 multi-query", (Hq, Hkv, rows), "partition", P)
        out = pa.decode(dq, dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale), case.max_context_len,
                        partition_tokens=P, query_start_loc=dqsl, max_query_len=rows)
        torch.cuda.synchronize()
        err = max_err(out.cpu().numpy().astype(np.float64), expect)
        assert err <= TOL_BF16, (Hq, Hkv, rows, P, err)


@pytest.mark.parametrize("S", [8, 40])
def test_fused_write_head_dim64(S):
    """The newest token's K row (8 chunks of 16 bytes) and V row (16 pieces
    of 8 bytes) written by the wave that attends to it: caches bit-exact,
    output as the oracle's after the oracle's write (40 sequences x 8 kv
    heads: a grouped launch)."""
    rng = np.random.default_rng(S)
    lens = [int(x) for x in rng.integers(1, 1500, size=S)]
    lens[0] = 1
    case = synth.make_case("d64-fused", 350 + S, lens, 32, 8, D, 16, free_frac=0.1)
    nk = synth.bf16_bits(rng.standard_normal((S, 8, D), dtype=np.float32))
    nv = synth.bf16_bits(rng.standard_normal((S, 8, D), dtype=np.float32))
    dev = case_on_device(case)
    say("head_dim 64 fused write, sequences", S)
    out = pa.decode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale), case.max_context_len,
                    new_key=to_dev(nk), new_value=to_dev(nv))
    torch.cuda.synchronize()
    slots = oracle.slot_mapping(case.block_tables, case.context_lens - 1, case.block_size)
    oracle.reshape_and_cache(nk, nv, case.k_cache, case.v_cache, slots)
    assert np.array_equal(to_host(dev["k"]), case.k_cache)
    assert np.array_equal(to_host(dev["v"]), case.v_cache)
    err = max_err(out.cpu().numpy().astype(np.float64), run_oracle(case))
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("kv,mode,BS", [(synth.I8, pa.PA_SCALE_BLOCK, 16), (synth.I8, pa.PA_SCALE_TOKEN, 32),
                                        (synth.FP8, pa.PA_SCALE_TOKEN, 16), (synth.FP8, pa.PA_SCALE_BLOCK, 32)])
def test_quantised_head_dim64(kv, mode, BS):
    """1-byte caches at head_dim 64: plain, grouped (256 items) and balanced
    (skewed lengths with the hint) launches."""
    rng = np.random.default_rng(6)
    lens = [0, 1, 15, 16, 17, 255, 256, 257] + [int(x) for x in rng.integers(1, 1500, size=23)] + [3000]
    case = synth.make_case("d64-q", 360 + BS, lens, 64, 8, D, BS, kv_dtype=kv, free_frac=0.1)
    if kv == synth.I8 and mode == pa.PA_SCALE_BLOCK:
        quantize_case(case)
    else:
        quantize_case_by_token(case, mode)
    expect = oracle.paged_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                 float(case.scale), case.k_scales, case.v_scales, scale_mode=mode)
    dev = case_on_device(case)
    for kern, P, hint in ((pa.KERNEL_MFMA, 0, False), (pa.KERNEL_MFMA, 0, True), (pa.KERNEL_MFMA, 16, False),
                          (pa.KERNEL_MFMA, 512, False), (pa.KERNEL_VALU, 0, False)):
        say("head_dim 64 quantised", kv, mode, BS, "kernel", kern, "partition", P, "hint", hint)
        got = run_decode(case, dev, partition_tokens=P, kernel=kern, length_hint=hint)
        err = max_err(got, expect)
        assert err <= TOL_BF16, (kv, mode, BS, kern, P, hint, err)
