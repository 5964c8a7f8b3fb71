"""Seeded random decode configurations on the GPU against the CPU oracle.

Each case draws a shape, a length distribution, a cache dtype and scale
layout, a length hint (exact, too small, too large or none), a partition
size, the kernel, and optionally a shared prefix and the fused cache write
(into a per-token-scaled 1-byte cache too, quantising in the kernel),
so that the partition plans (near-equal, ragged, balanced, shared prefix,
given partitions, vector-ALU) meet in combinations the targeted tests do
not list.  The oracle knows nothing of plans or prefixes: each result must
be the attention over the sequence's table.  max |gpu - oracle| <= 2e-3
(bf16 or 1-byte inputs) or 1e-5 (fp32 q and cache); the fused write
bit-exact over the whole pool, codes and scales included."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import case_on_device, max_err, quantize_case_by_token, say, to_dev, to_host, tolerance

pytestmark = pytest.mark.gpu

N_CASES = 60
MAX_TOKENS = 30000          # per case, all sequences (keeps the oracle and host copies small)

# (Hq, Hkv, D)
SHAPES = [(8, 8, 64), (8, 2, 64), (16, 4, 128), (32, 8, 128), (64, 8, 128), (16, 16, 128), (16, 1, 128)]


def _lengths(rng, S, BS):
    kind = rng.choice(["lognormal", "lognormal", "uniform", "equal", "zeros", "one-long", "one-long"])
    if kind == "lognormal":
        x = rng.lognormal(math.log(rng.uniform(20, 800)), 1.0, S)
    elif kind == "uniform":
        x = rng.uniform(0, rng.uniform(50, 2000), S)
    elif kind == "equal":
        x = np.full(S, rng.uniform(1, 1500))
    elif kind == "zeros":
        x = rng.uniform(0, 300, S) * (rng.random(S) < 0.5)
    else:
        x = rng.uniform(1, 100, S)
        x[rng.integers(0, S)] = rng.uniform(1000, 6000)
    lens = np.rint(x).astype(np.int64)
    if lens.sum() > MAX_TOKENS:
        lens = np.floor(lens * (MAX_TOKENS / lens.sum())).astype(np.int64)
    return kind, lens.astype(np.int32)


def _draw(seed):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = SHAPES[rng.integers(0, len(SHAPES))]
    BS = int(rng.choice([16, 32]))
    if D == 64:
        q_dt, kv_dt = [(synth.F32, synth.F32), (synth.BF16, synth.BF16), (synth.BF16, synth.I8),
                       (synth.BF16, synth.FP8)][int(rng.integers(0, 4))]
    else:
        q_dt, kv_dt = synth.BF16, str(rng.choice([synth.BF16, synth.BF16, synth.I8, synth.FP8, synth.F32]))
        if kv_dt == synth.F32:
            q_dt = synth.F32
    S = int(rng.integers(1, 200))
    kind, lens = _lengths(rng, S, BS)
    lens[0] = max(int(lens[0]), 1)                   # a table of at least one block
    matrix_ok = q_dt == synth.BF16 and kv_dt in (synth.BF16, synth.I8, synth.FP8)
    kernel = pa.KERNEL_VALU if (not matrix_ok or rng.random() < 0.15) else pa.KERNEL_AUTO
    prefix_blocks = 0
    if matrix_ok and kernel == pa.KERNEL_AUTO and rng.random() < 0.3:
        prefix_blocks = int(rng.integers(1, 8))
        lens[0] = max(int(lens[0]), prefix_blocks * BS)
    P = 0 if rng.random() < 0.7 else 16 * int(rng.integers(1, 8 * BS // 16 + 1))
    scale_mode = int(rng.choice([pa.PA_SCALE_BLOCK, pa.PA_SCALE_TOKEN]))
    quant_fused_ok = (kv_dt in (synth.I8, synth.FP8) and D == 128 and kernel == pa.KERNEL_AUTO
                      and scale_mode == pa.PA_SCALE_TOKEN)
    fused = (kv_dt in (synth.BF16, synth.F32) or quant_fused_ok) and rng.random() < (0.8 if quant_fused_ok else 0.4)
    hint_kind = str(rng.choice(["exact", "exact", "exact", "under", "over", "none"]))
    return dict(seed=seed, Hq=Hq, Hkv=Hkv, D=D, BS=BS, q_dt=q_dt, kv_dt=kv_dt, S=S, kind=kind, lens=lens,
                kernel=kernel, prefix_blocks=prefix_blocks, P=P, scale_mode=scale_mode, fused=fused,
                hint_kind=hint_kind)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_plan(seed):
    c = _draw(1000 + seed)
    lens, BS, S = c["lens"], c["BS"], c["S"]
    say("random plan", {k: v for k, v in c.items() if k != "lens"}, "total", int(lens.sum()), "max", int(lens.max()))
    case = synth.make_case("random_%d" % seed, 2000 + seed, lens, c["Hq"], c["Hkv"], c["D"], BS, q_dtype=c["q_dt"],
                           kv_dtype=c["kv_dt"], free_frac=0.05)
    pb = c["prefix_blocks"]
    if pb:
        case.block_tables[:, :pb] = case.block_tables[0, :pb]
    mode = pa.PA_SCALE_BLOCK
    if c["kv_dt"] in (synth.I8, synth.FP8):
        mode = c["scale_mode"]
        quantize_case_by_token(case, mode)
    mcl = case.max_context_len
    total = int(lens.sum())
    hint = {"exact": total, "under": total // 3, "over": S * mcl, "none": 0}[c["hint_kind"]]
    dev = case_on_device(case)
    new = None
    if c["fused"]:
        rng = np.random.default_rng(3000 + seed)
        rows = rng.standard_normal((2, S, c["Hkv"], c["D"]), dtype=np.float32)
        new = [r if c["kv_dt"] == synth.F32 else synth.bf16_bits(r) for r in rows]
    table = to_dev(np.ascontiguousarray(case.block_tables[0, :pb])) if pb else None
    out = pa.decode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale), mcl, k_scales=dev["ks"],
                    v_scales=dev["vs"], partition_tokens=c["P"], kernel=c["kernel"], total_context_len=hint,
                    new_key=None if new is None else to_dev(new[0]), new_value=None if new is None else to_dev(new[1]),
                    shared_prefix_table=table, shared_prefix_len=pb * BS)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    if new is not None:
        # every sequence's newest token is written, except (with a shared
        # prefix on the matrix-core kernel) those inside the prefix
        written = np.nonzero((lens >= 1) & (lens > pb * BS if pb else True))[0]
        quant = c["kv_dt"] in (synth.I8, synth.FP8)
        if len(written):
            slots = oracle.slot_mapping(case.block_tables[written], lens[written] - 1, BS)
            if quant:
                oracle.quantize_and_cache(new[0][written], new[1][written], case.k_cache, case.v_cache,
                                          case.k_scales, case.v_scales, slots, pa.PA_SCALE_TOKEN, 0.0, 0.0)
            else:
                oracle.reshape_and_cache(new[0][written], new[1][written], case.k_cache, case.v_cache, slots)
        # byte for byte: unused fp32 slots hold NaN poison
        assert np.array_equal(to_host(dev["k"]).view(np.uint8), case.k_cache.view(np.uint8))
        assert np.array_equal(to_host(dev["v"]).view(np.uint8), case.v_cache.view(np.uint8))
        if quant:
            assert np.array_equal(to_host(dev["ks"]).view(np.uint8), case.k_scales.view(np.uint8))
            assert np.array_equal(to_host(dev["vs"]).view(np.uint8), case.v_scales.view(np.uint8))
    expect = oracle.paged_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                 float(case.scale), case.k_scales, case.v_scales, scale_mode=mode)
    err = max_err(got, expect)
    assert err <= tolerance(case), (c["seed"], err)
