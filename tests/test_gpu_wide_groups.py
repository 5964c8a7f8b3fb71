"""More than 16 query heads per kv head on the GPU against the CPU oracle.

The matrix-core kernel takes the query heads of a kv head 16 at a time as
column groups (two per wave, the K/V tiles read once for both), as it takes
several query rows per sequence; the vector-ALU kernel takes them in head
groups of 8.  Shapes with 17, 24, 32, 64 and 128 heads per kv head, lengths
around tile and partition edges, given and automatic partitions with and
without the length hint, bf16 and quantised caches, the fused cache write
(bit-exact), and a shared prefix (read through each table row here; a
newest token inside it is neither stored nor attended).
max |gpu - oracle| <= 2e-3 (bf16, int8 or E4M3 inputs, fp32 accumulation)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import (TOL_BF16, case_on_device, max_err, quantize_case_by_token, run_decode, run_oracle, say,
                         to_dev, to_host)

pytestmark = pytest.mark.gpu

LENS = [0, 1, 15, 17, 300, 1000, 2049, 513]


@pytest.mark.parametrize("hq,hkv", [(34, 2), (48, 2), (64, 2), (128, 2), (256, 2)])
def test_wide_groups_match_oracle(hq, hkv):
    case = synth.make_case("wide_%d_%d" % (hq, hkv), 300 + hq, LENS, hq, hkv, 128, 16, free_frac=0.05)
    expect = run_oracle(case)
    dev = case_on_device(case)
    for kern in (0, pa.KERNEL_VALU):
        for P in (0, 64, 512):
            for hint in ((False, True) if P == 0 else (False,)):
                say("wide groups", hq, hkv, "kernel", kern, "partition", P, "hint", hint)
                err = max_err(run_decode(case, dev, partition_tokens=P, kernel=kern, length_hint=hint), expect)
                assert err <= TOL_BF16, (hq, hkv, kern, P, hint, err)


@pytest.mark.parametrize("kv,mode", [(synth.I8, pa.PA_SCALE_BLOCK), (synth.FP8, pa.PA_SCALE_TOKEN)])
def test_wide_groups_quantised(kv, mode):
    case = synth.make_case("wide_q", 77, LENS, 64, 2, 128, 32, kv_dtype=kv, free_frac=0.05)
    quantize_case_by_token(case, mode)
    expect = oracle.paged_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                                 float(case.scale), case.k_scales, case.v_scales, scale_mode=mode)
    dev = case_on_device(case)
    for kern in (0, pa.KERNEL_VALU):
        for hint in (False, True):
            say("wide groups quantised", kv, mode, "kernel", kern, "hint", hint)
            err = max_err(run_decode(case, dev, kernel=kern, length_hint=hint), expect)
            assert err <= TOL_BF16, (kv, mode, kern, hint, err)


@pytest.mark.parametrize("kernel", [0, pa.KERNEL_VALU])
def test_wide_groups_fused_write_and_shared_prefix(kernel):
    """The fused write of each newest token, with a shared prefix of 4 blocks
    passed: sequences past the prefix are written and attended with their new
    token; one whose newest token lies inside the prefix is not written."""
    pb, BS, hq, hkv = 4, 16, 64, 2
    L = pb * BS
    lens = [L + 70, L - 5, L + 1, L + 300, 0]
    case = synth.make_case("wide_write", 91, lens, hq, hkv, 128, BS, free_frac=0.1)
    case.block_tables[:, :pb] = case.block_tables[0, :pb]
    S = len(lens)
    rng = np.random.default_rng(5)
    k_new = synth.bf16_bits(rng.standard_normal((S, hkv, 128), dtype=np.float32))
    v_new = synth.bf16_bits(rng.standard_normal((S, hkv, 128), dtype=np.float32))
    dev = case_on_device(case)
    table = to_dev(np.ascontiguousarray(case.block_tables[0, :pb]))
    say("wide groups fused write + shared prefix, kernel", kernel)
    out = pa.decode(dev["q"], dev["k"], dev["v"], dev["bt"], dev["cl"], float(case.scale), case.max_context_len,
                    new_key=to_dev(k_new), new_value=to_dev(v_new), shared_prefix_table=table,
                    shared_prefix_len=L, kernel=kernel)
    torch.cuda.synchronize()
    written = [0, 2, 3]                                # past the prefix; 1 is inside it, 4 is empty
    slots = oracle.slot_mapping(case.block_tables[written], case.context_lens[written] - 1, BS)
    oracle.reshape_and_cache(k_new[written], v_new[written], case.k_cache, case.v_cache, slots)
    assert np.array_equal(to_host(dev["k"]), case.k_cache)
    assert np.array_equal(to_host(dev["v"]), case.v_cache)
    err = max_err(out.cpu().numpy().astype(np.float64), run_oracle(case))
    assert err <= TOL_BF16, (kernel, err)
