"""A bf16 output (out_dtype PA_BF16): the same call's fp32 result rounded to
the nearest bf16 (ties to even), bit for bit, in every launch form -- one
partition writing directly, partials and the merge, grouped workgroups, the
balanced split, a shared prefix, several query rows (the shared-tile
kernel) and the vector-ALU kernel -- and the entry point that allocates
nothing.  The fp32 results themselves are checked against the oracle by
the other tests."""
import numpy as np
import pytest
import torch

import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import case_on_device, quantize_case_by_token, say, to_dev

pytestmark = pytest.mark.gpu


def _pair(case, d, **kw):
    """(fp32 result, bf16 result) of the same call."""
    R = kw["q"].shape[0] if "q" in kw else d["q"].shape[0]
    q = kw.pop("q", d["q"])
    outs = []
    for dt in (torch.float32, torch.bfloat16):
        out = torch.full((R, case.num_q_heads, case.head_dim), float("nan"), dtype=dt, device="cuda:0")
        pa.decode(q, d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len, out=out,
                  k_scales=d["ks"], v_scales=d["vs"], **kw)
        outs.append(out)
    torch.cuda.synchronize()
    return outs


def _check(tag, f32, b16):
    assert torch.equal(b16, f32.to(torch.bfloat16)), tag


@pytest.mark.parametrize("kv", [synth.BF16, synth.I8])
def test_bf16_output_is_the_rounded_fp32_result(kv):
    rng = np.random.default_rng(8)
    lens = [0, 1, 17, 255, 256, 1000, 3000] + [int(x) for x in rng.integers(1, 1200, size=25)]
    case = synth.make_case("bf16-out", 970, lens, 32, 8, 128, 16, kv_dtype=kv, free_frac=0.1)
    if kv == synth.I8:
        quantize_case_by_token(case, pa.PA_SCALE_BLOCK)
    d = case_on_device(case)
    total = int(np.sum(case.context_lens, dtype=np.int64))
    forms = [("partials and merge", dict(partition_tokens=64)),
             ("automatic (grouped)", dict()),
             ("length hint", dict(total_context_len=total))]
    if kv == synth.BF16:
        forms.append(("vector-ALU kernel", dict(kernel=pa.KERNEL_VALU, partition_tokens=256)))
    for tag, kw in forms:
        say("bf16 output", kv, tag)
        f32, b16 = _pair(case, d, **kw)
        _check((kv, tag), f32, b16)


def test_bf16_output_shared_prefix_and_query_rows():
    pb, BS = 4, 32
    L = pb * BS
    lens = [L + 300, L - 7, L, L + 1, L + 40, 0, L + 129]
    case = synth.make_case("bf16-out-prefix", 971, lens, 64, 8, 128, BS, free_frac=0.1)
    case.block_tables[:, :pb] = case.block_tables[0, :pb]
    d = case_on_device(case)
    table = to_dev(np.ascontiguousarray(case.block_tables[0, :pb]))
    say("bf16 output, shared prefix")
    f32, b16 = _pair(case, d, shared_prefix_table=table, shared_prefix_len=L)
    _check("shared prefix", f32, b16)
    # 64 query rows per sequence (8 heads: the shared-tile kernel)
    rows = 64
    qlens = [min(rows, n) for n in lens]
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    rng = np.random.default_rng(12)
    q = to_dev(synth.bf16_bits(rng.standard_normal((int(qsl[-1]), 64, 128)).astype(np.float32)))
    say("bf16 output, query rows")
    f32, b16 = _pair(case, d, q=q, query_start_loc=to_dev(qsl), max_query_len=rows)
    _check("query rows", f32, b16)


def test_bf16_output_without_allocation():
    """pa_decode_noalloc with a bf16 output: the fp32 rows live in the
    library's fixed scratch; the result equals pa_decode's."""
    import ctypes
    case = synth.make_case("bf16-out-noalloc", 972, [5, 300, 1000, 77], 32, 8, 128, 16, free_frac=0.1)
    d = case_on_device(case)
    # one partition per sequence (32 items: not grouped): written directly
    say("bf16 output, one partition")
    f32, b16 = _pair(case, d, partition_tokens=1008)
    _check("one partition", f32, b16)
    ref = torch.empty(4, 32, 128, dtype=torch.bfloat16, device="cuda:0")
    pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len, out=ref,
              partition_tokens=64)
    out = torch.full((4, 32, 128), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    a = pa.make_decode_args(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                            out=out, partition_tokens=64)
    assert pa.decode_workspace_size(a) <= pa.library().pa_decode_noalloc_scratch_bytes()
    say("bf16 output without allocation")
    assert pa.library().pa_decode_noalloc(ctypes.byref(a)) == pa.PA_OK
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
