"""pa_decode_noalloc -- decode whose split-K workspace is the library's own
fixed device array, for callers that cannot allocate -- against pa_decode
with a caller-owned workspace, through the C ABI.

Same plan and kernels, so the results must agree bit for bit; they are
also checked against the oracle (2e-3, bf16 / int8 inputs).  Two calls in
a row on one GPU: a large ragged batch (balanced split, tens of MB of
partials), then a smaller one (int8, short given partitions), which must
not see the first call's leftovers.  A plan that needs more workspace than
the fixed array holds is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import TOL_BF16, case_on_device, max_err, quantize_case, run_oracle, say

pytestmark = pytest.mark.gpu


def _lib():
    return pa.library()


def _both(case, partition_tokens=0, hint=True):
    d = case_on_device(case)
    total = int(np.sum(case.context_lens, dtype=np.int64)) if hint else 0
    out_ref = torch.full((case.num_seqs, case.num_q_heads, case.head_dim), float("nan"), device="cuda:0")
    out = torch.full_like(out_ref, float("nan"))
    ref = pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len, out=out_ref,
                    k_scales=d["ks"], v_scales=d["vs"], partition_tokens=partition_tokens, total_context_len=total)
    args = pa.make_decode_args(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                               out=out, k_scales=d["ks"], v_scales=d["vs"], partition_tokens=partition_tokens,
                               total_context_len=total)
    need = pa.decode_workspace_size(args)
    st = _lib().pa_decode_noalloc(ctypes.byref(args))
    assert st == pa.PA_OK, _lib().pa_last_error()
    torch.cuda.synchronize()
    return ref, out, need


def test_noalloc_matches_pa_decode_on_two_calls():
    lib = _lib()
    cap = lib.pa_decode_noalloc_scratch_bytes()
    rng = np.random.default_rng(12)
    lens = np.clip(np.rint(rng.lognormal(np.log(600), 1.0, size=96)), 1, 12000).astype(np.int32)
    lens[3] = 12000
    big = synth.make_case("noalloc-big", 91, lens, 32, 8, 128, 16, free_frac=0.05)
    say("noalloc call 1: 96 ragged sequences, balanced split")
    ref, out, need = _both(big)
    assert 1 << 20 < need <= cap, need                     # the fixed array really carries the partials
    assert torch.equal(ref, out)
    assert max_err(out.cpu().numpy().astype(np.float64), run_oracle(big)) <= TOL_BF16

    small = synth.make_case("noalloc-small", 92, [1, 40, 300, 77, 0, 1000], 16, 4, 128, 16, kv_dtype=synth.I8,
                            free_frac=0.1)
    quantize_case(small)
    say("noalloc call 2: 6 int8 sequences, partitions of 64 tokens")
    ref, out, need = _both(small, partition_tokens=64, hint=False)
    assert 0 < need < 1 << 20, need
    assert torch.equal(ref, out)
    assert max_err(out.cpu().numpy().astype(np.float64), run_oracle(small)) <= TOL_BF16


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    lib = _lib()
    cap = lib.pa_decode_noalloc_scratch_bytes()
    S, Hq, Hkv, D, BS, MB = 256, 64, 8, 128, 16, 2048
    q = torch.zeros(S, Hq, D, dtype=torch.bfloat16, device="cuda:0")
    kc = torch.zeros(4, Hkv, BS, D, dtype=torch.bfloat16, device="cuda:0")
    bt = torch.zeros(S, MB, dtype=torch.int32, device="cuda:0")
    cl = torch.zeros(S, dtype=torch.int32, device="cuda:0")
    out = torch.zeros(S, Hq, D, dtype=torch.float32, device="cuda:0")
    args = pa.make_decode_args(q, kc, kc, bt, cl, 0.1, MB * BS, out=out)
    need = pa.decode_workspace_size(args)
    assert need > cap, need
    say("noalloc refusal")
    st = lib.pa_decode_noalloc(ctypes.byref(args))
    assert st == pa.PA_ERR_INVALID
    assert "fixed scratch" in lib.pa_last_error().decode()
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
