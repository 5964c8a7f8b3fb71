"""Helpers shared by the GPU tests: host arrays <-> device tensors, running
the library and the oracle on the same bytes, tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_192_amd as pa
import synth

# Attention tolerances (max |gpu - oracle| over all elements): bf16 or int8
# inputs with fp32 accumulation, and fp32 inputs.
TOL_BF16 = 2e-3
TOL_F32 = 1e-5

DEV = "cuda:0"


def say(*a):
    """Name the case on stdout before a GPU step (survives a dead box)."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bfloat16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy; bfloat16 comes back as uint16 bits."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def case_on_device(case: synth.DecodeCase):
    d = dict(q=to_dev(case.q), k=to_dev(case.k_cache), v=to_dev(case.v_cache),
             bt=to_dev(case.block_tables), cl=to_dev(case.context_lens))
    d["ks"] = to_dev(case.k_scales) if case.k_scales is not None else None
    d["vs"] = to_dev(case.v_scales) if case.v_scales is not None else None
    return d


def quantize_case(case: synth.DecodeCase) -> None:
    """int8 cases: codes and scales from the oracle's quantiser (inputs only;
    the kernels never quantise), tails and free blocks poisoned with +127."""
    valid = synth.valid_slots_per_block(case)
    case.k_cache, case.k_scales = oracle.quantize_int8(case.extra["k_f32"], valid)
    case.v_cache, case.v_scales = oracle.quantize_int8(case.extra["v_f32"], valid)
    synth.poison_unused(case.k_cache, case.block_tables, case.context_lens, case.free_blocks, synth.I8)
    synth.poison_unused(case.v_cache, case.block_tables, case.context_lens, case.free_blocks, synth.I8)


def run_decode(case: synth.DecodeCase, dev=None, partition_tokens=0, kernel=0, max_context_len=None,
               length_hint=False):
    """pa_decode on the case; length_hint passes the batch's total context
    length (the ragged-batch partition plan)."""
    d = dev or case_on_device(case)
    mcl = case.max_context_len if max_context_len is None else max_context_len
    total = int(np.sum(case.context_lens, dtype=np.int64)) if length_hint else 0
    out = pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), mcl, k_scales=d["ks"],
                    v_scales=d["vs"], partition_tokens=partition_tokens, kernel=kernel, total_context_len=total)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def run_oracle(case: synth.DecodeCase):
    return oracle.paged_decode(case.q, case.k_cache, case.v_cache, case.block_tables, case.context_lens,
                               float(case.scale), case.k_scales, case.v_scales)


def tolerance(case: synth.DecodeCase) -> float:
    return TOL_F32 if (case.q_dtype == synth.F32 and case.kv_dtype == synth.F32) else TOL_BF16


def max_err(a, b) -> float:
    assert a.shape == b.shape
    assert np.all(np.isfinite(a)), "non-finite output"
    return float(np.max(np.abs(a - b))) if a.size else 0.0
