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

# Regression guard beside the 2e-3 parity gate, on the rows of sequences of
# at least GUARD_MIN_LEN tokens (long contexts, ragged and balanced splits).
# There the outputs are small (|out| ~ 1e-2 at 8,000 tokens of N(0, 1)
# values, ~2e-2 at 131,072 with 8 heads) and one lost 16-token tile or
# merged partial can move them by less than 2e-3, but by more than this;
# below GUARD_MIN_LEN tokens a lost tile moves them by more than the gate
# itself (both pinned on the CPU with the oracle in
# tests/test_regression_guard.py).  The kernels' own errors on those rows
# are ~1e-8 .. 5e-6.  Not a parity tolerance: a breach means work was
# dropped or double-counted, or the arithmetic changed.
GUARD_BF16 = 2e-5
GUARD_MIN_LEN = 2048


def guard_err(got, expect, context_lens) -> float:
    """max |got - expect| over the output rows [S][Hq][D] of sequences with
    at least GUARD_MIN_LEN tokens (0 if there are none)."""
    long_rows = np.asarray(context_lens) >= GUARD_MIN_LEN
    if not np.any(long_rows):
        return 0.0
    return float(np.max(np.abs(got[long_rows] - expect[long_rows])))

DEV = "cuda:0"


def say(*a):
    """Name the case on stdout before a GPU step (survives a dead box)."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bfloat16 bit patterns and
    uint8 arrays E4M3 codes."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(DEV).view(torch.float8_e4m3fn)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy; bfloat16 comes back as uint16 bits, E4M3 as
    uint8 codes."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy().copy()
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


def quantize_case_by_token(case: synth.DecodeCase, scale_mode: int, static=(0.03, 0.03), poison=1e30) -> None:
    """int8 / E4M3 cases: every cached token's fp32 row quantised by the
    oracle's quantising write, per token (dynamic) or with static per-layer
    scales; unused slots keep poison codes and the scale poison (NaN is
    allowed: slots past a sequence's length are never read)."""
    slots = synth.token_slots(case)
    NB, Hkv, BS, D = case.k_cache.shape
    kf = case.extra["k_f32"]
    vf = case.extra["v_f32"]
    # the fp32 row of each token, in slot order
    key = np.stack([kf[sl // BS, :, sl % BS, :] for sl in slots]) if len(slots) else np.zeros((0, Hkv, D), np.float32)
    val = np.stack([vf[sl // BS, :, sl % BS, :] for sl in slots]) if len(slots) else np.zeros((0, Hkv, D), np.float32)
    dt = np.int8 if case.kv_dtype == synth.I8 else np.uint8
    case.k_cache = np.full(case.k_cache.shape, synth._poison_value(case.kv_dtype), dt)
    case.v_cache = case.k_cache.copy()
    sshape = oracle.scale_shape(NB, Hkv, BS, scale_mode)
    case.k_scales = np.full(sshape, poison, np.float32)
    case.v_scales = np.full(sshape, poison, np.float32)
    if len(slots):
        oracle.quantize_and_cache(key, val, case.k_cache, case.v_cache, case.k_scales, case.v_scales, slots,
                                  scale_mode, static[0], static[1])


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
