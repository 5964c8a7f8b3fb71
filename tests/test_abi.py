"""C ABI of libpa on the host: the library loads, exports every symbol pa.h
declares, rejects bad arguments before any launch, and its block pool
follows the pool policy model call for call.  No GPU is used."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import paged_kv_cache_192_amd as pa
from oracle import PoolModel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "pa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = pa.library()
    names = declared_functions()
    assert len(names) >= 16, names
    for n in names:
        assert hasattr(lib, n), "libpa.so does not export %s" % n
    assert lib.pa_abi_version() == pa.ABI_VERSION == 6


def test_status_strings():
    lib = pa.library()
    for code, name in pa.STATUS_NAMES.items():
        assert lib.pa_status_string(code).decode() == name


def _cpu_args(**over):
    """DecodeArgs with host tensors standing in for shapes only."""
    S, Hq, Hkv, D, BS, NB, MB = 3, 8, 2, 128, 16, 40, 10
    q = torch.zeros(S, Hq, D, dtype=torch.bfloat16)
    kc = torch.zeros(NB, Hkv, BS, D, dtype=torch.bfloat16)
    bt = torch.zeros(S, MB, dtype=torch.int32)
    cl = torch.zeros(S, dtype=torch.int32)
    a = pa.make_decode_args(q, kc, kc, bt, cl, 0.125, 100, device_pointers=False)
    a.out = 0x10000                                  # never dereferenced on these paths
    for k, v in over.items():
        setattr(a, k, v)
    return a


def _ws(a):
    n = ctypes.c_size_t(0)
    st = pa.library().pa_decode_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def test_struct_layout_and_workspace_size():
    a = _cpu_args(kernel=pa.KERNEL_VALU)
    st, n = _ws(a)
    assert st == pa.PA_OK, pa.library().pa_last_error()
    # 3 seqs x 2 kv heads, 7 tiles: the planner splits the 100 tokens into
    # partitions of 64 (4 tiles minimum) -> 2 partitions; on the vector-ALU
    # kernel the workspace is the partial (m, l) rows, then the acc rows,
    # 256-aligned
    nP = -(-100 // 64)
    rows = 3 * 8 * nP
    al = lambda b: (b + 255) // 256 * 256  # noqa: E731
    assert n == al(rows * 8) + al(rows * 128 * 4)
    # with at least 256 (sequence, kv head) items the matrix-core kernel
    # takes 2 .. 8 partitions of an item in one workgroup and combines them
    # there: no workspace, with the automatic split or a given one (100
    # tokens in 16-token partitions: 7); 128 sequences x 2 kv heads
    for over in ({}, {"kernel": pa.KERNEL_MFMA}, {"partition_tokens": 16}, {"partition_tokens": 32}):
        st, n = _ws(_cpu_args(num_seqs=128, **over))
        assert st == pa.PA_OK and n == 0, over
    # fewer items (the 3 x 2 above, or 127 x 2): partials and the merge
    st, n = _ws(_cpu_args())
    assert st == pa.PA_OK and n == al(rows * 8) + al(rows * 128 * 4)
    st, n = _ws(_cpu_args(num_seqs=127))
    assert st == pa.PA_OK and n == al(127 * 8 * 2 * 8) + al(127 * 8 * 2 * 128 * 4)
    # more than 8 partitions: partials again (10 blocks x 16 = 160 tokens in
    # 16-token partitions: 10)
    st, n = _ws(_cpu_args(num_seqs=128, partition_tokens=16, max_context_len=160))
    assert st == pa.PA_OK and n == al(128 * 8 * 10 * 8) + al(128 * 8 * 10 * 128 * 4)
    # a short ragged batch whose automatic split asks for more than 8
    # partitions (the longest sequence 2,048 tokens = 128 tiles, mean a
    # half): re-cut into 4-wave groups, no workspace; one tile longer keeps
    # the partials, and so does the vector-ALU kernel
    short = dict(num_seqs=128, max_blocks_per_seq=129, num_blocks=128 * 129, total_context_len=128 * 1024)
    st, n = _ws(_cpu_args(max_context_len=2048, **short))
    assert st == pa.PA_OK and n == 0
    st, n = _ws(_cpu_args(max_context_len=2049, **short))
    assert st == pa.PA_OK and n > 0
    st, n = _ws(_cpu_args(max_context_len=2048, kernel=pa.KERNEL_VALU, **short))
    assert st == pa.PA_OK and n > 0
    # one partition: no workspace
    st, n = _ws(_cpu_args(partition_tokens=128))
    assert st == pa.PA_OK and n == 0
    # a bf16 output adds the fp32 result rows (3 x 8 rows of 128) after the
    # partials, or alone
    st, n = _ws(_cpu_args(partition_tokens=128, out_dtype=pa.PA_BF16))
    assert st == pa.PA_OK and n == al(3 * 8 * 128 * 4)
    st, n = _ws(_cpu_args(out_dtype=pa.PA_BF16))
    assert st == pa.PA_OK and n == al(rows * 8) + al(rows * 128 * 4) + al(3 * 8 * 128 * 4)
    # distinctive values reach the right fields
    st, _ = _ws(_cpu_args(head_dim=96))
    assert st == pa.PA_ERR_INVALID and "head_dim 96" in pa.library().pa_last_error().decode()
    st, _ = _ws(_cpu_args(block_size=24))
    assert st == pa.PA_ERR_INVALID and "block_size 24" in pa.library().pa_last_error().decode()


def test_workspace_bytes_is_the_size_call_as_a_value():
    """pa_decode_workspace_bytes returns what pa_decode_workspace_size
    stores, SIZE_MAX where the latter fails, with the same message."""
    lib = pa.library()
    size_max = 2 ** (8 * ctypes.sizeof(ctypes.c_size_t)) - 1
    for over in ({}, {"partition_tokens": 128}, {"partition_tokens": 16}, {"total_context_len": 40},
                 {"max_context_len": 0}, {"num_seqs": 0}):
        a = _cpu_args(**over)
        st, n = _ws(a)
        assert st == pa.PA_OK, (over, lib.pa_last_error())
        assert lib.pa_decode_workspace_bytes(ctypes.byref(a)) == n, over
    for over, text in (({"head_dim": 96}, "head_dim 96"), ({"num_q_heads": 7}, "not a multiple"),
                       ({"struct_size": 8}, "struct_size"), ({"kernel": 3}, "kernel 3")):
        a = _cpu_args(**over)
        st, _ = _ws(a)
        assert st != pa.PA_OK
        lib.pa_last_error()
        assert lib.pa_decode_workspace_bytes(ctypes.byref(a)) == size_max, over
        assert text in lib.pa_last_error().decode(), (over, lib.pa_last_error())
    assert lib.pa_decode_workspace_bytes(None) == size_max


def test_partition_plan_follows_the_length_hint():
    """Near-equal lengths (hint absent or close to num_seqs * max): a few
    long partitions per sequence.  A ragged batch: short partitions, here
    the 4-tile minimum, up to 512 per sequence; a strongly skewed one (mean
    under a quarter of the maximum) on the matrix-core kernel: the balanced
    split, 640 waves over the heads' tiles."""
    al = lambda b: (b + 255) // 256 * 256  # noqa: E731

    def ws_for(nP):
        rows = 3 * 8 * nP
        return al(rows * 8) + al(rows * 128 * 4)

    big = dict(max_blocks_per_seq=2048, num_blocks=6144, max_context_len=32768)
    for hint in (0, 3 * 32768, 3 * 32768 - 1000):
        st, n = _ws(_cpu_args(total_context_len=hint, **big))
        assert st == pa.PA_OK
        assert n == ws_for(32)                          # 1024-token partitions
    st, n = _ws(_cpu_args(total_context_len=40000, **big))
    assert st == pa.PA_OK and n == ws_for(512)          # 64-token partitions
    st, n = _ws(_cpu_args(total_context_len=20000, kernel=pa.KERNEL_VALU, **big))
    assert st == pa.PA_OK and n == ws_for(512)
    # balanced: 320 waves per kv head, ranges of ceil((1250 + 3) / 320) = 4
    # tiles, so a 2,048-tile sequence meets at most 513 ranges; then the
    # per-sequence partial counts
    st, n = _ws(_cpu_args(total_context_len=20000, **big))
    assert st == pa.PA_OK and n == ws_for(513) + al(3 * 4)
    # an explicit partition size ignores the hint
    st, n = _ws(_cpu_args(total_context_len=40000, partition_tokens=2048, **big))
    assert st == pa.PA_OK and n == ws_for(16)


def test_balanced_split_up_to_1024_sequences():
    """A strongly skewed batch (mean an eighth of the 32,768-token maximum)
    takes the balanced split up to 1,024 sequences (lengths in sixteen
    64-lane register chunks past 256): 2 kv heads, t = 4,194,304 / 16 +
    1,024 = 263,168 tiles per head by the hint, max(320, ceil(t / 64)) = 4,112
    waves per head of 64-tile ranges, so a 2,048-tile sequence meets at most
    33 ranges: 33 partial slots per row and the per-sequence counts.  1,025
    sequences fall back to the ragged rule's partitions (no counts)."""
    al = lambda b: (b + 255) // 256 * 256  # noqa: E731
    big = dict(max_blocks_per_seq=2048, num_blocks=6144, max_context_len=32768)

    def balanced_ws(S, slots):
        rows = S * 8 * slots
        return al(rows * 8) + al(rows * 128 * 4) + al(S * 4)

    st, n = _ws(_cpu_args(num_seqs=1024, total_context_len=1024 * 32768 // 8, **big))
    assert st == pa.PA_OK and n == balanced_ws(1024, 33)
    st, n = _ws(_cpu_args(num_seqs=1025, total_context_len=1025 * 32768 // 8, **big))
    # the ragged rule's partitions, here the 128-block cap: 16 per row, no counts
    rows = 1025 * 8 * 16
    assert st == pa.PA_OK and n == al(rows * 8) + al(rows * 128 * 4)


@pytest.mark.parametrize("field,value,status", [
    ("struct_size", 8, pa.PA_ERR_INVALID),
    ("num_q_heads", 7, pa.PA_ERR_INVALID),            # not a multiple of 2 kv heads
    ("num_q_heads", 0, pa.PA_ERR_INVALID),
    ("head_dim", 256, pa.PA_ERR_INVALID),
    ("block_size", 8, pa.PA_ERR_INVALID),
    ("out_dtype", pa.PA_I8, pa.PA_ERR_UNSUPPORTED),
    ("q_dtype", pa.PA_I8, pa.PA_ERR_UNSUPPORTED),
    ("kv_dtype", 7, pa.PA_ERR_INVALID),
    ("kv_dtype", pa.PA_I8, pa.PA_ERR_INVALID),        # int8 without scales
    ("k_scales", 64, pa.PA_ERR_INVALID),              # scales for a bf16 cache
    ("scale", float("nan"), pa.PA_ERR_INVALID),
    ("scale", float("inf"), pa.PA_ERR_INVALID),
    ("max_context_len", 161, pa.PA_ERR_INVALID),      # > 10 blocks x 16
    ("max_context_len", -1, pa.PA_ERR_INVALID),
    ("partition_tokens", 24, pa.PA_ERR_INVALID),
    ("partition_tokens", 2064, pa.PA_ERR_INVALID),    # > 128 blocks
    ("kernel", 3, pa.PA_ERR_INVALID),
    ("num_seqs", -1, pa.PA_ERR_INVALID),
    ("total_context_len", -1, pa.PA_ERR_INVALID),
    ("total_context_len", 301, pa.PA_ERR_INVALID),    # > 3 seqs x 100
    ("kv_dtype", pa.PA_FP8_E4M3, pa.PA_ERR_INVALID),  # E4M3 without scales
])
def test_decode_rejects_bad_arguments(field, value, status):
    a = _cpu_args(**{field: value})
    lib = pa.library()
    assert lib.pa_decode(ctypes.byref(a)) == status
    assert lib.pa_last_error().decode()
    assert _ws(a)[0] == status


def test_decode_rejects_null_alignment_and_workspace_before_launch():
    lib = pa.library()
    a = _cpu_args(out=None)
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_INVALID
    a = _cpu_args(q=0x1008)                            # 8-byte aligned only
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_INVALID
    assert "aligned" in lib.pa_last_error().decode()
    a = _cpu_args(workspace=None, workspace_bytes=0, kernel=pa.KERNEL_VALU)   # 2 partitions need one
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_INVALID
    assert "workspace" in lib.pa_last_error().decode()
    a = _cpu_args(kernel=2, q_dtype=pa.PA_F32)
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_UNSUPPORTED


def test_multi_query_argument_checks():
    lib = pa.library()
    qsl = 0x30000
    a = _cpu_args(query_start_loc=qsl, num_queries=5, max_query_len=0)
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_INVALID
    a = _cpu_args(query_start_loc=qsl, num_queries=-1, max_query_len=2)
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_INVALID
    a = _cpu_args(query_start_loc=qsl, num_queries=5, max_query_len=2, kernel=pa.KERNEL_VALU)
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_UNSUPPORTED
    a = _cpu_args(query_start_loc=qsl, num_queries=5, max_query_len=2, q_dtype=pa.PA_F32)
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_UNSUPPORTED
    a = _cpu_args(query_start_loc=qsl, num_queries=5, max_query_len=2, new_key=0x20000, new_value=0x30000)
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_UNSUPPORTED
    # workspace rows are query rows: 5 rows x 8 heads x 2 partitions of 64
    # tokens, with 5 rows x 4 heads per kv head = 2 column groups per item
    st, n = _ws(_cpu_args(query_start_loc=qsl, num_queries=5, max_query_len=5, partition_tokens=64))
    al = lambda b: (b + 255) // 256 * 256  # noqa: E731
    assert st == pa.PA_OK and n == al(5 * 8 * 2 * 8) + al(5 * 8 * 2 * 128 * 4)
    # one column group per item (up to 4 rows of 4 heads) and 128 x 2
    # items: grouped, no workspace
    st, n = _ws(_cpu_args(query_start_loc=qsl, num_seqs=128, num_queries=5, max_query_len=4, partition_tokens=64))
    assert st == pa.PA_OK and n == 0


def test_shared_prefix_argument_checks_and_plan():
    lib = pa.library()
    tbl = 0x40000
    al = lambda b: (b + 255) // 256 * 256  # noqa: E731
    for over in (dict(shared_prefix_len=32),                               # no table
                 dict(shared_prefix_table=tbl, shared_prefix_len=40),      # not whole blocks
                 dict(shared_prefix_table=tbl, shared_prefix_len=112),     # > max_context_len 100
                 dict(shared_prefix_table=tbl, shared_prefix_len=-16)):
        a = _cpu_args(**over)
        assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_INVALID
        assert "shared_prefix" in lib.pa_last_error().decode()
    a = _cpu_args(shared_prefix_table=0x40002, shared_prefix_len=64)
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_INVALID
    # partials per row: prefix partitions, then the sequences' own -- given
    # 32-token partitions: 64 prefix tokens -> 2, the other <= 36 -> 2
    st, n = _ws(_cpu_args(shared_prefix_table=tbl, shared_prefix_len=64, partition_tokens=32))
    assert st == pa.PA_OK and n == al(24 * 4 * 8) + al(24 * 4 * 128 * 4)
    # automatic: one partition for each part -> 2 partials per row
    st, n = _ws(_cpu_args(shared_prefix_table=tbl, shared_prefix_len=64))
    assert st == pa.PA_OK and n == al(24 * 2 * 8) + al(24 * 2 * 128 * 4)
    # the whole context shared: only prefix partials (given 32-token
    # partitions: 3); automatic: one partition of 96 (at least 4 tiles per
    # wave of an item) -> written directly, no workspace
    st, n = _ws(_cpu_args(shared_prefix_table=tbl, shared_prefix_len=96, max_context_len=96, partition_tokens=32))
    assert st == pa.PA_OK and n == al(24 * 3 * 8) + al(24 * 3 * 128 * 4)
    st, n = _ws(_cpu_args(shared_prefix_table=tbl, shared_prefix_len=96, max_context_len=96))
    assert st == pa.PA_OK and n == 0
    # ignored by the vector-ALU kernel: the plan without a prefix
    st0, n0 = _ws(_cpu_args(kernel=pa.KERNEL_VALU))
    st, n = _ws(_cpu_args(shared_prefix_table=tbl, shared_prefix_len=64, kernel=pa.KERNEL_VALU))
    assert st == st0 == pa.PA_OK and n == n0


def test_fused_write_argument_checks():
    lib = pa.library()
    a = _cpu_args(new_key=0x20000)                      # new_value missing
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_INVALID
    a = _cpu_args(new_key=0x20000, new_value=0x20008)   # misaligned
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_INVALID
    a = _cpu_args(new_key=0x20000, new_value=0x30000, kv_dtype=pa.PA_I8, k_scales=64, v_scales=64)
    assert lib.pa_decode(ctypes.byref(a)) == pa.PA_ERR_UNSUPPORTED
    # into a 1-byte cache only with per-token scales, head_dim 128 and the
    # matrix-core kernel (the write quantises bf16 rows in the kernel)
    quant = dict(new_key=0x20000, new_value=0x30000, k_scales=64, v_scales=64, kv_scale_mode=pa.PA_SCALE_TOKEN)
    for kv in (pa.PA_I8, pa.PA_FP8_E4M3):
        assert _ws(_cpu_args(kv_dtype=kv, **quant))[0] == pa.PA_OK
        for bad in (dict(head_dim=64), dict(kernel=pa.KERNEL_VALU), dict(q_dtype=pa.PA_F32)):
            st, _ = _ws(_cpu_args(kv_dtype=kv, **quant, **bad))
            assert st == pa.PA_ERR_UNSUPPORTED, bad
            assert "fused write into a quantised cache" in lib.pa_last_error().decode()


def test_zero_sequences_is_a_no_op():
    a = _cpu_args(num_seqs=0)
    assert pa.library().pa_decode(ctypes.byref(a)) == pa.PA_OK


def test_cache_ops_reject_bad_arguments():
    lib = pa.library()
    P = 0x10000
    # reshape: quantised caches go through pa_quantize_and_cache; bad shapes, misalignment
    assert lib.pa_reshape_and_cache(P, P, P, P, pa.PA_I8, P, 1, 8, 128, 16, 10, None) == pa.PA_ERR_UNSUPPORTED
    assert lib.pa_reshape_and_cache(P, P, P, P, pa.PA_FP8_E4M3, P, 1, 8, 128, 16, 10, None) == pa.PA_ERR_UNSUPPORTED
    assert lib.pa_reshape_and_cache(P, P, P, P, pa.PA_BF16, P, 1, 8, 96, 16, 10, None) == pa.PA_ERR_INVALID
    assert lib.pa_reshape_and_cache(P, P, P, P, pa.PA_BF16, P, 1, 8, 128, 12, 10, None) == pa.PA_ERR_INVALID
    assert lib.pa_reshape_and_cache(P, P, P, P, pa.PA_BF16, P, -1, 8, 128, 16, 10, None) == pa.PA_ERR_INVALID
    assert lib.pa_reshape_and_cache(P + 4, P, P, P, pa.PA_BF16, P, 1, 8, 128, 16, 10, None) == pa.PA_ERR_INVALID
    assert lib.pa_reshape_and_cache(None, P, P, P, pa.PA_BF16, P, 1, 8, 128, 16, 10, None) == pa.PA_ERR_INVALID
    assert lib.pa_reshape_and_cache(None, None, None, None, pa.PA_BF16, None, 0, 8, 128, 16, 10, None) == pa.PA_OK
    # copy: scales exactly for quantised caches, a known scale layout
    B, T = pa.PA_SCALE_BLOCK, pa.PA_SCALE_TOKEN
    assert lib.pa_copy_blocks(P, P, pa.PA_BF16, P, P, B, P, 1, 8, 128, 16, 10, None) == pa.PA_ERR_INVALID
    assert lib.pa_copy_blocks(P, P, pa.PA_I8, None, None, B, P, 1, 8, 128, 16, 10, None) == pa.PA_ERR_INVALID
    assert lib.pa_copy_blocks(P, P, pa.PA_FP8_E4M3, None, None, T, P, 1, 8, 128, 16, 10, None) == pa.PA_ERR_INVALID
    assert lib.pa_copy_blocks(P, P, pa.PA_I8, P, P, 7, P, 1, 8, 128, 16, 10, None) == pa.PA_ERR_INVALID
    assert lib.pa_copy_blocks(P, P, pa.PA_BF16, None, None, B, P, -2, 8, 128, 16, 10, None) == pa.PA_ERR_INVALID
    assert lib.pa_copy_blocks(P, P, pa.PA_BF16, None, None, B, None, 0, 8, 128, 16, 10, None) == pa.PA_OK
    assert lib.pa_copy_blocks(P, P, pa.PA_I8, P, P, T, None, 0, 8, 128, 16, 10, None) == pa.PA_OK
    # swap: scales all or none and only for quantised pools; pool ids; empty is fine
    sw = lib.pa_swap_blocks
    assert sw(P, P, P, None, P, P, P, P, pa.PA_I8, B, P, 1, 8, 128, 16, 10, 10, None) == pa.PA_ERR_INVALID
    assert sw(P, P, P, P, P, P, P, P, pa.PA_BF16, B, P, 1, 8, 128, 16, 10, 10, None) == pa.PA_ERR_INVALID
    assert sw(P, P, P, P, P, P, P, P, pa.PA_I8, 5, P, 1, 8, 128, 16, 10, 10, None) == pa.PA_ERR_INVALID
    assert sw(P, P, None, None, P, P, None, None, pa.PA_BF16, B, P, 1, 8, 128, 16, 0, 10, None) == pa.PA_ERR_INVALID
    assert sw(P, P, None, None, P, P, None, None, pa.PA_BF16, B, P, -1, 8, 128, 16, 4, 10, None) == pa.PA_ERR_INVALID
    assert sw(P + 8, P, None, None, P, P, None, None, pa.PA_BF16, B, P, 1, 8, 128, 16, 4, 10, None) == \
        pa.PA_ERR_INVALID
    assert sw(None, None, None, None, None, None, None, None, pa.PA_BF16, B, None, 0, 8, 128, 16, 4, 10, None) == pa.PA_OK
    # quantising write: quantised cache, fp32/bf16 source, valid static scales
    qc = lib.pa_quantize_and_cache
    assert qc(P, P, pa.PA_BF16, P, P, pa.PA_BF16, P, P, T, 0.0, 0.0, P, 1, 8, 128, 16, 10, None) == pa.PA_ERR_INVALID
    assert qc(P, P, pa.PA_I8, P, P, pa.PA_I8, P, P, T, 0.0, 0.0, P, 1, 8, 128, 16, 10, None) == pa.PA_ERR_INVALID
    assert qc(P, P, pa.PA_BF16, P, P, pa.PA_I8, P, P, B, 0.0, 1.0, P, 1, 8, 128, 16, 10, None) == pa.PA_ERR_INVALID
    assert qc(P, P, pa.PA_BF16, P, P, pa.PA_I8, P, P, B, 1.0, float("inf"), P, 1, 8, 128, 16, 10, None) == \
        pa.PA_ERR_INVALID
    assert qc(P, P, pa.PA_BF16, P, P, pa.PA_I8, P, P, 3, 1.0, 1.0, P, 1, 8, 128, 16, 10, None) == pa.PA_ERR_INVALID
    assert qc(P, P, pa.PA_BF16, P, P, pa.PA_I8, None, P, T, 0.0, 0.0, P, 1, 8, 128, 16, 10, None) == \
        pa.PA_ERR_INVALID
    assert qc(P, P, pa.PA_F32, P, P, pa.PA_FP8_E4M3, P, P, T, 0.0, 0.0, P, 1, 8, 96, 16, 10, None) == \
        pa.PA_ERR_INVALID
    assert qc(None, None, pa.PA_F32, None, None, pa.PA_FP8_E4M3, None, None, T, 0.0, 0.0, None, 0, 8, 128, 16, 10,
              None) == pa.PA_OK
    # slot mapping: exactly one of positions / context_lens
    assert lib.pa_slot_mapping(P, 4, 2, None, P, P, 2, 16, P, None) == pa.PA_ERR_INVALID
    assert lib.pa_slot_mapping(P, 4, 2, None, None, None, 2, 16, P, None) == pa.PA_ERR_INVALID
    assert lib.pa_slot_mapping(P, 4, 2, None, P, None, 3, 16, P, None) == pa.PA_ERR_INVALID  # T > S, no seq_idx
    assert lib.pa_slot_mapping(P, 0, 2, None, P, None, 2, 16, P, None) == pa.PA_ERR_INVALID
    assert lib.pa_slot_mapping(P, 4, 2, None, P, None, 0, 16, P, None) == pa.PA_OK


# --------------------------------------------------------------------------
# block pool vs the policy model
# --------------------------------------------------------------------------

def test_pool_create_validation():
    lib = pa.library()
    h = ctypes.c_void_p()
    assert lib.pa_pool_create(0, None, ctypes.byref(h)) == pa.PA_ERR_INVALID
    bad = (ctypes.c_int32 * 3)(0, 0, 2)
    assert lib.pa_pool_create(3, bad, ctypes.byref(h)) == pa.PA_ERR_INVALID
    assert lib.pa_pool_num_free(None) == -1 and lib.pa_block_refcount(None, 0) == -1


@pytest.mark.parametrize("seed", range(8))
def test_pool_matches_model_on_random_scripts(seed):
    """Random alloc / free / share scripts, including over-frees, shares of
    free blocks and out-of-range ids: identical ids, statuses and counts."""
    rng = np.random.default_rng(seed)
    NB = int(rng.integers(1, 60))
    order = rng.permutation(NB) if seed % 2 else None
    pool = pa.BlockPool(NB, order)
    model = PoolModel(NB, order)
    for _ in range(500):
        op = int(rng.integers(0, 3))
        held = [i for i in range(NB) if model.refcount(i) > 0]
        if op == 0:
            n = int(rng.integers(-1, 8))
            st_m, ids_m = model.alloc(n)
            if st_m == 0:
                assert pool.alloc(n) == ids_m
            else:
                assert pool.status_of("alloc", n) == st_m
        else:
            k = int(rng.integers(0, 5))
            ids = [int(i) for i in rng.choice(held, size=k)] if held and rng.random() < 0.8 else \
                [int(i) for i in rng.integers(-2, NB + 2, size=k)]
            fn = "free" if op == 1 else "share"
            st_m = getattr(model, fn)(ids)
            assert pool.status_of(fn, ids) == st_m, (fn, ids)
        assert pool.num_free() == model.num_free()
        for i in range(-1, NB + 1):
            assert pool.refcount(i) == model.refcount(i)
    for i in range(NB):
        ids = [i] * model.refcount(i)
        assert model.free(ids) == 0
        pool.free(ids)
    assert pool.num_free() == model.num_free() == NB


def test_pool_leak_free_after_cancel_and_fragmentation(golden):
    """Cancelled requests return every block; 32 blocks for a 500-token
    request come from ten scattered holes."""
    g = golden("fragmentation.json")
    pool = pa.BlockPool(80)
    ids = pool.alloc(80)
    for i in range(10):
        pool.free(ids[i * 8:i * 8 + 4])
    got = pool.alloc(g["blocks_needed"])
    assert len(set(got)) == 32 and pool.num_free() == 8
    pool.free(got)
    for i in range(10):
        pool.free(ids[i * 8 + 4:i * 8 + 8])
    assert pool.num_free() == 80
    with pytest.raises(pa.PaError) as e:
        pool.free([3])
    assert e.value.status == pa.PA_ERR_STATE
    with pytest.raises(pa.PaError) as e:
        pool.alloc(81)
    assert e.value.status == pa.PA_ERR_OOM and pool.num_free() == 80


def test_workload_tables_are_what_the_pool_hands_out():
    """The workloads' seeded placement (perm = a seeded permutation, each
    sequence's logical blocks laid out on perm[0], perm[1], ...) is exactly
    what a pool created with initial_order = perm returns when each
    sequence's blocks are allocated in sequence order -- through the
    library's pool and the oracle's pool model alike."""
    import synth

    st = synth.config3_structure()
    cases = [(st["block_tables"], st["context_lens"], st["perm"], 16)]
    for c in (synth.config1(), synth.config2()):
        cases.append((c.block_tables, c.context_lens, c.perm, c.block_size))
    for tables, lens, perm, BS in cases:
        NB = len(perm)
        pool = pa.BlockPool(NB, initial_order=perm)
        model = PoolModel(NB, initial_order=perm)
        for s, n in enumerate(lens):
            nb = -(-int(n) // BS)
            got = pool.alloc(nb)
            rc, exp = model.alloc(nb)
            assert rc == 0 and got == exp == tables[s, :nb].tolist(), s
            assert np.all(tables[s, nb:] == -1)
        assert pool.num_free() == NB - int(np.sum(-(-lens // BS)))
        pool.close()


def test_noalloc_refuses_on_the_host_what_its_scratch_cannot_hold():
    """pa_decode_noalloc checks the plan's workspace against its fixed array
    before touching the device: 256 sequences of up to 32,768 tokens with
    64 query heads need more than it holds; no GPU is used."""
    lib = pa.library()
    cap = lib.pa_decode_noalloc_scratch_bytes()
    assert cap == 64 << 20
    S, Hq, Hkv, D, BS, MB = 256, 64, 8, 128, 16, 2048
    q = torch.zeros(S, Hq, D, dtype=torch.bfloat16)
    kc = torch.zeros(4, Hkv, BS, D, dtype=torch.bfloat16)
    bt = torch.zeros(S, MB, dtype=torch.int32)
    cl = torch.zeros(S, dtype=torch.int32)
    a = pa.make_decode_args(q, kc, kc, bt, cl, 0.1, MB * BS, device_pointers=False)
    a.out = 0x10000
    st, need = _ws(a)
    assert st == pa.PA_OK and need > cap
    assert lib.pa_decode_noalloc(ctypes.byref(a)) == pa.PA_ERR_INVALID
    assert "fixed scratch" in lib.pa_last_error().decode()
    # invalid arguments are refused as pa_decode refuses them
    b = _cpu_args(head_dim=96)
    assert lib.pa_decode_noalloc(ctypes.byref(b)) == pa.PA_ERR_INVALID
    assert "head_dim 96" in lib.pa_last_error().decode()


def test_wide_query_groups_are_planned_as_column_groups():
    """More than 16 query heads per kv head: the matrix-core plan takes them
    16 at a time (two groups per wave), as it does query rows; the
    workspace holds one partial row per query head."""
    lib = pa.library()
    al = lambda b: (b + 255) // 256 * 256  # noqa: E731
    for hq in (34, 64, 256):                           # 17, 32 and 128 per kv head
        a = _cpu_args(num_q_heads=hq, partition_tokens=64)
        st, n = _ws(a)
        assert st == pa.PA_OK, lib.pa_last_error()
        rows = 3 * hq * 2                              # 3 sequences, 2 partitions of 64 tokens
        assert n == al(rows * 8) + al(rows * 128 * 4)
    a = _cpu_args(num_q_heads=64, kernel=pa.KERNEL_VALU, partition_tokens=64)
    assert _ws(a)[0] == pa.PA_OK
    # the shared prefix is read through each row; the balanced split is not used
    big = dict(num_seqs=3, num_q_heads=64, max_blocks_per_seq=2048, max_context_len=32768, num_blocks=6000)
    st, n = _ws(_cpu_args(total_context_len=20000, **big))
    assert st == pa.PA_OK
    st2, n2 = _ws(_cpu_args(total_context_len=20000, shared_prefix_table=0x40000, shared_prefix_len=160, **big))
    assert st2 == pa.PA_OK and n2 == n


def test_build_flags_kernels_that_use_scratch():
    """The build fails when a kernel spills vector registers or keeps an
    array in scratch memory (read from the compiler's resource remarks)."""
    from paged_kv_cache_192_amd import build
    ok = ("x.hip:1:1: remark: Function Name: _Z1kv [-Rpass-analysis=kernel-resource-usage]\n"
          "x.hip:1:1: remark:     VGPRs: 120 [-Rpass-analysis=kernel-resource-usage]\n"
          "x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]\n"
          "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n")
    assert build._scratch_users(ok) == []
    bad = ok.replace("ScratchSize [bytes/lane]: 0", "ScratchSize [bytes/lane]: 880")
    assert build._scratch_users(bad) == ["_Z1kv: ScratchSize [bytes/lane] 880"]
    spill = ok.replace("VGPRs Spill: 0", "VGPRs Spill: 12")
    assert build._scratch_users(spill) == ["_Z1kv: VGPRs Spill 12"]


def test_binding_checks_new_rows_dtype():
    """new_key/new_value hold the cache's element type for a bf16 or fp32
    cache, and bf16 rows (quantised by the call) for an int8 or E4M3 cache."""
    S, Hq, Hkv, D, BS, NB, MB = 3, 8, 2, 128, 16, 40, 10
    q = torch.zeros(S, Hq, D, dtype=torch.bfloat16)
    bt = torch.zeros(S, MB, dtype=torch.int32)
    cl = torch.zeros(S, dtype=torch.int32)
    rows = {dt: torch.zeros(S, Hkv, D, dtype=dt) for dt in (torch.bfloat16, torch.float32)}
    for cache_dt, good, bad in ((torch.bfloat16, torch.bfloat16, torch.float32),
                                (torch.int8, torch.bfloat16, torch.float32)):
        kc = torch.zeros(NB, Hkv, BS, D, dtype=cache_dt)
        sc = {} if cache_dt == torch.bfloat16 else dict(k_scales=torch.zeros(NB, Hkv, BS),
                                                        v_scales=torch.zeros(NB, Hkv, BS))
        pa.make_decode_args(q, kc, kc, bt, cl, 0.125, 100, new_key=rows[good], new_value=rows[good],
                            device_pointers=False, **sc)
        with pytest.raises(ValueError):
            pa.make_decode_args(q, kc, kc, bt, cl, 0.125, 100, new_key=rows[bad], new_value=rows[bad],
                                device_pointers=False, **sc)
