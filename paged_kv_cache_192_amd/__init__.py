"""Python binding of libpa (paged-KV-cache decode for MI355X).

Argument marshalling only: every entry point hands torch tensors' device
pointers, shapes and the current HIP stream to the C ABI declared in
``include/pa.h``; all work runs in the library's kernels.  PyTorch supplies
device memory and streams.  There is no fallback: if ``libpa.so`` is not
built, importing the binding's functions raises.

Build the library with ``python -m paged_kv_cache_192_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_OOM, PA_ERR_STATE, PA_ERR_HIP = range(6)
PA_F32, PA_BF16, PA_I8, PA_FP8_E4M3 = 0, 1, 2, 3
PA_SCALE_BLOCK, PA_SCALE_TOKEN = 0, 1
KERNEL_AUTO, KERNEL_VALU, KERNEL_MFMA = 0, 1, 2
ABI_VERSION = 6

STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_INVALID", 2: "PA_ERR_UNSUPPORTED", 3: "PA_ERR_OOM",
                4: "PA_ERR_STATE", 5: "PA_ERR_HIP"}


class PaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status
        self.message = message


class DecodeArgs(ctypes.Structure):
    """Mirror of ``pa_decode_args`` (field order and types as in pa.h)."""

    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("out", ctypes.c_void_p),
        ("out_dtype", ctypes.c_int),
        ("q", ctypes.c_void_p),
        ("q_dtype", ctypes.c_int),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("kv_dtype", ctypes.c_int),
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("context_lens", ctypes.c_void_p),
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_context_len", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("partition_tokens", ctypes.c_int32),
        ("kernel", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("new_key", ctypes.c_void_p),
        ("new_value", ctypes.c_void_p),
        ("total_context_len", ctypes.c_int64),
        ("kv_scale_mode", ctypes.c_int32),
        ("query_start_loc", ctypes.c_void_p),
        ("num_queries", ctypes.c_int32),
        ("max_query_len", ctypes.c_int32),
        ("shared_prefix_table", ctypes.c_void_p),
        ("shared_prefix_len", ctypes.c_int32),
    ]


_lib = None


def library() -> ctypes.CDLL:
    """The loaded libpa.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libpa.so is not built (%s); run `python -m paged_kv_cache_192_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_abi_version.argtypes = []
    lib.pa_abi_version.restype = i32
    lib.pa_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(ctypes.c_size_t)]
    lib.pa_decode_workspace_size.restype = ctypes.c_int
    lib.pa_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeArgs)]
    lib.pa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pa_decode.argtypes = [ctypes.POINTER(DecodeArgs)]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_read_probe.argtypes = [P, i64, P, i32, i32, P, P]
    lib.pa_read_probe.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs)]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_decode_noalloc_scratch_bytes.argtypes = []
    lib.pa_decode_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.pa_slot_mapping.argtypes = [P, i32, i32, P, P, P, i32, i32, P, P]
    lib.pa_slot_mapping.restype = ctypes.c_int
    lib.pa_reshape_and_cache.argtypes = [P, P, P, P, ctypes.c_int, P, i32, i32, i32, i32, i32, P]
    lib.pa_reshape_and_cache.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [P, P, ctypes.c_int, P, P, i32, P, i32, i32, i32, i32, i32, P]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_swap_blocks.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int, i32, P, i32, i32, i32, i32, i32, i32, P]
    lib.pa_swap_blocks.restype = ctypes.c_int
    f32 = ctypes.c_float
    lib.pa_quantize_and_cache.argtypes = [P, P, ctypes.c_int, P, P, ctypes.c_int, P, P, i32, f32, f32, P, i32, i32,
                                          i32, i32, i32, P]
    lib.pa_quantize_and_cache.restype = ctypes.c_int
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_pool_create.argtypes = [i32, P, ctypes.POINTER(ctypes.c_void_p)]
    lib.pa_pool_create.restype = ctypes.c_int
    lib.pa_pool_destroy.argtypes = [P]
    lib.pa_pool_destroy.restype = None
    lib.pa_block_alloc.argtypes = [P, i32, P]
    lib.pa_block_alloc.restype = ctypes.c_int
    lib.pa_block_share.argtypes = [P, i32, P]
    lib.pa_block_share.restype = ctypes.c_int
    lib.pa_block_free.argtypes = [P, i32, P]
    lib.pa_block_free.restype = ctypes.c_int
    lib.pa_block_refcount.argtypes = [P, i32]
    lib.pa_block_refcount.restype = i32
    lib.pa_pool_num_free.argtypes = [P]
    lib.pa_pool_num_free.restype = i32
    lib.pa_pool_num_blocks.argtypes = [P]
    lib.pa_pool_num_blocks.restype = i32
    del i64
    if lib.pa_abi_version() != ABI_VERSION:
        raise RuntimeError("libpa ABI version %d, binding expects %d" % (lib.pa_abi_version(), ABI_VERSION))
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != PA_OK:
        raise PaError(status, library().pa_last_error().decode(errors="replace"))


def _torch():
    import torch  # noqa: PLC0415

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: PA_F32, torch.bfloat16: PA_BF16, torch.int8: PA_I8}
    if hasattr(torch, "float8_e4m3fn"):
        codes[torch.float8_e4m3fn] = PA_FP8_E4M3
    try:
        return codes[t.dtype]
    except KeyError:
        raise TypeError("unsupported tensor dtype %s (float32, bfloat16, int8 or float8_e4m3fn)" % t.dtype)


def scale_mode_of(k_cache, k_scales) -> int:
    """PA_SCALE_TOKEN when the scales are ``[NB][Hkv][BS]``, else PA_SCALE_BLOCK."""
    return PA_SCALE_TOKEN if (k_scales is not None and k_scales.dim() == 3) else PA_SCALE_BLOCK


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _ptr_pool(t) -> Optional[int]:
    """Device tensor, or pinned host tensor (pa_swap_blocks)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if not t.is_cuda and not t.is_pinned():
        raise ValueError("host pool tensors must be pinned (pin_memory=True)")
    return t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------

def make_decode_args(q, k_cache, v_cache, block_tables, context_lens, scale: float, max_context_len: int,
                     out=None, k_scales=None, v_scales=None, workspace=None, partition_tokens: int = 0,
                     kernel: int = KERNEL_AUTO, stream=None, device_pointers: bool = True, new_key=None,
                     new_value=None, total_context_len: int = 0, query_start_loc=None,
                     max_query_len: int = 0, shared_prefix_table=None, shared_prefix_len: int = 0) -> DecodeArgs:
    """Fill a DecodeArgs from tensors.  q ``[S][Hq][D]``; caches
    ``[NB][Hkv][BS][D]``; block_tables int32 ``[S][max_blocks]``;
    context_lens int32 ``[S]``; out float32 ``[S][Hq][D]``; optional
    new_key/new_value ``[S][Hkv][D]`` for the fused cache write;
    total_context_len: optional sum of the context lengths (partition
    hint, 0 = unknown); query_start_loc int32 ``[S+1]`` with max_query_len:
    several causal query rows per sequence (q and out ``[R][Hq][D]``);
    shared_prefix_table int32 ``[shared_prefix_len / BS]``: blocks every
    table row starts with (read once for the whole batch)."""
    R, Hq, D = q.shape
    S = int(context_lens.shape[0])
    if query_start_loc is None and R != S:
        raise ValueError("q has %d rows for %d sequences (pass query_start_loc for several rows each)" % (R, S))
    NB, Hkv, BS, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache shapes %s / %s do not match q %s" % (tuple(k_cache.shape), tuple(v_cache.shape),
                                                                      tuple(q.shape)))
    a = DecodeArgs()
    a.struct_size = ctypes.sizeof(DecodeArgs)
    get = _ptr if device_pointers else (lambda t: None if t is None else t.data_ptr())
    a.out = get(out)
    a.out_dtype = PA_F32 if out is None else _dtype_code(out)
    a.q = get(q)
    a.q_dtype = _dtype_code(q)
    a.k_cache = get(k_cache)
    a.v_cache = get(v_cache)
    a.kv_dtype = _dtype_code(k_cache)
    a.k_scales = get(k_scales)
    a.v_scales = get(v_scales)
    a.block_tables = get(block_tables)
    a.max_blocks_per_seq = int(block_tables.shape[1])
    a.context_lens = get(context_lens)
    a.num_seqs = S
    a.num_q_heads = Hq
    a.num_kv_heads = Hkv
    a.head_dim = D
    a.block_size = BS
    a.num_blocks = NB
    a.max_context_len = int(max_context_len)
    a.scale = float(scale)
    a.partition_tokens = int(partition_tokens)
    a.kernel = int(kernel)
    a.workspace = get(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.stream = _stream(stream) if device_pointers else None
    quantised = _dtype_code(k_cache) in (PA_I8, PA_FP8_E4M3)
    for name, t in (("new_key", new_key), ("new_value", new_value)):
        if t is not None and tuple(t.shape) != (S, Hkv, D):
            raise ValueError("%s must be [%d][%d][%d]" % (name, S, Hkv, D))
        want = PA_BF16 if quantised else _dtype_code(k_cache)
        if t is not None and _dtype_code(t) != want:
            raise ValueError("%s must hold %s rows (%s)" % (name, "bfloat16" if quantised else "the cache's type",
                                                            "quantised by the call" if quantised else "copied"))
    a.new_key = get(new_key)
    a.new_value = get(new_value)
    a.total_context_len = int(total_context_len)
    a.kv_scale_mode = scale_mode_of(k_cache, k_scales)
    if query_start_loc is not None:
        if tuple(query_start_loc.shape) != (S + 1,):
            raise ValueError("query_start_loc must be int32 [%d]" % (S + 1))
        a.query_start_loc = get(query_start_loc)
        a.num_queries = R
        a.max_query_len = int(max_query_len)
    if shared_prefix_table is not None:
        if shared_prefix_table.dim() != 1 or int(shared_prefix_table.shape[0]) * BS != int(shared_prefix_len):
            raise ValueError("shared_prefix_table must be int32 [shared_prefix_len / block_size]")
        a.shared_prefix_table = get(shared_prefix_table)
    a.shared_prefix_len = int(shared_prefix_len)
    return a


def decode_workspace_size(args: DecodeArgs) -> int:
    n = ctypes.c_size_t(0)
    _check(library().pa_decode_workspace_size(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, max_context_len: int, out=None,
           k_scales=None, v_scales=None, workspace=None, partition_tokens: int = 0, kernel: int = KERNEL_AUTO,
           stream=None, new_key=None, new_value=None, total_context_len: int = 0, query_start_loc=None,
           max_query_len: int = 0, shared_prefix_table=None, shared_prefix_len: int = 0):
    """Paged decode attention (``pa_decode``).  Returns ``out`` (float32
    ``[S][Hq][D]``, allocated on q's device when not given, or the
    bfloat16 tensor passed: the fp32 result rounded).  A workspace
    is allocated when the plan needs one and none is passed (its contents
    are scratch of the call)."""
    torch = _torch()
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    args = make_decode_args(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len, out=out,
                            k_scales=k_scales, v_scales=v_scales, workspace=workspace,
                            partition_tokens=partition_tokens, kernel=kernel, stream=stream, new_key=new_key,
                            new_value=new_value, total_context_len=total_context_len,
                            query_start_loc=query_start_loc, max_query_len=max_query_len,
                            shared_prefix_table=shared_prefix_table, shared_prefix_len=shared_prefix_len)
    need = decode_workspace_size(args)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        args.workspace = workspace.data_ptr()
        args.workspace_bytes = need
    _check(library().pa_decode(ctypes.byref(args)))
    return out


# --------------------------------------------------------------------------
# slot mapping, cache writes, copies
# --------------------------------------------------------------------------

def slot_mapping(block_tables, block_size: int, positions=None, context_lens=None, seq_idx=None, out=None,
                 stream=None):
    """``pa_slot_mapping``: int64 slot of each new token (-1 = none)."""
    torch = _torch()
    T = (positions if positions is not None else (seq_idx if seq_idx is not None else context_lens)).shape[0]
    if out is None:
        out = torch.empty(T, dtype=torch.int64, device=block_tables.device)
    _check(library().pa_slot_mapping(_ptr(block_tables), int(block_tables.shape[1]), int(block_tables.shape[0]),
                                     _ptr(seq_idx), _ptr(positions), _ptr(context_lens), T, int(block_size),
                                     _ptr(out), _stream(stream)))
    return out


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """``pa_reshape_and_cache``: key/value ``[T][Hkv][D]`` into their slots."""
    NB, Hkv, BS, D = k_cache.shape
    T = key.shape[0]
    if tuple(key.shape) != (T, Hkv, D) or tuple(value.shape) != (T, Hkv, D):
        raise ValueError("key/value must be [T][%d][%d]" % (Hkv, D))
    if key.dtype != k_cache.dtype or value.dtype != v_cache.dtype:
        raise TypeError("key/value dtype must match the caches")
    _check(library().pa_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                          _dtype_code(k_cache), _ptr(slot_mapping), T, Hkv, D, BS, NB,
                                          _stream(stream)))


def copy_blocks(k_cache, v_cache, block_pairs, k_scales=None, v_scales=None, stream=None) -> None:
    """``pa_copy_blocks``: block_pairs int64 ``[P][2]`` of (src, dst)."""
    prepare_copy_blocks(k_cache, v_cache, block_pairs, k_scales, v_scales, stream=stream)()


def swap_blocks(src_k, src_v, dst_k, dst_v, block_pairs, src_k_scales=None, src_v_scales=None, dst_k_scales=None,
                dst_v_scales=None, stream=None) -> None:
    """``pa_swap_blocks``: whole blocks from one pool to another; either
    pool may be a pinned host tensor.  block_pairs int64 ``[P][2]`` of
    (source id, destination id), on the device or pinned."""
    prepare_swap_blocks(src_k, src_v, dst_k, dst_v, block_pairs, src_k_scales, src_v_scales, dst_k_scales,
                        dst_v_scales, stream=stream)()


def quantize_and_cache(key, value, k_cache, v_cache, k_scales, v_scales, slot_mapping, k_static_scale: float = 0.0,
                       v_static_scale: float = 0.0, stream=None) -> None:
    """``pa_quantize_and_cache``: key/value ``[T][Hkv][D]`` (float32 or
    bfloat16) quantised into int8 or float8_e4m3fn caches.  Scales
    ``[NB][Hkv]`` select the static per-layer scale (k/v_static_scale);
    ``[NB][Hkv][BS]`` the dynamic per-token scale."""
    prepare_quantize_and_cache(key, value, k_cache, v_cache, k_scales, v_scales, slot_mapping, k_static_scale,
                               v_static_scale, stream=stream)()


def prepare_read_probe(base, num_chunks: int, sink, chunk_ids=None, num_waves: int = 4096, chunk_bytes: int = 4096,
                       stream=None) -> "PreparedCall":
    """``pa_read_probe``: read num_chunks chunks of chunk_bytes (1, 2 or 4
    KiB) of ``base`` (a device tensor), in address order or in the order of
    ``chunk_ids`` (device int32); ``sink`` is a device int32 tensor of
    num_waves * 64 words."""
    if sink.numel() < num_waves * 64:
        raise ValueError("sink must hold num_waves * 64 words")
    if num_chunks * chunk_bytes > base.numel() * base.element_size() and chunk_ids is None:
        raise ValueError("chunks reach past the tensor")
    ids = None if chunk_ids is None else _ptr(chunk_ids)
    return PreparedCall("pa_read_probe", (_ptr(base), int(num_chunks), ids, int(chunk_bytes), int(num_waves),
                                          _ptr(sink), _stream(stream)), keep=(base, sink, chunk_ids))


# --------------------------------------------------------------------------
# block pool (host)
# --------------------------------------------------------------------------

class BlockPool:
    """Host block pool (``pa_pool``): stack of free ids with refcounts."""

    def __init__(self, num_blocks: int, initial_order: Optional[Sequence[int]] = None):
        lib = library()
        h = ctypes.c_void_p()
        order = None
        if initial_order is not None:
            order = (ctypes.c_int32 * num_blocks)(*[int(i) for i in initial_order])
        _check(lib.pa_pool_create(int(num_blocks), order, ctypes.byref(h)))
        self._h = h

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            library().pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass

    def alloc(self, n: int):
        ids = (ctypes.c_int32 * max(n, 1))()
        _check(library().pa_block_alloc(self._h, int(n), ids))
        return list(ids[:n])

    def _ids(self, ids):
        arr = (ctypes.c_int32 * max(len(ids), 1))(*[int(i) for i in ids])
        return len(ids), arr

    def free(self, ids) -> None:
        n, arr = self._ids(ids)
        _check(library().pa_block_free(self._h, n, arr))

    def share(self, ids) -> None:
        n, arr = self._ids(ids)
        _check(library().pa_block_share(self._h, n, arr))

    def status_of(self, op: str, ids) -> int:
        """Raw status of alloc/free/share without raising (for tests)."""
        lib = library()
        if op == "alloc":
            out = (ctypes.c_int32 * max(int(ids), 1))()
            return lib.pa_block_alloc(self._h, int(ids), out)
        n, arr = self._ids(ids)
        return (lib.pa_block_free if op == "free" else lib.pa_block_share)(self._h, n, arr)

    def refcount(self, i: int) -> int:
        return library().pa_block_refcount(self._h, int(i))

    def num_free(self) -> int:
        return library().pa_pool_num_free(self._h)

    @property
    def num_blocks(self) -> int:
        return library().pa_pool_num_blocks(self._h)


# --------------------------------------------------------------------------
# prepared calls: arguments marshalled once, launched many times (decode
# loops, graph capture).  The stream is fixed when the call is prepared.
# --------------------------------------------------------------------------

class PreparedDecode:
    """``pa_decode`` with its arguments packed once.  A workspace is
    allocated here when the plan needs one and none is given."""

    def __init__(self, q, k_cache, v_cache, block_tables, context_lens, scale: float, max_context_len: int, out,
                 k_scales=None, v_scales=None, workspace=None, partition_tokens: int = 0, kernel: int = KERNEL_AUTO,
                 stream=None, new_key=None, new_value=None, total_context_len: int = 0, query_start_loc=None,
                 max_query_len: int = 0, shared_prefix_table=None, shared_prefix_len: int = 0):
        torch = _torch()
        self.args = make_decode_args(q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                                     out=out, k_scales=k_scales, v_scales=v_scales, workspace=workspace,
                                     partition_tokens=partition_tokens, kernel=kernel, stream=stream,
                                     new_key=new_key, new_value=new_value, total_context_len=total_context_len,
                                     query_start_loc=query_start_loc, max_query_len=max_query_len,
                                     shared_prefix_table=shared_prefix_table, shared_prefix_len=shared_prefix_len)
        need = decode_workspace_size(self.args)
        if need and (workspace is None or self.args.workspace_bytes < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            self.args.workspace = workspace.data_ptr()
            self.args.workspace_bytes = need
        self.workspace_bytes = need
        self._keep = (q, k_cache, v_cache, block_tables, context_lens, out, k_scales, v_scales, workspace, new_key,
                      new_value, query_start_loc, shared_prefix_table)
        self._fn = library().pa_decode
        self._ref = ctypes.byref(self.args)

    def __call__(self) -> None:
        st = self._fn(self._ref)
        if st != PA_OK:
            _check(st)


class PreparedCall:
    """Any other entry point with its argument tuple packed once."""

    def __init__(self, name: str, args: tuple, keep: tuple = ()):
        self._fn = getattr(library(), name)
        self._args = args
        self._keep = keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != PA_OK:
            _check(st)


def prepare_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None) -> PreparedCall:
    NB, Hkv, BS, D = k_cache.shape
    T = key.shape[0]
    if tuple(key.shape) != (T, Hkv, D) or tuple(value.shape) != (T, Hkv, D):
        raise ValueError("key/value must be [T][%d][%d]" % (Hkv, D))
    args = (_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache), _ptr(slot_mapping), T, Hkv,
            D, BS, NB, _stream(stream))
    return PreparedCall("pa_reshape_and_cache", args, (key, value, k_cache, v_cache, slot_mapping))


def prepare_slot_mapping(block_tables, block_size: int, out, positions=None, context_lens=None, seq_idx=None,
                         stream=None) -> PreparedCall:
    T = out.shape[0]
    args = (_ptr(block_tables), int(block_tables.shape[1]), int(block_tables.shape[0]), _ptr(seq_idx),
            _ptr(positions), _ptr(context_lens), T, int(block_size), _ptr(out), _stream(stream))
    return PreparedCall("pa_slot_mapping", args, (block_tables, out, positions, context_lens, seq_idx))


def prepare_copy_blocks(k_cache, v_cache, block_pairs, k_scales=None, v_scales=None, stream=None) -> PreparedCall:
    NB, Hkv, BS, D = k_cache.shape
    args = (_ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache), _ptr(k_scales), _ptr(v_scales),
            scale_mode_of(k_cache, k_scales), _ptr(block_pairs), int(block_pairs.shape[0]), Hkv, D, BS, NB,
            _stream(stream))
    return PreparedCall("pa_copy_blocks", args, (k_cache, v_cache, block_pairs, k_scales, v_scales))


def prepare_swap_blocks(src_k, src_v, dst_k, dst_v, block_pairs, src_k_scales=None, src_v_scales=None,
                        dst_k_scales=None, dst_v_scales=None, stream=None) -> PreparedCall:
    sNB, Hkv, BS, D = src_k.shape
    dNB = dst_k.shape[0]
    if tuple(dst_k.shape[1:]) != (Hkv, BS, D) or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination pools differ in shape or dtype")
    args = (_ptr_pool(src_k), _ptr_pool(src_v), _ptr_pool(src_k_scales), _ptr_pool(src_v_scales), _ptr_pool(dst_k),
            _ptr_pool(dst_v), _ptr_pool(dst_k_scales), _ptr_pool(dst_v_scales), _dtype_code(src_k),
            scale_mode_of(src_k, src_k_scales), _ptr_pool(block_pairs), int(block_pairs.shape[0]), Hkv, D, BS,
            sNB, dNB, _stream(stream))
    return PreparedCall("pa_swap_blocks", args, (src_k, src_v, dst_k, dst_v, block_pairs, src_k_scales,
                                                 src_v_scales, dst_k_scales, dst_v_scales))


def prepare_quantize_and_cache(key, value, k_cache, v_cache, k_scales, v_scales, slot_mapping,
                               k_static_scale: float = 0.0, v_static_scale: float = 0.0, stream=None) -> PreparedCall:
    NB, Hkv, BS, D = k_cache.shape
    T = key.shape[0]
    if tuple(key.shape) != (T, Hkv, D) or tuple(value.shape) != (T, Hkv, D):
        raise ValueError("key/value must be [T][%d][%d]" % (Hkv, D))
    args = (_ptr(key), _ptr(value), _dtype_code(key), _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache),
            _ptr(k_scales), _ptr(v_scales), scale_mode_of(k_cache, k_scales), float(k_static_scale),
            float(v_static_scale), _ptr(slot_mapping), T, Hkv, D, BS, NB, _stream(stream))
    return PreparedCall("pa_quantize_and_cache", args, (key, value, k_cache, v_cache, k_scales, v_scales,
                                                        slot_mapping))
