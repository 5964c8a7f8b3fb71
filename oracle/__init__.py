"""CPU oracle for paged-KV-cache decode.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
the two share no code: this package loads its own C file (``pa_oracle.c``,
built with gcc) and adds three pure-Python/NumPy pieces:

* :func:`contiguous_attention` -- unpaged attention over per-sequence arrays,
  an independent second implementation used to cross-check the paged one;
* :class:`PoolModel` -- the block pool's allocation policy written out;
* thin ctypes wrappers around the C functions.

Element types: ``numpy.float32`` is fp32, ``numpy.uint16`` holds the bits of
bfloat16 values, ``numpy.int8`` is int8, ``numpy.uint8`` holds OCP E4M3 fp8
codes.  Quantised caches (int8, E4M3) come with fp32 scales laid out per
(block, KV head) ``[NB][Hkv]`` (scale mode 0) or per token ``[NB][Hkv][BS]``
(scale mode 1).

Sources, by page and section (the pages are French web articles on the KV
cache and PagedAttention):

* "Cache KV en production", opening section -- attention of the current
  token's query over the keys of all earlier tokens, weighting their values.
* deeplearn.tn KV-cache article, "La taille réelle du cache KV" -- only the
  newest query is needed when decoding.
* "PagedAttention & Gestion du KV-Cache", section 2 figure -- logical blocks
  of 16 tokens, block table, scattered physical blocks, a free block in the
  pool; section 3 scenario 01 -- shared pages, copy on write; section 4 --
  pages must return to the free pool when a request is cancelled.
* "Cache KV en production", "PagedAttention : la pagination appliquée au
  cache KV" -- pages taken one at a time as the request grows, returned to
  the common pool as soon as it ends.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libpa_oracle.so")

F32, BF16, I8, FP8 = 0, 1, 2, 3
_DTYPE_CODE = {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16, np.dtype(np.int8): I8,
               np.dtype(np.uint8): FP8}
SCALE_BLOCK, SCALE_TOKEN = 0, 1


def scale_shape(NB: int, Hkv: int, BS: int, scale_mode: int):
    return (NB, Hkv, BS) if scale_mode == SCALE_TOKEN else (NB, Hkv)

# Status codes of the pool policy (same meaning as the library's, defined
# here independently).
OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_OOM, ERR_STATE = 0, 1, 2, 3, 4


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile a copy of pa_oracle.c with gcc into a shared library."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-Wno-unused-parameter", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _bind(lib):
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    lib.oracle_paged_decode.argtypes = [P, P, i32, P, P, i32, P, P, i32, P, i32, P,
                                        i32, i32, i32, i32, i32, i32, ctypes.c_double]
    lib.oracle_paged_decode.restype = i32
    lib.oracle_paged_attention.argtypes = [P, P, i32, P, P, i32, P, P, i32, P, i32, P, P,
                                           i32, i32, i32, i32, i32, i32, ctypes.c_double]
    lib.oracle_paged_attention.restype = i32
    lib.oracle_fp8_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_fp8_e4m3_value.restype = ctypes.c_double
    lib.oracle_fp8_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_fp8_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_swap_blocks.argtypes = [P, P, P, P, P, P, P, P, i32, i32, P, i32, i32, i32, i32, i32, i32]
    lib.oracle_swap_blocks.restype = i32
    lib.oracle_quantize_and_cache.argtypes = [P, P, i32, P, P, i32, P, P, i32, ctypes.c_float, ctypes.c_float,
                                              P, i32, i32, i32, i32, i32]
    lib.oracle_quantize_and_cache.restype = i32
    lib.oracle_slot_mapping.argtypes = [P, P, i32, P, P, i32, i32]
    lib.oracle_slot_mapping.restype = None
    lib.oracle_reshape_and_cache.argtypes = [P, P, P, P, i32, P, i32, i32, i32, i32, i32]
    lib.oracle_reshape_and_cache.restype = i32
    lib.oracle_copy_blocks.argtypes = [P, P, i32, P, P, i32, P, i32, i32, i32, i32, i32]
    lib.oracle_copy_blocks.restype = i32
    lib.oracle_quantize_int8.argtypes = [P, P, P, P, i32, i32, i32, i32]
    lib.oracle_quantize_int8.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


_lib = None
_lib_override = None


def _load():
    global _lib
    if _lib_override is not None:
        return _lib_override
    if _lib is None:
        build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


class use_library:
    """Context manager: route this module's functions through another build
    of the oracle source (used by the planted-mistake test)."""

    def __init__(self, path: str):
        self._lib = _bind(ctypes.CDLL(path))

    def __enter__(self):
        global _lib_override
        self._prev = _lib_override
        _lib_override = self._lib
        return self

    def __exit__(self, *exc):
        global _lib_override
        _lib_override = self._prev
        return False


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _code(a: np.ndarray) -> int:
    try:
        return _DTYPE_CODE[a.dtype]
    except KeyError:
        raise TypeError("oracle element type must be float32, uint16 (bf16 bits), int8 or uint8 (E4M3 codes), "
                        "got %s" % a.dtype)


def fp8_e4m3_value(code: int) -> float:
    """Value of one OCP E4M3 code (NaN for 0x7F / 0xFF)."""
    return float(_load().oracle_fp8_e4m3_value(int(code) & 0xFF))


def fp8_e4m3_encode(x: float) -> int:
    """Nearest E4M3 code to the fp32 value x (ties to even mantissa,
    saturating at +-448)."""
    return int(_load().oracle_fp8_e4m3_encode(float(np.float32(x))))


def fp8_table() -> np.ndarray:
    """float64[256]: the value of every E4M3 code."""
    return np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)


def as_float64(a: np.ndarray) -> np.ndarray:
    """Exact fp64 image of an fp32 / bf16-bits / int8 / E4M3-codes array."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.uint8:
        return fp8_table()[a]
    return a.astype(np.float64)


def num_threads() -> int:
    """Threads the C oracle's decode loop uses (OpenMP maximum)."""
    return int(_load().oracle_num_threads())


# --------------------------------------------------------------------------
# decode attention (C, fp64)
# --------------------------------------------------------------------------

def paged_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                 k_scales: Optional[np.ndarray] = None, v_scales: Optional[np.ndarray] = None,
                 scale_mode: int = SCALE_BLOCK) -> np.ndarray:
    """fp64 paged decode attention, ``out[S][Hq][D]``.

    q ``[S][Hq][D]``; caches ``[NB][Hkv][BS][D]``; block_tables
    ``int32[S][max_blocks]``; context_lens ``int32[S]``; int8 and E4M3
    caches need ``k_scales``/``v_scales`` in the layout of ``scale_mode``.
    ``scale`` is applied as given (pass the fp32 value a kernel receives to
    compare like with like).
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    S, Hq, D = q.shape
    NB, Hkv, BS, D2 = k_cache.shape
    assert D2 == D and v_cache.shape == k_cache.shape and k_cache.dtype == v_cache.dtype
    assert bt.ndim == 2 and bt.shape[0] == S and cl.shape == (S,)
    kv = _code(k_cache)
    if kv in (I8, FP8):
        assert k_scales is not None and v_scales is not None
        k_scales = np.ascontiguousarray(k_scales, dtype=np.float32)
        v_scales = np.ascontiguousarray(v_scales, dtype=np.float32)
        shp = scale_shape(NB, Hkv, BS, scale_mode)
        assert k_scales.shape == shp and v_scales.shape == shp
    else:
        k_scales = v_scales = None
    out = np.zeros((S, Hq, D), dtype=np.float64)
    rc = lib.oracle_paged_decode(_ptr(out), _ptr(q), _code(q), _ptr(k_cache), _ptr(v_cache), kv,
                                 _ptr(k_scales), _ptr(v_scales), int(scale_mode), _ptr(bt), bt.shape[1],
                                 _ptr(cl), S, Hq, Hkv, D, BS, NB, float(scale))
    if rc != 0:
        raise ValueError("oracle_paged_decode: a table entry or context length is out of range")
    return out


def paged_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                    block_tables: np.ndarray, context_lens: np.ndarray, query_start_loc: np.ndarray,
                    scale: float, k_scales: Optional[np.ndarray] = None, v_scales: Optional[np.ndarray] = None,
                    scale_mode: int = SCALE_BLOCK) -> np.ndarray:
    """fp64 paged attention with several causal query rows per sequence,
    ``out[R][Hq][D]``; ``q [R][Hq][D]``, ``query_start_loc int32[S+1]`` from
    0 to R: the rows of sequence s are its last L_s tokens."""
    lib = _load()
    q = np.ascontiguousarray(q)
    k_cache = np.ascontiguousarray(k_cache)
    v_cache = np.ascontiguousarray(v_cache)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    R, Hq, D = q.shape
    NB, Hkv, BS, _ = k_cache.shape
    S = cl.shape[0]
    assert qsl.shape == (S + 1,) and qsl[0] == 0 and qsl[-1] == R
    kv = _code(k_cache)
    if kv in (I8, FP8):
        k_scales = np.ascontiguousarray(k_scales, dtype=np.float32)
        v_scales = np.ascontiguousarray(v_scales, dtype=np.float32)
    else:
        k_scales = v_scales = None
    out = np.zeros((R, Hq, D), dtype=np.float64)
    rc = lib.oracle_paged_attention(_ptr(out), _ptr(q), _code(q), _ptr(k_cache), _ptr(v_cache), kv,
                                    _ptr(k_scales), _ptr(v_scales), int(scale_mode), _ptr(bt), bt.shape[1],
                                    _ptr(cl), _ptr(qsl), S, Hq, Hkv, D, BS, NB, float(scale))
    if rc != 0:
        raise ValueError("oracle_paged_attention: bad table entry, length or offsets")
    return out


# --------------------------------------------------------------------------
# contiguous (unpaged) attention, NumPy -- independent cross-check
# --------------------------------------------------------------------------

def contiguous_attention(q64: np.ndarray, keys: Sequence[np.ndarray], values: Sequence[np.ndarray],
                         scale: float) -> np.ndarray:
    """Attention of one query row per sequence over that sequence's own
    contiguous key/value arrays (the pre-paging layout the pages contrast
    with: one contiguous buffer per request).

    q64 ``[S][Hq][D]`` float64; ``keys[s]``/``values[s]`` ``[n_s][Hkv][D]``
    float64.  Query head h reads KV head ``h // (Hq // Hkv)``.
    """
    S, Hq, D = q64.shape
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        K, V = keys[s], values[s]
        n = K.shape[0]
        if n == 0:
            continue
        G = Hq // K.shape[1]
        Kh = np.repeat(K, G, axis=1)  # [n][Hq][D]
        Vh = np.repeat(V, G, axis=1)
        logits = scale * np.einsum("hd,thd->ht", q64[s], Kh)
        logits -= logits.max(axis=1, keepdims=True)
        w = np.exp(logits)
        w /= w.sum(axis=1, keepdims=True)
        out[s] = np.einsum("ht,thd->hd", w, Vh)
    return out


def gather_logical(cache: np.ndarray, block_tables: np.ndarray, context_lens: np.ndarray,
                   scales: Optional[np.ndarray] = None) -> List[np.ndarray]:
    """Per-sequence contiguous fp64 copies ``[n_s][Hkv][D]`` read through the
    block tables (for building inputs of :func:`contiguous_attention` from a
    paged cache); scales ``[NB][Hkv]`` or per token ``[NB][Hkv][BS]``."""
    NB, Hkv, BS, D = cache.shape
    c64 = as_float64(cache)
    if scales is not None:
        sc = np.asarray(scales, dtype=np.float64)
        c64 = c64 * (sc[:, :, :, None] if sc.ndim == 3 else sc[:, :, None, None])
    res = []
    for s, n in enumerate(np.asarray(context_lens)):
        rows = [c64[block_tables[s][t // BS], :, t % BS, :] for t in range(int(n))]
        res.append(np.stack(rows) if rows else np.zeros((0, Hkv, D)))
    return res


# --------------------------------------------------------------------------
# slot mapping, cache writes, block copies (C, byte exact)
# --------------------------------------------------------------------------

def slot_mapping(block_tables: np.ndarray, positions: np.ndarray, block_size: int,
                 seq_idx: Optional[np.ndarray] = None) -> np.ndarray:
    lib = _load()
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    si = None if seq_idx is None else np.ascontiguousarray(seq_idx, dtype=np.int32)
    out = np.empty(pos.shape[0], dtype=np.int64)
    lib.oracle_slot_mapping(_ptr(out), _ptr(bt), bt.shape[1], _ptr(si), _ptr(pos), pos.shape[0],
                            int(block_size))
    return out


def reshape_and_cache(key: np.ndarray, value: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                      slots: np.ndarray) -> None:
    """In place on k_cache / v_cache ``[NB][Hkv][BS][D]``; key/value ``[T][Hkv][D]``."""
    lib = _load()
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    sl = np.ascontiguousarray(slots, dtype=np.int64)
    NB, Hkv, BS, D = k_cache.shape
    assert key.dtype == k_cache.dtype == value.dtype == v_cache.dtype
    assert key.shape == value.shape == (sl.shape[0], Hkv, D)
    rc = lib.oracle_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                      key.dtype.itemsize, _ptr(sl), sl.shape[0], Hkv, D, BS, NB)
    if rc != 0:
        raise ValueError("oracle_reshape_and_cache: slot beyond the pool")


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs: np.ndarray,
                k_scales: Optional[np.ndarray] = None, v_scales: Optional[np.ndarray] = None,
                scale_mode: int = SCALE_BLOCK) -> None:
    """In place; ``pairs`` is ``int64[P][2]`` of (src, dst) block ids."""
    lib = _load()
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    pr = np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    NB, Hkv, BS, D = k_cache.shape
    for a in (k_scales, v_scales):
        assert a is None or (a.flags.c_contiguous and a.dtype == np.float32 and
                             a.shape == scale_shape(NB, Hkv, BS, scale_mode))
    rc = lib.oracle_copy_blocks(_ptr(k_cache), _ptr(v_cache), k_cache.dtype.itemsize,
                                _ptr(k_scales), _ptr(v_scales), int(scale_mode), _ptr(pr), pr.shape[0],
                                Hkv, D, BS, NB)
    if rc != 0:
        raise ValueError("oracle_copy_blocks: block id out of range")


def swap_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray, pairs: np.ndarray,
                src_ks: Optional[np.ndarray] = None, src_vs: Optional[np.ndarray] = None,
                dst_ks: Optional[np.ndarray] = None, dst_vs: Optional[np.ndarray] = None,
                scale_mode: int = SCALE_BLOCK) -> None:
    """In place on the destination pool; pools ``[NB][Hkv][BS][D]`` of one
    element type, ``pairs`` ``int64[P][2]`` of (source id, destination id)."""
    lib = _load()
    for a in (src_k, src_v, dst_k, dst_v):
        assert a.flags.c_contiguous
    assert src_k.dtype == dst_k.dtype and src_k.shape[1:] == dst_k.shape[1:]
    pr = np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    sNB, Hkv, BS, D = src_k.shape
    dNB = dst_k.shape[0]
    rc = lib.oracle_swap_blocks(_ptr(src_k), _ptr(src_v), _ptr(src_ks), _ptr(src_vs), _ptr(dst_k), _ptr(dst_v),
                                _ptr(dst_ks), _ptr(dst_vs), src_k.dtype.itemsize, int(scale_mode), _ptr(pr),
                                pr.shape[0], Hkv, D, BS, sNB, dNB)
    if rc != 0:
        raise ValueError("oracle_swap_blocks: block id out of range")


def quantize_and_cache(key: np.ndarray, value: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                       k_scales: np.ndarray, v_scales: np.ndarray, slots: np.ndarray, scale_mode: int,
                       k_static: float = 0.0, v_static: float = 0.0) -> None:
    """Quantising cache write, in place.  key/value ``[T][Hkv][D]`` float32
    or bf16 bits; caches int8 or uint8 (E4M3 codes) ``[NB][Hkv][BS][D]``;
    scales in the layout of ``scale_mode`` (0: static scale per layer, given
    as k_static / v_static and stamped per (block, head); 1: per token)."""
    lib = _load()
    for a in (k_cache, v_cache, k_scales, v_scales):
        assert a.flags.c_contiguous
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    sl = np.ascontiguousarray(slots, dtype=np.int64)
    NB, Hkv, BS, D = k_cache.shape
    assert key.dtype == value.dtype and key.shape == value.shape == (sl.shape[0], Hkv, D)
    assert k_cache.dtype == v_cache.dtype and _code(k_cache) in (I8, FP8)
    assert k_scales.dtype == np.float32 and k_scales.shape == scale_shape(NB, Hkv, BS, scale_mode)
    rc = lib.oracle_quantize_and_cache(_ptr(key), _ptr(value), _code(key), _ptr(k_cache), _ptr(v_cache),
                                       _code(k_cache), _ptr(k_scales), _ptr(v_scales), int(scale_mode),
                                       float(k_static), float(v_static), _ptr(sl), sl.shape[0], Hkv, D, BS, NB)
    if rc != 0:
        raise ValueError("oracle_quantize_and_cache: slot beyond the pool or bad static scale")


def quantize_int8(x: np.ndarray, valid: np.ndarray):
    """Per-(block, KV head) symmetric int8 codes and fp32 scales of
    ``x float32[NB][Hkv][BS][D]``; ``valid int32[NB]`` leading slots count."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    NB, Hkv, BS, D = x.shape
    va = np.ascontiguousarray(valid, dtype=np.int32)
    assert va.shape == (NB,)
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty((NB, Hkv), dtype=np.float32)
    lib.oracle_quantize_int8(_ptr(codes), _ptr(scales), _ptr(x), _ptr(va), NB, Hkv, BS, D)
    return codes, scales


# --------------------------------------------------------------------------
# block pool policy (pure Python)
# --------------------------------------------------------------------------

class PoolModel:
    """The block pool's policy written out.

    * A stack of free ids; ``initial_order[0]`` is the first id handed out
      (default 0, 1, 2, ...).
    * ``alloc(n)``: all or nothing -- OOM with nothing changed when fewer
      than n ids are free; otherwise pops n ids, each with refcount 1.
    * ``share(ids)``: refcount + 1 per occurrence (a second sequence now
      points at the block: prefix sharing / fork).
    * ``free(ids)``: refcount - 1 per occurrence, in array order; an id whose
      count reaches 0 is pushed back on the stack at once.
    * The whole call is validated before anything changes: an id outside
      [0, NB) is INVALID; freeing or sharing a block more times than it is
      held is STATE.
    """

    def __init__(self, num_blocks: int, initial_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        order = list(range(num_blocks)) if initial_order is None else [int(i) for i in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self._stack = order[::-1]  # top of stack = end of list
        self._ref = [0] * num_blocks

    def num_free(self) -> int:
        return len(self._stack)

    def refcount(self, i: int) -> int:
        return self._ref[i] if 0 <= i < self.num_blocks else -1

    def alloc(self, n: int):
        if n < 0:
            return ERR_INVALID, []
        if n > len(self._stack):
            return ERR_OOM, []
        ids = [self._stack.pop() for _ in range(n)]
        for i in ids:
            self._ref[i] = 1
        return OK, ids

    def _validate(self, ids, need_held: bool):
        counts = {}
        for i in ids:
            if not (0 <= i < self.num_blocks):
                return ERR_INVALID
            counts[i] = counts.get(i, 0) + 1
        for i, c in counts.items():
            if self._ref[i] == 0 or (need_held and c > self._ref[i]):
                return ERR_STATE
        return OK

    def share(self, ids) -> int:
        ids = [int(i) for i in ids]
        rc = self._validate(ids, need_held=False)
        if rc != OK:
            return rc
        for i in ids:
            self._ref[i] += 1
        return OK

    def free(self, ids) -> int:
        ids = [int(i) for i in ids]
        rc = self._validate(ids, need_held=True)
        if rc != OK:
            return rc
        for i in ids:
            self._ref[i] -= 1
            if self._ref[i] == 0:
                self._stack.append(i)
        return OK
