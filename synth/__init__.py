"""Seeded synthetic inputs for paged decode (shapes, lengths, block tables, values).

Shared by the tests, the smoke check and the benchmark, and by nothing in
the product library.  It holds none of the method's arithmetic: it draws
lengths, permutations and N(0, 1) values, lays out block tables from a
permutation, rounds fp32 samples to bfloat16 (input formatting) and poisons
unused memory.  Attention, slot mapping, cache writes, copies, quantisation
and the pool policy live elsewhere.

Workload shapes follow the sizing examples on the pages: a Llama-13B-like
model on a 40 GB card (forum thread and deeplearn.tn article), Llama-3-70B
serving 20 requests of 8,000 tokens (ia-vox article, "Pourquoi le KV cache
domine"), 50 users sharing one prompt (glossary, section 3 scenario 01), an
int8 KV cache (ia-vox "Quantization du KV cache").

Element conventions: fp32 as ``numpy.float32``; bfloat16 as its bit pattern
in ``numpy.uint16``; int8 codes as ``numpy.int8``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

F32, BF16, I8, FP8 = "f32", "bf16", "i8", "fp8"   # fp8: OCP E4M3 codes held as uint8

BF16_NAN = np.uint16(0x7FC0)
F32_NAN = np.float32("nan")
I8_POISON = np.int8(127)
FP8_POISON = np.uint8(0x7F)   # the E4M3 NaN code


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 samples to bfloat16 (round to nearest even) and return the bits."""
    import torch  # noqa: PLC0415 - torch is only needed for this conversion

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern -> fp32 with the same value (exact)."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


@dataclass
class DecodeCase:
    """One decode batch over one layer's paged cache."""

    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    q_dtype: str
    kv_dtype: str
    scale: np.float32
    context_lens: np.ndarray            # int32 [S]
    block_tables: np.ndarray            # int32 [S][max_blocks], -1 padded
    q: np.ndarray                       # [S][Hq][D] float32 or uint16 bits
    k_cache: np.ndarray                 # [NB][Hkv][BS][D]
    v_cache: np.ndarray
    k_scales: Optional[np.ndarray] = None   # float32 [NB][Hkv] (int8 only)
    v_scales: Optional[np.ndarray] = None
    free_blocks: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    perm: Optional[np.ndarray] = None   # the physical permutation used
    extra: Dict[str, object] = field(default_factory=dict)

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0


def _values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    return bf16_bits(x) if dtype == BF16 else x


def _poison_value(dtype: str):
    return {F32: F32_NAN, BF16: BF16_NAN, I8: I8_POISON, FP8: FP8_POISON}[dtype]


def assign_tables(rng: np.random.Generator, num_blocks: int, blocks_per_seq: List[int],
                  max_blocks: Optional[int] = None):
    """Seeded physical placement: perm = rng.permutation(NB); logical blocks
    are laid out in sequence order (seq 0 block 0, 1, ..., then seq 1 ...) on
    perm[0], perm[1], ...  Returns (tables int32 [S][max_blocks] padded with
    -1, perm, free ids)."""
    perm = rng.permutation(num_blocks).astype(np.int32)
    total = int(sum(blocks_per_seq))
    if total > num_blocks:
        raise ValueError("pool too small: %d blocks needed, %d in the pool" % (total, num_blocks))
    mb = max(max(blocks_per_seq, default=0), 1) if max_blocks is None else max_blocks
    tables = np.full((len(blocks_per_seq), mb), -1, dtype=np.int32)
    k = 0
    for s, nb in enumerate(blocks_per_seq):
        tables[s, :nb] = perm[k:k + nb]
        k += nb
    return tables, perm, perm[total:].copy()


def poison_unused(cache: np.ndarray, tables: np.ndarray, context_lens: np.ndarray,
                  free_blocks: np.ndarray, dtype: str) -> None:
    """Fill tail slots of each sequence's last block and every free block
    with NaN (float) or +127 (int8), so a kernel that reads them fails."""
    bad = _poison_value(dtype)
    BS = cache.shape[2]
    if len(free_blocks):
        cache[free_blocks] = bad
    for s, n in enumerate(context_lens):
        n = int(n)
        if n % BS:
            cache[tables[s, n // BS], :, n % BS:, :] = bad


def make_case(name: str, seed: int, context_lens, num_q_heads: int, num_kv_heads: int,
              head_dim: int, block_size: int, num_blocks: Optional[int] = None,
              q_dtype: str = BF16, kv_dtype: str = BF16, scale: Optional[float] = None,
              poison: bool = True, free_frac: float = 0.0, max_blocks: Optional[int] = None
              ) -> DecodeCase:
    """Generic seeded decode batch.  For int8 and E4M3 caches the fp32
    samples are returned in ``extra['k_f32']``/``extra['v_f32']`` with zero
    codes; the caller quantises them (the quantiser is not input
    generation)."""
    rng = np.random.default_rng(seed)
    cl = np.asarray(context_lens, dtype=np.int32)
    S = cl.shape[0]
    bps = [-(-int(n) // block_size) for n in cl]
    used = sum(bps)
    NB = num_blocks if num_blocks is not None else max(1, math.ceil(used * (1.0 + free_frac)))
    tables, perm, free = assign_tables(rng, NB, bps, max_blocks)
    shape = (NB, num_kv_heads, block_size, head_dim)
    q = _values(rng, (S, num_q_heads, head_dim), q_dtype)
    extra: Dict[str, object] = {}
    if kv_dtype in (I8, FP8):
        extra["k_f32"] = rng.standard_normal(shape, dtype=np.float32)
        extra["v_f32"] = rng.standard_normal(shape, dtype=np.float32)
        k = np.zeros(shape, np.int8 if kv_dtype == I8 else np.uint8)
        v = np.zeros_like(k)
    else:
        k = _values(rng, shape, kv_dtype)
        v = _values(rng, shape, kv_dtype)
    if poison and kv_dtype not in (I8, FP8):
        poison_unused(k, tables, cl, free, kv_dtype)
        poison_unused(v, tables, cl, free, kv_dtype)
    sc = np.float32(1.0 / math.sqrt(head_dim)) if scale is None else np.float32(scale)
    return DecodeCase(name, S, num_q_heads, num_kv_heads, head_dim, block_size, NB, q_dtype,
                      kv_dtype, sc, cl, tables, q, k, v, free_blocks=free, perm=perm, extra=extra)


def valid_slots_per_block(case: DecodeCase) -> np.ndarray:
    """int32[NB]: how many leading slots of each physical block hold tokens."""
    valid = np.zeros(case.num_blocks, np.int32)
    BS = case.block_size
    for s, n in enumerate(case.context_lens):
        n = int(n)
        for j in range(-(-n // BS)):
            valid[case.block_tables[s, j]] = min(BS, n - j * BS)
    return valid


# --------------------------------------------------------------------------
# The five workload configurations
# --------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny-fp32",
    2: "llama13b-mha-bf16",
    3: "llama3-70b-gqa-bf16-80layers",
    4: "prefix-share-cow-bf16",
    5: "int8-kv-lognormal",
}


def config1() -> DecodeCase:
    """4 sequences of 17, 33, 100, 200 tokens; 8 = 8 heads of 64; fp32;
    blocks of 16 in a pool of 64 placed by a seeded permutation; scale 1/8."""
    return make_case(CONFIG_NAMES[1], 1, [17, 33, 100, 200], 8, 8, 64, 16, num_blocks=64,
                     q_dtype=F32, kv_dtype=F32, scale=1.0 / 8.0)


def config2_lengths(rng: np.random.Generator) -> np.ndarray:
    return rng.integers(200, 2048, size=32, endpoint=True).astype(np.int32)


def config2() -> DecodeCase:
    """Llama-13B-shaped layer: 32 sequences, lengths uniform in [200, 2048],
    40 = 40 heads of 128, bf16, blocks of 16, pool = used + 10 % free."""
    rng = np.random.default_rng(2)
    cl = config2_lengths(rng)
    seed2 = int(rng.integers(0, 2**31))
    return make_case(CONFIG_NAMES[2], seed2, cl, 40, 40, 128, 16, free_frac=0.10)


CFG3 = dict(layers=80, num_seqs=20, num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
            context_len=8000)


def config3_structure():
    """Tables, lengths and scale shared by all 80 layers of the 70B-shaped
    batch: 20 sequences of 8,000 tokens, 500 blocks each, pool of exactly
    10,000 blocks per layer, seeded permutation."""
    c = CFG3
    rng = np.random.default_rng(3)
    nbs = c["context_len"] // c["block_size"]
    tables, perm, free = assign_tables(rng, c["num_seqs"] * nbs, [nbs] * c["num_seqs"])
    cl = np.full(c["num_seqs"], c["context_len"], np.int32)
    return dict(context_lens=cl, block_tables=tables, perm=perm, free_blocks=free,
                num_blocks=c["num_seqs"] * nbs, scale=np.float32(1.0 / math.sqrt(c["head_dim"])))


def config3_layer_values(layer: int, device, num_blocks: Optional[int] = None):
    """Device-generated bf16 q, K, V, new-token K/V of one layer (torch
    generator seeded 3000 + layer).  Returns torch tensors on ``device``."""
    import torch  # noqa: PLC0415

    c = CFG3
    NB = config3_structure()["num_blocks"] if num_blocks is None else num_blocks
    g = torch.Generator(device=device)
    g.manual_seed(3000 + layer)
    shape = (NB, c["num_kv_heads"], c["block_size"], c["head_dim"])

    def randn(*shp):
        return torch.randn(*shp, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)

    k = randn(*shape)
    v = randn(*shape)
    q = randn(c["num_seqs"], c["num_q_heads"], c["head_dim"])
    k_new = randn(c["num_seqs"], c["num_kv_heads"], c["head_dim"])
    v_new = randn(c["num_seqs"], c["num_kv_heads"], c["head_dim"])
    return q, k, v, k_new, v_new


def config3_layer_case(layer: int = 0) -> DecodeCase:
    """Host copy of one 70B-shaped layer (CPU generator; used where a GPU
    is absent).  Values come from the same seeded torch generator on CPU,
    which differs from the device stream, so parity always reads back the
    device bytes."""
    st = config3_structure()
    c = CFG3
    q, k, v, _, _ = config3_layer_values(layer, "cpu")
    u16 = lambda t: t.view(__import__("torch").int16).numpy().view(np.uint16)  # noqa: E731
    return DecodeCase(CONFIG_NAMES[3], c["num_seqs"], c["num_q_heads"], c["num_kv_heads"],
                      c["head_dim"], c["block_size"], st["num_blocks"], BF16, BF16, st["scale"],
                      st["context_lens"], st["block_tables"], u16(q), u16(k), u16(v),
                      free_blocks=st["free_blocks"], perm=st["perm"])


CFG4 = dict(num_seqs=50, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=32,
            prefix_len=2000, suffix_lo=50, suffix_hi=500, scratch=50)


def config4() -> DecodeCase:
    """Prefix sharing + copy-on-write.  A 2,000-token prefix (62 full blocks
    of 32 and a partial block holding 16 tokens) is stored once and every
    table points at its full blocks; each sequence owns a copy of the
    partial block, continued by its suffix (uniform 50..500 tokens, the
    newest token included), and a scratch block that receives the per-step
    copy of the shared partial block.  Pool = used + 50 scratch + 10 %.

    extra: 'shared' (62 ids), 'partial' (the shared partial block),
    'private' (list of per-sequence id lists, first = its partial copy),
    'scratch' (50 ids), 'new_pos' (position of each newest token),
    'k_new'/'v_new' [S][Hkv][D] bits of the newest tokens."""
    c = CFG4
    rng = np.random.default_rng(4)
    S, BS = c["num_seqs"], c["block_size"]
    suffix = rng.integers(c["suffix_lo"], c["suffix_hi"], size=S, endpoint=True).astype(np.int32)
    n_full = c["prefix_len"] // BS                  # 62
    part = c["prefix_len"] - n_full * BS            # 16 tokens in the partial block
    priv_counts = [-(-(part + int(n)) // BS) for n in suffix]
    used = n_full + 1 + sum(priv_counts)
    NB = math.ceil((used + c["scratch"]) * 1.10)
    perm = rng.permutation(NB).astype(np.int32)
    shared = perm[:n_full]
    partial = int(perm[n_full])
    k0 = n_full + 1
    private = []
    for cnt in priv_counts:
        private.append(perm[k0:k0 + cnt].copy())
        k0 += cnt
    scratch = perm[k0:k0 + c["scratch"]].copy()
    free = perm[k0 + c["scratch"]:].copy()
    cl = (c["prefix_len"] + suffix).astype(np.int32)
    mb = n_full + max(priv_counts)
    tables = np.full((S, mb), -1, np.int32)
    for s in range(S):
        tables[s, :n_full] = shared
        tables[s, n_full:n_full + priv_counts[s]] = private[s]
    H, D = c["num_kv_heads"], c["head_dim"]
    shape = (NB, H, BS, D)
    k = _values(rng, shape, BF16)
    v = _values(rng, shape, BF16)
    q = _values(rng, (S, c["num_q_heads"], D), BF16)
    k_new = _values(rng, (S, H, D), BF16)
    v_new = _values(rng, (S, H, D), BF16)
    # Every sequence starts from an exact copy of the shared partial block
    # (the copy-on-write that happened when it began its own answer); the
    # setup copy here is input preparation, the per-step copy is timed.
    # Its own tokens continue the copied block from slot `part` on.
    for s in range(S):
        k[private[s][0], :, :part, :] = k[partial, :, :part, :]
        v[private[s][0], :, :part, :] = v[partial, :, :part, :]
    # poison: the shared partial block's tail, sequence tails, scratch, free
    bad = BF16_NAN
    for arr in (k, v):
        arr[partial, :, part:, :] = bad
        arr[scratch] = bad
        if len(free):
            arr[free] = bad
        for s in range(S):
            n = int(cl[s])
            if n % BS:
                arr[tables[s, n // BS], :, n % BS:, :] = bad
    case = DecodeCase(CONFIG_NAMES[4], S, c["num_q_heads"], H, D, BS, NB, BF16, BF16,
                      np.float32(1.0 / math.sqrt(D)), cl, tables, q, k, v, free_blocks=free,
                      perm=perm)
    case.extra.update(shared=shared, partial=partial, private=private, scratch=scratch,
                      new_pos=(cl - 1).astype(np.int32), k_new=k_new, v_new=v_new,
                      suffix=suffix)
    return case


def config5_lengths(rng: np.random.Generator, n: int = 64) -> np.ndarray:
    """round(LogNormal(ln 1500, sigma 1.0)), clipped to [16, 32768]."""
    x = rng.lognormal(mean=math.log(1500.0), sigma=1.0, size=n)
    return np.clip(np.rint(x), 16, 32768).astype(np.int32)


def config5() -> DecodeCase:
    """int8 KV: 64 sequences, log-normal lengths (median 1,500), 32 query /
    8 KV heads of 128, blocks of 16, bf16 q; fp32 samples in extra for the
    quantiser; pool = exactly the used blocks."""
    rng = np.random.default_rng(5)
    cl = config5_lengths(rng)
    seed2 = int(rng.integers(0, 2**31))
    return make_case(CONFIG_NAMES[5], seed2, cl, 32, 8, 128, 16, q_dtype=BF16, kv_dtype=I8,
                     poison=False)


def random_int8_cache(case: DecodeCase, seed: int = 0, per_token: bool = False) -> None:
    """Fill an int8 case with random codes in [-127, 127] and positive fp32
    scales, per (block, head) or per token (timing inputs; parity tests
    quantise fp32 samples instead)."""
    rng = np.random.default_rng(seed)
    shape = case.k_cache.shape
    case.k_cache = rng.integers(-127, 128, shape).astype(np.int8)
    case.v_cache = rng.integers(-127, 128, shape).astype(np.int8)
    sshape = shape[:3] if per_token else shape[:2]
    case.k_scales = (rng.random(sshape) * 0.03 + 0.005).astype(np.float32)
    case.v_scales = (rng.random(sshape) * 0.03 + 0.005).astype(np.float32)


def random_fp8_cache(case: DecodeCase, seed: int = 0, per_token: bool = False) -> None:
    """Fill a case with random finite E4M3 codes (exponent field 0..14) and
    positive fp32 scales (timing inputs)."""
    rng = np.random.default_rng(seed)
    shape = case.k_cache.shape
    case.k_cache = rng.integers(0, 256, shape).astype(np.uint8) & np.uint8(0xF7)
    case.v_cache = rng.integers(0, 256, shape).astype(np.uint8) & np.uint8(0xF7)
    case.kv_dtype = FP8
    sshape = shape[:3] if per_token else shape[:2]
    case.k_scales = (rng.random(sshape) * 0.01 + 0.002).astype(np.float32)
    case.v_scales = (rng.random(sshape) * 0.01 + 0.002).astype(np.float32)


def token_slots(case: DecodeCase) -> np.ndarray:
    """int64[sum n_s]: the slot of every cached token, sequence by sequence."""
    BS = case.block_size
    out = []
    for s, n in enumerate(case.context_lens):
        for t in range(int(n)):
            out.append(int(case.block_tables[s, t // BS]) * BS + t % BS)
    return np.asarray(out, np.int64)
