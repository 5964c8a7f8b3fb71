"""Planted mistakes: each mutant is a copy of the oracle's C source with one
plausible bug (a dropped term, a wrong index or sign, swapped operands),
built with gcc into a temporary library.  Every mutant must fail at least
one pin, which shows the pins constrain each part of the oracle.  CPU only;
the real oracle source is never modified."""
import os

import pytest

import oracle
import pins

MUTANTS = [
    ("drop the softmax scale", "x[t] = scale * dot;", "x[t] = dot;"),
    ("query head -> KV head by modulo", "g = h / G;", "g = h % Hkv;"),
    ("logical block by modulo", "int logical_block = t / BS;", "int logical_block = t % BS;"),
    ("K read from the V cache", "kv_value(k_cache, k_scales, kv_dtype, scale_mode, b, g, t % BS",
     "kv_value(v_cache, v_scales, kv_dtype, scale_mode, b, g, t % BS"),
    ("V read from the K cache", "kv_value(v_cache, v_scales, kv_dtype, scale_mode, b, g, t % BS",
     "kv_value(k_cache, k_scales, kv_dtype, scale_mode, b, g, t % BS"),
    ("weights not normalised", "double w = x[t] / z;", "double w = x[t];"),
    ("V dequantised with the K scale", "kv_value(v_cache, v_scales,", "kv_value(v_cache, k_scales,"),
    ("sign flipped in the exponent", "x[t] = exp(x[t] - m);", "x[t] = exp(m - x[t]);"),
    ("every head uses query head 0", "const int64_t qoff = row * D;",
     "const int64_t qoff = (int64_t)s * Hq * D;"),
    ("cache layout with slot and head swapped", "return (((b * Hkv + g) * BS) + slot) * (int64_t)D + d;",
     "return (((b * BS + slot) * Hkv) + g) * (int64_t)D + d;"),
    ("last token dropped", "for (int t = 0; t < n; ++t) {\n      int64_t b = physical_block(block_tables, max_blocks, s, t, BS, NB);\n      double dot",
     "for (int t = 0; t < n - 1; ++t) {\n      int64_t b = physical_block(block_tables, max_blocks, s, t, BS, NB);\n      double dot"),
    ("int8 scale not applied", "x *= (double)scales[scale_index(b, g, slot, Hkv, BS, scale_mode)];",
     "(void)scales;"),
    ("bf16 decoded from the wrong half", "bits = ((uint32_t)h) << 16;", "bits = ((uint32_t)h);"),
    ("slot without the block stride", "slots[t] = (int64_t)b * BS + pos % BS;", "slots[t] = (int64_t)b + pos % BS;"),
    ("slot offset by division", "slots[t] = (int64_t)b * BS + pos % BS;", "slots[t] = (int64_t)b * BS + pos / BS;"),
    ("reshape writes the key into the V cache",
     "memcpy(v_cache + dst * elem_bytes, value + src * elem_bytes",
     "memcpy(v_cache + dst * elem_bytes, key + src * elem_bytes"),
    ("reshape ignores the slot offset", "off = (int)(slot % BS);\n    if (b >= NB) return -1;\n    for (int h = 0; h < Hkv; ++h)\n      for (int d",
     "off = 0;\n    if (b >= NB) return -1;\n    for (int h = 0; h < Hkv; ++h)\n      for (int d"),
    ("copy skips the V cache",
     "memmove(v_cache + dst * block_bytes, v_cache + src * block_bytes, (size_t)block_bytes);", ""),
    ("copy skips the scales",
     "for (int64_t i = 0; i < nsc; ++i) k_scales[dst * nsc + i] = k_scales[src * nsc + i];", ""),
    ("E4M3 exponent bias 8", "else v = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "else v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("E4M3 subnormals read as normals", "if (e == 0) v = ldexp((double)m / 8.0, 1 - 7);",
     "if (e == 0) v = ldexp(1.0 + (double)m / 8.0, -7);"),
    ("E4M3 ties to odd", "(above == below && (hi & 1) == 0)", "(above == below && (hi & 1) == 1)"),
    ("E4M3 rounds down always", "best = (above < below ||", "best = (0 && above < below ||"),
    ("per-token scale read per block",
     "return scale_mode == OR_SCALE_TOKEN ? (b * Hkv + g) * BS + slot : b * Hkv + g;",
     "return scale_mode == OR_SCALE_TOKEN ? (b * Hkv + g) * BS : b * Hkv + g;"),
    ("per-token scale from qmax 128", "s = amax > 0.0f ? amax / qmax : 1.0f;",
     "s = amax > 0.0f ? amax / (qmax + 1.0f) : 1.0f;"),
    ("static V scale taken from K", "s = kv ? v_static : k_static;", "s = k_static;"),
    ("quantising write truncates", "float c = rintf(r);", "float c = truncf(r);"),
    ("swap copies V from the K pool",
     "memcpy(dst_v + dst * block_bytes, src_v + src * block_bytes",
     "memcpy(dst_v + dst * block_bytes, src_k + src * block_bytes"),
    ("causal limit one token short", "n = context_lens[s] - L + i + 1;", "n = context_lens[s] - L + i;"),
    ("query row found in the next sequence", "while (query_start_loc[s + 1] <= r) ++s;",
     "while (query_start_loc[s + 1] < r) ++s;"),
    ("query rows counted from the chunk's end", "i = r - query_start_loc[s];", "i = query_start_loc[s + 1] - 1 - r;"),
    ("swap skips the destination scales",
     "for (int64_t i = 0; i < nsc; ++i) dst_ks[dst * nsc + i] = src_ks[src * nsc + i];", ""),
    ("quantiser truncates", "r = rintf(x[i] / s);", "r = truncf(x[i] / s);"),
    ("quantiser divides by 128", "amax / 127.0f", "amax / 128.0f"),
    ("quantiser keeps codes past the valid slots", "if (t >= n || amax == 0.0f)", "if (amax == 0.0f)"),
]


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, mutant_dir):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, "mutation site not unique or missing: %r" % old
    idx = MUTANTS.index((name, old, new))
    path = os.path.join(str(mutant_dir), "m%02d.c" % idx)
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(force=True, src=path, out=path[:-2] + ".so")
    caught = []
    with oracle.use_library(lib):
        for pin in pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError):
                caught.append(pin.__name__)
    assert caught, "planted mistake %r passed every pin" % name
