"""PA_DEBUG: the device-side preconditions pa.h leaves to the caller are
checked before any launch.

Every bad input here is one the kernels already survive (an out-of-range id
contributes nothing, a bad slot or pair is skipped); under PA_DEBUG the call
instead returns PA_ERR_INVALID naming the violation, and nothing on the
device is touched.  Valid calls give exactly the result they give without
the checks, and a call captured into a HIP graph is not checked (a capture
cannot synchronise) but still runs."""
import numpy as np
import pytest
import torch

import paged_kv_cache_192_amd as pa
import synth
from gpu_helpers import TOL_BF16, case_on_device, max_err, run_oracle, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug(monkeypatch):
    monkeypatch.setenv("PA_DEBUG", "1")


def _case():
    return synth.make_case("debug", 77, [1, 17, 300, 0, 129], 16, 4, 128, 16, free_frac=0.3)


def _decode(case, d, **kw):
    return pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len, **kw)


def _rejected(fn, needle):
    with pytest.raises(pa.PaError) as e:
        fn()
    assert e.value.status == pa.PA_ERR_INVALID and "PA_DEBUG" in e.value.message, e.value.message
    assert needle in e.value.message, e.value.message


def test_valid_calls_are_unchanged(debug, monkeypatch):
    case = _case()
    d = case_on_device(case)
    say("PA_DEBUG valid decode")
    got = _decode(case, d)
    torch.cuda.synchronize()
    assert max_err(got.cpu().numpy().astype(np.float64), run_oracle(case)) <= TOL_BF16
    monkeypatch.setenv("PA_DEBUG", "0")
    ref = _decode(case, d)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_decode_table_entry_outside_the_pool(debug):
    case = _case()
    NB = case.k_cache.shape[0]
    case.block_tables[2, 5] = NB + 3            # in use: sequence 2 has 19 blocks
    case.block_tables[0, 4] = NB + 9            # past sequence 0's one block: unused, not checked
    d = case_on_device(case)
    out = torch.full(tuple(case.q.shape), 7.0, dtype=torch.float32, device="cuda")
    say("PA_DEBUG table entry outside the pool")
    _rejected(lambda: _decode(case, d, out=out), "block_tables[2][5]")
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())             # nothing launched


def test_decode_length_above_max_context_len(debug):
    case = _case()
    d = case_on_device(case)
    say("PA_DEBUG length above max_context_len")
    _rejected(lambda: pa.decode(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), 200),
              "context_lens[2] = 300")


def test_decode_query_rows_and_shared_prefix(debug):
    case = synth.make_case("debug-mq", 78, [40, 64, 33], 8, 1, 128, 16)
    d = case_on_device(case)
    qsl = np.array([0, 2, 5, 7], np.int32)
    q = to_dev(synth.bf16_bits(np.random.default_rng(1).standard_normal((7, 8, 128)).astype(np.float32)))
    say("PA_DEBUG query rows")
    out = pa.decode(q, d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                    query_start_loc=to_dev(qsl), max_query_len=3)
    torch.cuda.synchronize()
    bad = qsl.copy()
    bad[3] = 6                                   # does not end at num_queries = 7
    _rejected(lambda: pa.decode(q, d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                                query_start_loc=to_dev(bad), max_query_len=3), "query_start_loc")
    _rejected(lambda: pa.decode(q, d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                                query_start_loc=to_dev(qsl), max_query_len=2), "3 query rows")
    # a "shared prefix" that is not what the table rows start with
    say("PA_DEBUG shared prefix")
    prefix = case.block_tables[1, :2].copy()
    _rejected(lambda: _decode(case, d, shared_prefix_table=to_dev(prefix), shared_prefix_len=32), "shared prefix")
    assert out.shape == (7, 8, 128)


def test_fused_write_to_one_slot_from_two_sequences(debug):
    case = synth.make_case("debug-fused", 79, [20, 20, 5], 8, 2, 128, 16)
    case.block_tables[1, 1] = case.block_tables[0, 1]   # both newest tokens: block b, slot 3
    d = case_on_device(case)
    rng = np.random.default_rng(2)
    nk = to_dev(synth.bf16_bits(rng.standard_normal((3, 2, 128)).astype(np.float32)))
    nv = to_dev(synth.bf16_bits(rng.standard_normal((3, 2, 128)).astype(np.float32)))
    k_before = to_host(d["k"])
    say("PA_DEBUG fused write slot clash")
    _rejected(lambda: _decode(case, d, new_key=nk, new_value=nv), "same slot")
    torch.cuda.synchronize()
    assert np.array_equal(to_host(d["k"]), k_before)


def test_cache_write_slots(debug):
    rng = np.random.default_rng(3)
    NB, H, BS, D, T = 10, 2, 16, 64, 6
    kc = to_dev(synth.bf16_bits(rng.standard_normal((NB, H, BS, D)).astype(np.float32)))
    vc = to_dev(synth.bf16_bits(rng.standard_normal((NB, H, BS, D)).astype(np.float32)))
    key = to_dev(synth.bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32)))
    before = to_host(kc)
    say("PA_DEBUG cache write slots")
    pa.reshape_and_cache(key, key, kc, vc, to_dev(np.array([0, 5, -1, 159, -1, 17], np.int64)))
    torch.cuda.synchronize()
    _rejected(lambda: pa.reshape_and_cache(key, key, kc, vc, to_dev(np.array([0, 5, -1, 5, 7, 8], np.int64))),
              "slot 5 appears twice")
    _rejected(lambda: pa.reshape_and_cache(key, key, kc, vc, to_dev(np.array([0, 1, 2, 3, 4, 160], np.int64))),
              "slot_mapping[5] = 160")
    after_valid = to_host(kc)
    assert not np.array_equal(after_valid, before)
    # quantising write: same rule
    q8 = torch.zeros((NB, H, BS, D), dtype=torch.int8, device="cuda")
    sc = torch.zeros((NB, H, BS), dtype=torch.float32, device="cuda")
    keyf = to_dev(rng.standard_normal((T, H, D)).astype(np.float32))
    _rejected(lambda: pa.quantize_and_cache(keyf, keyf, q8, q8.clone(), sc, sc.clone(),
                                            to_dev(np.array([3, 3, -1, 4, 5, 6], np.int64))), "slot 3 appears twice")
    torch.cuda.synchronize()
    assert int(q8.abs().sum()) == 0


def test_copy_pairs(debug):
    rng = np.random.default_rng(4)
    NB, H, BS, D = 12, 2, 16, 64
    kc = to_dev(synth.bf16_bits(rng.standard_normal((NB, H, BS, D)).astype(np.float32)))
    vc = to_dev(synth.bf16_bits(rng.standard_normal((NB, H, BS, D)).astype(np.float32)))
    before = to_host(kc)
    say("PA_DEBUG copy pairs")
    for pairs, needle in (([[1, 2], [3, 2]], "destination block 2 appears twice"),
                          ([[1, 2], [2, 5]], "both a source and a destination"),
                          ([[1, 2], [3, NB]], "outside [0, 12)")):
        _rejected(lambda: pa.copy_blocks(kc, vc, to_dev(np.array(pairs, np.int64))), needle)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(kc), before)
    pa.copy_blocks(kc, vc, to_dev(np.array([[1, 2], [1, 3]], np.int64)))   # one source twice is fine
    torch.cuda.synchronize()
    k = to_host(kc)
    assert np.array_equal(k[2], before[1]) and np.array_equal(k[3], before[1])


def test_swap_destinations(debug):
    rng = np.random.default_rng(5)
    NB, H, BS, D = 8, 2, 16, 64
    dk = to_dev(synth.bf16_bits(rng.standard_normal((NB, H, BS, D)).astype(np.float32)))
    dv = to_dev(synth.bf16_bits(rng.standard_normal((NB, H, BS, D)).astype(np.float32)))
    hk = torch.zeros((NB, H, BS, D), dtype=torch.bfloat16).pin_memory()
    hv = torch.zeros((NB, H, BS, D), dtype=torch.bfloat16).pin_memory()
    say("PA_DEBUG swap destinations")
    _rejected(lambda: pa.swap_blocks(dk, dv, hk, hv, to_dev(np.array([[0, 1], [2, 1]], np.int64))),
              "destination block 1 appears twice")
    torch.cuda.synchronize()
    assert int(hk.view(torch.int16).abs().sum()) == 0
    # ids outside a pool skip the pair (documented), not an error
    pa.swap_blocks(dk, dv, hk, hv, to_dev(np.array([[0, 1], [2, NB + 4]], np.int64)))
    torch.cuda.synchronize()
    assert torch.equal(hk[1].cpu(), dk[0].cpu())


def test_graph_capture_skips_the_checks(debug):
    case = _case()
    d = case_on_device(case)
    out = torch.empty(tuple(case.q.shape), dtype=torch.float32, device="cuda")
    ref = _decode(case, d)
    torch.cuda.synchronize()
    args = pa.make_decode_args(d["q"], d["k"], d["v"], d["bt"], d["cl"], float(case.scale), case.max_context_len,
                               out=out)
    need = pa.decode_workspace_size(args)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    say("PA_DEBUG graph capture")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            _decode(case, d, out=out, workspace=ws, stream=s)
    for _ in range(3):
        out.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
