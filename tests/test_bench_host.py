"""Host side of the benchmark: the byte accounting its roofline is priced on
and the one-GPU guard.  No GPU is used.

* The KV bytes of the 70B-shaped step equal the KV-size formula of the
  ia-vox article ("Pourquoi le KV cache domine") applied to its own example
  (tests/golden/kv_size_formula.json).
* One layer's algorithmic bytes are that KV share plus, term by term, the
  table entries in use, the context lengths, q and the fp32 output; the
  quantised variants add the per-(block, head) or per-token scales.
* Contiguous reservation wastes what the pages' fragmentation examples
  give (tests/golden/waste_examples.json); paged storage wastes only the
  tail of the last block.
* `bench.py --gpus 2` stops with a message before touching a GPU.
* The warm-up before a timed region runs at least the asked steps and at
  least the asked wall time, synchronising as it goes and once at the end
  (synchronisation stubbed out: no GPU)."""
import os
import subprocess
import sys

import time

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kv_bytes_match_the_page_formula(golden):
    g = golden("kv_size_formula.json")
    lens = [g["context"]] * g["batch"]
    assert bench.kv_bytes(lens, g["kv_heads"], g["head_dim"], g["bytes_per_value"], g["layers"]) == g["kv_bytes"]


def test_algorithmic_bytes_of_the_70b_shaped_layer():
    S, Hq, Hkv, D, BS, n = 20, 64, 8, 128, 16, 8000
    lens = [n] * S
    kv = 2 * Hkv * D * n * S * 2                       # K and V, bf16
    tables = S * (n // BS) * 4                         # 500 int32 entries per sequence
    ctx = S * 4
    q_out = S * Hq * D * (2 + 4)                       # bf16 q, fp32 out
    assert kv == 655_360_000
    assert bench.decode_algorithmic_bytes(lens, Hq, Hkv, D, BS, 2, 2) == kv + tables + ctx + q_out == 656_383_120


def test_algorithmic_bytes_count_tokens_not_padded_blocks_and_scales():
    lens = [1, 16, 17, 0]
    Hq, Hkv, D, BS = 8, 2, 64, 16
    blocks = 1 + 1 + 2 + 0
    base = 2 * Hkv * D * 34 * 1 + blocks * 4 + 4 * 4 + 4 * Hq * D * (2 + 4)
    assert bench.decode_algorithmic_bytes(lens, Hq, Hkv, D, BS, 1, 2) == base
    assert bench.decode_algorithmic_bytes(lens, Hq, Hkv, D, BS, 1, 2, int8_scales=True) == base + blocks * Hkv * 8
    assert bench.decode_algorithmic_bytes(lens, Hq, Hkv, D, BS, 1, 2, token_scales=True) == base + 34 * Hkv * 8
    # several query rows per sequence: q and out per row
    assert (bench.decode_algorithmic_bytes(lens, Hq, Hkv, D, BS, 1, 2, query_rows=10)
            == base + 6 * Hq * D * (2 + 4))


def test_waste_of_contiguous_and_paged_storage(golden):
    g = golden("waste_examples.json")
    pg = g["paged_case"]
    for c in g["contiguous_cases"]:
        w = bench.waste_report([c["used"]], pg["block_size"], c["reserved"])
        assert abs(w["contiguous_waste"] - c["waste_fraction"]) < 1e-12
        assert abs(w["paged_waste"] - pg["waste_fraction"]) < 1e-12


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_warm_up_runs_the_asked_steps_and_the_time_floor(monkeypatch):
    import torch

    log = []
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: log.append("sync"))

    def step():
        log.append("step")

    # no time floor: exactly the asked steps, then a synchronisation
    assert bench.warm_up(step, 6, 0.0) == 6
    assert log.count("step") == 6 and log[-1] == "sync"
    assert log.index("sync") == 4                      # one synchronisation every four steps
    log.clear()
    assert bench.warm_up(step, 0, 0.0) == 0 and log == ["sync"]

    # a time floor: steps continue until it has passed, the last one synchronised
    log.clear()
    slow = lambda: (log.append("step"), time.sleep(0.002))  # noqa: E731
    t0 = time.perf_counter()
    n = bench.warm_up(slow, 2, 30.0)
    assert (time.perf_counter() - t0) * 1e3 >= 30.0
    assert n == log.count("step") and n > 2
    assert log[-1] == "sync"
