"""The CPU oracle against its pins (closed forms, the architecture figure,
an independent unpaged implementation, invariances), and the pool policy
model against hand-derived scripts."""
import numpy as np
import pytest

import oracle
import pins
from oracle import ERR_INVALID, ERR_OOM, ERR_STATE, OK, PoolModel


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()


def test_oracle_rejects_out_of_range_table():
    q = np.zeros((1, 1, 64), np.float32)
    kc = np.zeros((2, 1, 16, 64), np.float32)
    with pytest.raises(ValueError):
        oracle.paged_decode(q, kc, kc, np.array([[5]], np.int32), np.array([3], np.int32), 1.0)
    with pytest.raises(ValueError):  # context past the table row
        oracle.paged_decode(q, kc, kc, np.array([[0]], np.int32), np.array([17], np.int32), 1.0)


# --------------------------------------------------------------------------
# pool policy model
# --------------------------------------------------------------------------

def test_pool_model_hand_script():
    """Stack policy, worked by hand: initial order [2, 0, 3, 1] hands out 2
    first; freed ids come back last-in first-out."""
    p = PoolModel(4, [2, 0, 3, 1])
    assert p.alloc(2) == (OK, [2, 0])
    assert p.alloc(1) == (OK, [3])
    assert p.num_free() == 1
    assert p.free([2]) == OK
    assert p.alloc(2) == (OK, [2, 1])
    assert p.alloc(1) == (ERR_OOM, [])
    assert p.share([0, 0]) == OK and p.refcount(0) == 3
    assert p.free([0, 3]) == OK and p.refcount(0) == 2 and p.num_free() == 1
    assert p.alloc(1) == (OK, [3])
    assert p.free([0, 0]) == OK and p.num_free() == 1
    assert p.alloc(1) == (OK, [0])


def test_pool_model_errors_leave_state_unchanged():
    p = PoolModel(5)
    assert p.alloc(3) == (OK, [0, 1, 2])
    assert p.alloc(3) == (ERR_OOM, []) and p.num_free() == 2
    assert p.free([0, 7]) == ERR_INVALID and p.refcount(0) == 1
    assert p.free([1, 1]) == ERR_STATE and p.refcount(1) == 1      # freed twice, held once
    assert p.free([4]) == ERR_STATE                                 # never allocated
    assert p.share([3]) == ERR_STATE and p.refcount(3) == 0
    assert p.share([-1]) == ERR_INVALID
    assert p.alloc(-1)[0] == ERR_INVALID
    assert p.refcount(99) == -1 and p.refcount(-1) == -1
    assert p.num_free() == 2


def test_pool_model_no_leak_after_cancel():
    """Every page goes back to the pool when requests finish or are
    cancelled mid-generation (glossary, section 4)."""
    rng = np.random.default_rng(0)
    p = PoolModel(64, rng.permutation(64))
    held = []
    for _ in range(200):
        if held and rng.random() < 0.4:
            seq = held.pop(int(rng.integers(len(held))))
            assert p.free(seq) == OK
        else:
            rc, ids = p.alloc(int(rng.integers(1, 6)))
            if rc == OK:
                held.append(ids)
        assert p.num_free() + sum(len(h) for h in held) == 64
    for seq in held:
        assert p.free(seq) == OK
    assert p.num_free() == 64


def test_pool_model_external_fragmentation(golden):
    """Ten separated holes: a contiguous allocator cannot place the 500-token
    request, the block pool can (deeplearn.tn, 'La fragmentation')."""
    g = golden("fragmentation.json")
    BS = g["block_size"]
    need = -(-g["request_tokens"] // BS)
    assert need == g["blocks_needed"]
    NB = 80
    p = PoolModel(NB)
    ok, ids = p.alloc(NB)
    assert ok == OK
    holes = [ids[i * 8:i * 8 + 4] for i in range(10)]       # ten holes of 4 blocks, 4 apart
    for h in holes:
        assert p.free(h) == OK
    free_ids = sorted(i for h in holes for i in h)
    runs, run = [], 1
    for a, b in zip(free_ids, free_ids[1:]):
        if b == a + 1:
            run += 1
        else:
            runs.append(run)
            run = 1
    runs.append(run)
    assert max(runs) * BS < g["request_tokens"]              # no contiguous room
    assert p.num_free() * BS >= g["request_tokens"]
    rc, got = p.alloc(need)
    assert rc == OK and len(set(got)) == need
