"""The read-bandwidth probe (pa_read_probe, a diagnostic beside the
attention path) reads exactly the chunks it is given: every lane's fold of
its 16-byte words over the chunks its wave visits equals the same fold done
on the host, for 1, 2 and 4 KiB chunks, in address order and in a given
order.  Bit-exact (integer XOR)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_192_amd as pa
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _expected(data: np.ndarray, ids: np.ndarray, chunk: int, waves: int) -> np.ndarray:
    """Host fold: wave w, lane l XORs the 16-byte words at byte l*16 + 1024*k
    of chunks ids[c] and ids[c + W] for c = w, w + 2W, ...  (n a multiple
    of 2W), then the four 32-bit words together."""
    words = data.view(np.uint32).reshape(-1, chunk // 4)           # [chunks][words]
    n = ids.shape[0]
    out = np.zeros((waves, 64), np.uint32)
    for w in range(waves):
        acc = np.zeros((64, 4), np.uint32)
        for c in range(w, n, 2 * waves):
            for cid in (ids[c], ids[c + waves]):
                row = words[cid].reshape(chunk // 1024, 64, 4)      # [k][lane][word]
                acc ^= np.bitwise_xor.reduce(row, axis=0)
        out[w] = acc[:, 0] ^ acc[:, 1] ^ acc[:, 2] ^ acc[:, 3]
    return out.reshape(-1)


@pytest.mark.parametrize("chunk", [1024, 2048, 4096])
def test_read_probe_reads_the_given_chunks(chunk):
    rng = np.random.default_rng(chunk)
    n, waves = 96, 12
    data = rng.integers(0, 2**32, size=n * chunk // 4, dtype=np.uint32).view(np.uint8)
    base = torch.from_numpy(data.copy()).to("cuda:0")
    sink = torch.empty(waves * 64, dtype=torch.int32, device="cuda:0")
    for order in ("address", "permuted"):
        ids = np.arange(n, dtype=np.int32) if order == "address" else rng.permutation(n).astype(np.int32)
        say("read probe, chunk", chunk, order)
        dev_ids = None if order == "address" else torch.from_numpy(ids).to("cuda:0")
        pa.prepare_read_probe(base, n, sink, chunk_ids=dev_ids, num_waves=waves, chunk_bytes=chunk)()
        torch.cuda.synchronize()
        got = sink.cpu().numpy().view(np.uint32)
        assert np.array_equal(got, _expected(data, ids, chunk, waves)), (chunk, order)
