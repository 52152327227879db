"""The streaming-read probe behind the measured HBM ceiling reads every byte:
its per-range XORs equal the host's, including a short last range."""
import numpy as np
import pytest
import torch

import bit_quantized_grouped_amd as bq
from gpu_cases import DEV, announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("nbytes", [16, 32768, (1 << 20) + 48, 3 * 32768 - 16])
def test_read_probe_reads_every_word(nbytes):
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 1 << 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(DEV)
    n_sink = bq.read_probe_sink_words(nbytes)
    sink = torch.full((n_sink + 3,), -1, dtype=torch.int32, device=DEV)
    announce(f"read probe {nbytes} bytes")
    bq.moe_read_probe(buf, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = [np.bitwise_xor.reduce(words[i:i + 8192]) for i in range(0, words.size, 8192)]
    assert np.array_equal(got[:n_sink], np.array(want, dtype=np.uint32))
    assert np.all(got[n_sink:] == 0xFFFFFFFF)     # nothing past the documented sink length
