"""GPU streaming-read probe (the bench's practical HBM read ceiling): its XOR of
the buffer's 32-bit words equals numpy's, bit for bit, so every byte was read
exactly once (needs an MI355X)."""
import sys

import numpy as np
import pytest

from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (33 << 20) + 48, 1 << 28])
def test_hbm_read_probe_reads_every_word_once(nbytes):
    from quantized_expert_ffn_moe_amd import binding as B
    print(f"[probe] bytes={nbytes}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.moe_hbm_read_probe(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host)
    assert np.uint32(sink.cpu().numpy().view(np.uint32)[0]) == want
    # a second read XORs the same value in again: the sink returns to zero
    B.moe_hbm_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().item()) == 0
