"""The measurement aid w4a4_read_probe (a plain streaming read used for the
HBM read ceiling): it must read every byte it is given once, which its
checksum (the XOR of all 32-bit words) shows against numpy's, for sizes
that leave ragged tails in the four-load main loop and in the grid."""
import numpy as np
import pytest

from gpu_common import log, torch_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words", [4, 1028, 262148, 2621444, 30750000])
def test_read_probe_checksum(words):
    import w4a4_post_quantized_amd as L
    torch, dev = torch_dev()
    log(f"read_probe {4 * words} bytes")
    rng = np.random.default_rng(words)
    h = rng.integers(0, 2**32, size=words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(h.view(np.int32)).to(dev)
    out = torch.zeros(1, dtype=torch.int32, device=dev)
    L.read_probe(buf, out)
    got = np.uint32(out.cpu().numpy().view(np.uint32)[0])
    want = np.bitwise_xor.reduce(h)
    assert got == want
    # a second call XORs the same checksum in again
    L.read_probe(buf, out)
    assert out.cpu().numpy()[0] == 0
