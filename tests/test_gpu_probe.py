"""The read probe (a measuring stick for the benchmark, not a step of the method): the XOR of
the words it reports as written is the XOR of the 32-bit words of exactly the bytes it was
asked to read (so every byte is read once and no byte outside the range counts), in both
launch shapes, and it writes nothing past those words."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_tiered_amd as spax
    return torch, spax, torch.device("cuda:0")


@pytest.mark.parametrize("nbytes,offset", [(16, 0), (4096, 16), (16 * 1001, 48),
                                           (64 << 20, 0), ((64 << 20) - 32, 16),
                                           ((1 << 30) + 48, 16)])
def test_read_probe_xor(env, nbytes, offset):
    """Both launch shapes (grid-stride below 1 GiB, chunked from 1 GiB), ragged ends."""
    torch, spax, dev = env
    rng = np.random.default_rng(nbytes + offset)
    host = rng.integers(0, 256, size=nbytes + offset + 64, dtype=np.uint8)  # bytes around the range
    buf = torch.from_numpy(host).to(dev)
    out = torch.full((8192,), -1, dtype=torch.int32, device=dev)
    print(f"read_probe nbytes={nbytes} offset={offset}", flush=True)
    n = spax.spax_read_probe(buf, out, nbytes=nbytes, offset=offset)
    torch.cuda.synchronize()
    assert 8 <= n <= 8192 and n % 8 == 0
    words = out.cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(host[offset:offset + nbytes].view(np.uint32))
    assert int(np.bitwise_xor.reduce(words[:n])) == int(want)
    assert (words[n:] == 0xFFFFFFFF).all()  # nothing written past the reported words


def test_read_probe_fewer_words_fewer_workgroups(env):
    torch, spax, dev = env
    rng = np.random.default_rng(5)
    host = rng.integers(0, 256, size=1 << 22, dtype=np.uint8)
    buf = torch.from_numpy(host).to(dev)
    out = torch.full((24,), -1, dtype=torch.int32, device=dev)
    n = spax.spax_read_probe(buf, out)
    torch.cuda.synchronize()
    assert n == 24
    assert int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))) == \
        int(np.bitwise_xor.reduce(host.view(np.uint32)))


def test_read_probe_rejects_a_range_outside_the_buffer(env):
    torch, spax, dev = env
    buf = torch.zeros(64, dtype=torch.uint8, device=dev)
    out = torch.zeros(8, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        spax.spax_read_probe(buf, out, nbytes=64, offset=16)
