"""ft_read_checksum against numpy: the XOR of a buffer's 32-bit words, for sizes from one 16-byte
word to a grid of many workgroups with a ragged last piece, XORed into the sink's start value."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from expert_cached_ffn_amd import ops as _ops
    _ops.version()
    return _ops


@pytest.mark.parametrize("nbytes", [16, 1024, 16384, 16384 + 48, 16384 * 8 * 512 + 4096 + 16, 100 << 20])
def test_read_checksum_matches_numpy(ops, nbytes):
    rng = np.random.default_rng(nbytes % 1000)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.uint8).copy()).cuda()
    start = np.uint32(0x5A5A1234)
    sink = torch.tensor([int(start)], dtype=torch.int64).to(torch.int32).cuda()
    print(f"checksum {nbytes} bytes", flush=True)
    ops.ft_read_checksum(buf, nbytes, sink)
    torch.cuda.synchronize()
    got = np.uint32(sink.cpu().numpy().view(np.uint32)[0])
    want = np.bitwise_xor.reduce(host) ^ start
    assert got == want, f"{nbytes}: {got:#010x} != {want:#010x}"
