"""The measurement aids behind bench.py's probe legs do what their rates
assume: the copy moves every byte, the write stores every byte, the read
touches the data and stores nothing unless its fold matches."""
import numpy as np
import pytest

from gpu_helpers import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sharded_optimizer_step_shard_amd as m
    return m


@pytest.mark.parametrize("nbytes", [16, 4096 + 13, (1 << 20) + 7, (5 << 20) + 16])
def test_probe_copy_and_write_move_every_byte(zs, nbytes):
    say(f"case: probes over {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    src_h = rng.integers(0, 256, nbytes + 64, dtype=np.uint8)
    src = torch.from_numpy(src_h).cuda()
    dst = torch.full((nbytes + 64,), 0xAB, dtype=torch.uint8, device="cuda")
    zs.zero_probe_copy(src, dst, nbytes)
    d = dst.cpu().numpy()
    assert np.array_equal(d[:nbytes], src_h[:nbytes]) and np.all(d[nbytes:] == 0xAB)
    dst.fill_(0xAB)
    zs.zero_probe_write(dst, nbytes, 0x11223344)
    d = dst.cpu().numpy()
    full = nbytes // 16 * 16
    assert np.all(d[:full].view(np.uint32) == 0x11223344)
    assert np.all(d[full:nbytes] == 0x44) and np.all(d[nbytes:] == 0xAB)


def test_probe_read_stores_only_on_a_match(zs):
    say("case: read probe over 4 MiB of zeros")
    n = 4 << 20
    buf = torch.zeros(n, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    zs.zero_probe_read(buf, n, sink, magic=1)           # every fold is 0: no store
    torch.cuda.synchronize()
    assert sink.item() == -1
    zs.zero_probe_read(buf, n, sink, magic=0)           # every fold matches: stores 0
    torch.cuda.synchronize()
    assert sink.item() == 0
