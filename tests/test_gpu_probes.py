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


@pytest.mark.parametrize("k,n", [(1, 1), (2, 3), (3, 255), (5, 256), (8, 257), (16, 1000003),
                                 (16, (1 << 24) + 5)])
def test_probe_sum_adds_in_order(zs, k, n):
    """dst = src[0] + ... + src[k-1] in fp32, added in that order, bitwise
    against numpy's float32 additions; the floats past dst are untouched and
    a source named twice is read twice."""
    say(f"case: sum probe, k = {k}, n = {n}")
    rng = np.random.default_rng(k * 1000 + n)
    hs = [(rng.standard_normal(n) * 10.0 ** rng.integers(-3, 4, n)).astype(np.float32) for _ in range(k)]
    srcs = [torch.from_numpy(h).cuda() for h in hs]
    if k >= 3:
        srcs[2], hs[2] = srcs[0], hs[0]
    dst = torch.full((n + 8,), 7.5, device="cuda")
    zs.zero_probe_sum(srcs, dst, n)
    want = hs[0].copy()
    for h in hs[1:]:
        want = (want + h).astype(np.float32)
    got = dst.cpu().numpy()
    assert np.array_equal(got[:n].view(np.uint32), want.view(np.uint32))
    assert np.all(got[n:] == 7.5)
