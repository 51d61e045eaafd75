"""The fused step captured in a HIP graph (through torch.cuda.graph) and
replayed gives the same bits as the same calls made eagerly.

The kernels use no memset and no library collective, so a capture records
only kernel nodes.  Hyper-parameters are kernel arguments, fixed at capture:
each replay applies step t again, so every replay is compared with an eager
call at that same t from the same starting state.  Between replays the test
does eager work of its own (resetting the state with copies) and
synchronises, and it checks every replay, not just the first.
"""
import numpy as np
import pytest

import oracle
from synth import workloads as W
from gpu_helpers import assert_bitwise, host_master, host_partials, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


@pytest.fixture(scope="module")
def zs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sharded_optimizer_step_shard_amd as m
    return m


def dev(x):
    a = np.ascontiguousarray(x)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


@pytest.mark.parametrize("bucketed", [False, True])
def test_graph_replays_equal_eager_calls(zs, bucketed):
    say(f"case: graph capture of the fused step, bucketed={bucketed}")
    n_ranks, total, rank, t = 8, 300_001, 3, 7
    w = W.Workload("graph", 99, [total], n_ranks, "bf16", 1e-3)
    lo, hi = w.shard_range(rank)
    n = hi - lo
    idx = np.arange(lo, hi, dtype=np.int64)
    parts = [dev(p) for p in host_partials(w, t, idx)]
    rng = np.random.default_rng(1)
    th0 = host_master(w, idx)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-8).astype(np.float32)
    init = [dev(th0), dev(m0), dev(v0)]

    def make():
        slot = torch.zeros(n, dtype=torch.int16, device="cuda")
        table, _ = zs.zero_build_chunks([total], n_ranks, rank, slot_dst=slot, max_chunk=512)
        bufs = [x.clone() for x in init]
        return slot, table, zs.chunks_to_device(table), bufs

    def launch(slot, table, d_table, bufs):
        hp = zs.hparams(t, **HP)
        if not bucketed:
            zs.zero_shard_step(parts, *bufs, n, d_table, len(table), hp)
            return
        base = d_table.data_ptr()
        step = 97                                 # chunks per bucket; the last bucket is short
        for first in range(0, len(table), step):
            count = min(step, len(table) - first)
            zs.zero_shard_step(parts, *bufs, n, base + 32 * first, count, hp)

    # eager reference from the initial state
    e_slot, e_table, e_dtab, e_bufs = make()
    launch(e_slot, e_table, e_dtab, e_bufs)
    torch.cuda.synchronize()
    want = [host(b) for b in e_bufs] + [host(e_slot)]
    # and the oracle agrees with it
    th, mm, vv, p = oracle.shard_step(host_partials(w, t, idx), th0, m0, v0, oracle.hparams(t, **HP))
    for got, ref, what in zip(want, (th, mm, vv, p), ("master", "m", "v", "param")):
        assert_bitwise(got, ref, f"eager vs oracle {what}")

    g_slot, g_table, g_dtab, g_bufs = make()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            launch(g_slot, g_table, g_dtab, g_bufs)
    torch.cuda.current_stream().wait_stream(side)
    for replay in range(4):
        for b, x in zip(g_bufs, init):          # eager work between replays
            b.copy_(x)
        g_slot.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [host(b) for b in g_bufs] + [host(g_slot)]
        for k, (a, b) in enumerate(zip(got, want)):
            assert_bitwise(a, b, f"replay {replay} array {k}", strict_nan=True)
