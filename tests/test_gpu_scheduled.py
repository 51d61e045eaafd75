"""The fused steps with their constants in device memory
(zero_shard_step_scheduled and its 12-byte and pure-bf16 forms,
zero_step_index_advance).

- Eager calls: entry i of the table gives the bits of zero_shard_step with
  the hparams entry i was made from; the call leaves the index as it is; an
  index outside the table changes nothing.
- Graph capture, for each state layout: one step (the scheduled launch and
  the index advance) is captured once and replayed six times with a
  learning-rate schedule in the table.  The state carries over from replay to replay, as in training; the
  partials are refilled eagerly between replays.  After every replay the
  state equals the oracle's run of that many steps with the scheduled
  hparams, and the index has moved on by one.  Replays past the end of the
  table change nothing.
"""
import numpy as np
import pytest

import oracle
from synth import workloads as W
from gpu_helpers import assert_bitwise, host_master, host_partials, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


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


def schedule(n):
    """Warm-up then decay of the learning rate, weight decay switched off on
    one step: one hparams per step t = 1..n."""
    out = []
    for t in range(1, n + 1):
        lr = 1e-3 * min(1.0, t / 3) * (0.9 ** max(0, t - 3))
        out.append(dict(lr=lr, beta1=0.9, beta2=0.999, eps=1e-8,
                        weight_decay=0.0 if t == 4 else 0.1))
    return out


def setup(zs, n_ranks=8, total=1_000_003, gdt="bf16"):
    w = W.Workload("scheduled", 101, [total], n_ranks, gdt, 1e-3)
    rank = min(5, n_ranks - 1)
    lo, hi = w.shard_range(rank)
    n = hi - lo
    idx = np.arange(lo, hi, dtype=np.int64)
    slot = torch.zeros(n, dtype=torch.int16, device="cuda")
    table, _ = zs.zero_build_chunks([total], n_ranks, rank, slot_dst=slot, max_chunk=1024)
    return w, rank, n, idx, slot, zs.chunks_to_device(table), len(table)


@pytest.mark.parametrize("gdt,n_ranks", [("bf16", 8), ("f32", 3)])
def test_eager_entries_equal_host_hparams(zs, gdt, n_ranks):
    say(f"case: scheduled step, eager, {gdt} N={n_ranks}")
    w, rank, n, idx, slot, d_table, nc = setup(zs, n_ranks=n_ranks, gdt=gdt)
    hps = [zs.hparams(t, **h) for t, h in enumerate(schedule(5), start=1)]
    consts = torch.from_numpy(zs.zero_make_step_consts(hps).view(np.uint8)).cuda()
    index = torch.zeros(1, dtype=torch.int64, device="cuda")
    parts = [dev(p) for p in host_partials(w, 2, idx)]
    th0 = dev(host_master(w, idx))
    rng = np.random.default_rng(3)
    m0 = dev((rng.standard_normal(n) * 1e-4).astype(np.float32))
    v0 = dev((rng.random(n) * 1e-8).astype(np.float32))
    slot_b = torch.zeros_like(slot)
    table_b, _ = zs.zero_build_chunks(w.numels, n_ranks, rank, slot_dst=slot_b, max_chunk=1024)
    d_table_b = zs.chunks_to_device(table_b)
    for e in (0, 3, 4):
        a = [x.clone() for x in (th0, m0, v0)]
        b = [x.clone() for x in (th0, m0, v0)]
        zs.zero_shard_step(parts, *a, n, d_table, nc, hps[e])
        index.fill_(e)
        zs.zero_shard_step_scheduled(parts, *b, n, d_table_b, len(table_b), consts, len(hps), index)
        torch.cuda.synchronize()
        for x, y, what in zip(a + [slot], b + [slot_b], ("master", "m", "v", "param")):
            assert_bitwise(host(y), host(x), f"entry {e} {what}", strict_nan=True)
        assert int(index.item()) == e, "the step call must not move the index"
    # an index outside the table: nothing changes
    for bad in (-1, len(hps), 1 << 40):
        b = [x.clone() for x in (th0, m0, v0)]
        index.fill_(bad)
        zs.zero_shard_step_scheduled(parts, *b, n, d_table, nc, consts, len(hps), index)
        torch.cuda.synchronize()
        for x, y in zip(b, (th0, m0, v0)):
            assert torch.equal(x, y)
        assert int(index.item()) == bad


def test_index_advance_stops_at_the_end(zs):
    say("case: index advance")
    index = torch.zeros(1, dtype=torch.int64, device="cuda")
    for _ in range(7):
        zs.zero_step_index_advance(index, 5)
    torch.cuda.synchronize()
    assert int(index.item()) == 5
    index.fill_(-3)
    zs.zero_step_index_advance(index, 5)
    torch.cuda.synchronize()
    assert int(index.item()) == -3


@pytest.mark.parametrize("layout", ["fp32", "bf16-moments", "bf16-kahan"])
def test_graph_replays_follow_the_schedule(zs, layout):
    say(f"case: scheduled {layout} step captured in a graph, six replays with a learning-rate schedule")
    n_steps = 6
    w, rank, n, idx, slot, d_table, nc = setup(zs)
    sch = schedule(n_steps)
    hps = [zs.hparams(t, **h) for t, h in enumerate(sch, start=1)]
    consts = torch.from_numpy(zs.zero_make_step_consts(hps).view(np.uint8)).cuda()
    index = torch.zeros(1, dtype=torch.int64, device="cuda")
    parts_h = {t: host_partials(w, t, idx) for t in range(1, n_steps + 1)}
    parts = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(w.n_ranks)]
    th0 = host_master(w, idx)
    z16 = np.zeros(n, np.uint16)
    if layout == "fp32":
        state_h = (th0, np.zeros(n, np.float32), np.zeros(n, np.float32))
        fn, oracle_step = zs.zero_shard_step_scheduled, oracle.shard_step
    elif layout == "bf16-moments":
        state_h = (th0, z16, z16)
        fn, oracle_step = zs.zero_shard_step_bf16_moments_scheduled, oracle.shard_step_bf16m
    else:
        state_h = (oracle.bf16_round(th0), z16, z16, z16)
        slot.copy_(dev(state_h[0]))
        fn, oracle_step = zs.zero_shard_step_kahan_scheduled, oracle.shard_step_kahan
    bufs = [dev(x) for x in (state_h if layout != "bf16-kahan" else state_h[1:])]

    def one_step():
        fn(parts, *bufs, n, d_table, nc, consts, len(hps), index)
        zs.zero_step_index_advance(index, len(hps))

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            one_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capture only records: nothing ran
    assert int(index.item()) == 0
    assert_bitwise(host(bufs[0]), state_h[0] if layout != "bf16-kahan" else state_h[1],
                   "state untouched by the capture")

    st = state_h
    for t in range(1, n_steps + 1):
        for d, h in zip(parts, parts_h[t]):        # eager work between replays
            d.copy_(dev(h))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out = oracle_step(parts_h[t], *st, oracle.hparams(t, **sch[t - 1]))
        if layout == "bf16-kahan":
            st = out
            want = list(out[1:]) + [out[0]]        # comp, m, v, then the parameters
        else:
            st = out[:3]
            want = list(out)                        # master, m, v, parameters
        for k, (got, w_) in enumerate(zip(bufs + [slot], want)):
            assert_bitwise(host(got), w_, f"{layout} replay {t} array {k}")
        assert int(index.item()) == t
    # past the end of the table: replays change nothing
    before = [x.clone() for x in bufs + [slot]]
    graph.replay()
    graph.replay()
    torch.cuda.synchronize()
    for x, y in zip(bufs + [slot], before):
        assert torch.equal(x, y)
    assert int(index.item()) == n_steps
