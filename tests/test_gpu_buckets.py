"""zero_shard_step_buckets: the whole bucketed step enqueued by one call.

Equal bits to one launch over the same chunks; and with per-bucket ready
events the stream really waits: the partials start as NaN, a producer stream
writes each bucket's slice only after a delay and then records that
bucket's event, and the step still matches the oracle bit for bit (a bucket
stepped before its event would have read NaN).
"""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from gpu_helpers import assert_bitwise, host_master, host_partials, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


@pytest.fixture(scope="module")
def env():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    import sharded_optimizer_step_shard_amd as zs
    return bench, zs


def host(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def shard(bench, t):
    w = W.Workload("buckets", 91, [123_457, 300_001, 77], 4, "bf16", 1e-3)
    sh = bench.Shard(w, rank=1, dst_mode="slot", max_chunk=512)
    sh.fill_partials(t)
    return w, sh


def test_buckets_equal_one_launch(env):
    bench, zs = env
    t = 3
    say("case: bucketed step (one call) vs one launch")
    w, a = shard(bench, t)
    _, b = shard(bench, t)
    runs = bench.bucket_runs(a.table["len"], 5_000)
    assert len(runs) > 10
    hp = zs.hparams(t, **HP)
    zs.zero_shard_step(a.partials, a.master, a.m, a.v, a.n, a.d_table, len(a.table), hp)
    zs.zero_shard_step_buckets(b.partials, b.master, b.m, b.v, b.n, b.d_table, len(b.table), runs, hp)
    for x, y, what in ((a.master, b.master, "master"), (a.m, b.m, "m"), (a.v, b.v, "v"),
                       (a.params[0], b.params[0], "param")):
        assert_bitwise(host(y), host(x), f"buckets vs one launch {what}", strict_nan=True)
    # every other bucket only: the chunks of the skipped buckets keep their state
    _, c = shard(bench, t)
    m0 = host(c.master).copy()
    half = runs[::2]
    zs.zero_shard_step_buckets(c.partials, c.master, c.m, c.v, c.n, c.d_table, len(c.table), half, hp)
    got, ref = host(c.master), host(a.master)
    stepped = np.zeros(c.n, bool)
    for first, count in half:
        lo = int(c.table["shard_off"][first])
        hi = int(c.table["shard_off"][first + count - 1] + c.table["len"][first + count - 1])
        stepped[lo:hi] = True
    assert_bitwise(got[stepped], ref[stepped], "stepped buckets")
    assert_bitwise(got[~stepped], m0[~stepped], "skipped buckets untouched")


def test_buckets_wait_for_their_events(env):
    bench, zs = env
    t = 4
    say("case: bucketed step gated by per-bucket events from a producer stream")
    w, sh = shard(bench, t)
    runs = bench.bucket_runs(sh.table["len"], 20_000)
    assert len(runs) > 5
    for p in sh.partials:
        p.fill_(0x7FC0)                      # bf16 NaN until the producer writes
    consumer = torch.cuda.current_stream()
    producer = torch.cuda.Stream()
    producer.wait_stream(consumer)
    events = []
    with torch.cuda.stream(producer):
        for first, count in runs:
            torch.cuda._sleep(200_000)       # bounded spin: the bucket arrives late
            lo = int(sh.table["shard_off"][first])
            hi = int(sh.table["shard_off"][first + count - 1] + sh.table["len"][first + count - 1])
            for k, p in enumerate(sh.partials):
                synth.dev_fill(p[lo:hi], w.seed, sh.grad_stream(k, t), sh.lo + lo, w.sigma_grad,
                               sh.mask_stream(k, t), w.outlier_frac, w.outlier_mult)
            ev = torch.cuda.Event()
            ev.record(producer)
            events.append(ev)
    zs.zero_shard_step_buckets(sh.partials, sh.master, sh.m, sh.v, sh.n, sh.d_table, len(sh.table),
                               runs, zs.hparams(t, **HP), ready=events)
    torch.cuda.synchronize()
    idx = np.arange(sh.lo, sh.hi, dtype=np.int64)
    z = np.zeros(sh.n, np.float32)
    th, m, v, p = oracle.shard_step(host_partials(w, t, idx), host_master(w, idx), z, z,
                                    oracle.hparams(t, **HP))
    assert_bitwise(host(sh.master), th, "gated master", strict_nan=True)
    assert_bitwise(host(sh.m), m, "gated m", strict_nan=True)
    assert_bitwise(host(sh.v), v, "gated v", strict_nan=True)
    assert_bitwise(host(sh.params[0]), p, "gated param", strict_nan=True)
