"""GPU parity at the workloads' real sizes, in the configuration bench.py
times (its Shard setup: device-filled inputs, chunk table, launch).

GPT-2, the ragged fp32 case and the 7B shard (every state layout) are
compared in full, the 7B shard one slice of 2^26 elements at a time so that
host memory stays small.  The 70B shard (4.4e9 elements, 203 GB of device
inputs) is compared on sampled indices that the oracle replays one by one:
every chunk boundary +-8, the first and last 4096 elements, 2^20 hashed
indices and the indices around 2^32.
"""
import gc

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from gpu_helpers import assert_bitwise, check_state, host_master, host_partials, oracle_warm_prefix, sample_indices, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bench():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench as b
    return b


def host(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def release():
    gc.collect()
    torch.cuda.empty_cache()


def gather_state(sh, idx):
    i = torch.from_numpy(idx).to(sh.dev)
    return (sh.master[i].cpu().numpy(), sh.m[i].cpu().numpy(), sh.v[i].cpu().numpy(),
            sh.param_at(idx))


def test_gpt2_full_twenty_steps(bench):
    w = W.gpt2()
    say(f"case: {w.name} rank 3, {w.steps} steps, full compare")
    sh = bench.Shard(w, rank=3)
    idx = np.arange(sh.lo, sh.hi, dtype=np.int64)
    th = host_master(w, idx)
    m = np.zeros(sh.n, np.float32)
    v = np.zeros(sh.n, np.float32)
    for t in range(1, w.steps + 1):
        sh.fill_partials(t)
        sh.step(t)
        parts = host_partials(w, t, idx)
        th, m, v, p = oracle.shard_step(parts, th, m, v, oracle.hparams(t, **w.hparams()))
        if t in (1, 2, 10, w.steps):
            say(f"  step {t}: compare")
            flat = np.concatenate([host(x) for x in sh.params])
            check_state((host(sh.master), host(sh.m), host(sh.v), flat[sh.lo:sh.hi]),
                        (th, m, v, p), f"gpt2 step {t}")
    del sh
    release()


def test_ragged_fp32_full(bench):
    w = W.ragged()
    say(f"case: {w.name} rank 0, 2 steps, full compare ({len(w.zero_tensors)} zero tensors)")
    sh = bench.Shard(w, rank=0)
    idx = np.arange(sh.lo, sh.hi, dtype=np.int64)
    th = host_master(w, idx)
    m = np.zeros(sh.n, np.float32)
    v = np.zeros(sh.n, np.float32)
    for t in (1, 2):
        sh.fill_partials(t)
        sh.step(t)
        parts = host_partials(w, t, idx)
        oracle.shard_step(parts, th, m, v, oracle.hparams(t, **w.hparams()), in_place=True)
        del parts
    p = oracle.bf16_round(th)
    flat = np.concatenate([host(x) for x in sh.params])
    check_state((host(sh.master), host(sh.m), host(sh.v), flat[sh.lo:sh.hi]), (th, m, v, p),
                "ragged step 2")
    del sh
    release()


SLICE = 1 << 26


def shard_slices(n, size=SLICE):
    for a in range(0, n, size):
        yield a, min(n, a + size)


def params_range(sh, a, b):
    """bf16 bits the step wrote for shard elements [a, b)."""
    if sh.dst_mode == "slot":
        return host(sh.params[0][a:b])
    starts = np.cumsum([0] + list(sh.w.numels))
    g0, g1 = sh.lo + a, sh.lo + b
    out = []
    for t, p in enumerate(sh.params):
        s, e = int(starts[t]), int(starts[t + 1])
        lo, hi = max(s, g0), min(e, g1)
        if lo < hi:
            out.append(host(p[lo - s:hi - s]))
    return np.concatenate(out)


def warm_state(w, sh, prefix, a, b):
    """The 7B shard's state after the warm start, for shard elements [a, b):
    the prefix elements keep the oracle's own prefix run, later elements
    take m, v from prefix element src(i) and their master from the
    generator."""
    pth, pm, pv = prefix
    P = w.warm_prefix
    idx = np.arange(a, b, dtype=np.int64)
    src = synth.prefix_src(w.seed, synth.stream_id(synth.KIND_PREFIX_MAP), idx, P)
    if b <= P:
        th = pth[a:b].copy()
    else:
        th = host_master(w, sh.lo + idx)
        if a < P:
            th[:P - a] = pth[a:]
    return idx, th, pm[src], pv[src]


@pytest.mark.timeout(900)
def test_llama7b_warm_start_then_full_compare(bench):
    w = W.llama7b()
    say(f"case: {w.name} rank 0: warm start ({w.warm_steps} steps on {w.warm_prefix}), "
        "then 3 bench steps, full compare")
    sh = bench.Shard(w, rank=0)
    t0 = sh.prepare()
    assert t0 == w.warm_steps + 1
    P = w.warm_prefix
    prefix = oracle_warm_prefix(w, sh.lo)
    say("  warm-start prefix: full compare against the oracle's own prefix run")
    check_state((host(sh.master[:P]), host(sh.m[:P]), host(sh.v[:P])), prefix, "7b warm prefix")
    steps = [t0, t0 + 1, t0 + 2]
    for t in steps:
        sh.step(t)
    torch.cuda.synchronize()
    for a, b in shard_slices(sh.n):
        idx, th, m, v = warm_state(w, sh, prefix, a, b)
        parts = host_partials(w, t0, sh.lo + idx)     # the bench reuses step t0's partials
        for t in steps:
            th, m, v, p = oracle.shard_step(parts, th, m, v, oracle.hparams(t, **w.hparams()))
        check_state((host(sh.master[a:b]), host(sh.m[a:b]), host(sh.v[a:b]), params_range(sh, a, b)),
                    (th, m, v, p), f"7b [{a}, {b})")
        say(f"  [{a}, {b}) equal")
    del sh
    release()


def test_llama70b_sampled_two_steps(bench):
    w = W.llama70b()
    say(f"case: {w.name} rank 5 slot, 2 steps, sampled compare (shard {w.shard_len})")
    sh = bench.Shard(w, rank=5)
    assert sh.n > (1 << 32)
    t0 = sh.prepare()
    sh.step(t0)
    sh.step(t0 + 1)
    idx = sample_indices(sh.table, sh.n, seed=70, n_random=1 << 20)
    idx = np.unique(np.concatenate([idx, np.array([(1 << 32) - 1, 1 << 32, (1 << 32) + 7])]))
    say(f"  {idx.size} sampled indices")
    th = host_master(w, sh.lo + idx)
    m = np.zeros(idx.size, np.float32)
    v = np.zeros(idx.size, np.float32)
    parts = host_partials(w, t0, sh.lo + idx)
    for t in (t0, t0 + 1):
        th, m, v, p = oracle.shard_step(parts, th, m, v, oracle.hparams(t, **w.hparams()))
    check_state(gather_state(sh, idx), (th, m, v, p), "70b sampled")
    del sh
    release()


def gather_kahan(sh, idx):
    i = torch.from_numpy(idx).to(sh.dev)
    return (sh.param_at(idx), sh.comp[i].cpu().numpy().view(np.uint16),
            sh.m[i].cpu().numpy().view(np.uint16), sh.v[i].cpu().numpy().view(np.uint16))


def assert_kahan_state(got, want, what):
    for name, g, w_ in zip(("parameters", "compensation", "m", "v"), got, want):
        assert_bitwise(g, w_, f"{what} {name}")


def test_gpt2_kahan_full_five_steps(bench):
    """The pure-bf16 state in the bench's set-up (parameters written from the
    initial fp32 master, zero compensation and moments), five steps, full
    compare."""
    w = W.gpt2()
    say(f"case: {w.name} rank 2, pure-bf16 Kahan state, 5 steps, full compare")
    sh = bench.Shard(w, rank=2)
    sh.use_kahan()
    idx = np.arange(sh.lo, sh.hi, dtype=np.int64)
    th = oracle.bf16_round(host_master(w, idx))
    c = np.zeros(sh.n, np.uint16)
    m = np.zeros(sh.n, np.uint16)
    v = np.zeros(sh.n, np.uint16)
    for t in range(1, 6):
        sh.fill_partials(t)
        sh.step_kahan(t)
        th, c, m, v = oracle.shard_step_kahan(host_partials(w, t, idx), th, c, m, v,
                                              oracle.hparams(t, **w.hparams()))
    flat = np.concatenate([host(x) for x in sh.params])
    assert_kahan_state((flat[sh.lo:sh.hi], host(sh.comp), host(sh.m), host(sh.v)), (th, c, m, v),
                       "gpt2 Kahan step 5")
    del sh
    release()


@pytest.mark.timeout(900)
def test_llama7b_kahan_full(bench):
    """bench.py --state bf16-kahan on the 7B shard: warm start, switch to the
    pure-bf16 state, three steps; full compare."""
    w = W.llama7b()
    say(f"case: {w.name} rank 0, warm start then pure-bf16 Kahan state, 3 steps, full compare")
    sh = bench.Shard(w, rank=0)
    t0 = sh.prepare()
    sh.use_kahan()
    steps = [t0, t0 + 1, t0 + 2]
    for t in steps:
        sh.step_kahan(t)
    torch.cuda.synchronize()
    prefix = oracle_warm_prefix(w, sh.lo)
    for a, b in shard_slices(sh.n):
        idx, th32, m32, v32 = warm_state(w, sh, prefix, a, b)
        th, m, v = oracle.bf16_round(th32), oracle.bf16_round(m32), oracle.bf16_round(v32)
        c = np.zeros(idx.size, np.uint16)
        parts = host_partials(w, t0, sh.lo + idx)     # the bench reuses step t0's partials
        for t in steps:
            th, c, m, v = oracle.shard_step_kahan(parts, th, c, m, v, oracle.hparams(t, **w.hparams()))
        assert_kahan_state((params_range(sh, a, b), host(sh.comp[a:b]), host(sh.m[a:b]),
                            host(sh.v[a:b])), (th, c, m, v), f"7b Kahan [{a}, {b})")
        say(f"  [{a}, {b}) equal")
    del sh
    release()


@pytest.mark.timeout(900)
def test_llama7b_bf16_moments_full(bench):
    """bench.py --state bf16-moments on the 7B shard: warm start, moments
    rounded to bf16, three steps; full compare."""
    w = W.llama7b()
    say(f"case: {w.name} rank 0, warm start then 12-byte state, 3 steps, full compare")
    sh = bench.Shard(w, rank=0)
    t0 = sh.prepare()
    sh.use_bf16_moments()
    steps = [t0, t0 + 1, t0 + 2]
    for t in steps:
        sh.step_bf16_moments(t)
    torch.cuda.synchronize()
    prefix = oracle_warm_prefix(w, sh.lo)
    for a, b in shard_slices(sh.n):
        idx, th, m32, v32 = warm_state(w, sh, prefix, a, b)
        m, v = oracle.bf16_round(m32), oracle.bf16_round(v32)
        parts = host_partials(w, t0, sh.lo + idx)
        for t in steps:
            th, m, v, p = oracle.shard_step_bf16m(parts, th, m, v, oracle.hparams(t, **w.hparams()))
        assert_bitwise(host(sh.master[a:b]), th, f"7b 12-byte master [{a}, {b})")
        assert_bitwise(host(sh.m[a:b]), m, f"7b 12-byte m [{a}, {b})")
        assert_bitwise(host(sh.v[a:b]), v, f"7b 12-byte v [{a}, {b})")
        assert_bitwise(params_range(sh, a, b), p, f"7b 12-byte parameters [{a}, {b})")
        say(f"  [{a}, {b}) equal")
    del sh
    release()


def test_llama70b_kahan_sampled(bench):
    """bench.py --workload llama70b --state bf16-kahan: rank 5's slot (shard
    elements past 2^32), two steps; sampled compare."""
    w = W.llama70b()
    say(f"case: {w.name} rank 5 slot, pure-bf16 Kahan state, 2 steps, sampled")
    sh = bench.Shard(w, rank=5)
    assert sh.n > (1 << 32)
    t0 = sh.prepare()
    sh.use_kahan()
    sh.step_kahan(t0)
    sh.step_kahan(t0 + 1)
    idx = sample_indices(sh.table, sh.n, seed=75, n_random=1 << 20)
    idx = np.unique(np.concatenate([idx, np.array([(1 << 32) - 1, 1 << 32, (1 << 32) + 7])]))
    say(f"  {idx.size} sampled indices")
    th = oracle.bf16_round(host_master(w, sh.lo + idx))
    z = np.zeros(idx.size, np.uint16)
    c, m, v = z.copy(), z.copy(), z.copy()
    parts = host_partials(w, t0, sh.lo + idx)
    for t in (t0, t0 + 1):
        th, c, m, v = oracle.shard_step_kahan(parts, th, c, m, v, oracle.hparams(t, **w.hparams()))
    assert_kahan_state(gather_kahan(sh, idx), (th, c, m, v), "70b Kahan sampled")
    del sh
    release()


@pytest.mark.parametrize("bucket_params", [1 << 20, 3_000_000])
def test_gpt2_bucketed_step_equals_oracle(bench, bucket_params):
    """ZeRO-2 bucketed step: one launch per bucket (a contiguous run of the
    chunk table) gives the same bits as the oracle's whole-shard step."""
    w = W.gpt2()
    say(f"case: {w.name} rank 1, buckets of ~{bucket_params} params, 3 steps")
    sh = bench.Shard(w, rank=1)
    runs = sh.set_buckets(bucket_params)
    assert len(runs) > 1
    idx = np.arange(sh.lo, sh.hi, dtype=np.int64)
    th = host_master(w, idx)
    m = np.zeros(sh.n, np.float32)
    v = np.zeros(sh.n, np.float32)
    for t in (1, 2, 3):
        sh.fill_partials(t)
        sh.step_bucketed(t)
        th, m, v, p = oracle.shard_step(host_partials(w, t, idx), th, m, v,
                                        oracle.hparams(t, **w.hparams()))
    flat = np.concatenate([host(x) for x in sh.params])
    check_state((host(sh.master), host(sh.m), host(sh.v), flat[sh.lo:sh.hi]), (th, m, v, p),
                f"gpt2 bucketed {bucket_params}")
    del sh
    release()
