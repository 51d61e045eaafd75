"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every expected value comes from the oracle run on host-generated inputs
(the synth module's host generator, which the device fill reproduces bit for
bit: see test_device_generator_matches_host).  Each test prints the case
it is about to run before touching the GPU.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W
from gpu_helpers import (assert_bitwise, check_state, host_master, host_partials,
                         oracle_warm_prefix, sample_indices, say)

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
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def host(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


# ------------------------------------------------------------ generator twin

def test_device_generator_matches_host(zs):
    say("case: device fill vs host generator, bf16 with outliers and f32")
    n, start = 1_000_003, 123_456_789_012
    st, ms = synth.stream_id(synth.KIND_GRAD, 3, 7), synth.stream_id(synth.KIND_OUTLIER, 3, 7)
    d = torch.empty(n, dtype=torch.int16, device="cuda")
    synth.dev_fill(d, 42, st, start, 1e-3, ms, 0.01, 100.0)
    assert_bitwise(host(d), synth.fill("bf16", 42, st, start, n, 1e-3, ms, 0.01, 100.0), "bf16 fill")
    f = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.dev_fill(f, 43, st, start, 0.02)
    assert_bitwise(host(f), synth.fill("f32", 43, st, start, n, 0.02), "f32 fill")
    pre = torch.arange(4096, dtype=torch.float32, device="cuda")
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.dev_spread(out, pre, 44, st, 0)
    want = synth.prefix_src(44, st, np.arange(n), 4096).astype(np.float32)
    assert_bitwise(host(out), want, "spread")


# ------------------------------------------------------------ small cases

def _flat_case(zs, n_ranks, total, rank, gdt, steps, max_chunk=1024, seed=7, hp=HP, t0=1):
    """Flat parameter buffer (slot destination), fresh partials per step."""
    S = -(-total // n_ranks)
    lo, hi = min(rank * S, total), min((rank + 1) * S, total)
    n = hi - lo
    idx = np.arange(lo, hi, dtype=np.int64)
    w = W.Workload("case", 99, [total], n_ranks, gdt, 1e-3)
    th_h = host_master(w, idx)
    m_h = np.zeros(n, np.float32)
    v_h = np.zeros(n, np.float32)
    full = torch.full((max(total, 1),), -1, dtype=torch.int16, device="cuda")
    master, m, v = dev(th_h), dev(m_h), dev(v_h)
    table, S2 = zs.zero_build_chunks([total], n_ranks, rank, slot_dst=full.data_ptr() + 2 * lo,
                                     max_chunk=max_chunk)
    assert S2 == S
    d_table = zs.chunks_to_device(table)
    for t in range(t0, t0 + steps):
        parts_h = host_partials(w, t, idx)
        parts = [dev_bf16(p) if gdt == "bf16" else dev(p) for p in parts_h]
        zs.zero_shard_step(parts, master, m, v, n, d_table, len(table), zs.hparams(t, **hp))
        th_h, m_h, v_h, p_h = oracle.shard_step(parts_h, th_h, m_h, v_h, oracle.hparams(t, **hp))
        fb = host(full)
        check_state((host(master), host(m), host(v), fb[lo:hi]), (th_h, m_h, v_h, p_h),
                    f"N={n_ranks} {gdt} rank {rank} step {t}")
        assert np.all(fb[:lo] == 0xFFFF) and np.all(fb[hi:] == 0xFFFF), "write outside the slot"


def test_smoke_entry(zs):
    say("case: __graft_entry__.smoke()")
    import __graft_entry__
    __graft_entry__.smoke()


@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_tiny_all_shards_ten_steps(zs, rank):
    """Tiny: one flat tensor of 1,048,576, N=4, steps 1..10, every shard."""
    say(f"case: tiny rank {rank}")
    _flat_case(zs, 4, 1 << 20, rank, "bf16", 10, max_chunk=65536, seed=0)


@pytest.mark.parametrize("n_ranks,gdt", [(1, "bf16"), (2, "bf16"), (3, "bf16"), (5, "f32"),
                                         (7, "bf16"), (8, "f32"), (13, "bf16"), (16, "bf16"),
                                         (32, "f32"), (33, "bf16"), (64, "bf16"), (64, "f32")])
def test_rank_counts_and_dtypes(zs, n_ranks, gdt):
    """Every compile-time N and the run-time-N kernel, both partial dtypes,
    a ragged total (short last shard), chunks of 192 elements."""
    total = 50_000 + 37
    for rank in (0, n_ranks - 1):
        say(f"case: N={n_ranks} {gdt} rank {rank}")
        _flat_case(zs, n_ranks, total, rank, gdt, 2, max_chunk=192)


def test_tiny_sizes_and_empty_shards(zs):
    for total, n_ranks, ranks in [(1, 1, [0]), (7, 2, [0, 1]), (9, 4, [0, 3]), (63, 64, [0, 62, 63]),
                                  (130, 64, [0, 43, 44, 63]), (9, 8, [4, 5, 7])]:
        for rank in ranks:
            say(f"case: total={total} N={n_ranks} rank {rank}")
            _flat_case(zs, n_ranks, total, rank, "bf16", 1, max_chunk=64)


def test_tensor_list_odd_boundaries(zs):
    """Tensor-list destination: shards cut across tensors whose sizes are
    odd, so chunk starts and bf16 destinations are misaligned."""
    rng = np.random.default_rng(5)
    numels = [int(x) for x in rng.integers(1, 3000, 40)] + [64, 1, 1, 8191]
    total = sum(numels)
    starts = np.cumsum([0] + numels[:-1])
    for n_ranks, gdt in [(4, "bf16"), (8, "f32"), (3, "bf16")]:
        w = W.Workload("list", 98, numels, n_ranks, gdt, 1e-3)
        for rank in range(n_ranks):
            say(f"case: tensor list N={n_ranks} {gdt} rank {rank}")
            lo, hi = w.shard_range(rank)
            n = hi - lo
            idx = np.arange(lo, hi, dtype=np.int64)
            params = [torch.full((k,), -1, dtype=torch.int16, device="cuda") for k in numels]
            table, _ = zs.zero_build_chunks(numels, n_ranks, rank, tensor_dst=params, max_chunk=128)
            d_table = zs.chunks_to_device(table)
            th_h = host_master(w, idx)
            m_h = (np.random.default_rng(rank).standard_normal(n) * 1e-4).astype(np.float32)
            v_h = (np.random.default_rng(rank + 9).random(n) * 1e-8).astype(np.float32)
            master, m, v = dev(th_h), dev(m_h), dev(v_h)
            for t in (5, 6):
                parts_h = host_partials(w, t, idx)
                parts = [dev_bf16(p) if gdt == "bf16" else dev(p) for p in parts_h]
                zs.zero_shard_step(parts, master, m, v, n, d_table, len(table), zs.hparams(t, **HP))
                th_h, m_h, v_h, p_h = oracle.shard_step(parts_h, th_h, m_h, v_h, oracle.hparams(t, **HP))
            flat = np.concatenate([host(p) for p in params])
            check_state((host(master), host(m), host(v), flat[lo:hi]), (th_h, m_h, v_h, p_h),
                        f"tensor list N={n_ranks} rank {rank}")
            assert np.all(flat[:lo] == 0xFFFF) and np.all(flat[hi:] == 0xFFFF)


def test_nonfinite_and_zero_partials(zs):
    """NaN / inf in single partials propagate to exactly those elements;
    all-zero partials give the decay-only update; -0 partials stay -0."""
    say("case: non-finite and zero partials")
    n, n_ranks = 4096 + 5, 4
    w = W.Workload("nf", 97, [n], n_ranks, "bf16", 1e-3)
    idx = np.arange(n, dtype=np.int64)
    parts_h = host_partials(w, 1, idx)
    parts_h[1][10] = 0x7FC0
    parts_h[2][11] = 0x7F80
    parts_h[3][11] = 0xFF80
    parts_h[0][12] = 0x7F80
    for p in parts_h:
        p[100:300] = 0
        p[300:310] = 0x8000
    th_h = host_master(w, idx)
    th_h[13] = np.nan
    m_h = np.zeros(n, np.float32)
    v_h = np.zeros(n, np.float32)
    full = torch.empty(n, dtype=torch.int16, device="cuda")
    table, _ = zs.zero_build_chunks([n], 1, 0, slot_dst=full, max_chunk=1024)
    master, m, v = dev(th_h), dev(m_h), dev(v_h)
    zs.zero_shard_step([dev_bf16(p) for p in parts_h], master, m, v, n, zs.chunks_to_device(table),
                       len(table), zs.hparams(1, **HP))
    want = oracle.shard_step(parts_h, th_h, m_h, v_h, oracle.hparams(1, **HP))
    got = (host(master), host(m), host(v), host(full))
    check_state(got, want, "non-finite")
    assert np.isnan(got[0][[10, 11, 12, 13]]).all()
    assert np.all(got[1][100:300] == 0) and np.all(got[2][100:300] == 0)


def test_fused_equals_unfused(zs):
    """zero_reduce_shard -> zero_adamw_shard -> zero_gather_write gives the
    same bits as zero_shard_step, and the reduce alone matches the oracle."""
    for n_ranks, gdt in [(8, "bf16"), (32, "f32"), (6, "bf16")]:
        say(f"case: fused vs unfused N={n_ranks} {gdt}")
        n = 100_003
        w = W.Workload("fu", 96, [n * n_ranks], n_ranks, gdt, 1e-3)
        idx = np.arange(n, dtype=np.int64)
        parts_h = host_partials(w, 3, idx)
        parts = [dev_bf16(p) if gdt == "bf16" else dev(p) for p in parts_h]
        th_h = host_master(w, idx)
        m_h = (np.random.default_rng(1).standard_normal(n) * 1e-4).astype(np.float32)
        v_h = (np.random.default_rng(2).random(n) * 1e-8).astype(np.float32)
        hp = zs.hparams(3, **HP)
        a = [dev(x) for x in (th_h, m_h, v_h)]
        b = [dev(x) for x in (th_h, m_h, v_h)]
        pa = torch.empty(n, dtype=torch.int16, device="cuda")
        pb = torch.empty(n, dtype=torch.int16, device="cuda")
        ta, _ = zs.zero_build_chunks([n], 1, 0, slot_dst=pa, max_chunk=4096)
        tb, _ = zs.zero_build_chunks([n], 1, 0, slot_dst=pb, max_chunk=4096)
        zs.zero_shard_step(parts, *a, n, zs.chunks_to_device(ta), len(ta), hp)
        g = torch.empty(n, dtype=torch.float32, device="cuda")
        zs.zero_reduce_shard(parts, n, g)
        zs.zero_adamw_shard(g, *b, n, hp)
        zs.zero_gather_write(b[0], n, zs.chunks_to_device(tb), len(tb))
        assert_bitwise(host(g), oracle.reduce(parts_h), "reduce")
        for x, y, name in zip(a + [pa], b + [pb], ("master", "m", "v", "param")):
            assert_bitwise(host(x), host(y), f"fused vs unfused {name}")
        want = oracle.adamw(oracle.reduce(parts_h), th_h, m_h, v_h, oracle.hparams(3, **HP))
        check_state((host(b[0]), host(b[1]), host(b[2])), want, "unfused adamw")


def test_bf16_rounding_exhaustive(zs):
    """The kernel's fp32 -> bf16 rounding on all 2^32 fp32 patterns (through
    zero_gather_write) equals the oracle's."""
    n = 1 << 28
    src = torch.empty(n, dtype=torch.int32, device="cuda")
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    table, _ = zs.zero_build_chunks([n], 1, 0, slot_dst=out, max_chunk=1 << 16)
    d_table = zs.chunks_to_device(table)
    for c in range(16):
        say(f"case: bf16 rounding, patterns {c << 28:#x}..")
        base = (c << 28) - (1 << 32 if c >= 8 else 0)       # same bits as int32
        src.copy_(torch.arange(base, base + n, dtype=torch.int64, device="cuda"))
        zs.zero_gather_write(src.view(torch.float32), n, d_table, len(table))
        u = np.arange(c << 28, (c + 1) << 28, dtype=np.uint64).astype(np.uint32)
        want = oracle.bf16_round(u.view(np.float32))
        assert_bitwise(host(out), want, f"bf16 block {c}", strict_nan=True)


# ------------------------------------------------------------ extended reduce

def _ext_case(zs, n_ranks, group, G, gdt, total=70_001, rank=0, max_chunk=192, steps=2):
    """G micro-batches per step: G - 1 through zero_accumulate_shard, the last
    through zero_shard_step_ex, against oracle.accumulate / shard_step_ex."""
    w = W.Workload("ext", 95, [total], n_ranks, gdt, 1e-3)
    S = -(-total // n_ranks)
    lo, hi = min(rank * S, total), min((rank + 1) * S, total)
    n = hi - lo
    idx = np.arange(lo, hi, dtype=np.int64)
    th_h = host_master(w, idx)
    m_h = np.zeros(n, np.float32)
    v_h = np.zeros(n, np.float32)
    full = torch.full((total,), -1, dtype=torch.int16, device="cuda")
    master, m, v = dev(th_h), dev(m_h), dev(v_h)
    acc = torch.empty(max(n, 1), dtype=torch.float32, device="cuda")
    table, _ = zs.zero_build_chunks([total], n_ranks, rank, slot_dst=full.data_ptr() + 2 * lo,
                                    max_chunk=max_chunk)
    d_table = zs.chunks_to_device(table)
    for t in range(1, steps + 1):
        acc_h = None
        for j in range(G):
            parts_h = host_partials(w, 100 * t + j, idx)
            parts = [dev_bf16(p) if gdt == "bf16" else dev(p) for p in parts_h]
            if j < G - 1:
                zs.zero_accumulate_shard(parts, n, acc, reset=(j == 0), group=group)
                acc_h = oracle.accumulate(parts_h, acc_h, group=group or None)
                assert_bitwise(host(acc)[:n], acc_h, f"accumulator N={n_ranks} K={group} j={j}")
            else:
                zs.zero_shard_step_ex(parts, master, m, v, n, d_table, len(table), zs.hparams(t, **HP),
                                      group=group, micro_batches=G, acc=acc if G > 1 else None)
                th_h, m_h, v_h, p_h = oracle.shard_step_ex(parts_h, th_h, m_h, v_h, oracle.hparams(t, **HP),
                                                           group=group or None, acc=acc_h, micro_batches=G)
        fb = host(full)
        check_state((host(master), host(m), host(v), fb[lo:hi]), (th_h, m_h, v_h, p_h),
                    f"ext N={n_ranks} K={group} G={G} {gdt} step {t}")


@pytest.mark.parametrize("n_ranks,group,G,gdt", [
    (8, 0, 1, "bf16"), (8, 4, 1, "bf16"), (8, 2, 3, "bf16"), (8, 1, 2, "f32"),
    (16, 8, 1, "bf16"), (16, 4, 4, "bf16"), (32, 8, 2, "f32"), (6, 3, 3, "bf16"),
    (12, 4, 2, "f32"), (4, 2, 5, "bf16")])
def test_extended_reduce_two_level_and_accumulation(zs, n_ranks, group, G, gdt):
    say(f"case: extended reduce N={n_ranks} K={group} G={G} {gdt}")
    _ext_case(zs, n_ranks, group, G, gdt, rank=n_ranks - 1)


def test_extended_flat_equals_plain_step(zs):
    """group 0, one micro-batch: the extended kernel gives the bits of the
    plain fused kernel."""
    say("case: extended flat vs plain step")
    n, n_ranks = 50_003, 8
    w = W.Workload("ef", 94, [n], n_ranks, "bf16", 1e-3)
    idx = np.arange(n, dtype=np.int64)
    parts = [dev_bf16(p) for p in host_partials(w, 1, idx)]
    th = host_master(w, idx)
    a = [dev(th), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")]
    b = [dev(th), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")]
    pa = torch.empty(n, dtype=torch.int16, device="cuda")
    pb = torch.empty(n, dtype=torch.int16, device="cuda")
    ta, _ = zs.zero_build_chunks([n], 1, 0, slot_dst=pa)
    tb, _ = zs.zero_build_chunks([n], 1, 0, slot_dst=pb)
    for t in (1, 2):
        zs.zero_shard_step(parts, *a, n, zs.chunks_to_device(ta), len(ta), zs.hparams(t, **HP))
        zs.zero_shard_step_ex(parts, *b, n, zs.chunks_to_device(tb), len(tb), zs.hparams(t, **HP))
    for x, y, name in zip(a + [pa], b + [pb], ("master", "m", "v", "param")):
        assert_bitwise(host(x), host(y), f"flat ex vs plain {name}")


def test_grouping_decides_the_rounding_on_gpu(zs):
    """The hand-derived case of the oracle pins: 2^60, 1, -2^60, 1 gives 0 with
    two groups of two and 1/4 flat, through the GPU reduce."""
    say("case: grouping rounding case on the GPU")
    big = 2.0 ** 60
    vals = [np.full(16, v, np.float32) for v in (big, 1.0, -big, 1.0)]
    parts = [dev(x) for x in vals]
    acc = torch.empty(16, dtype=torch.float32, device="cuda")
    zs.zero_accumulate_shard(parts, 16, acc, reset=True, group=2)
    assert np.all(host(acc) == 0.0)
    zs.zero_accumulate_shard(parts, 16, acc, reset=True, group=0)
    assert np.all(host(acc) == 1.0)


# ------------------------------------------------------------ 12-byte state

def _m16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()


@pytest.mark.parametrize("n_ranks,gdt,total,rank", [(1, "bf16", 9_999, 0), (3, "bf16", 30_001, 2),
                                                    (8, "bf16", 80_003, 7), (16, "bf16", 64_000, 5),
                                                    (32, "f32", 50_021, 31), (5, "f32", 12_345, 1)])
def test_bf16_moment_state_matches_oracle(zs, n_ranks, gdt, total, rank):
    say(f"case: 12-byte state N={n_ranks} {gdt} total={total} rank={rank}")
    w = W.Workload("m16", 93, [total], n_ranks, gdt, 1e-3)
    lo, hi = w.shard_range(rank)
    n = hi - lo
    idx = np.arange(lo, hi, dtype=np.int64)
    rng = np.random.default_rng(n_ranks)
    th_h = host_master(w, idx)
    m_h = oracle.bf16_from_double(rng.standard_normal(n) * 1e-4)
    v_h = oracle.bf16_from_double(rng.random(n) * 1e-8)
    full = torch.full((total,), -1, dtype=torch.int16, device="cuda")
    master, m, v = dev(th_h), _m16_dev(m_h), _m16_dev(v_h)
    table, _ = zs.zero_build_chunks([total], n_ranks, rank, slot_dst=full.data_ptr() + 2 * lo,
                                    max_chunk=576)
    d_table = zs.chunks_to_device(table)
    for t in (3, 4, 5):
        parts_h = host_partials(w, t, idx)
        parts = [dev_bf16(p) if gdt == "bf16" else dev(p) for p in parts_h]
        zs.zero_shard_step_bf16_moments(parts, master, m, v, n, d_table, len(table), zs.hparams(t, **HP))
        th_h, m_h, v_h, p_h = oracle.shard_step_bf16m(parts_h, th_h, m_h, v_h, oracle.hparams(t, **HP))
    fb = host(full)
    assert_bitwise(host(master), th_h, "12-byte master")
    assert_bitwise(host(m), m_h, "12-byte m")
    assert_bitwise(host(v), v_h, "12-byte v")
    assert_bitwise(fb[lo:hi], p_h, "12-byte param")
    assert np.all(fb[:lo] == 0xFFFF) and np.all(fb[hi:] == 0xFFFF)


def test_bf16_moment_rounding_at_midpoints(zs):
    """Moments driven onto, and one fp32 ulp either side of, bf16 midpoints:
    beta1 = beta2 = 1/2 and one fp32 partial g make m' = (m + g)/2 exactly;
    g is chosen so that m' lands at t, t +- 2^-24 t, t +- 2^-40 t for bf16
    midpoints t.  Every stored moment must be the single nearest-even
    rounding the oracle computes."""
    say("case: 12-byte state rounding at bf16 midpoints")
    rng = np.random.default_rng(31)
    k = 20000
    base = rng.integers(0x3000, 0x4000, k).astype(np.uint32)
    lo_b = (base << 16).view(np.float32).astype(np.float64)
    hi_b = ((base + 1) << 16).view(np.float32).astype(np.float64)
    t = (lo_b + hi_b) / 2
    rel = np.array([0.0, 2.0 ** -24, -2.0 ** -24, 2.0 ** -40, -2.0 ** -40])[rng.integers(0, 5, k)]
    target = t * (1 + rel)
    m_bits = oracle.bf16_from_double(rng.standard_normal(k) * t)
    m_val = (m_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g = (2 * target - m_val).astype(np.float32)           # fp32 partial (one rank)
    hp = dict(lr=1e-3, beta1=0.5, beta2=0.5, eps=1e-8, weight_decay=0.0)
    th = (rng.standard_normal(k) * 0.02).astype(np.float32)
    v_bits = m_bits.copy()
    full = torch.empty(k, dtype=torch.int16, device="cuda")
    table, _ = zs.zero_build_chunks([k], 1, 0, slot_dst=full)
    master, m, v = dev(th), _m16_dev(m_bits), _m16_dev(v_bits)
    zs.zero_shard_step_bf16_moments([dev(g)], master, m, v, k, zs.chunks_to_device(table), len(table),
                                    zs.hparams(1, **hp))
    want = oracle.shard_step_bf16m([g], th, m_bits, v_bits, oracle.hparams(1, **hp))
    assert_bitwise(host(m), want[1], "moments at midpoints: m")
    assert_bitwise(host(v), want[2], "moments at midpoints: v")
    assert_bitwise(host(master), want[0], "moments at midpoints: master")


# ------------------------------------------------------------ checkpoint / resume

@pytest.mark.parametrize("state", ["fp32", "bf16-kahan"])
def test_checkpoint_resume_is_bitwise(zs, tmp_path, state):
    """Kill-and-replay: three steps, the shard state (and t) saved to .npy
    files, every device buffer freed, the state reloaded into new
    allocations with a newly built chunk table, three more steps.  The
    result equals the uninterrupted six-step run bit for bit, and both equal
    the oracle."""
    say(f"case: checkpoint/resume, {state} state")
    w = W.Workload("ckpt", 97, [5_000, 70_001, 3], 4, "bf16", 1e-3)
    rank = 1
    lo, hi = w.shard_range(rank)
    n = hi - lo
    idx = np.arange(lo, hi, dtype=np.int64)
    th0 = host_master(w, idx)

    def fresh(arrays):
        full = torch.full((sum(w.numels),), -1, dtype=torch.int16, device="cuda")
        table, _ = zs.zero_build_chunks(w.numels, w.n_ranks, rank, slot_dst=full.data_ptr() + 2 * lo,
                                        max_chunk=960)
        if state == "fp32":
            bufs = [dev(arrays[0]), dev(arrays[1]), dev(arrays[2])]
        else:
            full[lo:hi] = torch.from_numpy(arrays[0].view(np.int16)).cuda()
            bufs = [dev_bf16(arrays[1]), dev_bf16(arrays[2]), dev_bf16(arrays[3])]
        return full, bufs, zs.chunks_to_device(table), len(table)

    def run(full, bufs, d_table, n_chunks, steps):
        for t in steps:
            parts = [dev_bf16(p) for p in host_partials(w, t, idx)]
            if state == "fp32":
                zs.zero_shard_step(parts, *bufs, n, d_table, n_chunks, zs.hparams(t, **HP))
            else:
                zs.zero_shard_step_kahan(parts, *bufs, n, d_table, n_chunks, zs.hparams(t, **HP))
        torch.cuda.synchronize()

    def snapshot(full, bufs):
        p = host(full)[lo:hi].copy()
        return [host(b).copy() for b in bufs] + [p] if state == "fp32" else [p] + [host(b).copy() for b in bufs]

    z32, z16 = np.zeros(n, np.float32), np.zeros(n, np.uint16)
    init = [th0, z32, z32] if state == "fp32" else [oracle.bf16_round(th0), z16, z16, z16]
    # uninterrupted
    full, bufs, d_table, nc = fresh(init)
    run(full, bufs, d_table, nc, range(1, 7))
    straight = snapshot(full, bufs)
    del full, bufs, d_table
    # interrupted after step 3, resumed from files
    full, bufs, d_table, nc = fresh(init)
    run(full, bufs, d_table, nc, range(1, 4))
    saved = snapshot(full, bufs)
    for k, a in enumerate(saved):
        np.save(tmp_path / f"s{k}.npy", a)
    np.save(tmp_path / "t.npy", np.array([3], np.int64))
    del full, bufs, d_table
    torch.cuda.empty_cache()
    loaded = [np.load(tmp_path / f"s{k}.npy") for k in range(len(saved))]
    t_done = int(np.load(tmp_path / "t.npy")[0])
    arrays = loaded[:3] if state == "fp32" else loaded
    full, bufs, d_table, nc = fresh(arrays)
    if state == "fp32":
        full[lo:hi] = torch.from_numpy(loaded[3].view(np.int16)).cuda()
    run(full, bufs, d_table, nc, range(t_done + 1, 7))
    resumed = snapshot(full, bufs)
    for k, (a, b) in enumerate(zip(straight, resumed)):
        assert_bitwise(b, a, f"resume {state} array {k}", strict_nan=True)
    # and the oracle's six steps
    if state == "fp32":
        th, m, v = th0, z32, z32
        for t in range(1, 7):
            th, m, v, p = oracle.shard_step(host_partials(w, t, idx), th, m, v, oracle.hparams(t, **HP))
        want = [th, m, v, p]
    else:
        th, c, m, v = init
        for t in range(1, 7):
            th, c, m, v = oracle.shard_step_kahan(host_partials(w, t, idx), th, c, m, v, oracle.hparams(t, **HP))
        want = [th, c, m, v]
    for k, (a, b) in enumerate(zip(want, straight)):
        assert_bitwise(b, a, f"oracle {state} array {k}")
