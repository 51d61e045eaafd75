"""GPU parity of the pure-bf16 step with the Kahan-compensated update
(zero_shard_step_kahan) against the CPU oracle, bitwise: the parameters in
their slots, the compensation, m and v.  Each test prints its case before
touching the GPU."""
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
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).cuda()


def host(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def initial_state(n, seed, comp_scale=1e-6):
    """bf16 parameters, a non-zero compensation (as after earlier steps), m, v."""
    rng = np.random.default_rng(seed)
    th = oracle.bf16_from_double(rng.standard_normal(n) * 0.02)
    c = oracle.bf16_from_double(rng.standard_normal(n) * comp_scale)
    m = oracle.bf16_from_double(rng.standard_normal(n) * 1e-4)
    v = oracle.bf16_from_double(rng.random(n) * 1e-8)
    return th, c, m, v


@pytest.mark.parametrize("n_ranks,gdt,total,rank", [(1, "bf16", 9_999, 0), (3, "bf16", 30_001, 2),
                                                    (8, "bf16", 80_003, 7), (16, "bf16", 64_000, 5),
                                                    (32, "f32", 50_021, 31), (5, "f32", 12_345, 1),
                                                    (64, "bf16", 20_000, 63)])
def test_kahan_state_matches_oracle(zs, n_ranks, gdt, total, rank):
    """Flat parameter buffer: the shard's slot holds its parameters; the
    rest of the buffer (other ranks' slots) must stay untouched."""
    say(f"case: pure-bf16 Kahan step N={n_ranks} {gdt} total={total} rank={rank}")
    w = W.Workload("kahan", 94, [total], n_ranks, gdt, 1e-3)
    lo, hi = w.shard_range(rank)
    n = hi - lo
    idx = np.arange(lo, hi, dtype=np.int64)
    th_h, c_h, m_h, v_h = initial_state(n, n_ranks)
    full_h = np.full(total, 0x7FC1, np.uint16)          # a NaN pattern no step writes
    full_h[lo:hi] = th_h
    full = dev16(full_h)
    comp, m, v = dev16(c_h), dev16(m_h), dev16(v_h)
    table, _ = zs.zero_build_chunks([total], n_ranks, rank, slot_dst=full.data_ptr() + 2 * lo,
                                    max_chunk=576)
    d_table = zs.chunks_to_device(table)
    for t in (3, 4, 5):
        parts_h = host_partials(w, t, idx)
        parts = [dev16(p) if gdt == "bf16" else dev(p) for p in parts_h]
        zs.zero_shard_step_kahan(parts, comp, m, v, n, d_table, len(table), zs.hparams(t, **HP))
        th_h, c_h, m_h, v_h = oracle.shard_step_kahan(parts_h, th_h, c_h, m_h, v_h,
                                                      oracle.hparams(t, **HP))
    fb = host(full)
    assert_bitwise(fb[lo:hi], th_h, "kahan parameters")
    assert_bitwise(host(comp), c_h, "kahan compensation")
    assert_bitwise(host(m), m_h, "kahan m")
    assert_bitwise(host(v), v_h, "kahan v")
    assert np.all(fb[:lo] == 0x7FC1) and np.all(fb[hi:] == 0x7FC1)


def test_kahan_tensor_list_odd_boundaries(zs):
    """Per-tensor destinations with odd sizes: chunk starts and bf16
    destinations are misaligned, so the kernel mixes its vector and
    element paths for reading and writing the parameters."""
    rng = np.random.default_rng(15)
    numels = [int(x) for x in rng.integers(1, 3000, 40)] + [64, 1, 1, 8191]
    starts = np.cumsum([0] + numels[:-1])
    for n_ranks, gdt in [(4, "bf16"), (8, "f32"), (3, "bf16")]:
        w = W.Workload("klist", 95, numels, n_ranks, gdt, 1e-3)
        for rank in range(n_ranks):
            say(f"case: Kahan tensor list N={n_ranks} {gdt} rank {rank}")
            lo, hi = w.shard_range(rank)
            n = hi - lo
            idx = np.arange(lo, hi, dtype=np.int64)
            th_h, c_h, m_h, v_h = initial_state(n, 100 + rank)
            flat_h = np.full(sum(numels), 0x7FC1, np.uint16)
            flat_h[lo:hi] = th_h
            params = [dev16(flat_h[a:a + k]) for a, k in zip(starts, numels)]
            table, _ = zs.zero_build_chunks(numels, n_ranks, rank, tensor_dst=params, max_chunk=128)
            d_table = zs.chunks_to_device(table)
            comp, m, v = dev16(c_h), dev16(m_h), dev16(v_h)
            for t in (5, 6):
                parts_h = host_partials(w, t, idx)
                parts = [dev16(p) if gdt == "bf16" else dev(p) for p in parts_h]
                zs.zero_shard_step_kahan(parts, comp, m, v, n, d_table, len(table),
                                         zs.hparams(t, **HP))
                th_h, c_h, m_h, v_h = oracle.shard_step_kahan(parts_h, th_h, c_h, m_h, v_h,
                                                              oracle.hparams(t, **HP))
            flat = np.concatenate([host(p) for p in params])
            tag = f"Kahan tensor list N={n_ranks} rank {rank}"
            assert_bitwise(flat[lo:hi], th_h, tag + " parameters")
            assert_bitwise(host(comp), c_h, tag + " compensation")
            assert_bitwise(host(m), m_h, tag + " m")
            assert_bitwise(host(v), v_h, tag + " v")
            assert np.all(flat[:lo] == 0x7FC1) and np.all(flat[hi:] == 0x7FC1)


def test_kahan_pure_decay_long_run(zs):
    """Zero gradients for 300 steps: every increment is below half a bf16
    ulp, so the parameters move only through the compensation; each step is
    compared with the oracle, bit for bit."""
    say("case: Kahan pure decay, 300 steps")
    n = 20_000
    th_h, c_h, m_h, v_h = initial_state(n, 3, comp_scale=0.0)
    m_h[:] = 0
    v_h[:] = 0
    full = dev16(th_h)
    comp, m, v = dev16(c_h), dev16(m_h), dev16(v_h)
    table, _ = zs.zero_build_chunks([n], 1, 0, slot_dst=full)
    d_table = zs.chunks_to_device(table)
    zero = np.zeros(n, np.float32)
    parts = [dev(zero)]
    th0 = th_h.copy()
    for t in range(1, 301):
        zs.zero_shard_step_kahan(parts, comp, m, v, n, d_table, len(table), zs.hparams(t, **HP))
        th_h, c_h, m_h, v_h = oracle.shard_step_kahan([zero], th_h, c_h, m_h, v_h,
                                                      oracle.hparams(t, **HP))
        if t % 50 == 0:
            assert_bitwise(host(full), th_h, f"decay step {t} parameters")
            assert_bitwise(host(comp), c_h, f"decay step {t} compensation")
    assert np.count_nonzero(th_h != th0) > n // 2      # the parameters did move


def test_kahan_nonfinite_and_zero_partials(zs):
    """NaN and inf in single partials reach exactly those elements' state
    (NaN payloads may differ); -0 and 0 partials give the decay-only step."""
    say("case: Kahan non-finite and zero partials")
    n, N = 4096, 4
    rng = np.random.default_rng(8)
    parts_h = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(N)]
    parts_h[1][10] = np.nan
    parts_h[2][20] = np.inf
    parts_h[3][30] = -np.inf
    parts_h[0][40] = np.inf
    parts_h[2][40] = -np.inf
    for p in parts_h:
        p[100:200] = -0.0
    th_h, c_h, m_h, v_h = initial_state(n, 4)
    full = dev16(th_h)
    comp, m, v = dev16(c_h), dev16(m_h), dev16(v_h)
    table, _ = zs.zero_build_chunks([n], 1, 0, slot_dst=full)
    zs.zero_shard_step_kahan([dev(p) for p in parts_h], comp, m, v, n, zs.chunks_to_device(table),
                             len(table), zs.hparams(2, **HP))
    th_h, c_h, m_h, v_h = oracle.shard_step_kahan(parts_h, th_h, c_h, m_h, v_h, oracle.hparams(2, **HP))
    assert_bitwise(host(full), th_h, "non-finite parameters")
    assert_bitwise(host(comp), c_h, "non-finite compensation")
    assert_bitwise(host(m), m_h, "non-finite m")
    assert_bitwise(host(v), v_h, "non-finite v")
    nan = lambda b: (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0
    assert nan(th_h[10]) and nan(th_h[40])
