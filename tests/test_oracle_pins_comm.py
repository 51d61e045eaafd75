"""Pins of the communication model (oracle.ledger.ring_volume, step_volume)
by a brute-force ring: the collectives are run step by step on n simulated
ranks, counting what each rank sends.  The same simulation in fp32 pins the
reduce's rank order against a real ring order: the two differ by no more
than the floating-point error bound of an (N-1)-term sum."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import ledger


def ring_reduce_scatter(bufs, dtype=np.float64):
    """Ring reduce-scatter of n equal buffers split in n chunks: at step s
    rank r sends its running chunk (r - s) mod n to rank r + 1, which adds
    its own copy.  After n - 1 steps rank r holds the full sum of chunk
    (r + 1) mod n.  Returns (chunk sums by chunk index, elements sent per
    rank)."""
    n = len(bufs)
    chunks = [np.array_split(np.asarray(b, dtype=dtype), n) for b in bufs]
    acc = [[c.copy() for c in cs] for cs in chunks]
    sent = [0] * n
    for s in range(n - 1):
        msgs = []
        for r in range(n):
            c = (r - s) % n
            msgs.append(((r + 1) % n, c, acc[r][c].copy()))
            sent[r] += acc[r][c].size
        for dst, c, data in msgs:
            acc[dst][c] = (data + acc[dst][c]).astype(dtype)
    out = [None] * n
    for r in range(n):
        out[(r + 1) % n] = acc[r][(r + 1) % n]
    return out, sent


def ring_all_gather(pieces):
    """Ring all-gather: at step s rank r forwards piece (r - s) mod n."""
    n = len(pieces)
    have = [{r: pieces[r]} for r in range(n)]
    sent = [0] * n
    for s in range(n - 1):
        msgs = []
        for r in range(n):
            c = (r - s) % n
            msgs.append(((r + 1) % n, c, have[r][c]))
            sent[r] += len(have[r][c])
        for dst, c, data in msgs:
            have[dst][c] = data
    return [np.concatenate([h[c] for c in range(n)]) for h in have], sent


@pytest.mark.parametrize("n", [2, 3, 4, 8, 16])
def test_ring_volumes_match_the_model(n):
    m = 48 * n
    rng = np.random.default_rng(n)
    bufs = [rng.integers(-50, 50, m).astype(np.float64) for _ in range(n)]
    sums, sent_rs = ring_reduce_scatter(bufs)
    full = np.sum(bufs, axis=0)
    assert np.array_equal(np.concatenate(sums), full)            # exact small integers
    gathered, sent_ag = ring_all_gather(sums)
    assert all(np.array_equal(g, full) for g in gathered)       # all-reduce = RS + AG
    assert all(x == ledger.ring_volume("reduce-scatter", n, m) for x in sent_rs)
    assert all(x == ledger.ring_volume("all-gather", n, m) for x in sent_ag)
    assert ledger.ring_volume("all-reduce", n, m) == sent_rs[0] + sent_ag[0]


def test_step_volumes():
    """About 4 psi bytes of bf16 gradient per data-parallel step for large n,
    ZeRO-1/2 the same as plain data parallelism, ZeRO-3 half as much again."""
    psi = 7e9
    for n in (2, 8, 64, 4096):
        dp, z1, z3 = (ledger.step_volume(s, n, psi) for s in (0, 1, 3))
        assert dp == z1 and ledger.step_volume(2, n, psi) == z1
        assert Fraction(z3) / Fraction(z1) == Fraction(3, 2)
        assert dp == 2 * (n - 1) * psi / n
    assert 2 * ledger.step_volume(0, 4096, psi) == pytest.approx(4 * psi, rel=1e-3)


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32])
def test_fixed_order_is_within_the_ring_sums_error_bound(n):
    """The reduce's fixed rank order (double sum, one rounding) and an fp32
    ring reduce-scatter sum the same values in different orders.  Each
    element of the ring's fp32 sum is within gamma_(n-1) * sum |g_k| of the
    exact sum (gamma_k = k u / (1 - k u), u = 2^-24); the fixed-order double
    sum within (n-1) 2^-53 sum |g_k| of it (the values span up to about 55
    bits here, so it may round too); each mean is then rounded once to
    fp32.  So the two means differ by at most (gamma_(n-1) + (n-1) 2^-53)
    sum|g_k| / n plus two fp32 roundings of the mean."""
    rng = np.random.default_rng(100 + n)
    m = 64 * n
    parts16 = [oracle.bf16_round((rng.standard_normal(m) * np.exp2(rng.integers(-20, 20, m)))
                                 .astype(np.float32)) for _ in range(n)]
    parts = [(p.astype(np.uint32) << 16).view(np.float32) for p in parts16]
    ring, _ = ring_reduce_scatter(parts, dtype=np.float32)
    ring_mean = (np.concatenate(ring).astype(np.float64) / n).astype(np.float32)
    ours = oracle.reduce(parts16)
    u = 2.0 ** -24
    gamma = (n - 1) * u / (1 - (n - 1) * u)
    abs_sum = np.sum(np.abs(np.array(parts, dtype=np.float64)), axis=0)
    bound = ((gamma + (n - 1) * 2.0 ** -53) * abs_sum / n + 2 * u * np.abs(ours.astype(np.float64))
             + 1e-45)
    diff = np.abs(ring_mean.astype(np.float64) - ours.astype(np.float64))
    assert np.all(diff <= bound)
    assert np.any(diff > 0) or n <= 2       # the orders do differ somewhere
