"""Pins of the oracle's extended reduce: the two-level (hybrid-sharded) order
and gradient accumulation over micro-batches."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from test_oracle_pins import _random_bf16, f32_bits


@pytest.mark.parametrize("n_ranks", [1, 2, 4, 6, 8, 16, 32])
def test_one_group_and_singleton_groups_are_the_flat_order(n_ranks):
    """K = N (one group) and K = 1 (every rank its own group) both reduce to
    the flat rank-order fold, which the flat pins fix."""
    rng = np.random.default_rng(200 + n_ranks)
    parts = [(rng.standard_normal(3000) * np.exp2(rng.integers(-30, 10, 3000))).astype(np.float32)
             for _ in range(n_ranks)]
    flat = oracle.reduce(parts)
    assert np.array_equal(f32_bits(oracle.reduce_ex(parts, group=n_ranks)), f32_bits(flat))
    assert np.array_equal(f32_bits(oracle.reduce_ex(parts, group=1)), f32_bits(flat))


def test_grouping_decides_the_rounding():
    """Ranks 0..3 hold 2^60, 1, -2^60, 1 (fp32).  In double, 2^60 + 1 rounds
    back to 2^60.  Two groups of two (ranks {0,1}, {2,3}):
    (2^60 + 1) + (-2^60 + 1) -> 2^60 + (-2^60) = 0, so g = 0.  The flat fold
    gives ((2^60 + 1) - 2^60) + 1 = 1, g = 1/4; grouping by the other axis
    ({0,2}, {1,3}) gives 0 + 2, g = 1/2.  Catches a transposed group index
    or a flat fold where the two-level order is asked for."""
    big = np.float32(2.0 ** 60)
    parts = [np.array([v], np.float32) for v in (big, 1.0, -big, 1.0)]
    assert oracle.reduce_ex(parts, group=2)[0] == 0.0
    assert oracle.reduce_ex(parts, group=4)[0] == 0.25
    assert oracle.reduce(parts)[0] == 0.25


@pytest.mark.parametrize("n_ranks,group", [(4, 2), (6, 3), (8, 2), (8, 4), (16, 8), (12, 4)])
def test_grouped_mean_is_exact_when_sums_are_exact(n_ranks, group):
    rng = np.random.default_rng(300 + n_ranks * 10 + group)
    n = 800
    parts = [_random_bf16(rng, n) for _ in range(n_ranks)]
    got = oracle.reduce_ex(parts, group=group)
    vals = [(p.astype(np.uint32) << 16).view(np.float32).astype(np.float64) for p in parts]
    exp = np.array([np.float32(float(sum(Fraction(float(v[i])) for v in vals) / n_ranks))
                    for i in range(n)], np.float32)
    assert np.array_equal(f32_bits(got), f32_bits(exp))


@pytest.mark.parametrize("group", [None, 2])
def test_accumulated_micro_batches_give_the_full_batch_gradient(group):
    """The data-parallel identity extended to gradient accumulation: a batch
    of b samples split over N = 4 ranks and G = 4 micro-batches each; per
    micro-batch gradient g_kj = (N G / b) sum over its samples of grad l.
    Accumulating the first G - 1 micro-batches and reducing the last with
    the accumulator gives the full-batch gradient (1/b) sum grad l exactly
    (integer data: every value is a dyadic rational fp32 holds)."""
    rng = np.random.default_rng(17)
    n_ranks, G, per = 4, 4, 2
    b = n_ranks * G * per
    din, dout = 3, 2
    X = rng.integers(-2, 3, (b, din))
    Y = rng.integers(-2, 3, (b, dout))
    W = rng.integers(-2, 3, (dout, din))
    grads = [2 * np.outer(W @ x - y, x).ravel() for x, y in zip(X, Y)]
    full = [Fraction(int(sum(g[j] for g in grads)), b) for j in range(din * dout)]

    def micro(k, j):
        samples = range((j * n_ranks + k) * per, (j * n_ranks + k + 1) * per)
        vals = [Fraction(n_ranks * G * int(sum(grads[s][e] for s in samples)), b)
                for e in range(din * dout)]
        a = np.array([float(q) for q in vals], np.float32)
        assert all(Fraction(float(x)) == q for x, q in zip(a, vals))
        return a

    acc = None
    for j in range(G - 1):
        acc = oracle.accumulate([micro(k, j) for k in range(n_ranks)], acc, group=group)
    g = oracle.reduce_ex([micro(k, G - 1) for k in range(n_ranks)], group=group, acc=acc,
                         micro_batches=G)
    assert [Fraction(float(x)) for x in g] == full


def test_accumulator_rounds_once_per_micro_batch():
    """acc after micro-batch j is fp32(acc + s_j) with s_j the double sum of
    that micro-batch: one rounding.  Element 0: micro-batch 0 sums to 1,
    micro-batch 1 to 2^-24 + 2^-50 (exact in double); 1 + 2^-24 + 2^-50 lies
    above the fp32 midpoint, so acc = 1 + 2^-23, whereas rounding s_1 to fp32
    first would give the tie 1 + 2^-24 and then 1.  Element 1: a sum of -0
    starts the accumulator at -0 (no +0 added)."""
    mb0 = [np.array([1.0, -0.0], np.float32), np.array([0.0, -0.0], np.float32)]
    mb1 = [np.array([2.0 ** -24, 1.0], np.float32), np.array([2.0 ** -50, 0.0], np.float32)]
    a0 = oracle.accumulate(mb0)
    assert a0[0] == 1.0 and f32_bits(a0)[1] == 0x80000000
    a1 = oracle.accumulate(mb1, a0)
    assert a1[0] == np.float32(1.0 + 2.0 ** -23) and a1[1] == 1.0
    g = oracle.reduce_ex(mb1, acc=a0, micro_batches=2)
    assert g[0] == np.float32((1.0 + 2.0 ** -23) / 4)
