"""Pins of the oracle's pure-bf16 step with the compensated (Kahan) update:
bf16 parameter, compensation, m and v, no fp32 master.

The compensated add is pinned by what compensated summation guarantees,
not by its formula: no part of an increment is lost while the residual
fits the compensation buffer, and each stored value is the nearest bf16
of the exact quantity.  The step is pinned by closed forms: pure decay,
which a plain bf16 update cannot follow at all, and the first step from
zero moments.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import ledger
from test_oracle_pins_bf16m import brute_force_bf16


def bits_of(x) -> np.ndarray:
    """bf16 bits of float64 values that are bf16 values exactly."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64))
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "not a bf16 value"
    return (b >> 16).astype(np.uint16)


def value_of(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def test_compensation_recovers_increments_a_bf16_sum_drops():
    """theta = 1, five increments of 2^-10.  Each is below half of bf16's
    spacing at 1 (2^-8), so plain bf16 addition stays at 1 for ever.  By hand
    from the compensated add: c runs 2^-10, 2^-9, 3*2^-10, 2^-8 with theta
    still 1 (the fourth sum 1 + 2^-8 is a tie, kept at the even 1); at the
    fifth the pending 5*2^-10 carries theta to 1 + 2^-7 and leaves
    c = 5*2^-10 - 8*2^-10 = -3*2^-10."""
    th, c = bits_of([1.0]), bits_of([0.0])
    want_c = [2.0 ** -10, 2.0 ** -9, 3 * 2.0 ** -10, 2.0 ** -8, -3 * 2.0 ** -10]
    want_th = [1.0, 1.0, 1.0, 1.0, 1.0 + 2.0 ** -7]
    for k in range(5):
        th, c = oracle.kahan_add(th, c, 2.0 ** -10)
        assert value_of(th)[0] == want_th[k] and value_of(c)[0] == want_c[k], k


@pytest.mark.parametrize("seed", range(4))
def test_no_increment_is_lost_while_the_residual_fits(seed, K=400):
    """Increments on a 2^-16 grid, |delta| < 2^-9, theta kept in [0.5, 2):
    every residual is a multiple of 2^-16 no larger than half theta's
    spacing (2^-8), so it fits bf16 exactly, and compensated summation then
    loses nothing: theta_k + c_k equals theta_0 plus the exact sum of the
    increments after every step.  Plain bf16 accumulation of the same
    increments drifts far from it."""
    rng = np.random.default_rng(600 + seed)
    n = 64
    th = bits_of(np.where(rng.random(n) < 0.5, 1.0, 1.5))
    c = np.zeros(n, np.uint16)
    exact = [Fraction(float(x)) for x in value_of(th)]
    plain = value_of(th).copy()
    for k in range(K):
        d = rng.integers(-31, 32, n).astype(np.float64) * 2.0 ** -16
        # keep theta inside [0.5, 2): push the increments back toward the middle
        d = np.where(value_of(th) > 1.8, -np.abs(d), np.where(value_of(th) < 0.7, np.abs(d), d))
        th, c = oracle.kahan_add(th, c, d)
        for i in range(n):
            exact[i] += Fraction(float(d[i]))
        plain = value_of(bits_of_nearest(plain + d))
        got = [Fraction(float(a)) + Fraction(float(b)) for a, b in zip(value_of(th), value_of(c))]
        assert got == exact, (k, next(i for i in range(n) if got[i] != exact[i]))
    drift = max(abs(float(plain[i]) - float(exact[i])) for i in range(n))
    assert drift > 2.0 ** -9       # the uncompensated sum is off by more than a bf16 ulp


def bits_of_nearest(x):
    return np.array([brute_force_bf16(float(v)) for v in x], dtype=np.uint16)


def test_each_stored_value_is_the_nearest_bf16(n=3000):
    """theta' is the bf16 nearest to theta + c + delta and c' the bf16
    nearest to what remains, checked by exhaustive search over bf16 values,
    on sums exact in double (delta carries at most 28 significant bits
    within 20 binades below theta).  A quarter of the cases are sums
    2^-45 (relative) to either side of a bf16 midpoint: a detour through
    fp32 would land on the midpoint itself and round half of them the other
    way."""
    rng = np.random.default_rng(77)
    e = rng.integers(-6, 6, n)
    th_v = np.sign(rng.standard_normal(n)) * value_of(bits_of_nearest(
        (1 + rng.random(n)) * np.exp2(e.astype(np.float64))))
    c_v = value_of(bits_of_nearest(rng.standard_normal(n) * np.exp2(e - 10.0)))
    mant = rng.integers(1 << 27, 1 << 28, n).astype(np.float64) * np.sign(rng.standard_normal(n))
    d = mant * np.exp2((e - rng.integers(2, 20, n) - 27).astype(np.float64))
    # a quarter of the cases: theta + c + delta just off a bf16 midpoint
    k = n // 4
    spacing = np.exp2(np.floor(np.log2(np.abs(th_v[:k]))) - 7)
    target = th_v[:k] + spacing / 2 + rng.choice([-1, 1], k) * np.abs(th_v[:k]) * 2.0 ** -45
    d[:k] = target - th_v[:k] - c_v[:k]
    th1, c1 = oracle.kahan_add(bits_of(th_v), bits_of(c_v), d)
    for i in range(n):
        s = Fraction(float(th_v[i])) + Fraction(float(c_v[i])) + Fraction(float(d[i]))
        assert Fraction(float(th_v[i] + (d[i] + c_v[i]))) == s      # the test's sums are exact
        want_th = brute_force_bf16(float(s))
        assert th1[i] == want_th, (i, float(s), hex(th1[i]), hex(want_th))
        rest = s - Fraction(float(value_of([want_th])[0]))
        assert c1[i] == brute_force_bf16(float(rest)), i


def _step(theta, comp, m, v, g, hp):
    parts = [np.asarray(g, dtype=np.float32)]
    return oracle.shard_step_kahan(parts, theta, comp, m, v, hp)


def test_pure_decay_is_followed_where_plain_bf16_stalls():
    """Zero gradient, zero moments: the step is theta <- theta (1 - lr wd).
    With lr = 1e-3, wd = 0.1 each decrement is 1e-4 theta, under half of
    bf16's relative spacing (2^-9), so an uncompensated bf16 parameter never
    moves.  With the compensation the pair tracks theta_0 (1 - 1e-4)^2000:
    theta + c within a quarter of theta's ulp (each increment is taken off
    the bf16 theta, which differs from theta + c by at most half an ulp, so
    the 2000 increments drift by at most 2000 * 1e-4 / 2 = 0.1 ulp; the
    compensation's own roundings add 0.08 ulp at most here), and theta,
    its nearest bf16, within three quarters."""
    th0 = np.array([0.5, 0.75, 1.0, 1.25, 1.5, 3.0, -2.0, 100.0, 1e-3, -7e-5])
    th, c = bits_of_nearest(th0), np.zeros(th0.size, np.uint16)
    th0 = value_of(th)
    z = np.zeros(th0.size, np.uint16)
    K = 2000
    for t in range(1, K + 1):
        hp = oracle.hparams(t, lr=1e-3, weight_decay=0.1)
        th, c, m, v = _step(th, c, z, z, np.zeros(th0.size), hp)
        assert not m.any() and not v.any()
    want = th0 * (1 - 1e-4) ** K
    ulp = np.exp2(np.floor(np.log2(np.abs(want))) - 7)
    pair = value_of(th) + value_of(c)
    assert np.all(np.abs(pair - want) <= 0.25 * ulp), (pair - want) / ulp
    assert np.all(np.abs(value_of(th) - want) <= 0.75 * ulp), (value_of(th) - want) / ulp
    assert np.all(np.abs(value_of(th) - th0) > 20 * ulp)           # it did move


def test_first_step_closed_form(n=4000):
    """t = 1 from m = v = 0, c = 0: mhat = g and vhat = g^2 (up to double
    rounding), so theta_1 = theta_0 - lr (g / (|g| + eps) + wd theta_0),
    taken exactly in rationals.  theta' must be its nearest bf16 and c' the
    nearest bf16 of what is left.  Cases within 2^-40 (relative) of a bf16
    midpoint are skipped: double rounding inside the step may decide those
    either way."""
    rng = np.random.default_rng(5)
    th = bits_of_nearest(rng.standard_normal(n) * 0.02)
    g = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 2, n))).astype(np.float32)
    g[:n // 200] = 0.0
    lr, wd, eps = 1e-3, 0.1, 1e-8
    hp = oracle.hparams(1, lr=lr, weight_decay=wd, eps=eps)
    z = np.zeros(n, np.uint16)
    th1, c1, m1, v1 = _step(th, z, z, z, g, hp)
    checked = 0
    for i in range(n):
        t0, gi = Fraction(float(value_of([th[i]])[0])), Fraction(float(g[i]))
        x = t0 - Fraction(lr) * (gi / (abs(gi) + Fraction(eps)) + Fraction(wd) * t0)
        want = brute_force_bf16(float(x))
        near_boundary = any(brute_force_bf16(float(x) * (1 + r)) != want for r in (2.0 ** -40, -2.0 ** -40))
        if near_boundary:
            continue
        assert th1[i] == want, i
        rest = float(x - Fraction(float(value_of([want])[0])))
        r = float(value_of([c1[i]])[0])
        assert abs(r - rest) <= abs(rest) * 2.0 ** -8 + 1e-30, (i, r, rest)
        checked += 1
    assert checked > 0.99 * n


def test_moments_are_those_of_the_bf16_moment_step():
    """m' and v' do not depend on where the weight is kept: the same bits as
    the 12-byte step (fp32 master, bf16 m, v) from the same gradients and
    moments, whose moment arithmetic has its own pins."""
    rng = np.random.default_rng(9)
    n, N = 5000, 4
    parts = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(N)]
    m = bits_of_nearest(rng.standard_normal(n) * 1e-4)
    v = bits_of_nearest(np.abs(rng.standard_normal(n)) * 1e-7)
    th = bits_of_nearest(rng.standard_normal(n) * 0.02)
    hp = oracle.hparams(7)
    _, _, mk, vk = oracle.shard_step_kahan(parts, th, np.zeros(n, np.uint16), m, v, hp)
    _, mb, vb, _ = oracle.shard_step_bf16m(parts, value_of(th).astype(np.float32), m, v, hp)
    assert np.array_equal(mk, mb) and np.array_equal(vk, vb)


def test_pure_bf16_kahan_ledger():
    """bf16 parameter, gradient, m, v and compensation: 10 bytes per
    parameter held; the fused step reads N partials and the four bf16
    arrays and writes the four back: 2N + 16 bytes per shard element (32 at
    N = 8, against 42 for the 16-byte state)."""
    assert ledger.PURE_BF16_KAHAN.total == 10
    assert ledger.kahan_step_bytes_per_param(8) == 32
    assert ledger.kahan_step_bytes_per_param(16) == 48
    assert ledger.kahan_step_bytes_per_param(32, grad_bytes=4) == 144
