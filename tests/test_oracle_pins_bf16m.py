"""Pins of the oracle's 12-bytes-per-parameter state (bf16 Adam moments
beside the fp32 master)."""
import bisect
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import ledger
from test_oracle_pins import _random_bf16, f32_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _finite_bf16_table():
    """All finite bf16 values as exact fractions, sorted, with their bits."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    keep = np.isfinite(vals)
    pairs = sorted((Fraction(float(v)), int(b)) for v, b in zip(vals[keep], bits[keep])
                   if not (v == 0 and b == 0x8000))     # one zero; sign handled apart
    return [p[0] for p in pairs], [p[1] for p in pairs]


TABLE = None


def brute_force_bf16(d: float) -> int:
    """Nearest finite bf16 by search over every value; ties to the even
    pattern; beyond the largest finite value by half an ulp or more: inf."""
    global TABLE
    if TABLE is None:
        TABLE = _finite_bf16_table()
    vals, bits = TABLE
    if np.isinf(d):
        return 0x7F80 if d > 0 else 0xFF80
    x = Fraction(d)
    top, half_ulp = vals[-1], Fraction(2) ** 119     # 0x7F7F and half its ulp
    if x >= top + half_ulp:
        return 0x7F80
    if x <= -(top + half_ulp):
        return 0xFF80
    j = bisect.bisect_left(vals, x)
    cands = [k for k in (j - 1, j) if 0 <= k < len(vals)]
    best = min(abs(vals[k] - x) for k in cands)
    near = [k for k in cands if abs(vals[k] - x) == best]
    if len(near) == 2:
        near = [k for k in near if bits[k] % 2 == 0]
    b = bits[near[0]]
    if b == 0 and np.signbit(d):
        b = 0x8000
    return b


def test_double_to_bf16_matches_brute_force():
    rng = np.random.default_rng(21)
    xs = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 128, 3000)))
    # exact midpoints between neighbouring bf16 values, and one double ulp off them
    b = rng.integers(0, 0x7F7F, 1500).astype(np.uint32)
    lo = (b << 16).view(np.float32).astype(np.float64)
    hi = ((b + 1) << 16).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2                                   # exact in double
    xs += list(mid) + list(np.nextafter(mid, np.inf)) + list(np.nextafter(mid, -np.inf))
    xs += list(-mid[:300])
    xs += [0.0, -0.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -126,
           255 * 2.0 ** 120, 255.5 * 2.0 ** 120, np.nextafter(255.5 * 2.0 ** 120, 0), 1e300,
           -1e300, np.inf, -np.inf]
    xs = np.array(xs, dtype=np.float64)
    got = oracle.bf16_from_double(xs)
    want = np.array([brute_force_bf16(float(x)) for x in xs], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(xs[i], hex(got[i]), hex(want[i])) for i in bad[:5]]
    nan = oracle.bf16_from_double(np.array([np.nan, -np.nan]))
    assert all((h & 0x7F80) == 0x7F80 and (h & 0x40) for h in nan)


def test_double_to_bf16_is_one_rounding():
    """A double just above a bf16 tie whose fp32 rounding lands on the tie:
    one rounding goes up; rounding through fp32 first would go to even."""
    d = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert np.float32(d) == np.float32(1.0 + 2.0 ** -8)      # fp32 lands on the tie
    assert oracle.bf16_from_double(np.array([d]))[0] == 0x3F81


def test_bf16_moment_step_equals_fp32_step_when_moments_are_exact():
    """With beta1 = 1/2, beta2 = 3/4, m = v = 0 and gradients of few
    significant bits, m' = g/2 and v' = g^2/4 are exact in bf16, so the
    12-byte step must store the same m', v' (as bf16) and the same master
    and parameter as the 16-byte step (pinned separately): no term of the
    update may differ between the two layouts."""
    rng = np.random.default_rng(22)
    n, n_ranks = 4000, 4
    hp = dict(lr=1e-3, beta1=0.5, beta2=0.75, eps=1e-8, weight_decay=0.1)
    # every partial equal: the mean is the partial itself, exactly
    sign = rng.choice([-1.0, 1.0], n)
    g = (sign * (1 + rng.integers(0, 8, n) / 8.0) * np.exp2(rng.integers(-12, -6, n))).astype(np.float32)
    parts = [(f32_bits(g) >> 16).astype(np.uint16)] * n_ranks
    assert np.all((f32_bits(g) & 0xFFFF) == 0)
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    z32 = np.zeros(n, np.float32)
    z16 = np.zeros(n, np.uint16)
    for t in (1, 2, 3):
        a = oracle.shard_step(parts, th, z32, z32, oracle.hparams(t, **hp))
        b = oracle.shard_step_bf16m(parts, th, z16, z16, oracle.hparams(t, **hp))
        assert np.array_equal(f32_bits(a[0]), f32_bits(b[0]))
        assert np.array_equal(a[3], b[3])
        assert np.array_equal((f32_bits(a[1]) >> 16).astype(np.uint16), b[1])
        assert np.all((f32_bits(a[1]) & 0xFFFF) == 0) and np.all((f32_bits(a[2]) & 0xFFFF) == 0)
        assert np.array_equal((f32_bits(a[2]) >> 16).astype(np.uint16), b[2])


def test_bf16_moment_step_rounds_moments_to_nearest():
    """General inputs: the stored moments are the nearest-even bf16 of the
    fp32-state step's moments computed in double; master and parameter agree
    with the fp32-state step to within what the moment rounding moves them."""
    rng = np.random.default_rng(23)
    n, n_ranks = 20000, 8
    parts = [_random_bf16(rng, n, -16, -8) for _ in range(n_ranks)]
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m16 = oracle.bf16_from_double(rng.standard_normal(n) * 1e-4)
    v16 = oracle.bf16_from_double(rng.random(n) * 1e-8)
    m32 = (m16.astype(np.uint32) << 16).view(np.float32)
    v32 = (v16.astype(np.uint32) << 16).view(np.float32)
    hp = oracle.hparams(7)
    a = oracle.shard_step(parts, th, m32, v32, hp)
    b = oracle.shard_step_bf16m(parts, th, m16, v16, hp)
    # same double m', v'; a stores them in fp32, b in bf16: b == bf16(a) unless
    # the fp32 value sits exactly on a bf16 tie (then b may round differently)
    ra = oracle.bf16_round(a[1])
    tie = (f32_bits(a[1]) & 0xFFFF) == 0x8000
    assert np.array_equal(ra[~tie], b[1][~tie])
    assert np.array_equal(f32_bits(a[0]), f32_bits(b[0]))   # master: same double math


def test_twelve_byte_ledger():
    gold = json.load(open(os.path.join(GOLDEN, "ledger.json")))
    twelve = gold["bf16_moments_bytes_per_param"]
    assert ledger.BF16_MOMENTS_ADAM.total == twelve["value"] == 12
    cap = gold["zero_capacity_8xA100_80GB"]["ledger"]
    assert (ledger.BF16_MOMENTS_ADAM.param, ledger.BF16_MOMENTS_ADAM.grad,
            ledger.BF16_MOMENTS_ADAM.optimizer) == (cap["param"], cap["grad"], cap["optimizer"])
    assert ledger.shard_step_bytes_per_param(8, 2, 2) == 2 * 8 + 18


def test_bf16_moment_step_rounds_once():
    """A crafted element where rounding m' through fp32 first would differ:
    fp32 gradient 1 + 2^-7 + 2^-23 (one rank), m = 1.0, beta1 = 1/2 gives
    m' = 1 + 2^-8 + 2^-24 exactly in double.  In fp32 that is a tie that
    goes to 1 + 2^-8, itself a bf16 tie that goes to 1.0; the one rounding
    straight to bf16 gives 1 + 2^-7 (0x3F81)."""
    g = np.array([1.0 + 2.0 ** -7 + 2.0 ** -23], np.float32)
    m = np.array([0x3F80], np.uint16)
    v = np.array([0x3F80], np.uint16)
    th = np.array([0.5], np.float32)
    hp = oracle.hparams(1, lr=1e-3, beta1=0.5, beta2=0.5, eps=1e-8, weight_decay=0.0)
    _, m1, _, _ = oracle.shard_step_bf16m([g], th, m, v, hp)
    assert m1[0] == 0x3F81
