"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what it pins and the plausible mistake it would catch.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import ledger

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def ulp_diff(a, b):
    """Distance in fp32 ulps (monotone integer map of the bit patterns)."""
    def key(x):
        u = f32_bits(x).astype(np.int64)
        return np.where(u & 0x80000000, 0x80000000 - u, u)
    return np.abs(key(a) - key(b))


def bf16_bits_of(values):
    """Exact bf16 encodings of values known to be representable."""
    x = np.asarray(values, dtype=np.float32)
    u = f32_bits(x)
    assert np.all((u & 0xFFFF) == 0), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def bf16_to_f64(h):
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_round_exhaustive_against_torch():
    """Every fp32 bit pattern: the oracle's nearest-even rounding equals
    torch's float32->bfloat16 conversion (an independent library routine);
    NaNs stay NaN, quiet, with their sign.  Catches a wrong tie rule, a
    missing carry into the exponent, or overflow not going to inf."""
    chunk = 1 << 26
    for base in range(0, 1 << 32, chunk):
        u = np.arange(base, base + chunk, dtype=np.uint64).astype(np.uint32)
        x = u.view(np.float32)
        ours = oracle.bf16_round(x)
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(x)
        assert np.array_equal(ours[~nan], ref[~nan]), hex(base)
        on = ours[nan]
        assert np.all((on & 0x7F80) == 0x7F80) and np.all(on & 0x0040)
        assert np.array_equal(on >> 15, (u[nan] >> 31).astype(np.uint16))


def test_bf16_round_special_values():
    x = np.array([0.0, -0.0, np.inf, -np.inf, np.finfo(np.float32).max, 1.0 + 2.0 ** -8,
                  1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)
    got = oracle.bf16_round(x)
    # +0, -0, +inf, -inf, largest finite fp32 -> inf, tie to even (down),
    # tie to even (up), above half (up)
    assert list(got) == [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7F80, 0x3F80, 0x3F82, 0x3F81]


# ---------------------------------------------------------------- reduce

def _random_bf16(rng, n, lo_exp=-20, hi_exp=0):
    sign = rng.choice([-1.0, 1.0], n)
    mant = 1.0 + rng.integers(0, 128, n) / 128.0
    e = rng.integers(lo_exp, hi_exp + 1, n)
    return bf16_bits_of(sign * mant * np.exp2(e))


@pytest.mark.parametrize("n_ranks", [1, 2, 3, 4, 5, 7, 8, 16, 32, 64])
def test_reduce_equals_exact_rational_mean(n_ranks):
    """g = (1/N) sum_k g_k, the averaging identity.  With inputs spanning 20
    binades the double sum is exact, so the fp32 result must equal the
    exact rational mean rounded once to double and then to fp32.  Catches a
    dropped rank, a wrong divisor (N-1, or none), or a wrong element index."""
    rng = np.random.default_rng(100 + n_ranks)
    n = 1500
    parts = [_random_bf16(rng, n) for _ in range(n_ranks)]
    got = oracle.reduce(parts)
    vals = [bf16_to_f64(p) for p in parts]
    exp = np.empty(n, dtype=np.float32)
    for i in range(n):
        s = sum(Fraction(float(v[i])) for v in vals)
        exp[i] = np.float32(float(s / n_ranks))
    assert np.array_equal(f32_bits(got), f32_bits(exp))

    fparts = [(rng.standard_normal(n) * np.exp2(rng.integers(-20, 1, n))).astype(np.float32)
              for _ in range(n_ranks)]
    got = oracle.reduce(fparts)
    for i in range(n):
        s = sum(Fraction(float(p[i])) for p in fparts)
        exp[i] = np.float32(float(s / n_ranks))
    assert np.array_equal(f32_bits(got), f32_bits(exp))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gradient_averaging_identity_linear_model(dtype):
    """The pages' data-parallel identity: with a sample-additive loss, the
    mean of the N shards' gradients g_i = (N/b) sum_{x in shard i} grad l(x)
    equals the full-batch gradient (1/b) sum_x grad l(x).  Tiny linear model
    y = W x, squared error, small integer data: every quantity is a dyadic
    rational that fp32 and bf16 hold exactly, so equality is bitwise."""
    rng = np.random.default_rng(7)
    b, n_ranks, din, dout = 16, 4, 3, 2
    X = rng.integers(-2, 3, (b, din))
    Y = rng.integers(-2, 3, (b, dout))
    W = rng.integers(-2, 3, (dout, din))
    per_sample = [2 * np.outer(W @ x - y, x) for x, y in zip(X, Y)]   # grad of ||W x - y||^2
    full = [Fraction(int(sum(g.flat[j] for g in per_sample)), b) for j in range(dout * din)]
    shard = b // n_ranks
    parts = []
    for i in range(n_ranks):
        gi = [Fraction(n_ranks * int(sum(per_sample[s].flat[j]
                                         for s in range(i * shard, (i + 1) * shard))), b)
              for j in range(dout * din)]
        a = np.array([float(q) for q in gi], dtype=np.float32)
        assert all(Fraction(float(x)) == q for x, q in zip(a, gi))
        parts.append(bf16_bits_of(a) if dtype == "bf16" else a)
    got = oracle.reduce(parts)
    assert [Fraction(float(x)) for x in got] == full


def test_allreduce_equals_reduce_scatter_plus_all_gather():
    """all-reduce = reduce-scatter + all-gather: reducing each rank's own
    segment and concatenating the segments in rank order gives, bit for
    bit, the reduction of the whole vector.  Uses a total that N does not
    divide, so the short last shard is covered.  Catches a wrong shard
    offset or length in the geometry."""
    rng = np.random.default_rng(3)
    n_ranks, total = 4, 1003
    numels = [100, 1, 402, 500]
    assert sum(numels) == total
    parts = [_random_bf16(rng, total) for _ in range(n_ranks)]
    all_reduce = oracle.reduce(parts)
    pieces = []
    for r in range(n_ranks):
        seg, S = oracle.shard_segments(numels, n_ranks, r)
        lo, hi = min(r * S, total), min((r + 1) * S, total)
        assert int(seg[:, 3].sum()) == hi - lo
        pieces.append(oracle.reduce([p[lo:hi] for p in parts]))
    assert S == 251
    assert np.array_equal(f32_bits(np.concatenate(pieces)), f32_bits(all_reduce))


def test_reduce_propagates_nonfinite_per_element():
    rng = np.random.default_rng(4)
    parts = [_random_bf16(rng, 64) for _ in range(4)]
    parts[2][5] = 0x7FC0          # NaN
    parts[1][9] = 0x7F80          # +inf
    parts[3][9] = 0xFF80          # -inf -> inf + -inf = NaN
    parts[0][11] = 0x7F80         # +inf alone
    g = oracle.reduce(parts)
    assert np.isnan(g[5]) and np.isnan(g[9]) and g[11] == np.inf
    others = np.ones(64, bool)
    others[[5, 9, 11]] = False
    assert np.all(np.isfinite(g[others]))


# ---------------------------------------------------------------- AdamW

HP_VARIANTS = [
    dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1),
    dict(lr=3e-4, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.0),
    dict(lr=1e-2, beta1=0.0, beta2=0.5, eps=1e-3, weight_decay=0.01),
]


@pytest.mark.parametrize("hp", HP_VARIANTS)
def test_adamw_matches_torch_adamw_float64(hp):
    """Against torch.optim.AdamW run in float64 (an independent library
    implementation: lerp for m, addcmul for v, step size lr/(1-b1^t),
    denominator sqrt(v)/sqrt(1-b2^t) + eps, decay param *= 1 - lr*wd).
    Each step starts both from the oracle's fp32 state; torch's double
    result rounded to fp32 must be within 1 ulp.  Equality is not always
    reached: with decimal betas the exact m' often sits within a double ulp
    of an fp32 rounding midpoint, and torch's lerp form rounds differently
    from the plain form there (about 0.4% of elements).
    Catches a sign error, a dropped or misplaced bias correction, eps
    inside the root, coupled weight decay, or swapped betas."""
    rng = np.random.default_rng(11)
    n = 20000
    theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, 13):
        g = (rng.standard_normal(n) * 1e-3 * np.where(rng.random(n) < 0.01, 100, 1)).astype(np.float32)
        g[:7] = 0.0
        p = torch.tensor(theta.astype(np.float64))
        p.grad = torch.tensor(g.astype(np.float64))
        opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                                weight_decay=hp["weight_decay"], foreach=False)
        opt.state[p] = {"step": torch.tensor(float(t - 1), dtype=torch.float64),
                        "exp_avg": torch.tensor(m.astype(np.float64)),
                        "exp_avg_sq": torch.tensor(v.astype(np.float64))}
        opt.step()
        ref = [p.numpy().astype(np.float32), opt.state[p]["exp_avg"].numpy().astype(np.float32),
               opt.state[p]["exp_avg_sq"].numpy().astype(np.float32)]
        theta, m, v = oracle.adamw(g, theta, m, v, oracle.hparams(t, **hp))
        for ours, want in zip((theta, m, v), ref):
            d = ulp_diff(ours, want)
            assert d.max() <= 1, (t, d.max())
            assert (d == 0).mean() > 0.99


def test_adamw_step1_closed_form():
    """Step 1 from m = v = 0: the bias corrections cancel (1-b1) and (1-b2),
    so mhat = g and vhat = g^2 and theta1 = theta0 (1 - lr wd) - lr g/(|g|+eps):
    the update is lr * sign(g) plus the decay term.  Without bias correction
    the step would be ~3.16 lr."""
    rng = np.random.default_rng(12)
    n = 10000
    hp = HP_VARIANTS[0]
    theta0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    th, m, v = oracle.adamw(g, theta0, np.zeros(n, np.float32), np.zeros(n, np.float32),
                            oracle.hparams(1, **hp))
    g64 = g.astype(np.float64)
    closed = theta0.astype(np.float64) * (1 - hp["lr"] * hp["weight_decay"]) \
        - hp["lr"] * np.sign(g64) * (np.abs(g64) / (np.abs(g64) + hp["eps"]))
    assert ulp_diff(th, closed.astype(np.float32)).max() <= 1
    step = theta0.astype(np.float64) * (1 - hp["lr"] * hp["weight_decay"]) - th
    big = np.abs(g64) > 1e-4          # |g| >> eps: |g| / (|g| + eps) > 0.9999
    assert big.mean() > 0.9
    assert np.allclose(np.abs(step[big]), hp["lr"], rtol=1e-3)
    assert np.all(np.sign(step) == np.sign(g))


def test_adamw_zero_gradient_decay_only():
    """g = 0 from m = v = 0: the update term is 0/(0+eps) = 0, so only the
    decoupled decay acts: theta_t = theta_0 (1 - lr wd)^t, m and v stay 0.
    With nonzero m0, v0 and g = 0: m_t = b1^t m0, v_t = b2^t v0."""
    rng = np.random.default_rng(13)
    n, T = 5000, 10
    hp = HP_VARIANTS[0]
    theta0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    th, m, v = theta0, np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, T + 1):
        th, m, v = oracle.adamw(np.zeros(n, np.float32), th, m, v, oracle.hparams(t, **hp))
        want = (theta0.astype(np.float64) * (1 - hp["lr"] * hp["weight_decay"]) ** t).astype(np.float32)
        assert ulp_diff(th, want).max() <= t
        assert not m.any() and not v.any()

    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-7 + 1e-9).astype(np.float32)
    m, v = m0, v0
    for t in range(1, T + 1):
        _, m, v = oracle.adamw(np.zeros(n, np.float32), theta0, m, v, oracle.hparams(t + 5, **hp))
        assert ulp_diff(m, (m0 * hp["beta1"] ** t).astype(np.float32)).max() <= t
        assert ulp_diff(v, (v0 * hp["beta2"] ** t).astype(np.float32)).max() <= t


def test_adamw_zero_betas_reduce_to_normalised_step():
    """b1 = b2 = 0, wd = 0: m' = g, v' = g^2, no bias correction left
    (1 - 0^t = 1), so theta' = theta - lr g / (|g| + eps) at every t."""
    rng = np.random.default_rng(14)
    n = 5000
    hp = dict(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.0)
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n)).astype(np.float32)     # must be ignored
    v = (rng.random(n)).astype(np.float32)
    for t in (1, 2, 7):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        new, m, v = oracle.adamw(g, th, m, v, oracle.hparams(t, **hp))
        g64 = g.astype(np.float64)
        want = th.astype(np.float64) - hp["lr"] * g64 / (np.abs(g64) + hp["eps"])
        assert ulp_diff(new, want.astype(np.float32)).max() <= 1
        th = new


def test_adamw_constant_gradient_unbiased_moments():
    """A constant gradient c from m = v = 0: m_t = (1 - b1^t) c and
    v_t = (1 - b2^t) c^2, so the bias-corrected moments are exactly c and
    c^2 at every step and each update is lr c / (|c| + eps).  Catches a
    bias correction that uses t-1 or t+1, or skips one of the moments."""
    rng = np.random.default_rng(15)
    n = 5000
    hp = HP_VARIANTS[0]
    c = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    c64 = c.astype(np.float64)
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, 16):
        new, m, v = oracle.adamw(c, th, m, v, oracle.hparams(t, **hp))
        want = th.astype(np.float64) * (1 - hp["lr"] * hp["weight_decay"]) \
            - hp["lr"] * c64 / (np.abs(c64) + hp["eps"])
        # m and v are stored in fp32, so mhat and vhat carry a relative
        # error of at most ~t * 2^-24 each; the update (size lr) inherits it.
        tol = hp["lr"] * t * 2.0 ** -21 + np.spacing(np.abs(want).astype(np.float32))
        assert np.all(np.abs(new - want) <= tol), t
        assert ulp_diff(m, ((1 - hp["beta1"] ** t) * c64).astype(np.float32)).max() <= t
        th = new


# ---------------------------------------------------------------- shards

def _brute_force_owner(numels, n_ranks):
    total = sum(numels)
    S = -(-total // n_ranks)
    owner = np.arange(total) // S
    tensor = np.repeat(np.arange(len(numels)), numels)
    off = np.arange(total) - np.repeat(np.cumsum([0] + numels[:-1]), numels)
    return owner, tensor, off, S


@pytest.mark.parametrize("seed", range(6))
def test_shard_segments_brute_force(seed):
    """Each rank's pieces (tensor, offset in tensor, offset in shard, len)
    agree with a per-element brute-force owner map, and the pieces of all
    ranks cover every (tensor, element) exactly once."""
    rng = np.random.default_rng(seed)
    numels = [int(x) for x in rng.integers(1, 300, rng.integers(1, 12))]
    n_ranks = int(rng.integers(1, 9))
    owner, tensor, off, S_bf = _brute_force_owner(numels, n_ranks)
    seen = np.zeros(sum(numels), np.int64)
    starts = np.cumsum([0] + numels[:-1])
    for r in range(n_ranks):
        seg, S = oracle.shard_segments(numels, n_ranks, r)
        assert S == S_bf
        shard_pos = 0
        for t, toff, soff, ln in seg:
            assert soff == shard_pos
            flat = starts[t] + toff + np.arange(ln)
            assert np.all(owner[flat] == r) and np.all(tensor[flat] == t)
            assert np.array_equal(off[flat], toff + np.arange(ln))
            seen[flat] += 1
            shard_pos += ln
        assert shard_pos == np.sum(owner == r)
    assert np.all(seen == 1)


def test_sharded_update_equals_replicated_update():
    """ZeRO-1 is still data parallelism: every rank updating only its own
    segment with its own state gives, bit for bit, the same parameters,
    m and v as one replicated AdamW step on the all-reduced gradient."""
    rng = np.random.default_rng(16)
    n_ranks, total, T = 4, 4099, 5
    theta = (rng.standard_normal(total) * 0.02).astype(np.float32)
    full = [theta.copy(), np.zeros(total, np.float32), np.zeros(total, np.float32)]
    shards = [a.copy() for a in full]
    S = -(-total // n_ranks)
    for t in range(1, T + 1):
        parts = [_random_bf16(rng, total, -16, -8) for _ in range(n_ranks)]
        hp = oracle.hparams(t)
        g = oracle.reduce(parts)
        full[0], full[1], full[2] = oracle.adamw(g, *full, hp)
        full_param = oracle.bf16_round(full[0])
        params = []
        for r in range(n_ranks):
            lo, hi = r * S, min((r + 1) * S, total)
            th, m, v, p = oracle.shard_step([x[lo:hi] for x in parts], shards[0][lo:hi],
                                            shards[1][lo:hi], shards[2][lo:hi], hp)
            shards[0][lo:hi], shards[1][lo:hi], shards[2][lo:hi] = th, m, v
            params.append(p)
        for a, b in zip(full, shards):
            assert np.array_equal(f32_bits(a), f32_bits(b))
        assert np.array_equal(np.concatenate(params), full_param)


# ---------------------------------------------------------------- ledger

def test_ledger_against_the_pages():
    gold = json.load(open(os.path.join(GOLDEN, "ledger.json")))
    mp = gold["mixed_precision_adam_bytes_per_param"]
    assert ledger.MIXED_PRECISION_ADAM.total == mp["value"] == 16
    assert sum(ledger.STATE_ELEMENT_BYTES.values()) == 16
    ex = gold["seven_billion_replicated"]
    assert ledger.MIXED_PRECISION_ADAM.per_rank_bytes_per_param(0, 8) * ex["params"] == ex["bytes"]

    cap = gold["zero_capacity_8xA100_80GB"]
    L = ledger.Ledger(**cap["ledger"])
    for stage, want in cap["max_params_billion"].items():
        got = L.max_params(cap["hbm_gb"] * 1e9, int(stage), cap["n_ranks"]) / 1e9
        assert abs(got - want) <= 0.01, stage

    fs = gold["fsdp_100b_over_80_gpus"]
    L = ledger.Ledger(**fs["ledger"])
    assert L.total * fs["params"] == fs["total_bytes"]
    assert L.per_rank_bytes_per_param(3, fs["n_ranks"]) * fs["params"] == pytest.approx(fs["per_rank_bytes"])


def test_shard_step_byte_model():
    """Bytes the fused step moves per shard element: 2N + 26 for bf16
    partials, 4N + 26 for fp32 partials."""
    for n in (1, 4, 8, 16, 32, 64):
        assert ledger.shard_step_bytes_per_param(n) == 2 * n + 26
        assert ledger.shard_step_bytes_per_param(n, 4) == 4 * n + 26
        # run as three passes: + the fp32 gradient written and read back (8)
        # and the master read a second time for the parameter write (4)
        assert ledger.unfused_step_bytes_per_param(n) == 2 * n + 38
        assert ledger.unfused_step_bytes_per_param(n, 4) == ledger.shard_step_bytes_per_param(n, 4) + 12


def test_power_of_two_mean_is_a_scaling():
    """The mean's divisor, for a power-of-two count (N, or N times the
    micro-batches), is an exact scaling in double: s / 2^k equals s * 2^-k
    bit for bit at every magnitude a sum of bf16 or fp32 values can take, so
    a kernel may multiply where the definition divides (reading of the
    mean, §3 #5).  For other counts the two differ, so the division stays."""
    rng = np.random.default_rng(11)
    s = np.ldexp(rng.uniform(1.0, 2.0, 200_000) * rng.choice([-1.0, 1.0], 200_000),
                 rng.integers(-160, 140, 200_000))
    for k in range(0, 41):
        n = float(2 ** k)
        assert np.array_equal((s / n).view(np.uint64), (s * (1.0 / n)).view(np.uint64)), k
        with np.errstate(over="ignore"):              # sums past fp32's range round to inf
            assert np.array_equal((s / n).astype(np.float32).view(np.uint32),
                                  (s * (1.0 / n)).astype(np.float32).view(np.uint32)), k
    differs = [n for n in (3, 5, 6, 7, 12, 24, 48) if not np.array_equal(s / n, s * (1.0 / n))]
    assert differs == [3, 5, 6, 7, 12, 24, 48]
