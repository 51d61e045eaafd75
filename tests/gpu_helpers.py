"""Shared pieces of the GPU parity tests: tolerance checks and host-side
expected values from the CPU oracle (never from the GPU path)."""
import sys

import numpy as np

import oracle
import synth
from synth import workloads as W

# Tolerances of the method: fp32 state within 1e-6 relative (absolute floor
# 1e-12 near zero), bf16 parameters within 1 ulp.  Bitwise equality is the
# design target and is asserted separately.
REL_TOL = 1e-6
ABS_FLOOR = 1e-12


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f32_bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def assert_f32_close(got, want, what):
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    both_nan = np.isnan(g) & np.isnan(w)
    with np.errstate(invalid="ignore"):
        ok = both_nan | (g == w) | (np.abs(g - w) <= np.maximum(REL_TOL * np.abs(w), ABS_FLOOR))
    if not ok.all():
        i = int(np.nonzero(~ok)[0][0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance; "
                             f"first at {i}: got {got[i]!r} want {want[i]!r}")


def assert_bf16_close(got, want, what):
    def key(h):
        u = h.astype(np.int64)
        return np.where(u & 0x8000, 0x8000 - u, u)
    g = np.asarray(got, np.uint16)
    w = np.asarray(want, np.uint16)
    nan_g = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
    nan_w = ((w & 0x7F80) == 0x7F80) & ((w & 0x7F) != 0)
    ok = (nan_g & nan_w) | (~nan_g & ~nan_w & (np.abs(key(g) - key(w)) <= 1))
    if not ok.all():
        i = int(np.nonzero(~ok)[0][0])
        raise AssertionError(f"{what}: {int((~ok).sum())} bf16 values off by more than 1 ulp; "
                             f"first at {i}: got {g[i]:#06x} want {w[i]:#06x}")


def _is_nan_bits(b):
    if b.dtype == np.uint32:
        return (b & 0x7FFFFFFF) > 0x7F800000
    return (b & 0x7FFF) > 0x7F80


def assert_bitwise(got, want, what, strict_nan=False):
    """Equal bit patterns, except that any NaN matches any NaN: which
    operand's payload an IEEE operation propagates is left to the
    implementation, and x86 and the GPU choose differently.  strict_nan
    compares NaN patterns too (for pure bit manipulations such as rounding)."""
    g = np.ascontiguousarray(got)
    w = np.ascontiguousarray(want)
    gb = g.view(np.uint32) if g.dtype in (np.float32, np.uint32) else g.view(np.uint16)
    wb = w.view(np.uint32) if w.dtype in (np.float32, np.uint32) else w.view(np.uint16)
    bad = gb != wb
    if not strict_nan:
        bad &= ~(_is_nan_bits(gb) & _is_nan_bits(wb))
    if bad.any():
        i = int(np.nonzero(bad)[0][0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} not bitwise equal; "
                             f"first at {i}: got {g[i]!r} want {w[i]!r}")


def check_state(got, want, what):
    """Tolerance first (the acceptance bar), then bit equality."""
    for name, g, w in zip(("master", "m", "v"), got[:3], want[:3]):
        assert_f32_close(g, w, f"{what} {name}")
    if len(got) > 3:
        assert_bf16_close(got[3], want[3], f"{what} param")
    for name, g, w in zip(("master", "m", "v", "param"), got, want):
        assert_bitwise(g, w, f"{what} {name}")


def host_partials(w: W.Workload, t: int, flat_idx: np.ndarray):
    """Rank partials of step t at global flat indices (host generator)."""
    parts = []
    zero = W.zero_mask(w, flat_idx)
    for k in range(w.n_ranks):
        p = synth.gather(w.gdt, w.seed, synth.stream_id(synth.KIND_GRAD, k, t), flat_idx,
                         w.sigma_grad, synth.stream_id(synth.KIND_OUTLIER, k, t),
                         w.outlier_frac, w.outlier_mult)
        p[zero] = 0
        parts.append(p)
    return parts


def host_master(w: W.Workload, flat_idx: np.ndarray):
    return synth.gather("f32", w.seed, synth.stream_id(synth.KIND_MASTER), flat_idx,
                        w.sigma_master)


def oracle_warm_prefix(w: W.Workload, lo: int):
    """The oracle's own run of the warm-start prefix: warm_steps steps on the
    first warm_prefix shard elements from m = v = 0."""
    P = w.warm_prefix
    idx = lo + np.arange(P, dtype=np.int64)
    th = host_master(w, idx)
    m = np.zeros(P, np.float32)
    v = np.zeros(P, np.float32)
    for t in range(1, w.warm_steps + 1):
        parts = host_partials(w, t, idx)
        oracle.shard_step(parts, th, m, v, oracle.hparams(t, **w.hparams()), in_place=True)
    return th, m, v


def sample_indices(table: np.ndarray, n: int, seed: int, n_random: int = 1 << 16,
                   edge: int = 8):
    """Shard indices to check at full size: every chunk boundary +-edge, the
    first and last 4096 elements, and n_random hashed indices."""
    rng = np.random.default_rng(seed)
    parts = [rng.integers(0, n, n_random), np.arange(min(4096, n)),
             np.arange(max(0, n - 4096), n)]
    b = np.concatenate([table["shard_off"], table["shard_off"] + table["len"]])
    parts.append((b[:, None] + np.arange(-edge, edge)[None, :]).ravel())
    idx = np.unique(np.concatenate(parts))
    return idx[(idx >= 0) & (idx < n)].astype(np.int64)
