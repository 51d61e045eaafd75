"""Every compiled variant of the fused kernels against the oracle, bitwise.

The dispatchers compile each step for N in {1, 2, 4, 8, 16, 32, 64} (plus a
run-time N kernel) and both gradient dtypes; the extended step and the
accumulation pass also compile the two-level fold for groups of 4 and 8.
Each case below takes one (dtype, N), a small shard that is the short last
one, and runs every fused entry point on it: the 16-byte step, the 12-byte
step, the pure-bf16 Kahan step, and the extended step with every group size
the dispatcher distinguishes for that N (flat, compiled 4, compiled 8, a
group size folded at run time), each with one accumulated micro-batch.

The 16-byte, 12-byte and extended steps also compile two occupancies
each: launches of at most ZERO_SMALL_LAUNCH_CHUNKS chunks (the 12-byte
step: ZERO_SMALL_LAUNCH_CHUNKS_12B) run more waves per SIMD than longer
ones.  The small cases take the first; a second case per (dtype, N) builds
a table just over the larger limit to take the other, for the
launch-argument and scheduled forms and every fold of the extended step.
"""
import numpy as np
import pytest

import oracle
from synth import workloads as W
from gpu_helpers import assert_bitwise, host_master, host_partials, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
RANKS = [1, 2, 4, 8, 16, 32, 64, 7]      # 7: the run-time-N kernels


@pytest.fixture(scope="module")
def zs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sharded_optimizer_step_shard_amd as m
    return m


def dev(x):
    a = np.ascontiguousarray(x)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def groups_for(n):
    """Group sizes that reach each fold the dispatchers compile for N = n."""
    ks = [0]                                   # flat
    if n % 4 == 0 and n > 4:
        ks.append(4)
    if n % 8 == 0 and n > 8:
        ks.append(8)
    if n % 2 == 0 and n > 2:
        ks.append(2)                           # folded at run time
    return ks


@pytest.mark.parametrize("gdt", ["bf16", "f32"])
@pytest.mark.parametrize("n_ranks", RANKS)
def test_every_compiled_variant(zs, gdt, n_ranks):
    total = n_ranks * 2_083 + 5                # rank N-1 holds a short last shard
    w = W.Workload("variants", 96, [total], n_ranks, gdt, 1e-3)
    rank = n_ranks - 1
    lo, hi = w.shard_range(rank)
    n = hi - lo
    idx = np.arange(lo, hi, dtype=np.int64)
    th0 = host_master(w, idx)
    rng = np.random.default_rng(n_ranks)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-8).astype(np.float32)
    full = torch.full((total,), -1, dtype=torch.int16, device="cuda")
    table, _ = zs.zero_build_chunks([total], n_ranks, rank, slot_dst=full.data_ptr() + 2 * lo,
                                    max_chunk=448)
    d_table, nc = zs.chunks_to_device(table), len(table)
    steps = (4, 5)
    parts_h = {t: host_partials(w, t, idx) for t in steps}
    parts_d = {t: [dev(p) for p in parts_h[t]] for t in steps}
    tag = f"N={n_ranks} {gdt}"

    say(f"case: variants {tag}: 16-byte step")
    master, m, v = dev(th0), dev(m0), dev(v0)
    th, mm, vv = th0, m0, v0
    for t in steps:
        zs.zero_shard_step(parts_d[t], master, m, v, n, d_table, nc, zs.hparams(t, **HP))
        th, mm, vv, p = oracle.shard_step(parts_h[t], th, mm, vv, oracle.hparams(t, **HP))
    for got, want, what in ((host(master), th, "master"), (host(m), mm, "m"), (host(v), vv, "v"),
                            (host(full)[lo:hi], p, "param")):
        assert_bitwise(got, want, f"{tag} 16-byte {what}")

    say(f"case: variants {tag}: 12-byte step")
    m16, v16 = oracle.bf16_from_double(m0), oracle.bf16_from_double(v0)
    master, m, v = dev(th0), dev(m16), dev(v16)
    th, mm, vv = th0, m16, v16
    for t in steps:
        zs.zero_shard_step_bf16_moments(parts_d[t], master, m, v, n, d_table, nc, zs.hparams(t, **HP))
        th, mm, vv, p = oracle.shard_step_bf16m(parts_h[t], th, mm, vv, oracle.hparams(t, **HP))
    for got, want, what in ((host(master), th, "master"), (host(m), mm, "m"), (host(v), vv, "v"),
                            (host(full)[lo:hi], p, "param")):
        assert_bitwise(got, want, f"{tag} 12-byte {what}")

    say(f"case: variants {tag}: pure-bf16 Kahan step")
    th16 = oracle.bf16_round(th0)
    c16 = oracle.bf16_from_double(rng.standard_normal(n) * 1e-6)
    full[lo:hi] = dev(th16)
    comp, m, v = dev(c16), dev(m16), dev(v16)
    th, cc, mm, vv = th16, c16, m16, v16
    for t in steps:
        zs.zero_shard_step_kahan(parts_d[t], comp, m, v, n, d_table, nc, zs.hparams(t, **HP))
        th, cc, mm, vv = oracle.shard_step_kahan(parts_h[t], th, cc, mm, vv, oracle.hparams(t, **HP))
    for got, want, what in ((host(full)[lo:hi], th, "param"), (host(comp), cc, "comp"),
                            (host(m), mm, "m"), (host(v), vv, "v")):
        assert_bitwise(got, want, f"{tag} Kahan {what}")

    for k in groups_for(n_ranks):
        say(f"case: variants {tag}: extended step, group {k or 'flat'}, 2 micro-batches")
        acc = torch.empty(max(n, 1), dtype=torch.float32, device="cuda")
        master, m, v = dev(th0), dev(m0), dev(v0)
        zs.zero_accumulate_shard(parts_d[4], n, acc, reset=True, group=k)
        acc_h = oracle.accumulate(parts_h[4], None, group=k or None)
        assert_bitwise(host(acc)[:n], acc_h, f"{tag} accumulator group {k}")
        zs.zero_shard_step_ex(parts_d[5], master, m, v, n, d_table, nc, zs.hparams(5, **HP),
                              group=k, micro_batches=2, acc=acc)
        th, mm, vv, p = oracle.shard_step_ex(parts_h[5], th0, m0, v0, oracle.hparams(5, **HP),
                                             group=k or None, acc=acc_h, micro_batches=2)
        for got, want, what in ((host(master), th, "master"), (host(m), mm, "m"),
                                (host(v), vv, "v"), (host(full)[lo:hi], p, "param")):
            assert_bitwise(got, want, f"{tag} extended group {k} {what}")


@pytest.mark.parametrize("gdt", ["bf16", "f32"])
@pytest.mark.parametrize("n_ranks", RANKS)
def test_large_launch_variants_over_a_long_table(zs, gdt, n_ranks):
    limit = max(zs.ZERO_SMALL_LAUNCH_CHUNKS, zs.ZERO_SMALL_LAUNCH_CHUNKS_12B)
    n = limit * 64 + 777                             # chunks of 64: just over both limits
    w = W.Workload("variants-long", 97, [n * n_ranks], n_ranks, gdt, 1e-3)
    lo, hi = w.shard_range(0)
    assert hi - lo == n
    idx = np.arange(lo, hi, dtype=np.int64)
    slot = torch.full((n,), -1, dtype=torch.int16, device="cuda")
    table, _ = zs.zero_build_chunks([n * n_ranks], n_ranks, 0, slot_dst=slot, max_chunk=64)
    assert len(table) > limit
    d_table, nc = zs.chunks_to_device(table), len(table)
    t = 3
    parts_h = host_partials(w, t, idx)
    parts = [dev(p) for p in parts_h]
    th0 = host_master(w, idx)
    rng = np.random.default_rng(n_ranks)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-8).astype(np.float32)
    th, mm, vv, p = oracle.shard_step(parts_h, th0, m0, v0, oracle.hparams(t, **HP))
    tag = f"N={n_ranks} {gdt}, {nc} chunks"
    say(f"case: variants {tag}: 16-byte step, large-launch occupancy")
    master, m, v = dev(th0), dev(m0), dev(v0)
    zs.zero_shard_step(parts, master, m, v, n, d_table, nc, zs.hparams(t, **HP))
    for got, want, what in ((host(master), th, "master"), (host(m), mm, "m"), (host(v), vv, "v"),
                            (host(slot), p, "param")):
        assert_bitwise(got, want, f"{tag} {what}")
    say(f"case: variants {tag}: scheduled 16-byte step, large-launch occupancy")
    consts = torch.from_numpy(zs.zero_make_step_consts([zs.hparams(t, **HP)]).view(np.uint8)).cuda()
    index = torch.zeros(1, dtype=torch.int64, device="cuda")
    slot.fill_(-1)
    master, m, v = dev(th0), dev(m0), dev(v0)
    zs.zero_shard_step_scheduled(parts, master, m, v, n, d_table, nc, consts, 1, index)
    for got, want, what in ((host(master), th, "master"), (host(m), mm, "m"), (host(v), vv, "v"),
                            (host(slot), p, "param")):
        assert_bitwise(got, want, f"{tag} scheduled {what}")
    say(f"case: variants {tag}: 12-byte step and its scheduled form, large-launch occupancy")
    m16, v16 = oracle.bf16_from_double(m0), oracle.bf16_from_double(v0)
    th, mm, vv, p = oracle.shard_step_bf16m(parts_h, th0, m16, v16, oracle.hparams(t, **HP))
    for scheduled in (False, True):
        slot.fill_(-1)
        master, m, v = dev(th0), dev(m16), dev(v16)
        if scheduled:
            index.zero_()
            zs.zero_shard_step_bf16_moments_scheduled(parts, master, m, v, n, d_table, nc, consts, 1,
                                                      index)
        else:
            zs.zero_shard_step_bf16_moments(parts, master, m, v, n, d_table, nc, zs.hparams(t, **HP))
        for got, want, what in ((host(master), th, "master"), (host(m), mm, "m"),
                                (host(v), vv, "v"), (host(slot), p, "param")):
            assert_bitwise(got, want, f"{tag} 12-byte{' scheduled' if scheduled else ''} {what}")
    for k in groups_for(n_ranks):
        say(f"case: variants {tag}: extended step, group {k or 'flat'}, large-launch occupancy")
        acc = torch.empty(n, dtype=torch.float32, device="cuda")
        prev_h = [x[::-1].copy() for x in parts_h]            # an earlier micro-batch
        zs.zero_accumulate_shard([dev(x) for x in prev_h], n, acc, reset=True, group=k)
        acc_h = oracle.accumulate(prev_h, None, group=k or None)
        slot.fill_(-1)
        master, m, v = dev(th0), dev(m0), dev(v0)
        zs.zero_shard_step_ex(parts, master, m, v, n, d_table, nc, zs.hparams(t, **HP), group=k,
                              micro_batches=2, acc=acc)
        th, mm, vv, p = oracle.shard_step_ex(parts_h, th0, m0, v0, oracle.hparams(t, **HP),
                                             group=k or None, acc=acc_h, micro_batches=2)
        for got, want, what in ((host(master), th, "master"), (host(m), mm, "m"),
                                (host(v), vv, "v"), (host(slot), p, "param")):
            assert_bitwise(got, want, f"{tag} extended group {k} {what}")
