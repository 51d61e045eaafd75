"""Seeded random cases: the fused steps against the oracle, bitwise, over
shapes, rank counts, dtypes, destinations, chunk lengths, hyper-parameters
and value ranges that the hand-written cases do not pick.

Each seed draws one case: a tensor list (1 to 12 tensors, sizes from 1 to
200,000, many odd), a rank count (1 to 64) and rank, the gradient dtype,
per-tensor or slot destinations, a chunk length, a state layout (16-byte,
12-byte, pure bf16, the extended reduce with a group size and an
accumulated micro-batch, or the scheduled 16-byte step), hyper-parameters
(beta1, beta2 and weight decay including 0, eps including 0, t up to 10^6)
and the scale of the gradients (1e-6 to 1e2, with exact zeros, and a few
infinities and NaNs in some cases).  Elements of the parameter buffers
outside this rank's shard must keep their sentinel.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import assert_bitwise, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LAYOUTS = ("fp32", "bf16-moments", "bf16-kahan", "extended", "scheduled")


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


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    n_t = int(rng.integers(1, 13))
    numels = [int(x) for x in np.exp(rng.uniform(0, np.log(200_000), n_t)).astype(np.int64) + 1]
    if rng.random() < 0.3:
        numels[int(rng.integers(0, n_t))] = 1
    n_ranks = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 24, 32, 48, 64]))
    case = dict(
        numels=numels, n_ranks=n_ranks, rank=int(rng.integers(0, n_ranks)),
        gdt=str(rng.choice(["bf16", "f32"])), slot=bool(rng.random() < 0.5),
        max_chunk=64 * int(rng.integers(1, 129)), layout=LAYOUTS[seed % len(LAYOUTS)],
        t=int(rng.choice([1, 2, 3, 10, 1000, 10**6])),
        hp=dict(lr=float(10 ** rng.uniform(-5, -2)),
                beta1=float(rng.choice([0.0, 0.5, 0.9, 0.99])),
                beta2=float(rng.choice([0.0, 0.9, 0.999, 0.9999])),
                eps=float(rng.choice([0.0, 1e-12, 1e-8, 1e-3])),
                weight_decay=float(rng.choice([0.0, 0.01, 0.1, 1.0]))),
        scale=float(10 ** rng.uniform(-6, 2)), zeros=float(rng.random() * 0.2),
        specials=bool(rng.random() < 0.2), seed=seed)
    divisors = [k for k in range(1, n_ranks + 1) if n_ranks % k == 0]
    case["group"] = int(rng.choice(divisors))
    return case


def make_values(rng, c, n):
    parts = []
    for _ in range(c["n_ranks"]):
        x = rng.standard_normal(n) * c["scale"]
        x[rng.random(n) < c["zeros"]] = 0.0
        if c["specials"] and n > 0:
            k = max(1, n // 5000)
            x[rng.integers(0, n, k)] = rng.choice([np.inf, -np.inf, np.nan], k)
        x = x.astype(np.float32)
        parts.append(oracle.bf16_round(x) if c["gdt"] == "bf16" else x)
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * c["scale"] * 0.1).astype(np.float32)
    v = (rng.random(n) * (c["scale"] ** 2) * 0.01).astype(np.float32)
    return parts, th, m, v


@pytest.mark.parametrize("seed", range(50))
def test_random_case(zs, seed):
    c = draw(seed)
    total = sum(c["numels"])
    seg, S = oracle.shard_segments(c["numels"], c["n_ranks"], c["rank"])
    lo = min(c["rank"] * S, total)
    n = min(lo + S, total) - lo
    say(f"case: random seed {seed}: {c['layout']} N={c['n_ranks']} rank {c['rank']} {c['gdt']} "
        f"{len(c['numels'])} tensors, shard {n} of {total}, "
        f"{'slot' if c['slot'] else 'tensors'}, chunk {c['max_chunk']}, t={c['t']}, hp={c['hp']}, "
        f"scale {c['scale']:.2g}, specials {c['specials']}, group {c['group']}")
    rng = np.random.default_rng(seed)
    parts_h, th0, m0, v0 = make_values(rng, c, n)
    hp_h, hp_d = oracle.hparams(c["t"], **c["hp"]), zs.hparams(c["t"], **c["hp"])
    parts = [dev(p) for p in parts_h]
    if c["slot"]:
        flat = torch.full((total,), -1, dtype=torch.int16, device="cuda")
        table, S2 = zs.zero_build_chunks(c["numels"], c["n_ranks"], c["rank"],
                                         slot_dst=flat.data_ptr() + 2 * lo, max_chunk=c["max_chunk"])
        read_params = lambda: host(flat)                                    # noqa: E731
    else:
        bufs = [torch.full((k,), -1, dtype=torch.int16, device="cuda") for k in c["numels"]]
        table, S2 = zs.zero_build_chunks(c["numels"], c["n_ranks"], c["rank"], tensor_dst=bufs,
                                         max_chunk=c["max_chunk"])
        read_params = lambda: np.concatenate([host(b) for b in bufs])    # noqa: E731
    assert S2 == S
    zs.zero_check_chunks(table, n, parts)     # every built table passes the host check
    d_table, nc = zs.chunks_to_device(table), len(table)
    layout = c["layout"]

    if layout == "bf16-kahan":
        th16 = oracle.bf16_round(th0)
        c16 = oracle.bf16_from_double(rng.standard_normal(n) * 1e-6)
        m16, v16 = oracle.bf16_from_double(m0), oracle.bf16_from_double(v0)
        if c["slot"]:
            flat[lo:lo + n] = dev(th16)
        else:
            off = 0
            for b in bufs:
                a_, e_ = max(off, lo), min(off + b.numel(), lo + n)
                if a_ < e_:
                    b[a_ - off:e_ - off] = dev(th16[a_ - lo:e_ - lo])
                off += b.numel()
        comp, m, v = dev(c16), dev(m16), dev(v16)
        zs.zero_shard_step_kahan(parts, comp, m, v, n, d_table, nc, hp_d)
        th, cc, mm, vv = oracle.shard_step_kahan(parts_h, th16, c16, m16, v16, hp_h)
        got = [read_params()[lo:lo + n], host(comp), host(m), host(v)]
        want = [th, cc, mm, vv]
        names = ["param", "comp", "m", "v"]
    elif layout == "bf16-moments":
        m16, v16 = oracle.bf16_from_double(m0), oracle.bf16_from_double(v0)
        master, m, v = dev(th0), dev(m16), dev(v16)
        zs.zero_shard_step_bf16_moments(parts, master, m, v, n, d_table, nc, hp_d)
        th, mm, vv, p = oracle.shard_step_bf16m(parts_h, th0, m16, v16, hp_h)
        got = [host(master), host(m), host(v), read_params()[lo:lo + n]]
        want = [th, mm, vv, p]
        names = ["master", "m", "v", "param"]
    else:
        master, m, v = dev(th0), dev(m0), dev(v0)
        if layout == "fp32":
            zs.zero_shard_step(parts, master, m, v, n, d_table, nc, hp_d)
            th, mm, vv, p = oracle.shard_step(parts_h, th0, m0, v0, hp_h)
        elif layout == "scheduled":
            consts = torch.from_numpy(zs.zero_make_step_consts([hp_d]).view(np.uint8)).cuda()
            index = torch.zeros(1, dtype=torch.int64, device="cuda")
            zs.zero_shard_step_scheduled(parts, master, m, v, n, d_table, nc, consts, 1, index)
            th, mm, vv, p = oracle.shard_step(parts_h, th0, m0, v0, hp_h)
        else:
            k = c["group"] if c["group"] not in (1, c["n_ranks"]) else 0
            acc = torch.empty(max(n, 1), dtype=torch.float32, device="cuda")
            prev_h = [x[::-1].copy() for x in parts_h]          # an earlier micro-batch
            zs.zero_accumulate_shard([dev(x) for x in prev_h], n, acc, reset=True, group=k)
            acc_h = oracle.accumulate(prev_h, None, group=k or None)
            zs.zero_shard_step_ex(parts, master, m, v, n, d_table, nc, hp_d, group=k,
                                  micro_batches=2, acc=acc)
            th, mm, vv, p = oracle.shard_step_ex(parts_h, th0, m0, v0, hp_h, group=k or None,
                                                 acc=acc_h, micro_batches=2)
        got = [host(master), host(m), host(v), read_params()[lo:lo + n]]
        want = [th, mm, vv, p]
        names = ["master", "m", "v", "param"]
    torch.cuda.synchronize()
    for g, w_, name in zip(got, want, names):
        assert_bitwise(g, w_, f"seed {seed} {layout} {name}")
    outside = np.concatenate([read_params()[:lo], read_params()[lo + n:]])
    assert np.all(outside == 0xFFFF), f"seed {seed}: a parameter outside the shard was written"
