"""The chunk-table launches at their limits, against the oracle, bitwise.

- More chunks than the grid holds: a launch has at most 2^22 workgroups,
  and with a longer table each workgroup takes chunks blockIdx.x,
  blockIdx.x + 2^22, ...  A 268,436,456-element shard cut into chunks of 64
  gives 4,194,320 chunks, so the first 16 workgroups each step two.
- The longest chunk the builder accepts (2^24 elements, one wave looping
  over 32,768 groups of 512) followed by a ragged 1,237-element chunk.

Each case runs the 16-byte, 12-byte and pure-bf16 steps and the unfused
bf16 write over the same table.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_bitwise, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
SEED = 0x5EED0000 + 77


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


def run_all_layouts(zs, n, max_chunk, n_ranks, expect_chunks):
    t = 3
    parts_h = [synth.fill("bf16", SEED, synth.stream_id(synth.KIND_GRAD, k, t), 0, n, 1e-3)
               for k in range(n_ranks)]
    th0 = synth.fill("f32", SEED, synth.stream_id(synth.KIND_MASTER), 0, n, 0.02)
    rng = np.random.default_rng(n_ranks)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-8).astype(np.float32)
    parts = [dev(p) for p in parts_h]
    slot = torch.full((n,), -1, dtype=torch.int16, device="cuda")
    table, S = zs.zero_build_chunks([n], 1, 0, slot_dst=slot, max_chunk=max_chunk)
    assert S == n and len(table) == expect_chunks
    d_table, nc = zs.chunks_to_device(table), len(table)
    hp_h, hp_d = oracle.hparams(t, **HP), zs.hparams(t, **HP)

    say(f"  16-byte step over {nc} chunks")
    master, m, v = dev(th0), dev(m0), dev(v0)
    zs.zero_shard_step(parts, master, m, v, n, d_table, nc, hp_d)
    th, mm, vv, p = oracle.shard_step(parts_h, th0, m0, v0, hp_h)
    for got, want, what in ((master, th, "master"), (m, mm, "m"), (v, vv, "v"), (slot, p, "param")):
        assert_bitwise(host(got), want, f"16-byte {what}")
    say("  unfused bf16 write")
    slot.fill_(-1)
    zs.zero_gather_write(master, n, d_table, nc)
    assert_bitwise(host(slot), p, "gather write")
    del master, m, v, th, mm, vv

    say("  12-byte step")
    m16, v16 = oracle.bf16_from_double(m0), oracle.bf16_from_double(v0)
    master, m, v = dev(th0), dev(m16), dev(v16)
    slot.fill_(-1)
    zs.zero_shard_step_bf16_moments(parts, master, m, v, n, d_table, nc, hp_d)
    th, mm, vv, p = oracle.shard_step_bf16m(parts_h, th0, m16, v16, hp_h)
    for got, want, what in ((master, th, "master"), (m, mm, "m"), (v, vv, "v"), (slot, p, "param")):
        assert_bitwise(host(got), want, f"12-byte {what}")
    del master, m, v, th, mm, vv

    say("  pure-bf16 Kahan step")
    th16 = oracle.bf16_round(th0)
    c16 = oracle.bf16_from_double(rng.standard_normal(n) * 1e-6)
    slot.copy_(dev(th16))
    comp, m, v = dev(c16), dev(m16), dev(v16)
    zs.zero_shard_step_kahan(parts, comp, m, v, n, d_table, nc, hp_d)
    th, cc, mm, vv = oracle.shard_step_kahan(parts_h, th16, c16, m16, v16, hp_h)
    for got, want, what in ((slot, th, "param"), (comp, cc, "comp"), (m, mm, "m"), (v, vv, "v")):
        assert_bitwise(host(got), want, f"Kahan {what}")


@pytest.mark.timeout(600)
def test_more_chunks_than_the_grid(zs):
    n = (1 << 22) * 64 + 1000
    say(f"case: limits: {n} elements in chunks of 64 (more chunks than 2^22 workgroups)")
    run_all_layouts(zs, n, 64, 2, (1 << 22) + 16)
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_longest_chunk(zs):
    n = (1 << 24) + 1237
    say(f"case: limits: {n} elements, chunks of 2^24 then a ragged tail")
    run_all_layouts(zs, n, 1 << 24, 4, 2)
    torch.cuda.empty_cache()
