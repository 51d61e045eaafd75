"""The bf16 parameter stores on misaligned destinations, bitwise against the
oracle.

Each tensor of the list gets a destination that starts m elements past an
aligned slot, for every m in 1 .. VEC-1 (VEC = 8 with bf16 partials, 4 with
fp32 ones), with lengths that give chunks of one lane group, of one pass
minus one group, one pass, one pass plus one group, two passes plus one,
and several chunks per tensor.  Those chunks take the shuffled stores (the
lane owning group g writes the aligned slot that straddles groups g - 1 and
g); a few tensors with lengths off the group grid, and one aligned tensor,
take the other paths beside them.  Sentinel elements between the tensors
must survive.  Checked for the 16-byte step, the extended step, the 12-byte
step and the unfused bf16 write, and for the pure-bf16 step (which reads and
writes its parameters at the destinations element by element on those
chunks), with a short table (the two-wave launch) and a long one (the
one-wave launch)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_bitwise, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
SENTINEL = 0xFFFF
GAP = 24          # sentinel elements between two tensors' destinations


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


def layout(vec: int, repeat: int):
    """Tensor sizes and each tensor's destination offset (elements) in one
    flat buffer: every misalignment 1 .. vec-1 with every length, plus
    off-grid lengths and one aligned tensor."""
    lengths = [vec, 63 * vec, 64 * vec, 65 * vec, 129 * vec, 3000 * vec // 8 * 8]
    numels, mis = [], []
    for m in range(1, vec):
        for n in lengths:
            numels.append(n)
            mis.append(m)
    numels += [vec * 70 + 3, 5, vec * 64]        # off the grid, tiny, aligned
    mis += [vec - 1, 1, 0]
    numels *= repeat
    mis *= repeat
    offs, pos = [], 0
    for n, m in zip(numels, mis):
        pos = -(-(pos + GAP) // vec) * vec + m
        offs.append(pos)
        pos += n
    return numels, offs, pos + GAP


def expected_buffer(numels, offs, size, prm):
    want = np.full(size, SENTINEL, np.uint16)
    start = 0
    for n, o in zip(numels, offs):
        want[o:o + n] = prm[start:start + n]
        start += n
    return want


@pytest.mark.parametrize("long_table", [False, True])
@pytest.mark.parametrize("gdt", ["bf16", "f32"])
def test_misaligned_parameter_stores(zs, gdt, long_table):
    vec = 8 if gdt == "bf16" else 4
    max_chunk = 64 if long_table else (2048 if gdt == "bf16" else 1024)
    repeat = 1
    if long_table:     # enough 64-element chunks to exceed both small-launch limits
        limit = max(zs.ZERO_SMALL_LAUNCH_CHUNKS, zs.ZERO_SMALL_LAUNCH_CHUNKS_12B)
        repeat = -(-(limit + 512) * max_chunk // sum(layout(vec, 1)[0]))
    numels, offs, size = layout(vec, repeat)
    n = sum(numels)
    n_ranks, t, seed = 3, 4, 0x5EED0000 + 77
    parts_h = [synth.fill(gdt, seed, synth.stream_id(synth.KIND_GRAD, k, t), 0, n, 1e-3)
               for k in range(n_ranks)]
    th0 = synth.fill("f32", seed, synth.stream_id(synth.KIND_MASTER), 0, n, 0.02)
    rng = np.random.default_rng(5)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-8).astype(np.float32)
    parts = [dev(p) for p in parts_h]
    buf = torch.full((size,), -1, dtype=torch.int16, device="cuda")
    base = buf.data_ptr()
    dsts = [base + 2 * o for o in offs]
    table, S = zs.zero_build_chunks(numels, 1, 0, tensor_dst=dsts, max_chunk=max_chunk)
    assert S == n
    d_table, nc = zs.chunks_to_device(table), len(table)
    assert (nc > max(zs.ZERO_SMALL_LAUNCH_CHUNKS, zs.ZERO_SMALL_LAUNCH_CHUNKS_12B)) == long_table, nc
    assert long_table or nc <= zs.ZERO_SMALL_LAUNCH_CHUNKS, nc
    misaligned = int(((table["dst"].astype(np.int64) // 2) % vec != 0).sum())
    tag = f"{gdt} partials, {len(numels)} tensors, {nc} chunks ({misaligned} misaligned), chunk {max_chunk}"
    hp_h, hp_d = oracle.hparams(t, **HP), zs.hparams(t, **HP)

    say(f"case: misaligned stores, {tag}: 16-byte step")
    master, m, v = dev(th0), dev(m0), dev(v0)
    zs.zero_check_chunks(table, n, parts + [master, m, v])
    zs.zero_shard_step(parts, master, m, v, n, d_table, nc, hp_d)
    th, mm, vv, prm = oracle.shard_step(parts_h, th0, m0, v0, hp_h)
    for got, want, what in ((host(master), th, "master"), (host(m), mm, "m"), (host(v), vv, "v")):
        assert_bitwise(got, want, f"{tag} 16-byte {what}")
    want_buf = expected_buffer(numels, offs, size, prm)
    assert_bitwise(host(buf), want_buf, f"{tag} 16-byte parameters and sentinels", strict_nan=True)

    say(f"case: misaligned stores, {tag}: extended step (one group, one micro-batch)")
    buf.fill_(-1)
    master, m, v = dev(th0), dev(m0), dev(v0)
    zs.zero_shard_step_ex(parts, master, m, v, n, d_table, nc, hp_d, group=0, micro_batches=1)
    assert_bitwise(host(master), th, f"{tag} extended master")
    assert_bitwise(host(buf), want_buf, f"{tag} extended parameters and sentinels", strict_nan=True)

    say(f"case: misaligned stores, {tag}: unfused bf16 write")
    buf.fill_(-1)
    zs.zero_gather_write(dev(th), n, d_table, nc)
    assert_bitwise(host(buf), want_buf, f"{tag} unfused write and sentinels", strict_nan=True)

    say(f"case: misaligned stores, {tag}: 12-byte step")
    buf.fill_(-1)
    m16, v16 = oracle.bf16_from_double(m0), oracle.bf16_from_double(v0)
    master, dm, dv = dev(th0), dev(m16), dev(v16)
    zs.zero_shard_step_bf16_moments(parts, master, dm, dv, n, d_table, nc, hp_d)
    th2, mm2, vv2, prm2 = oracle.shard_step_bf16m(parts_h, th0, m16, v16, hp_h)
    for got, want, what in ((host(master), th2, "master"), (host(dm), mm2, "m"), (host(dv), vv2, "v")):
        assert_bitwise(got, want, f"{tag} 12-byte {what}")
    assert_bitwise(host(buf), expected_buffer(numels, offs, size, prm2),
                   f"{tag} 12-byte parameters and sentinels", strict_nan=True)

    say(f"case: misaligned stores, {tag}: pure-bf16 step (parameters read and written in place)")
    th16 = oracle.bf16_round(th0)
    c16 = oracle.bf16_from_double(rng.standard_normal(n) * 1e-6)
    buf.copy_(dev(expected_buffer(numels, offs, size, th16)))
    dc, dm, dv = dev(c16), dev(m16), dev(v16)
    zs.zero_shard_step_kahan(parts, dc, dm, dv, n, d_table, nc, hp_d)
    th3, c3, mm3, vv3 = oracle.shard_step_kahan(parts_h, th16, c16, m16, v16, hp_h)
    for got, want, what in ((host(dc), c3, "compensation"), (host(dm), mm3, "m"), (host(dv), vv3, "v")):
        assert_bitwise(got, want, f"{tag} pure-bf16 {what}")
    assert_bitwise(host(buf), expected_buffer(numels, offs, size, th3),
                   f"{tag} pure-bf16 parameters and sentinels", strict_nan=True)
