"""Arrays mapped from several physical allocations back to back (HIP's
virtual memory API, as allocators with expandable segments build them):
the step accepts them and gives the oracle's bits, and an array with an
unmapped hole is refused with NOT_DEVICE before anything is launched."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import assert_bitwise, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
PIECE = 2 << 20          # bytes per physical allocation


class MemLocation(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int), ("id", ctypes.c_int)]


class AllocFlags(ctypes.Structure):
    _fields_ = [("compressionType", ctypes.c_ubyte), ("gpuDirectRDMACapable", ctypes.c_ubyte),
                ("usage", ctypes.c_ushort)]


class AllocProp(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int), ("requestedHandleType", ctypes.c_int),
                ("location", MemLocation), ("win32HandleMetaData", ctypes.c_void_p),
                ("allocFlags", AllocFlags)]


class AccessDesc(ctypes.Structure):
    _fields_ = [("location", MemLocation), ("flags", ctypes.c_int)]


assert ctypes.sizeof(AllocProp) == 32 and ctypes.sizeof(AccessDesc) == 12


@pytest.fixture(scope="module")
def hip():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.zeros(1, device="cuda")
    h = ctypes.CDLL("libamdhip64.so")
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    h.hipMemGetAllocationGranularity.argtypes = [ctypes.POINTER(sz), ctypes.POINTER(AllocProp), ctypes.c_int]
    h.hipMemAddressReserve.argtypes = [ctypes.POINTER(vp), sz, sz, vp, ctypes.c_ulonglong]
    h.hipMemCreate.argtypes = [ctypes.POINTER(vp), sz, ctypes.POINTER(AllocProp), ctypes.c_ulonglong]
    h.hipMemMap.argtypes = [vp, sz, sz, vp, ctypes.c_ulonglong]
    h.hipMemSetAccess.argtypes = [vp, sz, ctypes.POINTER(AccessDesc), sz]
    h.hipMemUnmap.argtypes = [vp, sz]
    h.hipMemRelease.argtypes = [vp]
    h.hipMemAddressFree.argtypes = [vp, sz]
    h.hipMemGetAddressRange.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(sz), vp]
    h.hipMemcpy.argtypes = [vp, vp, sz, ctypes.c_int]
    h.hipGetLastError.argtypes = []
    return h


class Mapped:
    """One virtual range of `pieces` physical allocations of PIECE bytes,
    mapped back to back; `hole` leaves that piece unmapped."""

    def __init__(self, h, pieces, hole=None):
        self.h, self.pieces = h, pieces
        self.prop = AllocProp(type=1, requestedHandleType=0, location=MemLocation(1, 0))
        g = ctypes.c_size_t()
        assert h.hipMemGetAllocationGranularity(ctypes.byref(g), ctypes.byref(self.prop), 0) == 0
        assert PIECE % g.value == 0
        self.size = pieces * PIECE
        base = ctypes.c_void_p()
        assert h.hipMemAddressReserve(ctypes.byref(base), self.size, PIECE, None, 0) == 0
        self.base = base.value
        self.handles = []          # (handle, mapped) per piece; None for the hole
        acc = AccessDesc(location=MemLocation(1, 0), flags=3)
        try:
            for i in range(pieces):
                if i == hole:
                    self.handles.append(None)
                    continue
                hd = ctypes.c_void_p()
                assert h.hipMemCreate(ctypes.byref(hd), PIECE, ctypes.byref(self.prop), 0) == 0
                self.handles.append([hd.value, False])
                at = self.base + i * PIECE
                assert h.hipMemMap(at, PIECE, 0, hd.value, 0) == 0
                self.handles[-1][1] = True
                assert h.hipMemSetAccess(at, PIECE, ctypes.byref(acc), 1) == 0
        except BaseException:
            self.free()
            raise

    def upload(self, a: np.ndarray):
        assert a.nbytes <= self.size
        assert self.h.hipMemcpy(self.base, a.ctypes.data, a.nbytes, 1) == 0     # host to device

    def download(self, a: np.ndarray):
        assert self.h.hipMemcpy(a.ctypes.data, self.base, a.nbytes, 2) == 0     # device to host

    def free(self):
        ok = True
        for i, e in enumerate(self.handles):
            if e is None:
                continue
            hd, mapped = e
            if mapped:
                ok &= self.h.hipMemUnmap(self.base + i * PIECE, PIECE) == 0
            ok &= self.h.hipMemRelease(hd) == 0
        self.handles = []
        ok &= self.h.hipMemAddressFree(self.base, self.size) == 0
        assert ok


def test_step_on_arrays_mapped_from_several_allocations(hip):
    import sharded_optimizer_step_shard_amd as zs
    n, n_ranks, t, seed = 2_500_003, 4, 3, 0x5EED0000 + 91
    say(f"case: mapped arrays, n = {n}, N = {n_ranks}, pieces of {PIECE} bytes")
    parts_h = [synth.fill("bf16", seed, synth.stream_id(synth.KIND_GRAD, k, t), 0, n, 1e-3)
               for k in range(n_ranks)]
    th0 = synth.fill("f32", seed, synth.stream_id(synth.KIND_MASTER), 0, n, 0.02)
    rng = np.random.default_rng(3)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v0 = (rng.random(n) * 1e-8).astype(np.float32)
    pieces16, pieces32 = -(-2 * n // PIECE), -(-4 * n // PIECE)
    assert pieces16 >= 3 and pieces32 >= 5
    arrays = []
    try:
        parts = [Mapped(hip, pieces16) for _ in range(n_ranks)]
        state = [Mapped(hip, pieces32) for _ in range(3)]
        arrays = parts + state
        for a, h in zip(parts, parts_h):
            a.upload(h)
        for a, h in zip(state, (th0, m0, v0)):
            a.upload(h)
        slot = torch.zeros(n, dtype=torch.int16, device="cuda")
        table, S = zs.zero_build_chunks([n * n_ranks], n_ranks, 0, slot_dst=slot)
        assert S == n
        d_table = zs.chunks_to_device(table)
        zs.zero_shard_step([a.base for a in parts], state[0].base, state[1].base, state[2].base, n,
                           d_table, len(table), zs.hparams(t, **HP), gdt=zs.ZERO_BF16)
        torch.cuda.synchronize()
        th, mm, vv, prm = oracle.shard_step(parts_h, th0, m0, v0, oracle.hparams(t, **HP))
        for a, want, what in zip(state, (th, mm, vv), ("master", "m", "v")):
            got = np.empty(n, np.float32)
            a.download(got)
            assert_bitwise(got, want, f"mapped arrays {what}")
        assert_bitwise(slot.cpu().numpy().view(np.uint16), prm, "mapped arrays parameters")
    finally:
        torch.cuda.synchronize()
        for a in arrays:
            a.free()


def test_array_with_an_unmapped_hole_is_refused(hip):
    import sharded_optimizer_step_shard_amd as zs
    n, n_ranks = 2_500_003, 2
    pieces16, pieces32 = -(-2 * n // PIECE), -(-4 * n // PIECE)
    arrays = []
    try:
        holed = Mapped(hip, pieces16, hole=1)
        arrays.append(holed)
        whole = Mapped(hip, pieces16)
        arrays.append(whole)
        state = [Mapped(hip, pieces32) for _ in range(3)]
        arrays += state
        # The step is called only if the runtime reports the hole, so that
        # nothing can be launched onto unmapped memory.
        base, size = ctypes.c_void_p(), ctypes.c_size_t()
        rc = hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), holed.base + PIECE)
        hip.hipGetLastError()
        if rc == 0:
            pytest.skip("the runtime reports an address range for the unmapped piece")
        rc = hip.hipMemGetAddressRange(ctypes.byref(base), ctypes.byref(size), holed.base)
        if rc != 0 or base.value + size.value > holed.base + PIECE:
            pytest.skip("the runtime's range for the first piece reaches over the hole")
        say("case: mapped partial with an unmapped hole")
        slot = torch.zeros(n, dtype=torch.int16, device="cuda")
        table, S = zs.zero_build_chunks([n * n_ranks], n_ranks, 0, slot_dst=slot)
        d_table = zs.chunks_to_device(table)
        with pytest.raises(zs.ZeroShardError) as e:
            zs.zero_shard_step([whole.base, holed.base], state[0].base, state[1].base, state[2].base,
                               n, d_table, len(table), zs.hparams(1, **HP), gdt=zs.ZERO_BF16)
        assert e.value.code == zs.ZERO_ERR_NOT_DEVICE
    finally:
        torch.cuda.synchronize()
        for a in arrays:
            a.free()
