"""Python binding of libzero_shard.so, the MI355X ZeRO shard-step library.

Same names as the C ABI in include/zero_shard.h.  This module only marshals
arguments (torch tensors or raw device addresses -> pointers, the current
torch stream -> hipStream_t) and turns non-zero return codes into
exceptions.  Every step of the computation runs in the library's HIP
kernels; there is no fallback.  If the library has not been built, importing
this package raises.

    import sharded_optimizer_step_shard_amd as zs
    table, S = zs.zero_build_chunks(numels, n_ranks, rank, slot_dst=slot_ptr)
    d_table = zs.chunks_to_device(table)
    zs.zero_shard_step(partials, master, m, v, S, d_table, len(table), hp)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libzero_shard.so")

ZERO_BF16, ZERO_FP32 = 0, 1
ZERO_OK, ZERO_ERR_INVALID, ZERO_ERR_MISALIGNED, ZERO_ERR_UNSUPPORTED = 0, 1, 2, 3
ZERO_ERR_ALIAS, ZERO_ERR_HIP, ZERO_ERR_CAPACITY, ZERO_ERR_NOT_DEVICE = 4, 5, 6, 7
ZERO_MAX_RANKS = 64
ZERO_MAX_LEN = 1 << 48          # largest element or byte count an entry point accepts
ZERO_DEFAULT_MAX_CHUNK = 2048        # bf16 partials
ZERO_DEFAULT_MAX_CHUNK_FP32 = 1024   # fp32 partials
# step launches up to this many chunks run at a higher occupancy
ZERO_SMALL_LAUNCH_CHUNKS = 2048        # 16-byte and extended steps
ZERO_SMALL_LAUNCH_CHUNKS_12B = 16384   # 12-byte step
ZERO_PROBE_SUM_MAX = 16

# Mirrors `zero_chunk` (32 bytes).
CHUNK_DTYPE = np.dtype([("shard_off", "<i8"), ("dst", "<u8"), ("len", "<i4"),
                        ("tensor_id", "<i4"), ("tensor_off", "<i8")], align=True)
assert CHUNK_DTYPE.itemsize == 32


class HParams(ctypes.Structure):
    """Mirrors `zero_adamw_hparams`."""
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64)]


def hparams(step: int, lr: float = 1e-3, beta1: float = 0.9, beta2: float = 0.999,
            eps: float = 1e-8, weight_decay: float = 0.1) -> HParams:
    return HParams(lr, beta1, beta2, eps, weight_decay, step)


# Mirrors `zero_step_consts` (80 bytes): the constants of one step.
STEP_CONSTS_DTYPE = np.dtype([(f, "<f8") for f in
                              ("b1", "c1", "b2", "c2", "bc1", "bc2", "eps", "lr", "dec", "wd")])
assert STEP_CONSTS_DTYPE.itemsize == 80


class ReduceSpec(ctypes.Structure):
    """Mirrors `zero_reduce_spec`."""
    _fields_ = [("group", ctypes.c_int32), ("micro_batches", ctypes.c_int32),
                ("acc", ctypes.c_void_p)]


class ZeroShardError(RuntimeError):
    def __init__(self, code: int, fn: str):
        self.code = code
        super().__init__(f"{fn} failed: {code} ({zero_strerror(code)})")


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first "
                      f"(python {os.path.join(_PKG, 'build.py')})")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_lib.zero_build_chunks.argtypes = [_vp, _i32, _i32, _i32, _vp, _vp, _i64, _vp, _i64,
                                   ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
_lib.zero_shard_step.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i64,
                                 ctypes.POINTER(HParams), _vp]
_lib.zero_shard_step_buckets.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp,
                                         _i32, _vp, ctypes.POINTER(HParams), _vp]
_lib.zero_shard_step_ex.argtypes = [_vp, _i32, _i32, ctypes.POINTER(ReduceSpec), _vp, _vp, _vp,
                                    _i64, _vp, _i64, ctypes.POINTER(HParams), _vp]
_lib.zero_accumulate_shard.argtypes = [_vp, _i32, _i32, _i32, _i64, _vp, _i32, _vp]
_lib.zero_shard_step_bf16_moments.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i64,
                                              ctypes.POINTER(HParams), _vp]
_lib.zero_shard_step_kahan.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i64,
                                       ctypes.POINTER(HParams), _vp]
_lib.zero_reduce_shard.argtypes = [_vp, _i32, _i32, _i64, _vp, _vp]
_lib.zero_adamw_shard.argtypes = [_vp, _vp, _vp, _vp, _i64, ctypes.POINTER(HParams), _vp]
_lib.zero_gather_write.argtypes = [_vp, _i64, _vp, _i64, _vp]
_lib.zero_probe_copy.argtypes = [_vp, _vp, _i64, _vp]
_lib.zero_probe_read.argtypes = [_vp, _i64, _vp, ctypes.c_uint32, _vp]
_lib.zero_probe_write.argtypes = [_vp, _i64, ctypes.c_uint32, _vp]
_lib.zero_probe_sum.argtypes = [_vp, _i32, _vp, _i64, _vp]
_lib.zero_make_step_consts.argtypes = [_vp, _i64, _vp]
_lib.zero_shard_step_scheduled.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _i64, _vp, _i64, _vp,
                                           _i64, _vp, _vp]
_lib.zero_shard_step_bf16_moments_scheduled.argtypes = _lib.zero_shard_step_scheduled.argtypes
_lib.zero_shard_step_kahan_scheduled.argtypes = _lib.zero_shard_step_scheduled.argtypes
_lib.zero_step_index_advance.argtypes = [_vp, _i64, _vp]
_lib.zero_check_chunks.argtypes = [_vp, _i64, _i64, _vp, _vp, _i32]
_lib.zero_strerror.argtypes = [_i32]
_lib.zero_strerror.restype = ctypes.c_char_p
for _f in ("zero_build_chunks", "zero_shard_step", "zero_reduce_shard", "zero_adamw_shard",
           "zero_gather_write", "zero_probe_copy", "zero_probe_read", "zero_probe_write",
           "zero_version", "zero_shard_step_ex",
           "zero_accumulate_shard", "zero_shard_step_bf16_moments", "zero_shard_step_kahan",
           "zero_shard_step_buckets", "zero_make_step_consts", "zero_shard_step_scheduled",
           "zero_step_index_advance", "zero_shard_step_bf16_moments_scheduled",
           "zero_shard_step_kahan_scheduled", "zero_check_chunks", "zero_probe_sum"):
    getattr(_lib, _f).restype = _i32

Ptr = Union[int, "torch.Tensor", None]  # noqa: F821


def lib() -> ctypes.CDLL:
    return _lib


def _addr(x: Ptr) -> Optional[int]:
    """Device address of a tensor (must be contiguous and on a GPU) or a raw int."""
    if x is None:
        return None
    if isinstance(x, (int, np.integer)):
        return int(x)
    if not x.is_cuda:
        raise ValueError("tensor arguments must live in device memory")
    if not x.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _gdt_of(partials) -> int:
    p0 = partials[0]
    if isinstance(p0, (int, np.integer)):
        raise ValueError("pass gdt explicitly with raw partial addresses")
    import torch
    if p0.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return ZERO_BF16
    if p0.dtype == torch.float32:
        return ZERO_FP32
    raise ValueError(f"unsupported partial dtype {p0.dtype}")


def _check(code: int, fn: str) -> None:
    if code != ZERO_OK:
        raise ZeroShardError(code, fn)


def zero_strerror(code: int) -> str:
    return _lib.zero_strerror(code).decode()


def zero_version() -> Tuple[int, int]:
    v = _lib.zero_version()
    return v >> 16, v & 0xFFFF


def zero_build_chunks(numels: Sequence[int], n_ranks: int, rank: int,
                      tensor_dst: Optional[Sequence[Ptr]] = None, slot_dst: Ptr = None,
                      max_chunk: int = ZERO_DEFAULT_MAX_CHUNK) -> Tuple[np.ndarray, int]:
    """Host chunk table (numpy array of CHUNK_DTYPE) and the shard length S."""
    nm = np.ascontiguousarray(numels, dtype=np.int64)
    td = None
    if tensor_dst is not None:
        td = (ctypes.c_void_p * len(tensor_dst))(*[_addr(t) for t in tensor_dst])
    n = _i64(0)
    S = _i64(0)
    _check(_lib.zero_build_chunks(nm.ctypes.data, len(nm), n_ranks, rank, td, _addr(slot_dst),
                                  max_chunk, None, 0, ctypes.byref(n), ctypes.byref(S)),
           "zero_build_chunks")
    out = np.zeros(n.value, dtype=CHUNK_DTYPE)
    if n.value:
        _check(_lib.zero_build_chunks(nm.ctypes.data, len(nm), n_ranks, rank, td,
                                      _addr(slot_dst), max_chunk, out.ctypes.data, n.value,
                                      ctypes.byref(n), ctypes.byref(S)), "zero_build_chunks")
    return out, S.value


def _byte_range(x) -> Tuple[int, int]:
    """(device address, byte count) of a tensor, or an (address, bytes) pair."""
    if isinstance(x, tuple):
        return int(x[0]), int(x[1])
    return _addr(x), x.numel() * x.element_size()


def zero_check_chunks(table: np.ndarray, shard_len: int, arrays: Sequence) -> None:
    """Check a host chunk table against the arrays a step reads or writes
    besides the destinations (tensors or (address, bytes) pairs): raises
    ZeroShardError with INVALID for a malformed table, ALIAS when a
    destination overlaps one of the arrays or another chunk's destination.
    Host only; call it once per table and set of step arrays."""
    tab = np.ascontiguousarray(table, dtype=CHUNK_DTYPE)
    rng = [_byte_range(a) for a in arrays]
    ptrs = (ctypes.c_void_p * max(len(rng), 1))(*[r[0] for r in rng])
    sizes = (ctypes.c_int64 * max(len(rng), 1))(*[r[1] for r in rng])
    _check(_lib.zero_check_chunks(tab.ctypes.data if len(tab) else None, len(tab), shard_len,
                                  ptrs, sizes, len(rng)), "zero_check_chunks")


def chunks_to_device(table: np.ndarray, device: str = "cuda"):
    """Copy a host chunk table into a device buffer (torch owns the memory)."""
    import torch
    raw = torch.from_numpy(np.ascontiguousarray(table).view(np.uint8).copy())
    return raw.to(device)


def _partial_array(partials):
    addrs = [_addr(p) for p in partials]
    return (ctypes.c_void_p * max(len(addrs), 1))(*addrs)


def zero_shard_step(partials: Sequence[Ptr], master: Ptr, m: Ptr, v: Ptr, shard_len: int,
                    d_chunks: Ptr, n_chunks: int, hp: HParams, gdt: Optional[int] = None,
                    stream=None) -> None:
    """Fused reduce + AdamW + bf16 write of one shard (asynchronous on `stream`)."""
    gdt = _gdt_of(partials) if gdt is None else gdt
    _check(_lib.zero_shard_step(_partial_array(partials), len(partials), gdt, _addr(master),
                                _addr(m), _addr(v), shard_len, _addr(d_chunks), n_chunks,
                                ctypes.byref(hp), _stream(stream)), "zero_shard_step")


def zero_make_step_consts(hps: Sequence[HParams]) -> np.ndarray:
    """Host table of step constants, one entry per hparams (STEP_CONSTS_DTYPE)."""
    n = len(hps)
    arr = (HParams * max(n, 1))(*hps)
    out = np.zeros(n, dtype=STEP_CONSTS_DTYPE)
    _check(_lib.zero_make_step_consts(ctypes.addressof(arr), n, out.ctypes.data if n else None),
           "zero_make_step_consts")
    return out


def zero_shard_step_scheduled(partials: Sequence[Ptr], master: Ptr, m: Ptr, v: Ptr,
                              shard_len: int, d_chunks: Ptr, n_chunks: int, consts: Ptr,
                              n_consts: int, index: Ptr, gdt: Optional[int] = None,
                              stream=None) -> None:
    """Fused step whose constants are consts[*index], read on the device."""
    gdt = _gdt_of(partials) if gdt is None else gdt
    _check(_lib.zero_shard_step_scheduled(_partial_array(partials), len(partials), gdt,
                                          _addr(master), _addr(m), _addr(v), shard_len,
                                          _addr(d_chunks), n_chunks, _addr(consts), n_consts,
                                          _addr(index), _stream(stream)),
           "zero_shard_step_scheduled")


def zero_shard_step_bf16_moments_scheduled(partials: Sequence[Ptr], master: Ptr, m: Ptr, v: Ptr,
                                           shard_len: int, d_chunks: Ptr, n_chunks: int,
                                           consts: Ptr, n_consts: int, index: Ptr,
                                           gdt: Optional[int] = None, stream=None) -> None:
    """12-byte-state step whose constants are consts[*index], read on the device."""
    gdt = _gdt_of(partials) if gdt is None else gdt
    _check(_lib.zero_shard_step_bf16_moments_scheduled(
        _partial_array(partials), len(partials), gdt, _addr(master), _addr(m), _addr(v), shard_len,
        _addr(d_chunks), n_chunks, _addr(consts), n_consts, _addr(index), _stream(stream)),
        "zero_shard_step_bf16_moments_scheduled")


def zero_shard_step_kahan_scheduled(partials: Sequence[Ptr], comp: Ptr, m: Ptr, v: Ptr,
                                    shard_len: int, d_chunks: Ptr, n_chunks: int, consts: Ptr,
                                    n_consts: int, index: Ptr, gdt: Optional[int] = None,
                                    stream=None) -> None:
    """Pure-bf16 step whose constants are consts[*index], read on the device."""
    gdt = _gdt_of(partials) if gdt is None else gdt
    _check(_lib.zero_shard_step_kahan_scheduled(
        _partial_array(partials), len(partials), gdt, _addr(comp), _addr(m), _addr(v), shard_len,
        _addr(d_chunks), n_chunks, _addr(consts), n_consts, _addr(index), _stream(stream)),
        "zero_shard_step_kahan_scheduled")


def zero_step_index_advance(index: Ptr, n_consts: int, stream=None) -> None:
    _check(_lib.zero_step_index_advance(_addr(index), n_consts, _stream(stream)),
           "zero_step_index_advance")


def zero_shard_step_buckets(partials: Sequence[Ptr], master: Ptr, m: Ptr, v: Ptr, shard_len: int,
                            d_chunks: Ptr, n_chunks: int, runs: Sequence[Tuple[int, int]],
                            hp: HParams, ready=None, gdt: Optional[int] = None,
                            stream=None) -> None:
    """The fused step in buckets, one C call: runs = [(first chunk, chunk
    count), ...] in increasing, disjoint order; ready = per-bucket events
    (torch.cuda.Event or None) the stream waits for before each bucket."""
    gdt = _gdt_of(partials) if gdt is None else gdt
    nb = len(runs)
    first = np.ascontiguousarray([r[0] for r in runs], dtype=np.int64)
    count = np.ascontiguousarray([r[1] for r in runs], dtype=np.int64)
    ev = None
    if ready is not None:
        if len(ready) != nb:
            raise ValueError("one ready event (or None) per bucket")
        ev = (ctypes.c_void_p * max(nb, 1))(*[None if e is None else e.cuda_event for e in ready])
    _check(_lib.zero_shard_step_buckets(_partial_array(partials), len(partials), gdt, _addr(master),
                                        _addr(m), _addr(v), shard_len, _addr(d_chunks), n_chunks,
                                        first.ctypes.data if nb else None,
                                        count.ctypes.data if nb else None, nb, ev,
                                        ctypes.byref(hp), _stream(stream)),
           "zero_shard_step_buckets")


def zero_shard_step_ex(partials: Sequence[Ptr], master: Ptr, m: Ptr, v: Ptr, shard_len: int,
                       d_chunks: Ptr, n_chunks: int, hp: HParams, group: int = 0,
                       micro_batches: int = 1, acc: Ptr = None, gdt: Optional[int] = None,
                       stream=None) -> None:
    """Fused step with the two-level reduce order and/or an accumulator of
    earlier micro-batches (see zero_reduce_spec)."""
    gdt = _gdt_of(partials) if gdt is None else gdt
    rs = ReduceSpec(group, micro_batches, _addr(acc))
    _check(_lib.zero_shard_step_ex(_partial_array(partials), len(partials), gdt, ctypes.byref(rs),
                                   _addr(master), _addr(m), _addr(v), shard_len, _addr(d_chunks),
                                   n_chunks, ctypes.byref(hp), _stream(stream)),
           "zero_shard_step_ex")


def zero_shard_step_bf16_moments(partials: Sequence[Ptr], master: Ptr, m: Ptr, v: Ptr,
                                 shard_len: int, d_chunks: Ptr, n_chunks: int, hp: HParams,
                                 gdt: Optional[int] = None, stream=None) -> None:
    """Fused step on the 12-byte state: fp32 master, bf16 m and v (int16 /
    bfloat16 tensors holding the bit patterns)."""
    gdt = _gdt_of(partials) if gdt is None else gdt
    _check(_lib.zero_shard_step_bf16_moments(_partial_array(partials), len(partials), gdt,
                                             _addr(master), _addr(m), _addr(v), shard_len,
                                             _addr(d_chunks), n_chunks, ctypes.byref(hp),
                                             _stream(stream)), "zero_shard_step_bf16_moments")


def zero_shard_step_kahan(partials: Sequence[Ptr], comp: Ptr, m: Ptr, v: Ptr, shard_len: int,
                          d_chunks: Ptr, n_chunks: int, hp: HParams, gdt: Optional[int] = None,
                          stream=None) -> None:
    """Fused step on the pure-bf16 state: the bf16 parameters at the chunks'
    destinations are read and written in place; comp (Kahan compensation),
    m and v are bf16 bit patterns in shard order."""
    gdt = _gdt_of(partials) if gdt is None else gdt
    _check(_lib.zero_shard_step_kahan(_partial_array(partials), len(partials), gdt, _addr(comp),
                                      _addr(m), _addr(v), shard_len, _addr(d_chunks), n_chunks,
                                      ctypes.byref(hp), _stream(stream)), "zero_shard_step_kahan")


def zero_accumulate_shard(partials: Sequence[Ptr], n: int, acc: Ptr, reset: bool,
                          group: int = 0, gdt: Optional[int] = None, stream=None) -> None:
    """acc = fp32((reset ? 0 : acc) + two-level sum of the partials)."""
    gdt = _gdt_of(partials) if gdt is None else gdt
    _check(_lib.zero_accumulate_shard(_partial_array(partials), len(partials), gdt, group, n,
                                      _addr(acc), 1 if reset else 0, _stream(stream)),
           "zero_accumulate_shard")


def zero_reduce_shard(partials: Sequence[Ptr], n: int, grad_out: Ptr,
                      gdt: Optional[int] = None, stream=None) -> None:
    gdt = _gdt_of(partials) if gdt is None else gdt
    _check(_lib.zero_reduce_shard(_partial_array(partials), len(partials), gdt, n,
                                  _addr(grad_out), _stream(stream)), "zero_reduce_shard")


def zero_adamw_shard(grad: Ptr, master: Ptr, m: Ptr, v: Ptr, n: int, hp: HParams,
                     stream=None) -> None:
    _check(_lib.zero_adamw_shard(_addr(grad), _addr(master), _addr(m), _addr(v), n,
                                 ctypes.byref(hp), _stream(stream)), "zero_adamw_shard")


def zero_gather_write(master: Ptr, shard_len: int, d_chunks: Ptr, n_chunks: int,
                      stream=None) -> None:
    _check(_lib.zero_gather_write(_addr(master), shard_len, _addr(d_chunks), n_chunks,
                                  _stream(stream)), "zero_gather_write")


def zero_probe_copy(src: Ptr, dst: Ptr, nbytes: int, stream=None) -> None:
    _check(_lib.zero_probe_copy(_addr(src), _addr(dst), nbytes, _stream(stream)),
           "zero_probe_copy")


def zero_probe_read(src: Ptr, nbytes: int, sink: Ptr, magic: int = 0x9E3779B9, stream=None) -> None:
    _check(_lib.zero_probe_read(_addr(src), nbytes, _addr(sink), magic, _stream(stream)),
           "zero_probe_read")


def zero_probe_write(dst: Ptr, nbytes: int, value: int = 0x3C003C00, stream=None) -> None:
    _check(_lib.zero_probe_write(_addr(dst), nbytes, value, _stream(stream)), "zero_probe_write")


def zero_probe_sum(srcs: Sequence[Ptr], dst: Ptr, n: int, stream=None) -> None:
    """dst = srcs[0] + ... + srcs[k-1] over n fp32 elements (measurement aid)."""
    arr = (ctypes.c_void_p * max(len(srcs), 1))(*[_addr(x) for x in srcs])
    _check(_lib.zero_probe_sum(arr, len(srcs), _addr(dst), n, _stream(stream)), "zero_probe_sum")


def raw_call(name: str, *args) -> int:
    """Call a C entry point with raw ctypes arguments and return its code
    (used by the boundary tests to reach the error paths directly)."""
    return getattr(_lib, name)(*args)
