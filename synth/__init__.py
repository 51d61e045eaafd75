"""Seeded synthetic inputs shared by the CPU oracle and the GPU library.

Holds no arithmetic of the optimizer step: only the counter-based input
generator (host C in ``gen.c``, device twin in ``fill.hip``), the stream
naming, and the tensor-list shapes of the workloads (``workloads.py``).
Every generated value is a pure function of (seed, stream, index), so any
sampled index can be regenerated on the host without a full host mirror.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

# Stream kinds.  A stream id packs (kind, rank, step) so that every rank's
# gradient at every step is an independent sequence indexed by the *global*
# flat parameter index.
KIND_GRAD = 1
KIND_MASTER = 2
KIND_OUTLIER = 3
KIND_PREFIX_MAP = 4
KIND_RAGGED_SIZE = 5
KIND_ZERO_TENSOR = 6
KIND_MOMENT = 7


def stream_id(kind: int, rank: int = 0, step: int = 0) -> int:
    assert 0 <= kind < 256 and 0 <= rank < 65536 and 0 <= step < (1 << 32)
    return (kind << 48) | (rank << 32) | step


def scale_for_std(sigma: float) -> np.float32:
    """fp32 multiplier that turns an Irwin-Hall(4) sum minus 2 into std sigma."""
    return np.float32(np.sqrt(3.0) * sigma)


def build(verbose: bool = False) -> None:
    """Compile the host generator with gcc (the device twin is built by the
    package build, since it needs hipcc)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-o", HOST_LIB, os.path.join(_HERE, "gen.c")]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)


def build_dev(verbose: bool = False) -> None:
    """Compile the device twin (fill.hip) for gfx950 with hipcc."""
    cmd = ["/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc",
           "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-o", DEV_LIB, os.path.join(_HERE, "fill.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


_host = None
_dev = None


def _devlib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise ImportError(f"{DEV_LIB} missing: run synth.build_dev() (hipcc)")
        lib = ctypes.CDLL(DEV_LIB)
        u64, i64, f32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        for name in ("synth_dev_fill_f32", "synth_dev_fill_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, u64, u64, i64, i64, f32, u64, f32, f32, vp]
            fn.restype = ctypes.c_int
        lib.synth_dev_spread.argtypes = [vp, vp, i64, u64, u64, i64, i64, vp]
        lib.synth_dev_spread.restype = ctypes.c_int
        _dev = lib
    return _dev


def dev_fill(out, seed: int, stream: int, start: int, sigma: float, mask_stream: int = 0,
             frac: float = 0.0, mult: float = 1.0) -> None:
    """Fill a contiguous device tensor (bf16/int16 -> bf16 bits, float32) with
    the values at global indices [start, start + out.numel()), on the current
    torch stream."""
    import torch
    assert out.is_cuda and out.is_contiguous()
    st = torch.cuda.current_stream().cuda_stream
    if out.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        fn = _devlib().synth_dev_fill_bf16
    elif out.dtype == torch.float32:
        fn = _devlib().synth_dev_fill_f32
    else:
        raise TypeError(out.dtype)
    rc = fn(out.data_ptr(), seed, stream, start, out.numel(), scale_for_std(sigma), mask_stream,
            frac, mult, st)
    if rc:
        raise RuntimeError("synth device fill failed to launch")


def dev_spread(dst, prefix, seed: int, stream: int, start: int) -> None:
    """dst[j] = prefix[src(start + j)] on the device (warm-start spreading)."""
    import torch
    assert dst.is_cuda and prefix.is_cuda and dst.dtype == prefix.dtype == torch.float32
    rc = _devlib().synth_dev_spread(dst.data_ptr(), prefix.data_ptr(), prefix.numel(), seed,
                                    stream, start, dst.numel(),
                                    torch.cuda.current_stream().cuda_stream)
    if rc:
        raise RuntimeError("synth device spread failed to launch")


def _lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build()
        lib = ctypes.CDLL(HOST_LIB)
        u64, i64, f32, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
        for name in ("synth_fill_f32", "synth_fill_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, u64, u64, i64, i64, f32, u64, f32, f32]
            fn.restype = None
        for name in ("synth_gather_f32", "synth_gather_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, u64, u64, vp, i64, f32, u64, f32, f32]
            fn.restype = None
        lib.synth_prefix_src.argtypes = [vp, u64, u64, vp, i64, i64]
        lib.synth_prefix_src.restype = None
        lib.synth_uniform.argtypes = [vp, u64, u64, vp, i64]
        lib.synth_uniform.restype = None
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_key.restype = u64
        _host = lib
    return _host


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def fill(dtype: str, seed: int, stream: int, start: int, count: int, sigma: float,
         mask_stream: int = 0, frac: float = 0.0, mult: float = 1.0) -> np.ndarray:
    """Values at global indices [start, start+count); dtype 'bf16' (uint16 bits) or 'f32'."""
    lib = _lib()
    if dtype == "bf16":
        out = np.empty(count, dtype=np.uint16)
        lib.synth_fill_bf16(_ptr(out), seed, stream, start, count, scale_for_std(sigma),
                            mask_stream, frac, mult)
    elif dtype == "f32":
        out = np.empty(count, dtype=np.float32)
        lib.synth_fill_f32(_ptr(out), seed, stream, start, count, scale_for_std(sigma),
                           mask_stream, frac, mult)
    else:
        raise ValueError(dtype)
    return out


def gather(dtype: str, seed: int, stream: int, idx: np.ndarray, sigma: float,
           mask_stream: int = 0, frac: float = 0.0, mult: float = 1.0) -> np.ndarray:
    """Values at an arbitrary list of global indices."""
    lib = _lib()
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    if dtype == "bf16":
        out = np.empty(idx.size, dtype=np.uint16)
        lib.synth_gather_bf16(_ptr(out), seed, stream, _ptr(idx), idx.size,
                              scale_for_std(sigma), mask_stream, frac, mult)
    elif dtype == "f32":
        out = np.empty(idx.size, dtype=np.float32)
        lib.synth_gather_f32(_ptr(out), seed, stream, _ptr(idx), idx.size,
                             scale_for_std(sigma), mask_stream, frac, mult)
    else:
        raise ValueError(dtype)
    return out


def prefix_src(seed: int, stream: int, idx: np.ndarray, plen: int) -> np.ndarray:
    """Warm-start source index for each shard index (identity below plen)."""
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.int64)
    _lib().synth_prefix_src(_ptr(out), seed, stream, _ptr(idx), idx.size, plen)
    return out


def uniform(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """Uniform [0,1) fp32 draws unif(key(seed, stream), i) at the given counters."""
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.float32)
    _lib().synth_uniform(_ptr(out), seed, stream, _ptr(idx), idx.size)
    return out
