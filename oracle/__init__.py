"""CPU oracle of the sharded optimizer step (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and the
two share no code.  The arithmetic lives in ``zero_oracle.c`` (plain C,
double precision, compiled with gcc without FMA contraction); this module
only marshals numpy arrays into it.  ``ledger.py`` holds the
bytes-per-parameter accounting.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, List, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(_HERE, "liboracle.so")
SRC = os.path.join(_HERE, "zero_oracle.c")

BF16, FP32 = 0, 1


class HParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64)]


def build(verbose: bool = False) -> None:
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-o", LIB, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)


_lib = None


def _load(path: str):
    L = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.oracle_bf16_round.argtypes = [ctypes.c_float]
    L.oracle_bf16_round.restype = ctypes.c_uint16
    L.oracle_bf16_round_array.argtypes = [vp, i64, vp]
    L.oracle_reduce.argtypes = [vp, i32, i32, i64, vp]
    L.oracle_adamw.argtypes = [vp, vp, vp, vp, i64, ctypes.POINTER(HParams)]
    L.oracle_shard_step.argtypes = [vp, i32, i32, i64, vp, vp, vp,
                                    ctypes.POINTER(HParams), vp]
    L.oracle_reduce_ex.argtypes = [vp, i32, i32, i32, vp, i64, i64, vp]
    L.oracle_accumulate.argtypes = [vp, i32, i32, i32, i64, vp, i32]
    L.oracle_shard_step_ex.argtypes = [vp, i32, i32, i32, vp, i64, i64, vp, vp, vp,
                                       ctypes.POINTER(HParams), vp]
    L.oracle_bf16_from_double.argtypes = [ctypes.c_double]
    L.oracle_bf16_from_double.restype = ctypes.c_uint16
    L.oracle_bf16_from_double_array.argtypes = [vp, i64, vp]
    L.oracle_shard_step_bf16m.argtypes = [vp, i32, i32, i64, vp, vp, vp,
                                          ctypes.POINTER(HParams), vp]
    L.oracle_kahan_add.argtypes = [vp, vp, vp, i64]
    L.oracle_shard_step_kahan.argtypes = [vp, i32, i32, i64, vp, vp, vp, vp,
                                          ctypes.POINTER(HParams)]
    L.oracle_shard_segments.argtypes = [vp, i32, i32, i32, vp, i64, ctypes.POINTER(i64)]
    L.oracle_shard_segments.restype = i64
    L.oracle_set_threads.argtypes = [i32]
    L.oracle_max_threads.restype = i32
    for f in (L.oracle_bf16_round_array, L.oracle_reduce, L.oracle_adamw,
              L.oracle_shard_step, L.oracle_set_threads, L.oracle_reduce_ex,
              L.oracle_accumulate, L.oracle_shard_step_ex, L.oracle_bf16_from_double_array,
              L.oracle_shard_step_bf16m, L.oracle_kahan_add, L.oracle_shard_step_kahan):
        f.restype = None
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = _load(LIB)
    return _lib


def use_library(path):
    """Point this module at another build of the oracle (the mutation tests
    load deliberately broken copies); returns the previous handle.  Pass
    None to go back to the default build."""
    global _lib
    prev = _lib
    _lib = None if path is None else _load(path)
    return prev


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
    return a.ctypes.data


def _gdt(partials: Sequence[np.ndarray]) -> int:
    dt = partials[0].dtype
    assert all(p.dtype == dt for p in partials)
    if dt == np.uint16:
        return BF16
    if dt == np.float32:
        return FP32
    raise TypeError(f"partials must be bf16 bits (uint16) or float32, got {dt}")


def _ptr_array(partials: Sequence[np.ndarray]):
    n = len(partials)
    arr = (ctypes.c_void_p * n)(*[_p(p) for p in partials])
    return arr


def hparams(step: int, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1) -> HParams:
    return HParams(lr, beta1, beta2, eps, weight_decay, step)


def bf16_round(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_bf16_round_array(_p(x), x.size, _p(out))
    return out


def reduce(partials: Sequence[np.ndarray]) -> np.ndarray:
    """fp32 average of the N partials, summed in double in rank order."""
    n = partials[0].size
    assert all(p.size == n for p in partials)
    out = np.empty(n, dtype=np.float32)
    lib().oracle_reduce(_ptr_array(partials), len(partials), _gdt(partials), n, _p(out))
    return out


def adamw(g: np.ndarray, master: np.ndarray, m: np.ndarray, v: np.ndarray,
          hp: HParams) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One AdamW update; returns new (master, m, v), inputs untouched."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    th, mm, vv = (np.array(a, dtype=np.float32, copy=True) for a in (master, m, v))
    lib().oracle_adamw(_p(g), _p(th), _p(mm), _p(vv), g.size, ctypes.byref(hp))
    return th, mm, vv


def shard_step(partials: Sequence[np.ndarray], master: np.ndarray, m: np.ndarray,
               v: np.ndarray, hp: HParams, in_place: bool = False):
    """Reduce + AdamW + bf16 parameter; returns (master, m, v, param_bf16_bits)."""
    n = master.size
    assert all(p.size == n for p in partials) and m.size == n and v.size == n
    if in_place:
        th, mm, vv = master, m, v
    else:
        th, mm, vv = (np.array(a, dtype=np.float32, copy=True) for a in (master, m, v))
    prm = np.empty(n, dtype=np.uint16)
    lib().oracle_shard_step(_ptr_array(partials), len(partials), _gdt(partials), n,
                            _p(th), _p(mm), _p(vv), ctypes.byref(hp), _p(prm))
    return th, mm, vv, prm


def _group_of(n_ranks: int, group) -> int:
    g = n_ranks if group in (None, 0) else int(group)
    assert 1 <= g <= n_ranks and n_ranks % g == 0, "group must divide the rank count"
    return g


def reduce_ex(partials: Sequence[np.ndarray], group=None, acc=None,
              micro_batches: int = 1) -> np.ndarray:
    """fp32(((acc +) grouped sum) / (N * micro_batches)); group = ranks per
    group of the two-level order (None: one group, the flat order)."""
    n = partials[0].size
    out = np.empty(n, dtype=np.float32)
    a = None if acc is None else np.ascontiguousarray(acc, dtype=np.float32)
    lib().oracle_reduce_ex(_ptr_array(partials), len(partials), _group_of(len(partials), group),
                           _gdt(partials), None if a is None else _p(a), micro_batches, n, _p(out))
    return out


def accumulate(partials: Sequence[np.ndarray], acc=None, group=None) -> np.ndarray:
    """One non-final micro-batch: new fp32 accumulator (acc None: start)."""
    n = partials[0].size
    out = np.zeros(n, np.float32) if acc is None else np.array(acc, dtype=np.float32, copy=True)
    lib().oracle_accumulate(_ptr_array(partials), len(partials), _group_of(len(partials), group),
                            _gdt(partials), n, _p(out), 1 if acc is None else 0)
    return out


def shard_step_ex(partials: Sequence[np.ndarray], master, m, v, hp: HParams, group=None,
                  acc=None, micro_batches: int = 1):
    """Shard step with the extended reduce; returns (master, m, v, param bits)."""
    n = master.size
    th, mm, vv = (np.array(x, dtype=np.float32, copy=True) for x in (master, m, v))
    prm = np.empty(n, dtype=np.uint16)
    a = None if acc is None else np.ascontiguousarray(acc, dtype=np.float32)
    lib().oracle_shard_step_ex(_ptr_array(partials), len(partials), _group_of(len(partials), group),
                               _gdt(partials), None if a is None else _p(a), micro_batches, n,
                               _p(th), _p(mm), _p(vv), ctypes.byref(hp), _p(prm))
    return th, mm, vv, prm


def bf16_from_double(x: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bits of float64 values, one rounding."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_bf16_from_double_array(_p(x), x.size, _p(out))
    return out


def shard_step_bf16m(partials: Sequence[np.ndarray], master, m_bits, v_bits, hp: HParams):
    """Shard step on the 12-byte state (bf16 m, v as uint16 bits); returns
    (master, m_bits, v_bits, param_bits)."""
    n = master.size
    th = np.array(master, dtype=np.float32, copy=True)
    mm = np.array(m_bits, dtype=np.uint16, copy=True)
    vv = np.array(v_bits, dtype=np.uint16, copy=True)
    prm = np.empty(n, dtype=np.uint16)
    lib().oracle_shard_step_bf16m(_ptr_array(partials), len(partials), _gdt(partials), n,
                                  _p(th), _p(mm), _p(vv), ctypes.byref(hp), _p(prm))
    return th, mm, vv, prm


def kahan_add(theta_bits, comp_bits, delta):
    """Compensated add of float64 increments into bf16 (theta, comp) pairs
    (uint16 bit patterns); returns the new (theta_bits, comp_bits)."""
    th = np.array(theta_bits, dtype=np.uint16, copy=True)
    c = np.array(comp_bits, dtype=np.uint16, copy=True)
    d = np.ascontiguousarray(np.broadcast_to(np.asarray(delta, dtype=np.float64), th.shape))
    lib().oracle_kahan_add(_p(th), _p(c), _p(d), th.size)
    return th, c


def shard_step_kahan(partials: Sequence[np.ndarray], theta_bits, comp_bits, m_bits, v_bits,
                     hp: HParams):
    """Shard step on the pure-bf16 state with the compensated update: the
    parameters (shard order), compensation, m and v as uint16 bf16 bits;
    returns the new (theta, comp, m, v) bits."""
    n = len(theta_bits)
    th = np.array(theta_bits, dtype=np.uint16, copy=True)
    c = np.array(comp_bits, dtype=np.uint16, copy=True)
    mm = np.array(m_bits, dtype=np.uint16, copy=True)
    vv = np.array(v_bits, dtype=np.uint16, copy=True)
    lib().oracle_shard_step_kahan(_ptr_array(partials), len(partials), _gdt(partials), n,
                                  _p(th), _p(c), _p(mm), _p(vv), ctypes.byref(hp))
    return th, c, mm, vv


def shard_segments(numels: Sequence[int], n_ranks: int, rank: int) -> Tuple[np.ndarray, int]:
    """Pieces of rank `rank`'s shard: rows (tensor, tensor_off, shard_off, len)."""
    nm = np.ascontiguousarray(numels, dtype=np.int64)
    S = ctypes.c_int64(0)
    cap = len(numels) + 1
    seg = np.zeros((cap, 4), dtype=np.int64)
    k = lib().oracle_shard_segments(_p(nm), len(numels), n_ranks, rank, _p(seg), cap,
                                    ctypes.byref(S))
    assert k <= cap
    return seg[:k].copy(), int(S.value)


def set_threads(n: int) -> None:
    lib().oracle_set_threads(n)


def max_threads() -> int:
    return int(lib().oracle_max_threads())
