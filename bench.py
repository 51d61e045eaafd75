"""Benchmark of the fused ZeRO shard step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama70b]
                    [--secondary llama7b] [--allocations 3]

A step is one call of zero_shard_step: reduce the N gradient partials of
this rank's shard, AdamW on the shard's fp32 master/m/v, write the bf16
parameters into their slots.  Inputs are synthetic, seeded, and resident
in HBM before timing starts.  The partials are the same for every timed
step (one batch); the optimizer state advances.

Prints one JSON line: params/s over the shard (the Llama-70B rank-0 shard by
default, the largest configuration that fits one GPU), the roofline block of
the step kernel (algorithmic HBM bytes per launch / measured launch time
against the 8 TB/s HBM peak; the median of several fresh allocations), the
same record for a secondary workload (the Llama-7B rank-0 shard), plain
read/write/copy streams of the library and of the vendor's libraries, the
library's sums of 1 to 16 arrays (the rate of a mixed stream against the
number of arrays it streams), and the CPU oracle timed on a bounded sample
of the same workload on this host.

The workload setup below (allocation, device fill, warm start) is also what
the full-size GPU parity tests run, so they check the configuration timed
here.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from synth import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
# What decides the step kernels' HBM traffic: the kernels, their argument
# layout, how the chunk table is cut, and the public header (the chunk
# record, the launch-size limits).  Recorded counters stay valid while the
# code (not the comments) of these files is unchanged.
KERNEL_SOURCES = [os.path.join(ROOT, "sharded_optimizer_step_shard_amd", "csrc", f)
                  for f in ("zero_kernels.hip", "zero_internal.h", "zero_chunks.cpp")] + \
                 [os.path.join(ROOT, "include", "zero_shard.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

# Optimizer-state layouts the fused step runs on: the kernel, the state bytes
# read and written per shard element besides the N gradient partials, and a
# description.
STATES = {
    "fp32": ("shard_step_kernel", 12, 14, "fp32 master, m, v; bf16 parameter written"),
    # the same step as three kernels: reduce (2N read, 4 written), AdamW (16
    # read, 12 written), bf16 write (4 read, 2 written)
    "unfused": ("reduce_kernel+adamw_kernel+gather_kernel", 20, 18,
                "fp32 master, m, v; fp32 gradient shard between the phases"),
    "bf16-moments": ("shard_step_m16_kernel", 8, 10, "fp32 master, bf16 m, v; bf16 parameter written"),
    "bf16-kahan": ("shard_step_kahan_kernel", 8, 8,
                   "bf16 parameter (read and written in place), bf16 Kahan compensation, m, v"),
}


def code_text(src: str) -> str:
    """C/C++/HIP source with comments removed and whitespace collapsed: what
    the compiler sees, so that editing a comment keeps recorded counters."""
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("//", i):
            i = src.find("\n", i)
            i = n if i < 0 else i
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif src[i] in "\"'":
            q, j = src[i], i + 1
            while j < n and src[j] != q:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(src[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(sources=None) -> str:
    """Hash of the code (not the comments) of the kernel and host sources."""
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        h.update(code_text(open(p).read()).encode())
    return h.hexdigest()[:16]


def default_dst_mode(w: W.Workload) -> str:
    # The 70B full parameter buffer (141 GB) does not fit beside the partials
    # and state; only this rank's slot is allocated there.
    return "slot" if w.name == "llama-70b" else "tensors"


class Shard:
    """Device buffers of one rank's shard step for a workload."""

    def __init__(self, w: W.Workload, rank: int = 0, dst_mode: str = None,
                 max_chunk: int = None, device: str = "cuda"):
        import torch
        import sharded_optimizer_step_shard_amd as zs

        self.w, self.rank, self.zs = w, rank, zs
        self.dst_mode = dst_mode or default_dst_mode(w)
        max_chunk = max_chunk or (zs.ZERO_DEFAULT_MAX_CHUNK if w.gdt == "bf16"
                                  else zs.ZERO_DEFAULT_MAX_CHUNK_FP32)
        self.lo, self.hi = w.shard_range(rank)
        self.n = self.hi - self.lo
        self.S = w.shard_len
        dev = torch.device(device)
        self.dev = dev
        gtype = torch.int16 if w.gdt == "bf16" else torch.float32
        self.partials = [torch.empty(self.n, dtype=gtype, device=dev) for _ in range(w.n_ranks)]
        self.master = torch.empty(self.n, dtype=torch.float32, device=dev)
        self.m = torch.zeros(self.n, dtype=torch.float32, device=dev)
        self.v = torch.zeros(self.n, dtype=torch.float32, device=dev)
        if self.dst_mode == "slot":
            self.params = [torch.zeros(self.n, dtype=torch.int16, device=dev)]
            table, S = zs.zero_build_chunks(w.numels, w.n_ranks, rank, slot_dst=self.params[0],
                                            max_chunk=max_chunk)
        elif self.dst_mode == "tensors":
            self.params = [torch.zeros(k, dtype=torch.int16, device=dev) for k in w.numels]
            table, S = zs.zero_build_chunks(w.numels, w.n_ranks, rank, tensor_dst=self.params,
                                            max_chunk=max_chunk)
        else:
            raise ValueError(self.dst_mode)
        assert S == self.S
        # once per table: no destination overlaps a partial, the state or
        # another chunk's destination
        zs.zero_check_chunks(table, self.n, self.partials + [self.master, self.m, self.v])
        self.table = table
        self.d_table = zs.chunks_to_device(table, dev)
        self.step_t = 0
        self.buckets = [(0, len(table))]
        synth.dev_fill(self.master, w.seed, synth.stream_id(synth.KIND_MASTER), self.lo,
                       w.sigma_master)

    # -- inputs -------------------------------------------------------------
    def grad_stream(self, k: int, t: int) -> int:
        return synth.stream_id(synth.KIND_GRAD, k, t)

    def mask_stream(self, k: int, t: int) -> int:
        return synth.stream_id(synth.KIND_OUTLIER, k, t)

    def fill_partials(self, t: int, count: int = None) -> None:
        """Partials of gradient step t (per rank k: stream (grad, k, t) at the
        global flat indices of this shard); zero tensors zeroed."""
        w = self.w
        for k, p in enumerate(self.partials):
            dst = p if count is None else p[:count]
            synth.dev_fill(dst, w.seed, self.grad_stream(k, t), self.lo, w.sigma_grad,
                           self.mask_stream(k, t), w.outlier_frac, w.outlier_mult)
            for a, b in W.zero_ranges(w, self.lo, self.hi):
                if count is not None:
                    b = min(b, count)
                if a < b:
                    dst[a:b].zero_()

    def warm_start(self) -> None:
        """m, v warm start: warm_steps steps on the first warm_prefix shard
        elements (fresh partials each step), then every later element takes
        m, v from prefix element src(i) = hash(i) mod warm_prefix."""
        import torch
        w = self.w
        P = w.warm_prefix
        assert 0 < P <= self.n and P % 64 == 0
        # Prefix steps write their bf16 parameters into a scratch slot.
        scratch = torch.empty(P, dtype=torch.int16, device=self.dev)
        table, _ = self.zs.zero_build_chunks([P], 1, 0, slot_dst=scratch)
        d_table = self.zs.chunks_to_device(table, self.dev)
        for t in range(1, w.warm_steps + 1):
            self.fill_partials(t, count=P)
            self.zs.zero_shard_step([p[:P] for p in self.partials], self.master[:P], self.m[:P],
                                    self.v[:P], P, d_table, len(table),
                                    self.zs.hparams(t, **w.hparams()))
        mp, vp = self.m[:P].clone(), self.v[:P].clone()
        st = synth.stream_id(synth.KIND_PREFIX_MAP)
        synth.dev_spread(self.m, mp, w.seed, st, 0)
        synth.dev_spread(self.v, vp, w.seed, st, 0)
        torch.cuda.synchronize()
        self.step_t = w.warm_steps

    def prepare(self) -> int:
        """Bench inputs: warm start if the workload has one, then the partials
        of the first timed step.  Returns that step number."""
        if self.w.warm_prefix:
            self.warm_start()
        t0 = self.step_t + 1
        self.fill_partials(t0)
        return t0

    # -- the step -------------------------------------------------------------
    def step(self, t: int) -> None:
        self.zs.zero_shard_step(self.partials, self.master, self.m, self.v, self.n,
                                self.d_table, len(self.table),
                                self.zs.hparams(t, **self.w.hparams()))
        self.step_t = t

    def use_bf16_moments(self) -> None:
        """Switch to the 12-byte state: bf16 m and v beside the fp32 master.
        Set-up only: the current fp32 moments (zero, or warm-started) are
        rounded to bf16 with torch; the step then keeps them in bf16."""
        import torch
        self.m = self.m.to(torch.bfloat16).view(torch.int16).contiguous()
        self.v = self.v.to(torch.bfloat16).view(torch.int16).contiguous()
        self.state = "bf16-moments"

    def use_kahan(self) -> None:
        """Switch to the pure-bf16 state: the bf16 parameters at the chunks'
        destinations become the weights (written from the current fp32 master
        by the library's bf16 write), with a zero Kahan compensation and the
        moments rounded to bf16 with torch.  Set-up only; the fp32 master is
        released."""
        import torch
        self.zs.zero_gather_write(self.master, self.n, self.d_table, len(self.table))
        self.comp = torch.zeros(self.n, dtype=torch.int16, device=self.dev)
        self.m = self.m.to(torch.bfloat16).view(torch.int16).contiguous()
        self.v = self.v.to(torch.bfloat16).view(torch.int16).contiguous()
        self.master = None
        self.state = "bf16-kahan"

    def step_kahan(self, t: int) -> None:
        self.zs.zero_shard_step_kahan(self.partials, self.comp, self.m, self.v, self.n,
                                      self.d_table, len(self.table),
                                      self.zs.hparams(t, **self.w.hparams()))
        self.step_t = t

    def step_bf16_moments(self, t: int) -> None:
        self.zs.zero_shard_step_bf16_moments(self.partials, self.master, self.m, self.v, self.n,
                                             self.d_table, len(self.table),
                                             self.zs.hparams(t, **self.w.hparams()))
        self.step_t = t

    def set_extended(self, group: int, micro_batches: int) -> None:
        """Use the extended reduce: two-level order with `group` ranks per
        group, and gradient accumulation over `micro_batches` (the same
        partial buffers stand for every micro-batch)."""
        import torch
        self.group, self.micro_batches = group, micro_batches
        self.acc = (torch.empty(self.n, dtype=torch.float32, device=self.dev)
                    if micro_batches > 1 else None)

    def step_extended(self, t: int) -> None:
        for j in range(self.micro_batches - 1):
            self.zs.zero_accumulate_shard(self.partials, self.n, self.acc, reset=(j == 0),
                                          group=self.group)
        self.zs.zero_shard_step_ex(self.partials, self.master, self.m, self.v, self.n,
                                   self.d_table, len(self.table),
                                   self.zs.hparams(t, **self.w.hparams()), group=self.group,
                                   micro_batches=self.micro_batches, acc=self.acc)
        self.step_t = t

    def use_schedule(self, t0: int, count: int) -> None:
        """Constants of steps t0 .. t0+count-1 in a device table, read by
        zero_shard_step_scheduled at a device index that
        zero_step_index_advance moves on after each step (so a captured
        graph replays consecutive steps)."""
        import torch
        hps = [self.zs.hparams(t, **self.w.hparams()) for t in range(t0, t0 + count)]
        host = self.zs.zero_make_step_consts(hps)
        self.consts = torch.from_numpy(host.view(np.uint8)).to(self.dev)
        self.n_consts = count
        self.sched_index = torch.zeros(1, dtype=torch.int64, device=self.dev)

    def step_scheduled(self, t: int) -> None:
        """One step with the table's next constants (t is the table's, not
        the argument's)."""
        state = getattr(self, "state", "fp32")
        if state == "bf16-kahan":
            fn, first = self.zs.zero_shard_step_kahan_scheduled, self.comp
        elif state == "bf16-moments":
            fn, first = self.zs.zero_shard_step_bf16_moments_scheduled, self.master
        else:
            fn, first = self.zs.zero_shard_step_scheduled, self.master
        fn(self.partials, first, self.m, self.v, self.n, self.d_table, len(self.table),
           self.consts, self.n_consts, self.sched_index)
        self.zs.zero_step_index_advance(self.sched_index, self.n_consts)
        self.step_t = t

    def use_unfused(self) -> None:
        """The three phases as separate kernels (reduce into an fp32 gradient
        shard, AdamW, bf16 write), for comparison with the fused step."""
        import torch
        self.grad = torch.empty(self.n, dtype=torch.float32, device=self.dev)
        self.state = "unfused"

    def step_unfused(self, t: int) -> None:
        self.zs.zero_reduce_shard(self.partials, self.n, self.grad)
        self.zs.zero_adamw_shard(self.grad, self.master, self.m, self.v, self.n,
                                 self.zs.hparams(t, **self.w.hparams()))
        self.zs.zero_gather_write(self.master, self.n, self.d_table, len(self.table))
        self.step_t = t

    def set_buckets(self, bucket_params: int) -> list:
        """ZeRO-2 style buckets: split the chunk table into contiguous runs of
        about bucket_params shard elements (whole chunks).  Each bucket is then
        stepped by its own launch over its sub-table, as when each gradient
        bucket's reduce-scatter completes separately.  Returns the
        (first chunk, chunk count) runs."""
        self.buckets = bucket_runs(self.table["len"], bucket_params)
        return self.buckets

    def step_bucketed(self, t: int) -> None:
        """All buckets enqueued by one call (zero_shard_step_buckets)."""
        self.zs.zero_shard_step_buckets(self.partials, self.master, self.m, self.v, self.n,
                                        self.d_table, len(self.table), self.buckets,
                                        self.zs.hparams(t, **self.w.hparams()))
        self.step_t = t

    def step_bucketed_loop(self, t: int) -> None:
        """One zero_shard_step call per bucket from Python."""
        hp = self.zs.hparams(t, **self.w.hparams())
        base = self.d_table.data_ptr()
        for first, count in self.buckets:
            self.zs.zero_shard_step(self.partials, self.master, self.m, self.v, self.n,
                                    base + 32 * first, count, hp)
        self.step_t = t

    def param_at(self, shard_idx: np.ndarray):
        """bf16 bits written for the given shard indices (device gather)."""
        import torch
        if self.dst_mode == "slot":
            flat = self.params[0]
            idx = torch.from_numpy(shard_idx).to(self.dev)
            return flat[idx].cpu().numpy().view(np.uint16)
        starts = np.cumsum([0] + self.w.numels[:-1])
        g = shard_idx + self.lo
        t = np.searchsorted(starts, g, side="right") - 1
        out = np.empty(len(g), np.uint16)
        for tt in np.unique(t):
            sel = np.nonzero(t == tt)[0]
            idx = torch.from_numpy(g[sel] - starts[tt]).to(self.dev)
            out[sel] = self.params[tt][idx].cpu().numpy().view(np.uint16)
        return out

    def bytes_per_launch(self) -> int:
        _, rd, wr, _ = STATES[getattr(self, "state", "fp32")]
        return (self.w.n_ranks * (2 if self.w.gdt == "bf16" else 4) + rd + wr) * self.n


def bucket_chunk_len(bucket_params: int) -> int:
    """Chunk length for a step launched per bucket of about bucket_params
    elements: bucket_params / 1024 rounded down to a power of two, within
    [512, 2048].  A launch's waves each walk their chunk in groups of 512
    elements (64 lanes x 8), one memory round trip per group, so a small
    bucket cut into 2048-element chunks is a few latency-bound waves; about
    a thousand chunks per bucket keeps the round trips in parallel.  Measured
    on MI355X (7B shard, replayed from a HIP graph): 262K-element buckets
    12.2 -> 6.4 us per launch with 512-element chunks, 1M-element buckets
    16.2 -> 13.7 us with 1024; from 4M on, 2048 stays best."""
    if bucket_params <= 0:
        raise ValueError("bucket_params must be positive")
    c = 2048
    while c > 512 and c * 1024 > bucket_params:
        c //= 2
    return c


def bucket_runs(chunk_lens, bucket_params: int) -> list:
    """Split a chunk table (its len column) into contiguous runs of whole
    chunks holding at least bucket_params elements each (the last run may
    hold fewer); returns (first chunk, chunk count) pairs covering every
    chunk once, in order."""
    lens = np.asarray(chunk_lens, dtype=np.int64)
    if bucket_params <= 0:
        raise ValueError("bucket_params must be positive")
    ends = np.cumsum(lens)
    runs, first = [], 0
    while first < len(lens):
        base = ends[first - 1] if first else 0
        last = int(np.searchsorted(ends, base + bucket_params, side="left"))
        last = min(max(last, first), len(lens) - 1)
        runs.append((first, last - first + 1))
        first = last + 1
    return runs


def cpu_baseline(w: W.Workload, rank: int, t: int, target_s: float = 10.0,
                 sample: int = 1 << 30, state: str = "fp32", single_sample: int = 1 << 24) -> dict:
    """The CPU oracle of the same step (the same state layout) on a bounded
    sample (the first `sample` shard elements) of the same workload, on all
    host threads, repeated until ~target_s of work; params/s.  Then the same
    on one thread over the first `single_sample` elements."""
    import oracle

    lo, hi = w.shard_range(rank)
    n = min(sample, hi - lo)
    t_gen = time.perf_counter()
    parts = [synth.fill(w.gdt, w.seed, synth.stream_id(synth.KIND_GRAD, k, t), lo, n,
                        w.sigma_grad, synth.stream_id(synth.KIND_OUTLIER, k, t),
                        w.outlier_frac, w.outlier_mult) for k in range(w.n_ranks)]
    for a, b in W.zero_ranges(w, lo, lo + n):
        for p in parts:
            p[a:b] = 0
    master = synth.fill("f32", w.seed, synth.stream_id(synth.KIND_MASTER), lo, n, w.sigma_master)
    gen_s = time.perf_counter() - t_gen

    def run(k: int, budget: float) -> tuple:
        """Oracle steps over the first k elements until `budget` seconds
        (at least one step)."""
        sub = [p[:k] for p in parts]
        if state in ("fp32", "unfused"):
            th, m, v = master[:k].copy(), np.zeros(k, np.float32), np.zeros(k, np.float32)
        elif state == "bf16-moments":
            th, m16, v16 = master[:k].copy(), np.zeros(k, np.uint16), np.zeros(k, np.uint16)
        else:
            th16, c16 = oracle.bf16_round(master[:k]), np.zeros(k, np.uint16)
            m16, v16 = np.zeros(k, np.uint16), np.zeros(k, np.uint16)
        done, elapsed, reps = 0, 0.0, 0
        while elapsed < budget or reps == 0:
            hp = oracle.hparams(t + reps, **w.hparams())
            t0 = time.perf_counter()
            if state in ("fp32", "unfused"):
                oracle.shard_step(sub, th, m, v, hp, in_place=True)
            elif state == "bf16-moments":
                th, m16, v16, _ = oracle.shard_step_bf16m(sub, th, m16, v16, hp)
            else:
                th16, c16, m16, v16 = oracle.shard_step_kahan(sub, th16, c16, m16, v16, hp)
            elapsed += time.perf_counter() - t0
            done += k
            reps += 1
        return done / elapsed, reps, elapsed

    cores = oracle.max_threads()
    value, reps, elapsed = run(n, target_s)
    n1 = max(1, min(n // 4, single_sample))
    oracle.set_threads(1)
    try:
        value1, reps1, elapsed1 = run(n1, target_s / 4)
    finally:
        oracle.set_threads(cores)
    _, rd, wr, _ = STATES[state]
    bpp = w.n_ranks * (2 if w.gdt == "bf16" else 4) + rd + wr
    return {"value": value, "unit": "params/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {n} elements of rank {rank}'s shard of {w.name}, N={w.n_ranks} "
                      f"{w.gdt} partials, {state} state, {reps} oracle steps in {elapsed:.1f} s "
                      f"(inputs generated on the host in {gen_s:.1f} s, not timed)",
            "sample_elements": n,
            "host_gbs": value * bpp / 1e9,
            "single_thread": {"value": value1, "unit": "params/s",
                              "sample": f"first {n1} elements, {reps1} steps in {elapsed1:.1f} s"},
            "cpu_model": cpu_model()}


def probe_copy(nbytes: int, reps: int = 5) -> dict:
    """Plain device-to-device copy of nbytes (read nbytes + write nbytes)
    with zero_probe_copy: the attainable streaming rate next to the step's."""
    import torch
    import sharded_optimizer_step_shard_amd as zs
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    zs.zero_probe_copy(src, dst, nbytes)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        zs.zero_probe_copy(src, dst, nbytes)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_copied": nbytes, "ms": ms, "gbs": 2 * nbytes / (ms * 1e-3) / 1e9,
            "frac_of_peak": 2 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def probe_read(nbytes: int, reps: int = 5) -> dict:
    """Read-only stream over nbytes with zero_probe_read: the attainable read
    rate beside the copy rate (the step is 2:1 read/write)."""
    import torch
    import sharded_optimizer_step_shard_amd as zs
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    src.fill_(1)
    zs.zero_probe_read(src, nbytes, sink)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        zs.zero_probe_read(src, nbytes, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, sink
    torch.cuda.empty_cache()
    return {"bytes_read": nbytes, "ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def launch_overhead(n_ranks: int = 8, n: int = 1 << 16, calls: int = 4000,
                    max_chunk: int = None) -> dict:
    """Per-call cost of zero_shard_step on a small shard (n elements, 32
    chunks): the C call through ctypes with no chunks (argument checks only),
    the full C call (checks, one device-range query per array, launch; host
    issue time and time including the GPU's completion), and the same through
    the Python binding.  Microseconds per call."""
    import ctypes
    import torch
    import sharded_optimizer_step_shard_amd as zs
    parts = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(n_ranks)]
    master, m, v = (torch.zeros(n, device="cuda") for _ in range(3))
    slot = torch.zeros(n, dtype=torch.int16, device="cuda")
    table, _ = zs.zero_build_chunks([n], 1, 0, slot_dst=slot,
                                    max_chunk=max_chunk or zs.ZERO_DEFAULT_MAX_CHUNK)
    d_table = zs.chunks_to_device(table)
    hp = zs.hparams(3)
    stream = torch.cuda.current_stream().cuda_stream
    pp = (ctypes.c_void_p * n_ranks)(*[p.data_ptr() for p in parts])
    full = (pp, n_ranks, 0, master.data_ptr(), m.data_ptr(), v.data_ptr(), n, d_table.data_ptr(),
            len(table), ctypes.byref(hp), stream)
    empty = full[:8] + (0,) + full[9:]
    lib = zs.lib()

    def per_call(fn):
        for _ in range(200):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(calls):
            fn()
        t1 = time.perf_counter()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        return (t1 - t0) / calls * 1e6, (t2 - t0) / calls * 1e6

    checks, _ = per_call(lambda: lib.zero_shard_step(*empty))
    c_issue, c_done = per_call(lambda: lib.zero_shard_step(*full))
    py_issue, py_done = per_call(lambda: zs.zero_shard_step(parts, master, m, v, n, d_table,
                                                            len(table), hp))
    # the same launches captured in a HIP graph and replayed: GPU time per launch
    in_graph, replays = 500, 10
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for _ in range(in_graph):
                zs.zero_shard_step(parts, master, m, v, n, d_table, len(table), hp)
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / (in_graph * replays)
    return {"elements": n, "chunks": len(table), "n_ranks": n_ranks, "calls": calls,
            "c_checks_only_us": checks, "c_full_issue_us": c_issue, "c_full_with_gpu_us": c_done,
            "python_issue_us": py_issue, "python_with_gpu_us": py_done,
            "graph_replay_per_launch_us": graph_us}


def probe_write(nbytes: int, reps: int = 5) -> dict:
    """Write-only stream over nbytes with zero_probe_write (the step kernels'
    non-temporal stores): the attainable write rate."""
    import torch
    import sharded_optimizer_step_shard_amd as zs
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    zs.zero_probe_write(dst, nbytes)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        zs.zero_probe_write(dst, nbytes)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del dst
    torch.cuda.empty_cache()
    return {"bytes_written": nbytes, "ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def mix_bound(read_bytes: float, write_bytes: float, read_gbs: float, write_gbs: float) -> float:
    """Attainable GB/s of a stream that moves read_bytes and write_bytes if
    the reads go at the read-only rate and the writes at the write-only rate,
    one after the other: (R + W) / (R / r + W / w)."""
    return (read_bytes + write_bytes) / (read_bytes / read_gbs + write_bytes / write_gbs)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def load_traffic(kernel_key: str) -> dict:
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec


def _csv_rows(path: str):
    import csv
    with open(path, newline="") as f:
        yield from csv.DictReader(f)


def _counter_per_dispatch(path: str, counter: str, name_part: str) -> tuple:
    """Mean of one rocprofv3 counter (KiB per dispatch) over the dispatches of
    the kernel whose name holds name_part, at its largest grid; returns
    (mean, dispatch count, grid)."""
    by_grid = {}
    for r in _csv_rows(path):
        if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
            by_grid.setdefault(int(r["Grid_Size"]), []).append(float(r["Counter_Value"]))
    if not by_grid:
        raise SystemExit(f"{path}: no {counter} rows for a kernel named *{name_part}*")
    grid = max(by_grid)
    vals = by_grid[grid]
    return sum(vals) / len(vals), len(vals), grid


def ingest_counters(fetch_csv: str, write_csv: str, w: "W.Workload", rank: int, state: str,
                    probe_bytes: int) -> dict:
    """HBM traffic of one full-shard step launch from two rocprofv3 counter
    passes (FETCH_SIZE, then WRITE_SIZE) over the same bench command with
    --probe-copy: the copy kernel's known bytes turn each counter's KiB into
    bytes.  Records the result in profiles/traffic.json under the kernel
    source's hash (bench reports it as roofline.traffic only while the
    source is unchanged) and returns the record."""
    kname, rd, wr, _ = STATES[state]
    kernel_key = f"{kname}<{w.gdt},{w.n_ranks}>/{w.name}"
    f_kb, f_n, grid = _counter_per_dispatch(fetch_csv, "FETCH_SIZE", kname)
    w_kb, w_n, _ = _counter_per_dispatch(write_csv, "WRITE_SIZE", kname)
    pf_kb, _, _ = _counter_per_dispatch(fetch_csv, "FETCH_SIZE", "probe_copy_kernel")
    pw_kb, _, _ = _counter_per_dispatch(write_csv, "WRITE_SIZE", "probe_copy_kernel")
    f_factor, w_factor = probe_bytes / pf_kb, probe_bytes / pw_kb
    lo, hi = w.shard_range(rank)
    n = hi - lo
    alg_read = (w.n_ranks * (2 if w.gdt == "bf16" else 4) + rd) * n
    alg_write = wr * n
    rec = {
        "source_hash": kernel_source_hash(),
        "bytes_per_launch": f_kb * f_factor + w_kb * w_factor,
        "fetch_bytes_per_launch": f_kb * f_factor,
        "write_bytes_per_launch": w_kb * w_factor,
        "algorithmic_read_bytes": alg_read,
        "algorithmic_write_bytes": alg_write,
        "fetch_over_algorithmic": f_kb * f_factor / alg_read,
        "write_over_algorithmic": w_kb * w_factor / alg_write,
        "total_over_algorithmic": (f_kb * f_factor + w_kb * w_factor) / (alg_read + alg_write),
        "fetch_size_counter_kb_per_launch": f_kb,
        "write_size_counter_kb_per_launch": w_kb,
        "dispatches": [f_n, w_n],
        "grid": grid,
        "calibration": {
            "kernel": "zs::probe_copy_kernel",
            "bytes_read": probe_bytes,
            "bytes_written": probe_bytes,
            "fetch_size_kb": pf_kb,
            "write_size_kb": pw_kb,
            "fetch_factor_bytes_per_kb": f_factor,
            "write_factor_bytes_per_kb": w_factor,
        },
    }
    try:
        table = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        table = {}
    table[kernel_key] = rec
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    return {kernel_key: rec}


def trace_summary(kernel_trace_csv: str) -> str:
    """Markdown table of a rocprofv3 --kernel-trace CSV: per kernel and grid,
    dispatch count and launch durations in microseconds."""
    import statistics
    groups, meta = {}, {}
    for r in _csv_rows(kernel_trace_csv):
        key = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        meta[key] = (r["VGPR_Count"], r["Accum_VGPR_Count"], r["SGPR_Count"], r["Scratch_Size"])
    lines = ["| kernel | grid (work-items) | workgroup | dispatches | avg us | median us | min us "
             "| max us | VGPR/AGPR/SGPR | scratch |", "|---|---|---|---|---|---|---|---|---|---|"]
    for key, d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        name = key[0].replace("|", "/")
        name = name if len(name) <= 70 else name[:67] + "..."
        v, a, sg, sc = meta[key]
        lines.append(f"| {name} | {key[1]} | {key[2]} | {len(d)} | {statistics.mean(d):.1f} | "
                     f"{statistics.median(d):.1f} | {min(d):.1f} | {max(d):.1f} | {v}/{a}/{sg} | {sc} |")
    return "\n".join(lines)


def setup_step(sh: Shard, args, t: int):
    """Select the step of the requested mode on a prepared shard; returns
    (step function, launches per step, extended?)."""
    import torch
    step = sh.step
    extended = args.group > 0 or args.micro_batches > 1
    if extended and args.bucket_params > 0:
        raise SystemExit("--bucket-params does not combine with --group/--micro-batches")
    if args.state != "fp32":
        if extended or args.bucket_params > 0:
            raise SystemExit(f"--state {args.state} runs the plain fused step only")
        if args.state == "unfused":
            if args.scheduled or args.graph:
                raise SystemExit("--state unfused runs eagerly with launch-argument constants")
            sh.use_unfused()
            step = sh.step_unfused
        elif args.state == "bf16-moments":
            sh.use_bf16_moments()
            step = sh.step_bf16_moments
        else:
            sh.use_kahan()
            step = sh.step_kahan
    if args.scheduled:
        if extended or args.bucket_params > 0:
            raise SystemExit("--scheduled runs the plain fused step of each state layout")
        sh.use_schedule(t, args.warmup + args.steps + 1)
        step = sh.step_scheduled
    if args.bucket_params > 0:
        sh.set_buckets(args.bucket_params)
        step = sh.step_bucketed if args.bucket_call == "one" else sh.step_bucketed_loop
    elif extended:
        sh.set_extended(args.group, args.micro_batches)
        step = sh.step_extended
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                step(t)
        torch.cuda.current_stream().wait_stream(side)
        step = lambda _t: graph.replay()        # noqa: E731
    launches = len(sh.buckets) if args.bucket_params > 0 else 1
    return step, launches, extended


def time_allocation(w: W.Workload, args, alloc: int) -> dict:
    """One fresh allocation of the shard: allocate (behind a spacer whose size
    differs per allocation, so that the buffers land elsewhere), fill, warm
    start, W untimed steps, then exactly K timed steps.  Returns the
    measurement; everything is freed before returning."""
    import torch
    # spacer: 0, 1 GiB + 2 MiB, 2 GiB + 4 MiB, ...
    spacer = torch.empty(alloc * ((1 << 30) + (2 << 20)), dtype=torch.uint8, device="cuda")
    max_chunk = args.max_chunk
    if max_chunk is None and args.bucket_params > 0:
        max_chunk = bucket_chunk_len(args.bucket_params)
    sh = Shard(w, args.rank, args.dst, max_chunk)
    t = sh.prepare()
    torch.cuda.synchronize()
    print(f"# {w.name} allocation {alloc}: shard {sh.n} params, N={w.n_ranks} {w.gdt}, "
          f"{len(sh.table)} chunks, dst={sh.dst_mode}, first timed step t={t + args.warmup}",
          file=sys.stderr, flush=True)
    step, launches, extended = setup_step(sh, args, t)
    for _ in range(args.warmup):
        step(t)
        t += 1
    stream = torch.cuda.current_stream()
    # one event between consecutive steps: launch k's time is evs[k] -> evs[k+1]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for k in range(args.steps):
        step(t)
        t += 1
        evs[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = wall * 1e3 / args.steps
    step_ms = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps))
    kernel_ms = evs[0].elapsed_time(evs[-1]) / args.steps / launches   # average launch
    ext = None
    if extended:
        # Time the final fused launch on its own (same state, next steps) so
        # the roofline is the fused kernel's; the step time above includes
        # the accumulation passes.
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e2.record(stream)
        for _ in range(args.steps):
            sh.zs.zero_shard_step_ex(sh.partials, sh.master, sh.m, sh.v, sh.n, sh.d_table,
                                     len(sh.table), sh.zs.hparams(t, **w.hparams()),
                                     group=args.group, micro_batches=args.micro_batches,
                                     acc=sh.acc)
            t += 1
        e3.record(stream)
        torch.cuda.synchronize()
        kernel_ms = e2.elapsed_time(e3) / args.steps
        ext = {"group": args.group, "micro_batches": args.micro_batches,
               "step_ms_including_accumulation": ms_per_step}
    bytes_launch = sh.bytes_per_launch() / launches
    if extended and args.micro_batches > 1:
        bytes_launch += 4 * sh.n           # the accumulator read by the fused launch
    res = {"alloc": alloc, "n": sh.n, "chunks": len(sh.table), "dst": sh.dst_mode,
           "max_chunk": int(sh.table["len"].max()) if len(sh.table) else 0,
           "bytes_per_param": sh.bytes_per_launch() // sh.n, "launches": launches,
           "ms_per_step": ms_per_step, "kernel_ms": kernel_ms, "step_ms": step_ms,
           "bytes_launch": bytes_launch, "extended": ext, "next_t": t,
           "achieved": bytes_launch / (kernel_ms * 1e-3) / 1e9}
    del step, sh, spacer
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def chunk_sweep(w: W.Workload, args, lengths, rounds: int = 3) -> dict:
    """The plain fused step with chunk tables cut at each of `lengths`, over
    the same buffers of one allocation, taken round-robin `rounds` times
    (W untimed and K timed steps per turn): the fraction of HBM peak per
    chunk length, free of the spread between allocations."""
    import torch
    zs_ = __import__("sharded_optimizer_step_shard_amd")
    sh = Shard(w, args.rank, args.dst, max(lengths))
    t = sh.prepare()
    kw = ({"slot_dst": sh.params[0]} if sh.dst_mode == "slot" else {"tensor_dst": sh.params})
    tables = {}
    for mc in lengths:
        table, _ = zs_.zero_build_chunks(w.numels, w.n_ranks, args.rank, max_chunk=mc, **kw)
        zs_.zero_check_chunks(table, sh.n, sh.partials + [sh.master, sh.m, sh.v])
        tables[mc] = (zs_.chunks_to_device(table), len(table))
    stream = torch.cuda.current_stream()
    res = {mc: [] for mc in lengths}
    for _ in range(rounds):
        for mc in lengths:
            dt, nc = tables[mc]

            def step():
                nonlocal t
                zs_.zero_shard_step(sh.partials, sh.master, sh.m, sh.v, sh.n, dt, nc,
                                    zs_.hparams(t, **w.hparams()))
                t += 1
            for _ in range(args.warmup):
                step()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                step()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            res[mc].append(sh.bytes_per_launch() / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    return {"workload": f"{w.name} rank-{args.rank} shard", "steps_per_turn": args.steps,
            "rounds": rounds,
            "by_max_chunk": {str(mc): {"chunks": tables[mc][1], "frac": fr,
                                       "median": sorted(fr)[len(fr) // 2]}
                             for mc, fr in res.items()}}


def measure_workload(w: W.Workload, args) -> dict:
    """The step on `args.allocations` fresh allocations of the shard; the
    record of the allocation with the median roofline fraction, with the
    fractions of all of them."""
    runs = [time_allocation(w, args, a) for a in range(args.allocations)]
    fr = [r["achieved"] / HBM_PEAK_GBS for r in runs]
    order = sorted(range(len(runs)), key=lambda i: fr[i])
    med = runs[order[len(order) // 2]]
    med["frac_by_allocation"] = {"min": min(fr), "median": fr[order[len(order) // 2]],
                                 "max": max(fr), "values": fr}
    return med


def workload_record(w: W.Workload, args, r: dict) -> dict:
    """The metric, config and roofline of one measured workload."""
    extended = r["extended"] is not None
    kname = "shard_step_sched_kernel" if args.scheduled else STATES[args.state][0]
    kernel_key = f"{kname}<{w.gdt},{w.n_ranks}{',ext' if extended else ''}>/{w.name}"
    traffic = load_traffic(kernel_key) if r["launches"] == 1 else None
    achieved = r["achieved"]
    out = {
        "value": r["n"] / (r["ms_per_step"] * 1e-3),
        "unit": "params/s",
        "ms_per_step": r["ms_per_step"],
        "config": {"workload": f"{w.name} rank-{args.rank} shard", "shard_params": r["n"],
                   "n_ranks": w.n_ranks, "grad_dtype": w.gdt,
                   "state_dtype": STATES[args.state][3],
                   "param_dtype": "bf16", "tensors": len(w.numels), "chunks": r["chunks"],
                   "dst": r["dst"], "bytes_per_param": r["bytes_per_param"],
                   "state": args.state,
                   "launches_per_step": r["launches"],
                   "max_chunk": r["max_chunk"],
                   "graph_replay": bool(args.graph),
                   "scheduled_constants": bool(args.scheduled),
                   "bucket_call": args.bucket_call if args.bucket_params > 0 else None,
                   "parallelism": "one data-parallel rank's ZeRO shard"},
        "hbm_gbs": achieved,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None if traffic is None else traffic["bytes_per_launch"],
                     "kernel": kernel_key, "kernel_ms": r["kernel_ms"],
                     "algorithmic_bytes_per_launch": r["bytes_launch"],
                     "step_ms_median": r["step_ms"][len(r["step_ms"]) // 2],
                     "step_ms_min": r["step_ms"][0],
                     "frac_by_allocation": r["frac_by_allocation"]},
    }
    if extended:
        out["extended_reduce"] = r["extended"]
    return out


def best_rates(probes: dict, vendor: dict = None) -> tuple:
    """The highest read-only and write-only rates measured in this run: the
    library's probes, and the vendor's write-only fill when it was timed."""
    read = probes["probe_read"]["gbs"]
    write = probes["probe_write"]["gbs"]
    if vendor and "torch_fill_" in vendor:
        write = max(write, vendor["torch_fill_"]["gbs"])
    return read, write


def add_mix_model(rec: dict, w: W.Workload, args, n: int, probes: dict,
                  vendor: dict = None, sums: dict = None) -> None:
    """The step's rate against the same run's plain-stream rates: the copy
    and read probes, the serial bound of its own read/write mix from the
    best read-only and write-only rates of the run, and (when timed) the
    library's sums of many arrays, the attainable rate of a stream with
    about as many arrays as the step's."""
    rl = rec["roofline"]
    achieved = rl["achieved"]
    rl["vs_copy_probe"] = achieved / probes["probe_copy"]["gbs"]
    rl["vs_read_probe"] = achieved / probes["probe_read"]["gbs"]
    _, rd, wr, _ = STATES[args.state]
    gb = 2 if w.gdt == "bf16" else 4
    rb, wb = (w.n_ranks * gb + rd) * n, wr * n
    if args.micro_batches > 1:
        rb += 4 * n
    read, write = best_rates(probes, vendor)
    bound = mix_bound(rb, wb, read, write)
    rl["mix_model"] = {"read_bytes": rb, "write_bytes": wb, "read_gbs": read, "write_gbs": write,
                       "bound_gbs": bound, "frac_of_bound": achieved / bound}
    if sums:
        rl["vs_sum_streams"] = {k: achieved / v["gbs"] for k, v in sums.items() if k in ("k8", "k16")}


def vendor_streams(nbytes: int, probes: dict, reps: int = 10) -> dict:
    """Element-wise streams of the vendor's libraries (torch's HIP kernels),
    which this library did not write, on fp32 operands of nbytes each: the
    2:1 read/write mix of torch.add, the 3:1 mix of torch.addcmul, the 1:1
    device-to-device copy and the write-only fill.  Each with its rate, its
    fraction of the 8 TB/s peak and of its own serial read/write bound from
    the same run's best read-only and write-only rates."""
    import torch
    n = nbytes // 4
    a = torch.full((n,), 1.0, device="cuda")
    b = torch.full((n,), 2.0, device="cuda")
    c = torch.empty(n, device="cuda")
    d = torch.empty(n, device="cuda")
    cases = {
        "torch_add_out": (lambda: torch.add(a, b, out=c), 2, 1),
        "torch_addcmul_out": (lambda: torch.addcmul(a, b, c, out=d), 3, 1),
        "torch_copy_": (lambda: c.copy_(a), 1, 1),
        "torch_fill_": (lambda: d.fill_(3.0), 0, 1),
    }
    out = {}
    stream = torch.cuda.current_stream()
    for name, (fn, r, wr) in cases.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        rb, wb = r * 4 * n, wr * 4 * n
        gbs = (rb + wb) / (ms * 1e-3) / 1e9
        out[name] = {"read_bytes": rb, "write_bytes": wb, "ms": ms, "gbs": gbs,
                     "frac_of_peak": gbs / HBM_PEAK_GBS}
    # bounds from the best read-only and write-only rates, the fill's included
    rates = best_rates(probes, out)
    for v in out.values():
        v["frac_of_mix_bound"] = v["gbs"] / mix_bound(v["read_bytes"], v["write_bytes"], *rates)
    del a, b, c, d
    torch.cuda.empty_cache()
    return out


def sum_streams(probes: dict, vendor: dict = None, n: int = 1 << 28, ks=(1, 2, 3, 4, 8, 16),
                reps: int = 10) -> dict:
    """The library's sum probe (dst = src[0] + ... + src[k-1], fp32, one
    64-lane workgroup per 1 KiB of dst) over k source arrays of n floats:
    how the rate of a mixed stream depends on the number of arrays streamed
    at once.  Each with its rate, fraction of the 8 TB/s peak and of its own
    serial read/write bound from the run's best read-only and write-only
    rates."""
    import torch
    import sharded_optimizer_step_shard_amd as zs
    srcs = [torch.full((n,), float(j + 1), device="cuda") for j in range(max(ks))]
    dst = torch.empty(n, device="cuda")
    rates = best_rates(probes, vendor)
    stream = torch.cuda.current_stream()
    out = {}
    for k in ks:
        def run():
            zs.zero_probe_sum(srcs[:k], dst, n)
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        rb, wb = k * 4 * n, 4 * n
        gbs = (rb + wb) / (ms * 1e-3) / 1e9
        out[f"k{k}"] = {"read_bytes": rb, "write_bytes": wb, "ms": ms, "gbs": gbs,
                        "frac_of_peak": gbs / HBM_PEAK_GBS,
                        "frac_of_mix_bound": gbs / mix_bound(rb, wb, *rates)}
    if not torch.equal(dst[:1024], torch.full((1024,), float(max(ks) * (max(ks) + 1) // 2),
                                              device="cuda")):
        raise RuntimeError("sum probe result is wrong")
    del srcs, dst
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama70b", choices=sorted(W.ALL),
                    help="the headline workload (default: the Llama-70B rank-0 shard, the "
                         "largest configuration that fits one GPU)")
    ap.add_argument("--secondary", default="llama7b", choices=sorted(W.ALL) + ["none"],
                    help="a second workload measured the same way and nested in the line "
                         "(default: the Llama-7B rank-0 shard); 'none' to skip")
    ap.add_argument("--allocations", type=int, default=3,
                    help="fresh allocations of each shard, each timed for K steps; the line "
                         "reports the allocation with the median roofline fraction")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--dst", default=None, choices=["slot", "tensors"])
    ap.add_argument("--max-chunk", type=int, default=None,
                    help="chunk-table cut length (default: the library's tuned value)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=1 << 30,
                    help="shard elements the CPU oracle is timed on")
    ap.add_argument("--no-vendor-streams", action="store_true",
                    help="skip the vendor streams and the library's sum streams")
    ap.add_argument("--state", default="fp32", choices=sorted(STATES),
                    help="optimizer state: fp32 master, m, v (16 B/param ledger); fp32 "
                         "master with bf16 m, v (12 B/param ledger); or pure bf16 with a "
                         "Kahan-compensated update (no master, 10 B/param).  'unfused' runs "
                         "the 16 B/param step as three kernels (reduce, AdamW, bf16 write)")
    ap.add_argument("--group", type=int, default=0,
                    help="two-level reduce: ranks per group (hybrid sharding); 0 = flat")
    ap.add_argument("--micro-batches", type=int, default=1,
                    help="gradient accumulation: micro-batches per optimizer step")
    ap.add_argument("--bucket-params", type=int, default=0,
                    help="step the shard in buckets of about this many params, one launch "
                         "per bucket (ZeRO-2 bucketed step); 0 = one launch per step")
    ap.add_argument("--bucket-call", default="one", choices=["one", "per-bucket"],
                    help="with --bucket-params: enqueue all buckets with one "
                         "zero_shard_step_buckets call, or call zero_shard_step per bucket")
    ap.add_argument("--scheduled", action="store_true",
                    help="take the step constants from a device table (zero_shard_step_"
                         "scheduled + zero_step_index_advance): with --graph every replay "
                         "is the next step")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step's launches in a HIP graph and time its replays "
                         "(the hyper-parameters, step t included, are fixed at capture; the "
                         "work per replay is the step's)")
    ap.add_argument("--probe-copy", type=int, default=1 << 32, metavar="BYTES",
                    help="after timing, copy BYTES with the library's plain copy kernel "
                         "(measured copy bandwidth of this GPU; the known-size kernel that "
                         "calibrates HBM traffic counters); 0 to skip")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn the counter_collection CSVs of two rocprofv3 passes "
                         "(--pmc FETCH_SIZE, --pmc WRITE_SIZE) over this same command into "
                         "calibrated HBM bytes per launch, recorded in profiles/traffic.json")
    ap.add_argument("--launch-overhead", action="store_true",
                    help="print the per-call cost of zero_shard_step on a small shard (JSON)")
    ap.add_argument("--chunk-sweep", metavar="LENGTHS",
                    help="comma-separated chunk lengths: time the plain step with a table cut "
                         "at each, round-robin over the same buffers (JSON), instead of the "
                         "benchmark line")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="no GPU: print a markdown table of a rocprofv3 kernel trace")
    args = ap.parse_args()

    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return 0
    if args.launch_overhead:
        print(json.dumps(launch_overhead(max_chunk=args.max_chunk)), flush=True)
        return 0
    if args.ingest_counters:
        rec = ingest_counters(*args.ingest_counters, W.get(args.workload), args.rank, args.state,
                              args.probe_copy)
        print(json.dumps(rec, indent=1))
        return 0

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs one rank's shard step on one GPU; "
                                   "--gpus above 1 is not supported (the collectives that "
                                   "would feed it are out of scope)"}), flush=True)
        return 2
    if args.allocations < 1:
        raise SystemExit("--allocations must be at least 1")

    import torch

    w = W.get(args.workload)
    if args.chunk_sweep:
        lengths = [int(x) for x in args.chunk_sweep.split(",")]
        print(json.dumps(chunk_sweep(w, args, lengths)), flush=True)
        return 0
    r = measure_workload(w, args)
    rec = workload_record(w, args, r)
    out = {
        "metric": "params updated/sec and achieved HBM GB/s (fraction of peak), fused shard step",
        "value": rec["value"],
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": rec["config"],
        "hbm_gbs": rec["hbm_gbs"],
        "roofline": rec["roofline"],
    }
    if "extended_reduce" in rec:
        out["extended_reduce"] = rec["extended_reduce"]
    sec = None
    if args.secondary != "none" and args.secondary != args.workload:
        w2 = W.get(args.secondary)
        r2 = measure_workload(w2, args)
        sec = workload_record(w2, args, r2)
        out["secondary"] = sec
    props = torch.cuda.get_device_properties(0)
    out["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                     "compute_units": props.multi_processor_count,
                     "memory_gib": round(props.total_memory / 2**30, 1)}
    if args.probe_copy > 0:
        probes = {"probe_copy": probe_copy(args.probe_copy),
                  "probe_read": probe_read(args.probe_copy),
                  "probe_write": probe_write(args.probe_copy)}
        out.update(probes)
        vendor = None
        if not args.no_vendor_streams:
            vendor = out["vendor_streams"] = vendor_streams(args.probe_copy, probes)
            out["sum_streams"] = sum_streams(probes, vendor)
        add_mix_model(out, w, args, r["n"], probes, vendor, out.get("sum_streams"))
        if sec is not None:
            add_mix_model(sec, w2, args, r2["n"], probes, vendor, out.get("sum_streams"))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.rank, r["next_t"], args.cpu_seconds,
                                           sample=args.cpu_sample, state=args.state)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
