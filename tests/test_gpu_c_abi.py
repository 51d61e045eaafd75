"""The C ABI from a plain C program (tests/c_abi/step_c.c, built by
__graft_entry__.build() with gcc against libzero_shard.so): no Python, no
torch on the library side.  The program's results are compared with the
oracle.  State 2 captures the scheduled step in a HIP graph with the HIP C
API and launches it once per step of its table (four steps, then one launch
past the end that must change nothing)."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from synth import workloads as W
from gpu_helpers import assert_bitwise, host_master, host_partials, say

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "step_c")


@pytest.mark.parametrize("state", [0, 1, 2])
def test_plain_c_program_matches_oracle(tmp_path, state):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} not built: run __graft_entry__.build()")
    numels = [1000, 7, 4093, 64, 20003]
    n_ranks, rank, t = 4, 2, 3
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
    w = W.Workload("c", 92, numels, n_ranks, "bf16", 1e-3)
    lo, hi = w.shard_range(rank)
    n = hi - lo
    idx = np.arange(lo, hi, dtype=np.int64)
    parts = host_partials(w, t, idx)
    master = host_master(w, idx)
    rng = np.random.default_rng(5)
    if state in (0, 2):
        m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v = (rng.random(n) * 1e-8).astype(np.float32)
    else:
        m = oracle.bf16_from_double(rng.standard_normal(n) * 1e-4)
        v = oracle.bf16_from_double(rng.random(n) * 1e-8)
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([n_ranks, len(numels), rank, state], np.int32).tobytes())
        f.write(np.array([t], np.int64).tobytes())
        f.write(np.array([hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"]],
                         np.float64).tobytes())
        f.write(np.array(numels, np.int64).tobytes())
        for p in parts:
            f.write(p.tobytes())
        f.write(master.tobytes())
        f.write(m.tobytes())
        f.write(v.tobytes())
    say(f"case: plain C program, state {state}, shard {n} of {sum(numels)}")
    r = subprocess.run([EXE, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = open(out, "rb").read()
    mb = 2 if state == 1 else 4
    mdt = np.uint16 if state == 1 else np.float32
    off = 0
    g_master = np.frombuffer(raw, np.float32, n, off); off += 4 * n
    g_m = np.frombuffer(raw, mdt, n, off); off += mb * n
    g_v = np.frombuffer(raw, mdt, n, off); off += mb * n
    g_params = np.frombuffer(raw, np.uint16, sum(numels), off)
    if state == 0:
        want = oracle.shard_step(parts, master, m, v, oracle.hparams(t, **hp))
    elif state == 2:
        want = (master, m, v, None)
        for tt in range(t, t + 4):              # the program's table: steps t .. t+3
            want = oracle.shard_step(parts, *want[:3], oracle.hparams(tt, **hp))
    else:
        want = oracle.shard_step_bf16m(parts, master, m, v, oracle.hparams(t, **hp))
    assert_bitwise(g_master, want[0], "C program master")
    assert_bitwise(g_m, want[1], "C program m")
    assert_bitwise(g_v, want[2], "C program v")
    assert_bitwise(g_params[lo:hi], want[3], "C program params")
    assert np.all(g_params[:lo] == 0xFFFF) and np.all(g_params[hi:] == 0xFFFF)
