"""The fp64 oracle over every (sequence, head) pair of a workload, in a pool of
host processes (TEST INFRASTRUCTURE ONLY, like the rest of this package: the
full-size parity tests compare each pair with the GPU's outputs, and the
benchmark's CPU-baseline leg times the oracle this way).

Every (sequence, head) pair of the mixer is independent (its own state, conv
filters and channels), so the oracle runs each pair on its own.  The parent
writes the inputs and the GPU's outputs once, head-major, into a scratch folder
(bf16 tensors as their raw 16-bit patterns); each worker memory-maps the slices
of its pair, runs the oracle and returns only error figures.  This module imports
numpy and the oracle, nothing of the GPU library (the workers never touch the
GPU), and holds none of the mixer's arithmetic itself.

Figures per pair: relative L2 of o over the whole sequence and of S_T (the
tolerance the tests assert), and the worst relative L2 over 64-token blocks of o
(an error confined to a few tokens shows there), with its block index.
"""
from __future__ import annotations

import json
import os
import shutil
import tempfile
import time
from concurrent.futures import ProcessPoolExecutor, as_completed

import numpy as np

BLOCK = 64  # tokens per block of the per-block figure


def pool_workers() -> int:
    """Host processes for the pool: the cores this process may run on, at most 16
    (one GPU's share of a host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def scratch_dir(nbytes: int) -> str:
    """A scratch folder for nbytes of arrays: /dev/shm when it has room, else the
    temporary directory."""
    shm = "/dev/shm"
    try:
        if os.path.isdir(shm) and shutil.disk_usage(shm).free > 1.5 * nbytes:
            return tempfile.mkdtemp(prefix="kda_parity_", dir=shm)
    except OSError:
        pass
    return tempfile.mkdtemp(prefix="kda_parity_")


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Array as stored (bf16 bit patterns in uint16, or float32) to float64."""
    a = np.asarray(a)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)


def save_array(d: str, name: str, a):
    """Store one array of a scratch folder (None: nothing, the oracle then takes
    zeros or skips that input)."""
    if a is not None:
        np.save(os.path.join(d, name + ".npy"), np.asarray(a))


def save_meta(d: str, dtype: str, D: int):
    """dtype: "bf16" (arrays hold bf16 bit patterns) or "fp32"; D: head_dim."""
    with open(os.path.join(d, "meta.json"), "w") as f:
        json.dump({"dtype": dtype, "D": D}, f)


def _load(d: str, name: str):
    p = os.path.join(d, name + ".npy")
    return np.load(p, mmap_mode="r") if os.path.exists(p) else None


def _meta(d: str) -> dict:
    with open(os.path.join(d, "meta.json")) as f:
        return json.load(f)


def block_errors(o, ref, block=BLOCK):
    """Worst relative L2 over consecutive token blocks of [T, D] outputs, and its block."""
    T = ref.shape[0]
    worst, at = 0.0, -1
    for t0 in range(0, T, block):
        e = rel_l2(o[t0:t0 + block], ref[t0:t0 + block])
        if e > worst:
            worst, at = e, t0 // block
    return worst, at


def oracle_pair(d: str, b: int, h: int):
    """The oracle over the whole sequence of pair (b, h); returns (o [1, T, 1, D],
    S_T [1, 1, D, D])."""
    from oracle.kda_oracle import kda_reference

    m = _meta(d)
    dt, D = m["dtype"], m["D"]
    one = lambda name: to_f64(_load(d, name)[b, h], dt)[None, :, None, :]  # [1, T, 1, D]
    q, k, v, g = one("q"), one("k"), one("v"), one("g")
    beta = to_f64(_load(d, "beta")[b, h], dt)[None, :, None]
    ch = slice(h * D, (h + 1) * D)
    cw = _load(d, "conv_w")
    cw = None if cw is None else np.asarray(cw[:, ch], dtype=np.float64)
    cs = _load(d, "conv_state")
    cs = None if cs is None else to_f64(cs[b:b + 1, :, :, ch], dt)
    s0 = _load(d, "S0")
    s0 = None if s0 is None else np.asarray(s0[b:b + 1, h:h + 1], dtype=np.float64)
    ro, rS, _ = kda_reference(q, k, v, g, beta, conv_w=cw, conv_state=cs, S0=s0)
    return ro, rS


def timed_pair(d: str, b: int, h: int):
    """The oracle on pair (b, h), for timing: returns only (b, h)."""
    oracle_pair(d, b, h)
    return b, h


def prefill_pair(d: str, b: int, h: int):
    """Oracle over the whole sequence of pair (b, h) against the GPU's o and S_T."""
    ro, rS = oracle_pair(d, b, h)
    dt = _meta(d)["dtype"]
    go = to_f64(_load(d, "o")[b, h], dt)
    gS = np.asarray(_load(d, "S_T")[b, h], dtype=np.float64)
    eblk, at = block_errors(go, ro[0, :, 0])
    return b, h, rel_l2(go, ro[0, :, 0]), rel_l2(gS, rS[0, 0]), eblk, at


def decode_seq(d: str, b: int):
    """Oracle decode step of sequence b (all heads) against the GPU's o, S and
    conv state; per head figures plus whether the conv state matches exactly."""
    from oracle.kda_oracle import kda_reference_decode_step

    m = _meta(d)
    dt = m["dtype"]
    one = lambda name: to_f64(_load(d, name)[b:b + 1], dt)
    ro, rS, rcs = kda_reference_decode_step(
        one("q"), one("k"), one("v"), one("g"), one("beta"),
        np.asarray(_load(d, "S0")[b:b + 1], dtype=np.float64),
        conv_w=np.asarray(_load(d, "conv_w"), dtype=np.float64), conv_state=one("conv_state"))
    go = one("o")
    gS = _load(d, "S")
    cs_ok = bool(np.array_equal(one("conv_state_out"), rcs))
    out = []
    for h in range(go.shape[1]):
        out.append((b, h, rel_l2(go[0, h], ro[0, h]),
                    rel_l2(np.asarray(gS[b, h], dtype=np.float64), rS[0, h]), cs_ok))
    return out


def backward_pair(d: str, b: int, h: int):
    """Oracle gradients of pair (b, h) against the GPU's; relative L2 per gradient
    (the conv filter gradient of the head's channels comes from that head alone)."""
    from oracle.kda_oracle import kda_reference_backward

    m = _meta(d)
    dt, D = m["dtype"], m["D"]
    one = lambda name: to_f64(_load(d, name)[b, h], dt)[None, :, None, :]
    ch = slice(h * D, (h + 1) * D)
    cw = _load(d, "conv_w")
    cw = None if cw is None else np.asarray(cw[:, ch], dtype=np.float64)
    cs = _load(d, "conv_state")
    cs = None if cs is None else to_f64(cs[b:b + 1, :, :, ch], dt)
    s0 = _load(d, "S0")
    s0 = None if s0 is None else np.asarray(s0[b:b + 1, h:h + 1], dtype=np.float64)
    ref = kda_reference_backward(one("q"), one("k"), one("v"), one("g"),
                                 to_f64(_load(d, "beta")[b, h], dt)[None, :, None], one("do"),
                                 conv_w=cw, conv_state=cs, S0=s0)
    f32 = lambda name: np.asarray(_load(d, name)[b, h], dtype=np.float64)
    got = {"dq": f32("dq")[None, :, None], "dk": f32("dk")[None, :, None],
           "dv": f32("dv")[None, :, None], "dg": f32("dg")[None, :, None],
           "dbeta": f32("dbeta")[None, :, None], "dS0": f32("dS0")[None, None]}
    if cw is not None:
        got["dconv_w"] = np.asarray(_load(d, "dconv_w")[:, ch], dtype=np.float64)
        got["dconv_state"] = np.asarray(_load(d, "dconv_state")[b:b + 1, :, :, ch], dtype=np.float64)
    return b, h, {n: rel_l2(got[n], ref[n]) for n in got if ref.get(n) is not None}


_ONE_THREAD = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


class _OneThreadEnv:
    """Workers inherit one BLAS/OpenMP thread each (set while the pool spawns them)."""

    def __enter__(self):
        self.saved = {k: os.environ.get(k) for k in _ONE_THREAD}
        for k in _ONE_THREAD:
            os.environ[k] = "1"

    def __exit__(self, *exc):
        for k, v in self.saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _pool(workers: int):
    import multiprocessing as mp

    return ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"))


def _warm(_):
    return 0


def run(fn, d: str, tasks, label: str, workers: int | None = None):
    """Run fn(d, *task) for every task in a spawned pool; progress lines go to
    stdout as tasks finish.  Returns the results in completion order."""
    workers = workers or pool_workers()
    out = []
    t0 = time.perf_counter()
    step = max(1, len(tasks) // 12)
    with _OneThreadEnv(), _pool(workers) as ex:
        futs = [ex.submit(fn, d, *t) for t in tasks]
        for i, f in enumerate(as_completed(futs), 1):
            out.append(f.result())
            if i % step == 0 or i == len(tasks):
                print(f"  {label}: {i}/{len(tasks)} done, {time.perf_counter() - t0:.1f} s "
                      f"({workers} host processes)", flush=True)
    return out


def time_pairs(d: str, tasks, budget_s: float, workers: int | None = None):
    """Time the oracle (timed_pair) over tasks in waves of `workers` pairs until
    budget_s has elapsed; the workers are started and warmed before the clock
    starts.  Returns (pairs done, seconds, workers)."""
    workers = workers or pool_workers()
    done = 0
    with _OneThreadEnv(), _pool(workers) as ex:
        list(ex.map(_warm, range(workers)))
        t0 = time.perf_counter()
        i = 0
        while i < len(tasks):
            wave = tasks[i:i + workers]
            for f in [ex.submit(timed_pair, d, *t) for t in wave]:
                f.result()
            done += len(wave)
            i += len(wave)
            if time.perf_counter() - t0 >= budget_s:
                break
        elapsed = time.perf_counter() - t0
    return done, elapsed, workers
