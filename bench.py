"""Benchmark of the KDA mixer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill-4k]

A step is one kda_prefill over the workload (conv + SiLU + L2, chunk preparation,
state walk with output, conv-state hand-over), inputs resident in HBM.  The
decode step (B=256 sequences, in-place state) is timed in the same run and
reported beside it.  A second leg ("stages") times the same prefill and decode
steps with the optional stages on (decay and write strength from raw
projections, output RMSNorm and sigmoid gate), the prefill's tokens packed as
sequences of mixed length, and the backward pass.  Prints one JSON line.

Roofline figures use algorithmic bytes (each tensor the kernel must read or
write, once) divided by the kernel's mean duration from HIP events recorded on
the launch stream; peaks are MI355X's published 8 TB/s HBM and 2.5 PFLOP/s dense
bf16.  The CPU baseline runs the fp64 oracle on a bounded sample of heads in a
process pool on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s
BF16_PEAK = 2.5e15         # flop/s, dense
# the stages kda_prefill enqueues: preparation, state walk with the conv-state
# hand-over, separate output-stage pass (empty unless that stage is on)
STAGE_IDS = [0, 4, 3]
STAGE_NAMES = ["kda_chunk_prep_kernel", "kda_chunk_state_kernel", "kda_out_stage_kernel"]
KERNEL_SOURCES = ["gated_delta_rule_80_amd/csrc/kda_prep.hip",
                  "gated_delta_rule_80_amd/csrc/kda_backward.hip",
                  "gated_delta_rule_80_amd/csrc/kda_prep_exact.hip",
                  "gated_delta_rule_80_amd/csrc/kda_state.hip",
                  "gated_delta_rule_80_amd/csrc/kda_decode.hip",
                  "gated_delta_rule_80_amd/csrc/kda_convnorm.h",
                  "gated_delta_rule_80_amd/csrc/kda_device.h",
                  "gated_delta_rule_80_amd/csrc/kda_layout.h"]


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def esize(io: str) -> int:
    return 2 if io == "bf16" else 4


def prefill_bytes(w) -> dict:
    """Algorithmic bytes per launch of each prefill kernel and of the whole path."""
    es = esize(w.io)
    C, D = w.chunk, w.D
    NT = -(-w.T // C)
    tok = w.B * w.T
    x = tok * w.H * D * es
    beta = tok * w.H * es
    conv_w = 3 * w.H * D * 4 * 4
    state = w.B * w.H * D * D * 4
    s0 = state if w.s0_std > 0 else 0
    cst = w.B * 3 * 3 * w.H * D * es if w.conv_state_std > 0 else 0
    record = (4 * C * D + C * C) * es + 4 * D  # what the preparation hands over per chunk
    records = w.B * w.H * NT * record
    return {
        "prep": 4 * x + beta + conv_w + cst + records,
        "state": records + s0 + x + state,
        "path": 4 * x + beta + conv_w + cst + s0 + x + state,  # fused minimum of the whole step
    }


def prefill_flops(w) -> float:
    """Useful flops of the chunked form per token and head: 6 d^2 + 5 C d + C^2 / 3."""
    d, C = w.D, w.chunk
    return w.B * w.T * w.H * (6 * d * d + 5 * C * d + C * C / 3)


def decode_bytes(w) -> int:
    es = esize(w.io)
    x = w.B * w.H * w.D * es
    return (2 * w.B * w.H * w.D * w.D * 4 + 5 * x + w.B * w.H * es
            + 2 * w.B * 3 * 3 * w.H * w.D * es + 3 * w.H * w.D * 16)


def backward_bytes(w) -> dict:
    """Algorithmic bytes per launch of each backward kernel (its inputs read once and
    its outputs written once, with the intermediate buffers the kernels hand over:
    records, checkpoints, per-chunk gradients and dy in the I/O type) and of the
    whole call ("path": raw inputs and dO in, every gradient and the recomputed
    forward outputs out).  dS_T is not given in the benchmark."""
    es = esize(w.io)
    C, D = w.chunk, w.D
    NT = -(-w.T // C)
    nrec = w.B * w.H * NT
    tok = w.B * w.T
    xe, x4 = tok * w.H * D * es, tok * w.H * D * 4
    bth4 = tok * w.H * 4
    state = w.B * w.H * D * D * 4
    cw = 3 * w.H * D * 4 * 4
    cst_e = w.B * 3 * 3 * w.H * D * es if w.conv_state_std > 0 else 0
    cst_4 = w.B * 3 * 3 * w.H * D * 4
    s0 = state if w.s0_std > 0 else 0
    cd, cc, dd = C * D, C * C, D * D
    tokb = 4 * (256 // (D // 8))
    nblk = -(-w.T // tokb)
    return {
        "walk": nrec * ((3 * cd + cc) * es + 4 * D) + xe + nrec * (cd + dd) * es + state,
        "prod": nrec * (2 * cd + 2 * dd) * es + xe + nrec * ((3 * cd + cc) * es + D * 4),
        # the front end's outputs k, v (and q) in the I/O type, Gamma in float32
        "t": nrec * (cc + cd + cd) * es + 2 * xe + x4 + bth4 + nrec * (2 * cd + cc) * es,
        # the gradients of the front end's outputs (dy) in the I/O type
        "pair": 3 * xe + x4 + bth4 + nrec * ((2 * cc + 4 * cd) * es + D * 4) + 3 * xe + x4 + bth4,
        "front": 3 * xe + cw + cst_e + 3 * xe + bth4 + 3 * x4 + w.B * nblk * 3 * w.H * D * 16
                 + cst_4 + bth4,
        "path": 4 * xe + tok * w.H * es + cw + cst_e + s0 + xe  # q, k, v, g, beta, filters, history, S0, dO
                + 4 * x4 + bth4 + state + cw + cst_4        # dq, dk, dv, dg, dbeta, dS0, dconv_w, dconv_state
                + xe + state + cst_e,                       # o, S_T, conv hand-over recomputed
    }


def stage_bytes(w) -> dict:
    """Extra algorithmic bytes of the optional stages: the gate pre-activation read
    once in the fused minimum; the separate output pass reads o and the gate and
    writes o.  (f and the beta logits replace g and beta byte for byte.)"""
    es = esize(w.io)
    x = w.B * w.T * w.H * w.D * es
    params = (w.H + 2 * w.H * w.D + w.D) * 4  # A_log, dt_bias (and its use), o_norm_w
    return {"path_extra": x + params, "out_pass": 3 * x + w.D * 4}


def traffic_for(kernel: str):
    """Measured HBM bytes per launch from the committed counter summary, or None
    when absent or taken on different kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(p) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def cpu_baseline(w, inp, budget_s: float):
    """Time the fp64 oracle on whole heads (full sequence) until ~budget_s elapsed."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    from kda_inputs import to_numpy
    from oracle import kda_reference

    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        ncpu = os.cpu_count() or 1
    workers = max(1, min(16, ncpu))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    D = w.D
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def job(b, h):
        ch = slice(h * D, (h + 1) * D)
        one = lambda x: to_numpy(x[b:b + 1, :, h:h + 1])
        return (one(inp["q"]), one(inp["k"]), one(inp["v"]), one(inp["g"]),
                to_numpy(inp["beta"][b:b + 1, :, h:h + 1]), to_numpy(inp["conv_w"][:, ch]),
                None if inp["conv_state"] is None else to_numpy(inp["conv_state"][b:b + 1, :, :, ch]),
                None if inp["S0"] is None else to_numpy(inp["S0"][b:b + 1, h:h + 1]))

    done = 0
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        # warm the workers (imports, first-call costs) outside the timed region
        list(ex.map(_warm, range(workers)))
        t0 = time.perf_counter()
        i = 0
        while i < len(heads):
            batch = heads[i:i + workers]
            futs = [ex.submit(kda_reference, *job(b, h)) for b, h in batch]
            for f in futs:
                f.result()
            done += len(batch)
            i += len(batch)
            if time.perf_counter() - t0 >= budget_s:
                break
        elapsed = time.perf_counter() - t0
    tokens_equiv = w.B * w.T * done / (w.B * w.H)
    return {"value": tokens_equiv / elapsed, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{done} of {w.B * w.H} heads, full T={w.T} each (fp64 sequential oracle, "
                      f"{elapsed:.1f} s); rate scaled to the whole {w.H}-head layer"}


def _warm(_):
    import numpy as np

    from oracle import kda_reference
    x = np.zeros((1, 4, 1, 16))
    kda_reference(x, x, x, -np.ones_like(x), np.zeros((1, 4, 1)))
    return 0


def time_prefill(kda, torch, a, ws, stream, steps, warmup):
    """Mean ms per kda_prefill and per stage, from HIP events on the launch stream.

    The throughput pass brackets `steps` kda_prefill calls with one pair of
    events; a second pass of the same number of steps runs the stages kda_prefill
    enqueues (STAGE_IDS) one call each, with an event after every stage, for the
    per-kernel durations (an event between two kernels costs the step several
    microseconds of drain, so those events stay out of the throughput pass)."""
    n = len(STAGE_NAMES)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        for s in range(n):
            kda.kda_prefill_stage(a, ws, STAGE_IDS[s], stream)
            if ev is not None:
                ev[s + 1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(steps):
        kda.kda_prefill_raw(a, ws, stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    stage_ms = [sum(e[s].elapsed_time(e[s + 1]) for e in evs) / steps for s in range(n)]
    return ms, stage_ms


def stages_leg(kda, torch, w, wd, args, stream, dev, plain_ms, plain_dms):
    """Prefill and decode with every optional stage on (same workloads and seeds)."""
    from kda_inputs import make_inputs, make_stage_inputs
    inp = make_inputs(w, seed=args.seed, device=dev)
    st = make_stage_inputs(w, seed=args.seed, device=dev)
    o = torch.empty_like(inp["q"])
    S_T = torch.empty(w.B, w.H, w.D, w.D, dtype=torch.float32, device=dev)
    cso = torch.empty(w.B, 3, 3, w.H * w.D, dtype=inp["q"].dtype, device=dev)
    a = kda.prefill_args(inp["q"], inp["k"], inp["v"], st["f"], st["b_logit"], inp["conv_w"],
                         inp["conv_state"], inp["S0"], o, S_T, cso, chunk=w.chunk,
                         A_log=st["A_log"], dt_bias=st["dt_bias"], beta_logits=True,
                         o_norm_w=st["o_norm_w"], o_gate=st["o_gate"])
    ws = torch.empty(kda.kda_prefill_workspace_bytes(a), dtype=torch.uint8, device=dev)
    ms, stage_ms = time_prefill(kda, torch, a, ws, stream, args.steps, args.warmup)
    sb = stage_bytes(w)
    path_bytes = prefill_bytes(w)["path"] + sb["path_extra"]
    out_ms = stage_ms[2]
    out = None
    if out_ms > 0.001:
        out = {"bound": "hbm", "kernel": STAGE_NAMES[2], "algorithmic_bytes": sb["out_pass"],
               "achieved": sb["out_pass"] / (out_ms / 1e3) / 1e9, "peak": HBM_PEAK / 1e9,
               "unit": "GB/s", "frac": sb["out_pass"] / (out_ms / 1e3) / HBM_PEAK,
               "traffic": traffic_for(STAGE_NAMES[2]), "mean_launch_ms": out_ms}
    prefill = {"workload": w.name, "ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms / 1e3),
               "extra_ms_vs_plain": ms - plain_ms,
               "output_stage_in_walk": out_ms <= 0.001,
               "stage_ms": {STAGE_NAMES[i]: stage_ms[i] for i in range(len(STAGE_NAMES))},
               "path_hbm_frac": path_bytes / (ms / 1e3) / HBM_PEAK, "out_pass_roofline": out}
    del ws, inp, st, o, S_T, cso
    torch.cuda.empty_cache()

    dinp = make_inputs(wd, seed=args.seed + 1, device=dev)
    dst = make_stage_inputs(wd, seed=args.seed + 1, device=dev)
    S = dinp["S0"]
    od = torch.empty_like(dinp["q"])
    da = kda.decode_args(dinp["q"], dinp["k"], dinp["v"], dst["f"], dst["b_logit"], S, od,
                         dinp["conv_w"], dinp["conv_state"], A_log=dst["A_log"],
                         dt_bias=dst["dt_bias"], beta_logits=True, o_norm_w=dst["o_norm_w"],
                         o_gate=dst["o_gate"])
    for _ in range(args.warmup):
        kda.kda_decode_raw(da, stream)
    torch.cuda.synchronize()
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for _ in range(args.steps):
        kda.kda_decode_raw(da, stream)
    d1.record(stream)
    torch.cuda.synchronize()
    dms = d0.elapsed_time(d1) / args.steps
    dbytes = decode_bytes(wd) + wd.B * wd.H * wd.D * esize(wd.io) + (wd.H + wd.H * wd.D + wd.D) * 4
    decode = {"workload": wd.name, "ms_per_step": dms, "seq_per_s": wd.B / (dms / 1e3),
              "extra_ms_vs_plain": dms - plain_dms,
              "roofline": {"bound": "hbm", "kernel": "kda_decode_kernel",
                           "achieved": dbytes / (dms / 1e3) / 1e9, "peak": HBM_PEAK / 1e9,
                           "unit": "GB/s", "frac": dbytes / (dms / 1e3) / HBM_PEAK,
                           "algorithmic_bytes": dbytes}}
    del dinp, dst, S, od
    torch.cuda.empty_cache()
    return {"what": "raw-projection decay and beta, output RMSNorm + sigmoid gate",
            "prefill": prefill, "decode": decode}


def backward_leg(kda, torch, w, args, stream, dev, plain_ms):
    """kda_prefill_backward on the same workload (forward recomputed inside)."""
    from kda_inputs import make_inputs
    inp = make_inputs(w, seed=args.seed, device=dev)
    gen = torch.Generator(device=dev).manual_seed(args.seed + 7)
    do = torch.randn(w.B, w.T, w.H, w.D, generator=gen, device=dev).to(inp["q"].dtype)
    f32 = dict(dtype=torch.float32, device=dev)
    o = torch.empty_like(inp["q"])
    S_T = torch.empty(w.B, w.H, w.D, w.D, **f32)
    cso = torch.empty(w.B, 3, 3, w.H * w.D, dtype=inp["q"].dtype, device=dev)
    fwd = kda.prefill_args(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["conv_w"],
                           inp["conv_state"], inp["S0"], o, S_T, cso, chunk=w.chunk)
    shape = (w.B, w.T, w.H, w.D)
    grads = dict(dq=torch.empty(*shape, **f32), dk=torch.empty(*shape, **f32),
                 dv=torch.empty(*shape, **f32), dg=torch.empty(*shape, **f32),
                 dbeta=torch.empty(w.B, w.T, w.H, **f32), dS0=torch.empty(w.B, w.H, w.D, w.D, **f32),
                 dconv_w=torch.empty(3, w.H * w.D, 4, **f32),
                 dconv_state=torch.empty(w.B, 3, 3, w.H * w.D, **f32))
    a = kda.backward_args(fwd, do, None, grads)
    ws = torch.empty(kda.kda_backward_workspace_bytes(a), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        kda.kda_prefill_backward_raw(a, ws, stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        kda.kda_prefill_backward_raw(a, ws, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nb = backward_bytes(w)["path"]
    out = {"workload": w.name, "ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms / 1e3),
           "ratio_to_forward": ms / plain_ms, "workspace_bytes": ws.numel(),
           "path_bytes": nb, "path_GBps": nb / (ms / 1e3) / 1e9,
           "path_frac_hbm": nb / (ms / 1e3) / HBM_PEAK,
           "includes": "recomputed forward + reverse walk + per-chunk gradient kernels + front end"}
    del ws, inp, grads, o, S_T, cso, do
    torch.cuda.empty_cache()
    return out


# The 4096 tokens of the 4k workload as 8 packed sequences of mixed length.
PACKED_LENGTHS = [1024, 512, 700, 300, 1000, 60, 400, 100]


def packed_leg(kda, torch, w, args, stream, dev, plain_ms):
    """Prefill over the same number of tokens packed as sequences of mixed length."""
    from kda_inputs import make_packed_inputs
    lengths = PACKED_LENGTHS if sum(PACKED_LENGTHS) == w.B * w.T else [w.T] * w.B
    inp = make_packed_inputs(w, lengths, seed=args.seed, device=dev)
    N = len(lengths)
    o = torch.empty_like(inp["q"])
    S_T = torch.empty(N, w.H, w.D, w.D, dtype=torch.float32, device=dev)
    cso = torch.empty(N, 3, 3, w.H * w.D, dtype=inp["q"].dtype, device=dev)
    a = kda.prefill_args(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["conv_w"],
                         inp["conv_state"], inp["S0"], o, S_T, cso, chunk=w.chunk,
                         cu_seqlens=inp["cu_seqlens"])
    ws = torch.empty(kda.kda_prefill_workspace_bytes(a), dtype=torch.uint8, device=dev)
    ms, stage_ms = time_prefill(kda, torch, a, ws, stream, args.steps, args.warmup)
    tokens = sum(lengths)
    nb = prefill_bytes(w)["path"]
    out = {"workload": f"{w.name} packed as {N} sequences", "lengths": lengths, "ms_per_step": ms,
           "tokens_per_s": tokens / (ms / 1e3), "ms_vs_unpacked": ms - plain_ms,
           "stage_ms": {STAGE_NAMES[i]: stage_ms[i] for i in range(len(STAGE_NAMES))},
           "path_hbm_frac": nb / (ms / 1e3) / HBM_PEAK}
    del ws, inp, o, S_T, cso
    torch.cuda.empty_cache()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill-4k")
    ap.add_argument("--decode-workload", default="decode-b256")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle timing (0 = skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-stages", action="store_true",
                    help="skip the legs with the optional stages (raw projections, output norm + "
                         "gate), packed sequences and the backward pass")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run the library's plain state-copy kernel (kda_prefill with T=0) "
                         "on this many MiB, to calibrate HBM byte counters")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: the KDA mixer shards over (sequence, head) with no "
              "collective, so only --gpus 1 is run here", file=sys.stderr)
        return 2

    import torch

    import gated_delta_rule_80_amd as kda
    from kda_inputs import WORKLOADS, make_inputs

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.workload]
    inp = make_inputs(w, seed=args.seed, device=dev)
    o = torch.empty_like(inp["q"])
    S_T = torch.empty(w.B, w.H, w.D, w.D, dtype=torch.float32, device=dev)
    cso = torch.empty(w.B, 3, 3, w.H * w.D, dtype=inp["q"].dtype, device=dev)
    a = kda.prefill_args(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["conv_w"],
                         inp["conv_state"], inp["S0"], o, S_T, cso, chunk=w.chunk)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(a), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    ms, stage_ms = time_prefill(kda, torch, a, ws, stream, args.steps, args.warmup)
    tokens_per_s = w.B * w.T / (ms / 1e3)

    nb = prefill_bytes(w)
    names = STAGE_NAMES
    dom = 0 if stage_ms[0] >= stage_ms[1] else 1
    dom_bytes = nb["prep"] if dom == 0 else nb["state"]
    achieved = dom_bytes / (stage_ms[dom] / 1e3)
    roofline = {"bound": "hbm", "kernel": names[dom], "achieved": achieved / 1e9,
                "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": achieved / HBM_PEAK,
                "traffic": traffic_for(names[dom]), "algorithmic_bytes": dom_bytes,
                "mean_launch_ms": stage_ms[dom]}
    flops = prefill_flops(w)
    path = {"algorithmic_bytes": nb["path"], "achieved_GBps": nb["path"] / (ms / 1e3) / 1e9,
            "hbm_frac": nb["path"] / (ms / 1e3) / HBM_PEAK,
            "mfma_frac_useful": flops / (ms / 1e3) / BF16_PEAK,
            "stage_ms": {names[i]: stage_ms[i] for i in range(2)}}
    plain_ms = ms
    del ws, inp, o, S_T, cso
    torch.cuda.empty_cache()

    # ---- decode leg
    wd = WORKLOADS[args.decode_workload]
    dinp = make_inputs(wd, seed=args.seed + 1, device=dev)
    S = dinp["S0"]
    cs = dinp["conv_state"]
    od = torch.empty_like(dinp["q"])
    da = kda.decode_args(dinp["q"], dinp["k"], dinp["v"], dinp["g"], dinp["beta"], S, od,
                         dinp["conv_w"], cs)
    for _ in range(args.warmup):
        kda.kda_decode_raw(da, stream)
    torch.cuda.synchronize()
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for _ in range(args.steps):
        kda.kda_decode_raw(da, stream)
    d1.record(stream)
    torch.cuda.synchronize()
    dms = d0.elapsed_time(d1) / args.steps
    dbytes = decode_bytes(wd)
    decode = {"metric": "KDA decode seq/s", "value": wd.B / (dms / 1e3), "unit": "seq/s",
              "ms_per_step": dms, "config": {"workload": wd.name, "B": wd.B, "H": wd.H, "D": wd.D},
              "roofline": {"bound": "hbm", "kernel": "kda_decode_kernel",
                           "achieved": dbytes / (dms / 1e3) / 1e9, "peak": HBM_PEAK / 1e9,
                           "unit": "GB/s", "frac": dbytes / (dms / 1e3) / HBM_PEAK,
                           "traffic": traffic_for("kda_decode_kernel"),
                           "algorithmic_bytes": dbytes}}
    del dinp, S, cs, od
    torch.cuda.empty_cache()

    stages = None
    if not args.no_stages:
        stages = stages_leg(kda, torch, w, wd, args, stream, dev, plain_ms, dms)
        stages["packed"] = packed_leg(kda, torch, w, args, stream, dev, plain_ms)
        stages["backward"] = backward_leg(kda, torch, w, args, stream, dev, plain_ms)

    if args.calib_copy_mib > 0:
        # kda_prefill with T = 0 copies S0 to S_T with one plain copy kernel
        # (kda_copy_state_kernel): exactly n bytes read and n bytes written.
        nb_state = 128 * 128 * 4
        nbh = max(1, args.calib_copy_mib * (1 << 20) // nb_state)
        src = torch.randn(nbh, 1, 128, 128, device=dev)
        dst = torch.empty_like(src)
        z = torch.empty(nbh, 0, 1, 128, dtype=torch.bfloat16, device=dev)
        ca = kda.prefill_args(z, z, z, z, z[..., 0], None, None, src, None, dst, None, chunk=64)
        for _ in range(3):
            kda.kda_prefill_raw(ca, None, stream)
        torch.cuda.synchronize()
        print(f"calibration copy: {nbh * nb_state} bytes read and written per launch",
              file=sys.stderr, flush=True)
        del src, dst

    cpu = None
    if args.cpu_budget > 0:
        cinp = make_inputs(w, seed=args.seed, device=dev)
        cpu = cpu_baseline(w, cinp, args.cpu_budget)
        del cinp

    line = {
        "metric": "KDA tokens/s per GPU (prefill, H=96 d=128) + decode seq/s; % of roofline",
        "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.io, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "D": w.D, "chunk": w.chunk,
                   "io": w.io, "state": "fp32"},
        "roofline": roofline, "path": path, "decode": decode, "stages": stages,
        "cpu_baseline": cpu,
        "source_hash": source_hash(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
