"""Benchmark of the KDA mixer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill-64k]
                    [--also prefill-4k,prefill-b4-8k-s0] [--no-stages] [--cpu-budget S]
    python bench.py --profile-commands DIR        (print the rocprofv3 commands of a profile)
    python bench.py --summarize-rocprof DIR       (turn their output into profiles/)

A step is one kda_prefill over the workload (conv + SiLU + L2, chunk preparation,
state walk with output, conv-state hand-over), inputs resident in HBM.  The
headline is the long-context layer (B=1, T=65536, H=96, D=128, bf16, chunk 64),
the largest single-GPU prefill; the one-layer 4k prefill and the batched 8k
prefill with an initial state are timed in the same run and reported beside it,
as is the decode step (B=256 sequences, in-place state).  A further leg
("stages", on the 4k prefill) times the optional stages (decay and write
strength from raw projections, output RMSNorm and sigmoid gate), the 4k tokens
packed as sequences of mixed length, and the backward pass.  Prints one JSON line.

Rooflines use the fused minimum of HBM traffic of the whole mixer (raw q, k, v,
g, beta read once, o written once: 5 H D + H elements per token; S_T written,
S0 read when given, the conv filters read once) against MI355X's published
8 TB/s.  `roofline` divides it by the dominant kernel's mean duration (HIP events
on the launch stream), `path` by the whole step's; the bytes the kernels
actually move are `traffic` (rocprofv3 counters, profiles/traffic.json).  The
CPU baseline times the fp64 oracle on whole (sequence, head) pairs of the
headline workload in a pool of host processes.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import shutil
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
                  "gated_delta_rule_80_amd/csrc/kda_bwd_stages.hip",
                  "gated_delta_rule_80_amd/csrc/kda_split.hip",
                  "gated_delta_rule_80_amd/csrc/kda_prep_exact.hip",
                  "gated_delta_rule_80_amd/csrc/kda_state.hip",
                  "gated_delta_rule_80_amd/csrc/kda_decode.hip",
                  "gated_delta_rule_80_amd/csrc/kda_convnorm.h",
                  "gated_delta_rule_80_amd/csrc/kda_device.h",
                  "gated_delta_rule_80_amd/csrc/kda_layout.h"]
HEADLINE = "prefill-64k"
ALSO = "prefill-4k,prefill-b4-8k-s0,prefill-64k-h12"
STAGES_WORKLOAD = "prefill-4k"
TP_SHARE_WORKLOAD = "prefill-64k-h12"
METRIC = "KDA tokens/s per GPU (prefill, H=96 d=128) + decode seq/s; % of roofline"


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def esize(io: str) -> int:
    return 2 if io == "bf16" else 4


def path_bytes(w) -> int:
    """Fused minimum of HBM traffic of one prefill: raw q, k, v, g (H D elements
    each per token), beta (H) read and o (H D) written once per token -- 123,072 B
    per token at H = 96, D = 128, bf16 -- plus S_T written, S0 read when given,
    the conv filters (and conv states, when given) once."""
    es = esize(w.io)
    tok = w.B * w.T
    state = w.B * w.H * w.D * w.D * 4
    cst = 2 * w.B * 3 * 3 * w.H * w.D * es if w.conv_state_std > 0 else 0
    return (tok * (5 * w.H * w.D + w.H) * es + state + (state if w.s0_std > 0 else 0)
            + 3 * w.H * w.D * 4 * 4 + cst)


def design_bytes(w) -> dict:
    """Bytes each prefill kernel of this design must move: the preparation reads
    the raw inputs and writes one record per chunk (W, Q Lambda, Ktil^T, U~ in the
    I/O type, P, Lambda_C); the walk reads the records and writes o and S_T."""
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
    records = w.B * w.H * NT * ((4 * C * D + C * C) * es + 4 * D)
    return {"kda_chunk_prep_kernel": 4 * x + beta + conv_w + cst + records,
            "kda_chunk_state_kernel": records + s0 + x + state}


def prefill_flops(w) -> float:
    """Useful flops of the chunked form per token and head: 6 d^2 + 5 C d + C^2 / 3."""
    d, C = w.D, w.chunk
    return w.B * w.T * w.H * (6 * d * d + 5 * C * d + C * C / 3)


def decode_bytes(w) -> int:
    es = esize(w.io)
    x = w.B * w.H * w.D * es
    return (2 * w.B * w.H * w.D * w.D * 4 + 5 * x + w.B * w.H * es
            + 2 * w.B * 3 * 3 * w.H * w.D * es + 3 * w.H * w.D * 16)


def backward_bytes(w) -> int:
    """Fused minimum of the backward call: raw inputs and dO in, every gradient and
    the recomputed forward outputs out (dS_T not given in the benchmark)."""
    es = esize(w.io)
    tok = w.B * w.T
    xe, x4 = tok * w.H * w.D * es, tok * w.H * w.D * 4
    bth4 = tok * w.H * 4
    state = w.B * w.H * w.D * w.D * 4
    cw = 3 * w.H * w.D * 4 * 4
    cst_e = w.B * 3 * 3 * w.H * w.D * es if w.conv_state_std > 0 else 0
    cst_4 = w.B * 3 * 3 * w.H * w.D * 4
    s0 = state if w.s0_std > 0 else 0
    return (4 * xe + tok * w.H * es + cw + cst_e + s0 + xe
            + 4 * x4 + bth4 + state + cw + cst_4
            + xe + state + cst_e)


def stage_bytes(w) -> dict:
    """Extra algorithmic bytes of the optional stages: the gate pre-activation read
    once in the fused minimum; the separate output pass reads o and the gate and
    writes o.  (f and the beta logits replace g and beta byte for byte.)"""
    es = esize(w.io)
    x = w.B * w.T * w.H * w.D * es
    params = (w.H + 2 * w.H * w.D + w.D) * 4  # A_log, dt_bias (and its use), o_norm_w
    return {"path_extra": x + params, "out_pass": 3 * x + w.D * 4}


def traffic_for(workload: str, kernel: str):
    """Measured HBM bytes per launch of a kernel at a workload, from the committed
    counter summary, or None when absent or taken on other kernel sources."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    wl = d.get("workloads", {}).get(workload, {})
    if wl.get("source_hash") != source_hash():
        return None
    k = wl.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(w, inp, budget_s: float):
    """Time the fp64 oracle on whole (sequence, head) pairs (full sequence each) for
    about budget_s seconds; the rate is scaled to the whole layer."""
    from kda_inputs import to_storage
    from oracle.pool import pool_workers, save_array, save_meta, scratch_dir, time_pairs

    # the pairs a budget can reach: heads of the first sequence, a few per host process
    nh = min(w.H, 4 * pool_workers())
    sub = {t: inp[t][:1, :, :nh] for t in ("q", "k", "v", "g", "beta")}
    sub["conv_w"] = inp["conv_w"][:, :nh * w.D]
    sub["conv_state"] = None if inp["conv_state"] is None else inp["conv_state"][:1, :, :, :nh * w.D]
    sub["S0"] = None if inp["S0"] is None else inp["S0"][:1, :nh]
    d = scratch_dir(5 * sub["q"].numel() * sub["q"].element_size())
    try:
        save_meta(d, w.io, w.D)
        for t in ("q", "k", "v", "g", "beta"):
            save_array(d, t, to_storage(sub[t], head_major=True))
        for t in ("conv_w", "conv_state", "S0"):
            save_array(d, t, to_storage(sub[t]))
        done, elapsed, workers = time_pairs(d, [(0, h) for h in range(nh)], budget_s)
    finally:
        shutil.rmtree(d, ignore_errors=True)
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    tokens_equiv = w.B * w.T * done / len(pairs)
    return {"value": tokens_equiv / elapsed, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "host_cores_visible": host_cores(),
            "sample": f"{done} of {len(pairs)} (sequence, head) pairs of {w.name}, full T={w.T} "
                      f"each (fp64 sequential oracle, {elapsed:.1f} s in {workers} host processes "
                      f"of one thread; the pool is capped at 16, one GPU's share of the host); "
                      f"rate scaled to the whole {w.H}-head layer"}


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


def measure_prefill(kda, torch, w, args, stream, dev, keep_inputs=False):
    """One workload's prefill: throughput, per-kernel times and rooflines."""
    from kda_inputs import make_inputs
    inp = make_inputs(w, seed=args.seed, device=dev)
    o = torch.empty_like(inp["q"])
    S_T = torch.empty(w.B, w.H, w.D, w.D, dtype=torch.float32, device=dev)
    cso = torch.empty(w.B, 3, 3, w.H * w.D, dtype=inp["q"].dtype, device=dev)
    a = kda.prefill_args(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["conv_w"],
                         inp["conv_state"], inp["S0"], o, S_T, cso, chunk=w.chunk)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(a), dtype=torch.uint8, device=dev)
    print(f"timing {w.name}: B={w.B} T={w.T} H={w.H} D={w.D} {w.io}", file=sys.stderr, flush=True)
    ms, stage_ms = time_prefill(kda, torch, a, ws, stream, args.steps, args.warmup)
    nb = path_bytes(w)
    db = design_bytes(w)
    flops = prefill_flops(w)
    dom = 0 if stage_ms[0] >= stage_ms[1] else 1
    kname = STAGE_NAMES[dom]
    achieved = nb / (stage_ms[dom] / 1e3)
    nseg = kda.kda_prefill_walk_segments(a)
    label = kname
    if dom == 1 and nseg > 1:
        label = (f"{kname} (walk split into {nseg} segments: kda_seg_map_kernel, "
                 f"kda_seg_combine_kernel, then {kname})")
    roofline = {"bound": "hbm", "kernel": label,
                "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": achieved / HBM_PEAK, "traffic": traffic_for(w.name, kname),
                "algorithmic_bytes": nb, "mean_launch_ms": stage_ms[dom],
                "design_bytes": db[kname],
                "design_bytes_frac": db[kname] / (stage_ms[dom] / 1e3) / HBM_PEAK}
    t = ms / 1e3
    path = {"algorithmic_bytes": nb, "achieved_GBps": nb / t / 1e9, "hbm_frac": nb / t / HBM_PEAK,
            "mfma_frac_useful": flops / t / BF16_PEAK,
            "attainable_frac": max(flops / BF16_PEAK, nb / HBM_PEAK) / t,
            "stage_ms": {STAGE_NAMES[i]: stage_ms[i] for i in range(2)}}
    out = {"workload": w.name, "config": {"B": w.B, "T": w.T, "H": w.H, "D": w.D, "chunk": w.chunk,
                                          "io": w.io, "state": "fp32", "S0": w.s0_std > 0,
                                          "walk_segments": nseg},
           "ms_per_step": ms, "tokens_per_s": w.B * w.T / t, "roofline": roofline, "path": path}
    del ws, o, S_T, cso, a
    if not keep_inputs:
        del inp
        inp = None
    torch.cuda.empty_cache()
    return out, inp


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
    pb = path_bytes(w) + sb["path_extra"]
    out_ms = stage_ms[2]
    out = None
    if out_ms > 0.001:
        out = {"bound": "hbm", "kernel": STAGE_NAMES[2], "algorithmic_bytes": sb["out_pass"],
               "achieved": sb["out_pass"] / (out_ms / 1e3) / 1e9, "peak": HBM_PEAK / 1e9,
               "unit": "GB/s", "frac": sb["out_pass"] / (out_ms / 1e3) / HBM_PEAK,
               "traffic": traffic_for(w.name, STAGE_NAMES[2]), "mean_launch_ms": out_ms}
    prefill = {"workload": w.name, "ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms / 1e3),
               "extra_ms_vs_plain": ms - plain_ms,
               "output_stage_in_walk": out_ms <= 0.001,
               "stage_ms": {STAGE_NAMES[i]: stage_ms[i] for i in range(len(STAGE_NAMES))},
               "path_hbm_frac": pb / (ms / 1e3) / HBM_PEAK, "out_pass_roofline": out}
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
    dms = time_decode(kda, torch, da, stream, args.steps, args.warmup)
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


def training_leg(kda, torch, w, args, stream, dev, plain_ms, backward_ms):
    """A training step's mixer work with the forward kept for the backward
    (kda_prefill_forward_saved, then kda_prefill_backward_saved), each timed on
    its own, against kda_prefill plus the recomputing kda_prefill_backward."""
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
    ws = torch.empty(kda.kda_training_workspace_bytes(fwd), dtype=torch.uint8, device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    f_ms = timed(lambda: kda.kda_prefill_forward_saved_raw(fwd, ws, stream))
    # the saved part of the workspace is only read by the backward: repeated
    # backward calls on one saved forward are the steady state
    b_ms = timed(lambda: kda.kda_prefill_backward_saved_raw(a, ws, stream))
    out = {"workload": w.name, "forward_saved_ms": f_ms, "backward_saved_ms": b_ms,
           "step_ms": f_ms + b_ms,
           "backward_ratio_to_forward": b_ms / plain_ms if plain_ms == plain_ms else None,
           "step_ms_recomputing": (plain_ms + backward_ms) if plain_ms == plain_ms else None,
           "workspace_bytes": ws.numel(),
           "includes": "forward kept for the backward (records, front-end outputs, decay sums, "
                       "chunk-start states) + backward without the forward recompute"}
    del ws, inp, grads, o, S_T, cso, do, a, fwd
    torch.cuda.empty_cache()
    return out


def hbm_probe(torch, dev, stream, steps):
    """A practical ceiling for the decode step's access pattern: torch's in-place
    multiply of 1.5 GiB of float32 (read once, written once, like the 256 x 96
    decode states)."""
    x = torch.zeros(1610612736 // 4, dtype=torch.float32, device=dev)
    for _ in range(3):
        x.mul_(1.0)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        x.mul_(1.0)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = 2 * x.numel() * 4
    del x
    torch.cuda.empty_cache()
    return {"what": "torch in-place multiply of 1.5 GiB float32", "ms": ms,
            "GBps": nbytes / (ms / 1e3) / 1e9, "frac": nbytes / (ms / 1e3) / HBM_PEAK}


def time_decode(kda, torch, da, stream, steps, warmup):
    for _ in range(warmup):
        kda.kda_decode_raw(da, stream)
    torch.cuda.synchronize()
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for _ in range(steps):
        kda.kda_decode_raw(da, stream)
    d1.record(stream)
    torch.cuda.synchronize()
    return d0.elapsed_time(d1) / steps


def backward_leg(kda, torch, w, args, stream, dev, plain_ms, stages=False, packed=False):
    """kda_prefill_backward on the same workload (forward recomputed inside); with
    every optional stage on, or the tokens packed as sequences of mixed length."""
    from kda_inputs import make_inputs, make_packed_inputs, make_stage_inputs
    if packed:
        lengths = PACKED_LENGTHS if sum(PACKED_LENGTHS) == w.B * w.T else [w.T] * w.B
        inp = make_packed_inputs(w, lengths, seed=args.seed, device=dev)
        B, T, NS = 1, sum(lengths), len(lengths)
    else:
        inp = make_inputs(w, seed=args.seed, device=dev)
        B, T, NS = w.B, w.T, w.B
    skw, g, beta = {}, inp["g"], inp["beta"]
    if stages:
        st = make_stage_inputs(w, seed=args.seed, device=dev)
        g, beta = st["f"], st["b_logit"]
        skw = dict(A_log=st["A_log"], dt_bias=st["dt_bias"], beta_logits=True,
                   o_norm_w=st["o_norm_w"], o_gate=st["o_gate"])
    gen = torch.Generator(device=dev).manual_seed(args.seed + 7)
    do = torch.randn(B, T, w.H, w.D, generator=gen, device=dev).to(inp["q"].dtype)
    f32 = dict(dtype=torch.float32, device=dev)
    o = torch.empty_like(inp["q"])
    S_T = torch.empty(NS, w.H, w.D, w.D, **f32)
    cso = torch.empty(NS, 3, 3, w.H * w.D, dtype=inp["q"].dtype, device=dev)
    fwd = kda.prefill_args(inp["q"], inp["k"], inp["v"], g, beta, inp["conv_w"],
                           inp["conv_state"], inp["S0"], o, S_T, cso, chunk=w.chunk,
                           cu_seqlens=inp.get("cu_seqlens"), **skw)
    shape = (B, T, w.H, w.D)
    grads = dict(dq=torch.empty(*shape, **f32), dk=torch.empty(*shape, **f32),
                 dv=torch.empty(*shape, **f32), dg=torch.empty(*shape, **f32),
                 dbeta=torch.empty(B, T, w.H, **f32), dS0=torch.empty(NS, w.H, w.D, w.D, **f32),
                 dconv_w=torch.empty(3, w.H * w.D, 4, **f32),
                 dconv_state=torch.empty(NS, 3, 3, w.H * w.D, **f32))
    if stages:
        grads.update(dA_log=torch.empty(w.H, **f32), ddt_bias=torch.empty(w.H * w.D, **f32),
                     do_norm_w=torch.empty(w.D, **f32), do_gate=torch.empty(*shape, **f32))
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
    nb = backward_bytes(w)
    what = "recomputed forward + reverse walk + per-chunk gradient kernels + front end"
    if stages:
        what += "; every optional stage on (their backward included)"
    if packed:
        what += f"; {NS} packed sequences of lengths {lengths}"
    out = {"workload": w.name, "ms_per_step": ms, "tokens_per_s": B * T / (ms / 1e3),
           "ratio_to_forward": ms / plain_ms if plain_ms == plain_ms else None,
           "workspace_bytes": ws.numel(),
           "path_bytes": nb, "path_GBps": nb / (ms / 1e3) / 1e9,
           "path_frac_hbm": nb / (ms / 1e3) / HBM_PEAK, "includes": what}
    del ws, inp, grads, o, S_T, cso, do, a, fwd
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
    nb = path_bytes(w)
    out = {"workload": f"{w.name} packed as {N} sequences", "lengths": lengths, "ms_per_step": ms,
           "tokens_per_s": tokens / (ms / 1e3), "ms_vs_unpacked": ms - plain_ms,
           "stage_ms": {STAGE_NAMES[i]: stage_ms[i] for i in range(len(STAGE_NAMES))},
           "path_hbm_frac": nb / (ms / 1e3) / HBM_PEAK}
    del ws, inp, o, S_T, cso
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- profiles
# One profile of a workload is four rocprofv3 runs of this script (the kernel
# trace with per-kernel statistics, then one counter per run: HBM bytes fetched,
# HBM bytes written, and the matrix-core / VALU counters); a plain copy kernel of
# known size runs in each (kda_prefill with T = 0 copies S0 to S_T) to calibrate
# the byte counters.
CALIB_KERNEL = "kda_copy_state_kernel"
CALIB_MIB = 1024
SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU",
               "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CYCLES", "SQ_WAVES", "GRBM_GUI_ACTIVE"]


# kernels that a profiled run also launches outside the prefill of its workload
OTHER_LEG_WORKLOAD = {"kda_decode_kernel": "decode-b256",
                      CALIB_KERNEL: f"calibration-copy-{CALIB_MIB}-MiB"}


def profile_args(workload: str, backward: bool = False) -> str:
    return (f"--workload {workload} --also none --no-stages --cpu-budget 0 --steps 5 "
            f"--warmup 20 --calib-copy-mib {CALIB_MIB}" + (" --backward-only" if backward else ""))


def profile_label(workload: str, backward: bool = False) -> str:
    """Name under which a profile's kernels are filed (the backward's own kernels and
    its recomputed forward under <workload>-backward)."""
    return f"{workload}-backward" if backward else workload


def profile_commands(d: str, workload: str, backward: bool = False) -> dict:
    args = profile_args(workload, backward)
    run = f"python3 bench.py {args}"
    return {
        "trace": f"rocprofv3 --kernel-trace --stats -f csv -d {d}/trace -o trace -- {run}",
        "fetch": f"rocprofv3 --pmc FETCH_SIZE -f csv -d {d}/fetch -o pmc -- {run}",
        "write": f"rocprofv3 --pmc WRITE_SIZE -f csv -d {d}/write -o pmc -- {run}",
        "sq": f"rocprofv3 --pmc {' '.join(SQ_COUNTERS)} -f csv -d {d}/sq -o pmc -- {run}",
    }


def _csv_rows(pattern: str):
    import csv
    rows = []
    for p in sorted(glob.glob(pattern, recursive=True)):
        with open(p, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _short(name: str) -> str:
    """Kernel name without template arguments or parameters (kda_..._kernel)."""
    import re
    m = re.search(r"(kda_[a-z0-9_]+_kernel)", name)
    return m.group(1) if m else name


def summarize_rocprof(d: str, workload: str, out_dir: str, backward: bool = False) -> dict:
    """Turn the four runs of profile_commands(d, workload, backward) into one
    summary file per kernel under out_dir (named for the kernel and the workload's
    profile label) and this label's entry of out_dir/traffic.json.  Returns the
    traffic entry."""
    cmds = profile_commands(d, workload, backward)
    label = profile_label(workload, backward)
    trace = _csv_rows(os.path.join(d, "trace", "**", "*kernel_trace.csv"))
    stats = {}
    for r in trace:
        k = _short(r["Kernel_Name"])
        if not k.startswith("kda_"):
            continue  # torch's input generation
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # us
        col = lambda *names: next((int(float(r[n])) for n in names if r.get(n) not in (None, "")), 0)
        s = stats.setdefault(k, {"full_name": r["Kernel_Name"], "durations": [],
                                 "grid": col("Grid_Size_X", "Grid_Size"),
                                 "wg": col("Workgroup_Size_X", "Workgroup_Size"),
                                 "lds": col("LDS_Block_Size", "Group_Segment_Size"),
                                 "scratch": col("Scratch_Size", "Private_Segment_Size"),
                                 "vgpr": col("VGPR_Count", "Arch_VGPR_Count"),
                                 "agpr": col("Accum_VGPR_Count")})
        s["durations"].append(dur)

    def counter(sub, name):
        per = {}
        for r in _csv_rows(os.path.join(d, sub, "**", "*counter_collection.csv")):
            if r["Counter_Name"] != name:
                continue
            k = _short(r["Kernel_Name"])
            per.setdefault(k, {}).setdefault(r["Dispatch_Id"], 0.0)
            per[k][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {k: sum(v.values()) / len(v) for k, v in per.items()}

    fetch = counter("fetch", "FETCH_SIZE")
    write = counter("write", "WRITE_SIZE")
    sq = {c: counter("sq", c) for c in SQ_COUNTERS}
    calib_bytes = (CALIB_MIB << 20) // (128 * 128 * 4) * (128 * 128 * 4)
    ff = calib_bytes / (fetch[CALIB_KERNEL] * 1024) if fetch.get(CALIB_KERNEL) else None
    wf = calib_bytes / (write[CALIB_KERNEL] * 1024) if write.get(CALIB_KERNEL) else None
    shash = source_hash()
    kernels = {}
    os.makedirs(out_dir, exist_ok=True)
    for k, s in sorted(stats.items()):
        # kernels of the other legs of the profiled run are filed under their own workload
        wl = OTHER_LEG_WORKLOAD.get(k, label)
        durs = s["durations"]
        avg = sum(durs) / len(durs)
        lines = [f"# {k} -- {wl}", "",
                 f"kernel: {s['full_name']}",
                 f"source hash of the kernel sources (bench.py KERNEL_SOURCES): {shash}", "",
                 "## Kernel trace (rocprofv3 --kernel-trace --stats)",
                 f"command: {cmds['trace']}",
                 f"dispatches: {len(durs)}   grid: {s['grid']} work-items, workgroup {s['wg']}   "
                 f"LDS: {s['lds']} B   scratch: {s['scratch']} B/lane   VGPRs: {s['vgpr']} "
                 f"(+{s['agpr']} AGPRs)",
                 f"duration avg: {avg:.2f} us   min: {min(durs):.2f} us   max: {max(durs):.2f} us"]
        entry = {"avg_us": avg, "dispatches": len(durs)}
        if k in fetch and k in write and ff and wf:
            nbytes = fetch[k] * 1024 * ff + write[k] * 1024 * wf
            entry.update({"fetch_KiB": fetch[k], "write_KiB": write[k], "bytes_per_launch": nbytes})
            lines += ["", "## HBM traffic (rocprofv3 --pmc, one counter per run)",
                      f"commands: {cmds['fetch']}", f"          {cmds['write']}",
                      f"FETCH_SIZE: {fetch[k]:.1f} KiB/dispatch   WRITE_SIZE: {write[k]:.1f} KiB/dispatch",
                      f"calibration ({CALIB_KERNEL}, {calib_bytes} B read and {calib_bytes} B written "
                      f"per launch): FETCH_SIZE x {ff:.3f}, WRITE_SIZE x {wf:.3f} give bytes",
                      f"HBM bytes per launch: read {fetch[k] * 1024 * ff / 1e6:.1f} MB + written "
                      f"{write[k] * 1024 * wf / 1e6:.1f} MB = {nbytes / 1e6:.1f} MB",
                      f"achieved on those bytes: {nbytes / (avg * 1e-6) / 1e9:.0f} GB/s = "
                      f"{nbytes / (avg * 1e-6) / HBM_PEAK * 100:.1f}% of 8 TB/s"]
        if all(k in sq[c] for c in SQ_COUNTERS):
            gui = sq["GRBM_GUI_ACTIVE"][k] / 8  # summed over the 8 XCDs
            simd_cycles = gui * 1024
            mfma_busy = sq["SQ_VALU_MFMA_BUSY_CYCLES"][k] / simd_cycles
            bf16_flops = sq["SQ_INSTS_VALU_MFMA_MOPS_BF16"][k] * 512
            waves = sq["SQ_WAVES"][k]
            entry.update({"mfma_busy": mfma_busy, "bf16_tflops": bf16_flops / (avg * 1e-6) / 1e12,
                          "valu_insts_per_wave": sq["SQ_INSTS_VALU"][k] / max(waves, 1),
                          "valu_active_frac": sq["SQ_ACTIVE_INST_VALU"][k] * 4 / simd_cycles,
                          "clock_GHz": gui / (avg * 1e-6) / 1e9})
            lines += ["", "## Matrix-core and VALU counters (rocprofv3 --pmc)",
                      f"command: {cmds['sq']}",
                      "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); "
                      "bf16 MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; VALU active = "
                      "SQ_ACTIVE_INST_VALU x 4 / SIMD cycles",
                      f"clock {entry['clock_GHz']:.2f} GHz   MFMA busy {mfma_busy * 100:.1f}%   "
                      f"bf16 MFMA {entry['bf16_tflops']:.1f} TFLOP/s = "
                      f"{entry['bf16_tflops'] * 1e12 / BF16_PEAK * 100:.2f}% of 2.5 PFLOP/s   "
                      f"VALU instructions per wave {entry['valu_insts_per_wave']:.0f}   "
                      f"VALU active {entry['valu_active_frac'] * 100:.1f}%"]
        kernels.setdefault(wl, {})[k] = entry
        with open(os.path.join(out_dir, f"{k}.{wl}.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
    tpath = os.path.join(out_dir, "traffic.json")
    try:
        with open(tpath) as f:
            tj = json.load(f)
    except (OSError, ValueError):
        tj = {}
    tj.setdefault("workloads", {})
    tj["calibration"] = {"kernel": CALIB_KERNEL, "bytes_read_and_written": calib_bytes}
    for wl, ks in kernels.items():
        tj["workloads"][wl] = {"source_hash": shash, "fetch_factor": ff, "write_factor": wf,
                               "commands": cmds, "kernels": ks}
    with open(tpath, "w") as f:
        json.dump(tj, f, indent=1)
    return tj["workloads"][label]


def calibration_copy(kda, torch, mib, stream, dev):
    """kda_prefill with T = 0 copies S0 to S_T with one plain copy kernel
    (kda_copy_state_kernel): exactly n bytes read and n bytes written."""
    nb_state = 128 * 128 * 4
    nbh = max(1, mib * (1 << 20) // nb_state)
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


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--also", default=ALSO, help="comma-separated prefill workloads timed beside "
                                                 "the headline ('none' for none)")
    ap.add_argument("--decode-workload", default="decode-b256")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle timing (0 = skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-stages", action="store_true",
                    help="skip the legs with the optional stages (raw projections, output norm + "
                         "gate), packed sequences and the backward pass")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run the library's plain state-copy kernel (kda_prefill with T=0) "
                         "on this many MiB, to calibrate HBM byte counters")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only kda_prefill_backward on --workload (the profile of the backward)")
    ap.add_argument("--profile-commands", metavar="DIR",
                    help="print the rocprofv3 commands of a profile of --workload into DIR and exit")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="summarize a profile of --workload taken by those commands into profiles/")
    args = ap.parse_args(argv)
    if args.profile_commands:
        for c in profile_commands(args.profile_commands.rstrip("/"), args.workload,
                                  args.backward_only).values():
            print(c)
        return 0
    if args.summarize_rocprof:
        e = summarize_rocprof(args.summarize_rocprof.rstrip("/"), args.workload,
                              os.path.join(ROOT, "profiles"), args.backward_only)
        print(json.dumps({k: {kk: vv for kk, vv in v.items()} for k, v in e["kernels"].items()},
                         indent=1))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU: the KDA mixer shards over (sequence, head) with no "
              "collective, so only --gpus 1 is run here", file=sys.stderr)
        return 2

    import torch

    import gated_delta_rule_80_amd as kda
    from kda_inputs import WORKLOADS, make_inputs

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    w = WORKLOADS[args.workload]
    if args.backward_only:
        print(f"timing the backward of {w.name}", file=sys.stderr, flush=True)
        bw = backward_leg(kda, torch, w, args, stream, dev, float("nan"))
        if args.calib_copy_mib > 0:
            calibration_copy(kda, torch, args.calib_copy_mib, stream, dev)
        print(json.dumps({"metric": "KDA backward tokens/s", "value": bw["tokens_per_s"],
                          "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
                          "warmup": args.warmup, "ms_per_step": bw["ms_per_step"],
                          "higher_is_better": True, "dtype": w.io, "data": "synthetic",
                          "config": {"workload": w.name}, "backward": bw,
                          "source_hash": source_hash()}), flush=True)
        return 0
    head, _ = measure_prefill(kda, torch, w, args, stream, dev)
    others = {}
    for name in [x for x in args.also.split(",") if x and x != "none" and x != w.name]:
        others[name] = measure_prefill(kda, torch, WORKLOADS[name], args, stream, dev)[0]

    # ---- decode leg
    wd = WORKLOADS[args.decode_workload]
    dinp = make_inputs(wd, seed=args.seed + 1, device=dev)
    S = dinp["S0"]
    cs = dinp["conv_state"]
    od = torch.empty_like(dinp["q"])
    da = kda.decode_args(dinp["q"], dinp["k"], dinp["v"], dinp["g"], dinp["beta"], S, od,
                         dinp["conv_w"], cs)
    print(f"timing {wd.name}", file=sys.stderr, flush=True)
    dms = time_decode(kda, torch, da, stream, args.steps, args.warmup)
    dbytes = decode_bytes(wd)
    decode = {"metric": "KDA decode seq/s", "value": wd.B / (dms / 1e3), "unit": "seq/s",
              "ms_per_step": dms, "config": {"workload": wd.name, "B": wd.B, "H": wd.H, "D": wd.D},
              "roofline": {"bound": "hbm", "kernel": "kda_decode_kernel",
                           "achieved": dbytes / (dms / 1e3) / 1e9, "peak": HBM_PEAK / 1e9,
                           "unit": "GB/s", "frac": dbytes / (dms / 1e3) / HBM_PEAK,
                           "traffic": traffic_for(wd.name, "kda_decode_kernel"),
                           "algorithmic_bytes": dbytes}}
    del dinp, S, cs, od, da
    torch.cuda.empty_cache()
    decode["hbm_probe"] = hbm_probe(torch, dev, stream, args.steps)

    stages = None
    if not args.no_stages:
        ws4 = WORKLOADS[STAGES_WORKLOAD]
        base = others.get(ws4.name) or (head if w.name == ws4.name else None)
        base_ms = base["ms_per_step"] if base else float("nan")
        print("timing the optional stages, packed sequences and the backward", file=sys.stderr,
              flush=True)
        stages = stages_leg(kda, torch, ws4, wd, args, stream, dev, base_ms, dms)
        stages["packed"] = packed_leg(kda, torch, ws4, args, stream, dev, base_ms)
        stages["backward"] = backward_leg(kda, torch, ws4, args, stream, dev, base_ms)
        stages["backward_every_stage"] = backward_leg(kda, torch, ws4, args, stream, dev, base_ms,
                                                      stages=True)
        stages["backward_packed"] = backward_leg(kda, torch, ws4, args, stream, dev, base_ms,
                                                 packed=True)
        # the backward of one GPU's share of the heads at long context (split walks)
        wtp = WORKLOADS[TP_SHARE_WORKLOAD]
        tp = others.get(wtp.name) or (head if w.name == wtp.name else None)
        stages["backward_tp_share"] = backward_leg(kda, torch, wtp, args, stream, dev,
                                                   tp["ms_per_step"] if tp else float("nan"))
        stages["training"] = training_leg(kda, torch, ws4, args, stream, dev, base_ms,
                                          stages["backward"]["ms_per_step"])
        # the backward of the headline workload itself
        stages["backward_headline"] = backward_leg(kda, torch, w, args, stream, dev,
                                                   head["ms_per_step"])

    if args.calib_copy_mib > 0:
        calibration_copy(kda, torch, args.calib_copy_mib, stream, dev)

    cpu = None
    if args.cpu_budget > 0:
        print(f"timing the oracle on the host (~{args.cpu_budget:.0f} s)", file=sys.stderr,
              flush=True)
        cinp = make_inputs(w, seed=args.seed, device=dev)
        cpu = cpu_baseline(w, cinp, args.cpu_budget)
        del cinp

    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.io, "data": "synthetic",
        "config": dict({"workload": w.name}, **head["config"]),
        "roofline": head["roofline"], "path": head["path"],
        "prefill_configs": others, "decode": decode, "stages": stages,
        "cpu_baseline": cpu,
        "source_hash": source_hash(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
