"""Parity at the workloads' full sizes, in the launch configuration the benchmark
times (same entry points, same shapes, hence the same kernels and grids), over
EVERY (sequence, head) pair.

The GPU runs the whole workload; the fp64 oracle then runs every pair's whole
sequence in a pool of host processes (pairs are independent: each has its own
state, conv filters and channels), and each pair is compared on its own.  The
conv-state hand-over is compared whole and exactly.

Tolerance: relative L2 2e-2 for bf16 inputs per (sequence, head) pair,
separately for o and S_T (the decode state S); the worst pair is printed.  The
worst 64-token block of o per pair must stay within 5e-2, so an error confined
to a few tokens cannot hide under a whole sequence's norm."""
import shutil

import numpy as np
import pytest
import torch

import gated_delta_rule_80_amd as kda
from kda_inputs import WORKLOADS, make_inputs, to_storage
from kda_testutil import TOL
from oracle.pool import (backward_pair, decode_seq, prefill_pair, run, save_array, save_meta,
                         scratch_dir)

pytestmark = pytest.mark.gpu

BLOCK_TOL = 5e-2
FULL = ["prefill-4k", "prefill-b4-8k-s0", "prefill-64k", "prefill-64k-h12"]


def summarize(label, res, tol):
    """res: (b, h, e_o, e_S, e_block, block) per pair."""
    wo = max(res, key=lambda x: x[2])
    wS = max(res, key=lambda x: x[3])
    wb = max(res, key=lambda x: x[4])
    print(f"{label}: {len(res)} pairs; worst o {wo[2]:.2e} at (b={wo[0]}, h={wo[1]}), "
          f"worst S_T {wS[3]:.2e} at (b={wS[0]}, h={wS[1]}), worst 64-token block "
          f"{wb[4]:.2e} at (b={wb[0]}, h={wb[1]}, block {wb[5]})", flush=True)
    bad = [x for x in res if not (x[2] <= tol and x[3] <= tol and x[4] <= BLOCK_TOL)]
    assert not bad, bad[:8]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_prefill_every_pair(name):
    w = WORKLOADS[name]
    print(f"full-size prefill {name}: B={w.B} T={w.T} H={w.H} D={w.D}", flush=True)
    inp = make_inputs(w, seed=0, device="cuda")
    o, S, cs = kda.kda_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["conv_w"],
                               inp["conv_state"], inp["S0"], chunk=w.chunk)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())
    # the conv hand-over: the last three raw inputs of every channel, whole tensor
    HD = w.H * w.D
    for x, t in enumerate(("q", "k", "v")):
        assert torch.equal(cs[:, x], inp[t][:, w.T - 3:].reshape(w.B, 3, HD)), t
    d = scratch_dir(6 * o.numel() * o.element_size())
    try:
        save_meta(d, w.io, w.D)
        for t in ("q", "k", "v", "g", "beta"):
            save_array(d, t, to_storage(inp[t], head_major=True))
        save_array(d, "conv_w", to_storage(inp["conv_w"]))
        save_array(d, "conv_state", to_storage(inp["conv_state"]))
        save_array(d, "S0", to_storage(inp["S0"]))
        save_array(d, "o", to_storage(o, head_major=True))
        save_array(d, "S_T", to_storage(S))
        del inp, o, S, cs
        torch.cuda.empty_cache()
        res = run(prefill_pair, d, [(b, h) for b in range(w.B) for h in range(w.H)], name)
    finally:
        shutil.rmtree(d, ignore_errors=True)
    summarize(name, res, TOL[w.io])


@pytest.mark.timeout(600)
def test_full_size_decode_every_pair():
    w = WORKLOADS["decode-b256"]
    print(f"full-size decode: B={w.B} H={w.H} D={w.D}", flush=True)
    inp = make_inputs(w, seed=1, device="cuda")
    S0 = inp["S0"].clone()
    cs0 = inp["conv_state"].clone()
    S, cs = inp["S0"], inp["conv_state"]
    o = kda.kda_decode_step(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], S,
                            inp["conv_w"], cs)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())
    d = scratch_dir(3 * S.numel() * 4)
    try:
        save_meta(d, w.io, w.D)
        for t in ("q", "k", "v", "g", "beta", "conv_w"):
            save_array(d, t, to_storage(inp[t]))
        save_array(d, "S0", to_storage(S0))
        save_array(d, "conv_state", to_storage(cs0))
        save_array(d, "o", to_storage(o))
        save_array(d, "S", to_storage(S))
        save_array(d, "conv_state_out", to_storage(cs))
        del inp, S0, cs0, S, cs, o
        torch.cuda.empty_cache()
        res = [x for part in run(decode_seq, d, [(b,) for b in range(w.B)], "decode") for x in part]
    finally:
        shutil.rmtree(d, ignore_errors=True)
    assert all(x[4] for x in res), "conv state after the step differs from the oracle's"
    summarize("decode-b256", [(b, h, eo, eS, 0.0, -1) for b, h, eo, eS, _ in res], TOL[w.io])


# (workload, oracle processes): the oracle keeps every step's state of a head
# (8.6 GB at T = 65536, D = 128), so the long case runs 6 heads at a time
BACKWARD_FULL = [("prefill-4k", None), ("prefill-64k-h12", 6)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,workers", BACKWARD_FULL)
def test_full_size_backward_every_head(name, workers):
    """The backward at a workload's full size (at 12 heads and T = 65536 both of
    its walks split into segments), every head against the oracle's reverse-mode
    gradients of that head (heads are independent; the conv filter gradient of a
    head's channels comes from that head alone)."""
    w = WORKLOADS[name]
    print(f"full-size backward {name}: B={w.B} T={w.T} H={w.H} D={w.D}", flush=True)
    inp = make_inputs(w, seed=0, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(5)
    do = torch.randn(w.B, w.T, w.H, w.D, generator=gen, device="cuda").to(torch.bfloat16)
    grads, o, S_T = kda.kda_prefill_backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                             inp["conv_w"], inp["conv_state"], inp["S0"], do=do,
                                             chunk=w.chunk)
    torch.cuda.synchronize()
    for n, t in grads.items():
        assert bool(torch.isfinite(t).all()), n
    d = scratch_dir(12 * do.numel() * 4)
    try:
        save_meta(d, w.io, w.D)
        for t in ("q", "k", "v", "g", "beta"):
            save_array(d, t, to_storage(inp[t], head_major=True))
        save_array(d, "do", to_storage(do, head_major=True))
        save_array(d, "conv_w", to_storage(inp["conv_w"]))
        save_array(d, "conv_state", to_storage(inp["conv_state"]))
        save_array(d, "S0", to_storage(inp["S0"]))
        for n in ("dq", "dk", "dv", "dg", "dbeta"):
            save_array(d, n, to_storage(grads[n], head_major=True))
        for n in ("dS0", "dconv_w", "dconv_state"):
            save_array(d, n, to_storage(grads[n]))
        del inp, do, grads, o, S_T
        torch.cuda.empty_cache()
        res = run(backward_pair, d, [(0, h) for h in range(w.H)], "backward", workers=workers)
    finally:
        shutil.rmtree(d, ignore_errors=True)
    tol = TOL[w.io]
    names = sorted(res[0][2])
    for n in names:
        worst = max(res, key=lambda x: x[2][n])
        print(f"  backward {n}: worst rel_l2 {worst[2][n]:.2e} at h={worst[1]}", flush=True)
    bad = [(b, h, n, e) for b, h, errs in res for n, e in errs.items() if not e <= tol]
    assert not bad, bad[:8]
