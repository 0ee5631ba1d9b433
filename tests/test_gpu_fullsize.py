"""Parity at the workloads' full sizes, in the launch configuration the benchmark
times (same entry points, same shapes, hence the same kernels and grids).

The GPU runs the whole workload; the fp64 oracle then runs whole sequences of a
few sampled (sequence, head) pairs -- every (b, h) pair is independent of the
others, so a sampled pair is an exact check of that pair's outputs.  Everything
else is checked through properties that hold at any size: finite outputs, the
conv-state hand-over equal to the raw inputs it copies, and untouched pairs of
the decode state staying finite.

Tolerance: relative L2 2e-2 for bf16 inputs (per sampled pair, separately for
o and S_T)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_80_amd as kda
from kda_inputs import WORKLOADS, make_inputs, to_numpy
from kda_testutil import TOL, oracle_heads, rel_l2
from oracle import kda_reference_backward, kda_reference_decode_step

pytestmark = pytest.mark.gpu

# sampled (b, h) pairs per workload: first / middle / last heads, every sequence
# of the batched case touched at least once
SAMPLES = {
    "prefill-4k": [(0, 0), (0, 57), (0, 95)],
    "prefill-b4-8k-s0": [(0, 3), (1, 50), (3, 95)],
    "prefill-64k": [(0, 41)],
}


@pytest.mark.parametrize("name", list(SAMPLES))
def test_full_size_prefill_sampled_pairs(name):
    w = WORKLOADS[name]
    print(f"full-size prefill {name}: B={w.B} T={w.T} H={w.H} D={w.D}", flush=True)
    inp = make_inputs(w, seed=0, device="cuda")
    o, S, _ = kda.kda_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["conv_w"],
                              inp["conv_state"], inp["S0"], chunk=w.chunk)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())
    tol = TOL[w.io]
    pairs = SAMPLES[name]
    for (b, h), (ro, rS) in zip(pairs, oracle_heads(inp, pairs)):
        go = o[b, :, h].float().cpu().numpy()
        gS = S[b, h].cpu().numpy()
        eo, eS = rel_l2(go, ro), rel_l2(gS, rS)
        print(f"  (b={b}, h={h}): rel_l2 o={eo:.2e} S_T={eS:.2e}", flush=True)
        assert eo <= tol, (b, h, eo)
        assert eS <= tol, (b, h, eS)


def test_full_size_conv_state_handover():
    """The conv state handed over at the end of the 4k prefill is exactly the last
    three raw inputs of every channel (whole tensor, not sampled)."""
    w = WORKLOADS["prefill-4k"]
    inp = make_inputs(w, seed=0, device="cuda")
    _, _, cs = kda.kda_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                               inp["conv_w"], inp["conv_state"], inp["S0"], chunk=w.chunk)
    torch.cuda.synchronize()
    HD = w.H * w.D
    for x, name in enumerate(("q", "k", "v")):
        want = inp[name][:, w.T - 3:].reshape(w.B, 3, HD)
        assert torch.equal(cs[:, x], want), name


def test_full_size_decode_sampled_pairs():
    w = WORKLOADS["decode-b256"]
    print(f"full-size decode: B={w.B} H={w.H} D={w.D}", flush=True)
    inp = make_inputs(w, seed=1, device="cuda")
    pairs = [(0, 0), (17, 40), (128, 95), (255, 63)]
    before = {p: to_numpy(inp["S0"][p[0], p[1]]) for p in pairs}
    S = inp["S0"]
    cs = inp["conv_state"]
    cs0 = cs.clone()
    o = kda.kda_decode_step(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], S,
                            inp["conv_w"], cs)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())
    tol = TOL[w.io]
    D = w.D
    for b, h in pairs:
        ch = slice(h * D, (h + 1) * D)
        one = lambda t: to_numpy(t[b:b + 1, h:h + 1])
        ro, rS, rcs = kda_reference_decode_step(
            one(inp["q"]), one(inp["k"]), one(inp["v"]), one(inp["g"]),
            to_numpy(inp["beta"][b:b + 1, h:h + 1]), before[(b, h)][None, None],
            conv_w=to_numpy(inp["conv_w"][:, ch]), conv_state=to_numpy(cs0[b:b + 1, :, :, ch]))
        eo = rel_l2(o[b, h].float().cpu().numpy(), ro[0, 0])
        eS = rel_l2(S[b, h].cpu().numpy(), rS[0, 0])
        print(f"  (b={b}, h={h}): rel_l2 o={eo:.2e} S={eS:.2e}", flush=True)
        assert eo <= tol and eS <= tol, (b, h, eo, eS)
        np.testing.assert_array_equal(cs[b:b + 1, :, :, ch].float().cpu().numpy(), rcs)


def test_full_size_backward_sampled_head():
    """The backward at the 4k workload's full size (every head and chunk on the
    GPU), checked on one sampled head against the oracle's reverse-mode gradients
    of that head (heads are independent; the conv filter gradient of the head's
    channels comes from that head alone)."""
    w = WORKLOADS["prefill-4k"]
    inp = make_inputs(w, seed=0, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(5)
    do = torch.randn(w.B, w.T, w.H, w.D, generator=gen, device="cuda").to(torch.bfloat16)
    grads, o, S_T = kda.kda_prefill_backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                             inp["conv_w"], inp["conv_state"], inp["S0"], do=do,
                                             chunk=w.chunk)
    torch.cuda.synchronize()
    for n, t in grads.items():
        assert bool(torch.isfinite(t).all()), n
    b, h = 0, 37
    D = w.D
    ch = slice(h * D, (h + 1) * D)
    one = lambda x: to_numpy(x[b:b + 1, :, h:h + 1])
    ref = kda_reference_backward(one(inp["q"]), one(inp["k"]), one(inp["v"]), one(inp["g"]),
                                 to_numpy(inp["beta"][b:b + 1, :, h:h + 1]), one(do),
                                 conv_w=to_numpy(inp["conv_w"][:, ch]))
    tol = TOL[w.io]
    pairs = {"dq": grads["dq"][b:b + 1, :, h:h + 1], "dk": grads["dk"][b:b + 1, :, h:h + 1],
             "dv": grads["dv"][b:b + 1, :, h:h + 1], "dg": grads["dg"][b:b + 1, :, h:h + 1],
             "dbeta": grads["dbeta"][b:b + 1, :, h:h + 1], "dS0": grads["dS0"][b:b + 1, h:h + 1],
             "dconv_w": grads["dconv_w"][:, ch], "dconv_state": grads["dconv_state"][b:b + 1, :, :, ch]}
    for n, t in pairs.items():
        e = rel_l2(t.cpu().numpy(), ref[n])
        print(f"  backward (b={b}, h={h}) {n}: rel_l2 {e:.2e}", flush=True)
        assert e <= tol, (n, e)
