"""Gradients of the prefill on the GPU against the fp64 oracle's reverse-mode
gradients (kda_reference_backward, itself pinned by finite differences).

Loss L = <o, do> + <S_T, dS_T> with random do, dS_T.  Tolerance: relative L2 per
gradient tensor, 2e-2 for bf16 inputs and 1e-4 for fp32 inputs (the same bar as
the forward), over dq, dk, dv, dg, dbeta, dS0, dconv_w and dconv_state."""
import numpy as np
import pytest
import torch

import gated_delta_rule_80_amd as kda
from kda_inputs import to_numpy
from kda_testutil import TOL, cuda, make, rel_l2, small
from oracle import kda_reference_backward

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0", "dconv_w", "dconv_state")


def check_backward(w, chunk, seed=0, conv=True, l2=True, scale=1.0, with_dST=True, g_head=None):
    inp = make(w, seed)
    if g_head is not None:
        # constant log-decay per token on the given heads: {head: g}
        g = inp["g"].clone()
        for hh, val in g_head.items():
            g[:, :, hh, :] = val
        inp = dict(inp, g=g)
    if not conv:
        inp = dict(inp, conv_w=None, conv_state=None)
    gen = torch.Generator().manual_seed(seed + 1000)
    do = torch.randn(w.B, w.T, w.H, w.D, generator=gen).to(inp["q"].dtype)
    dST = torch.randn(w.B, w.H, w.D, w.D, generator=gen) if with_dST else None
    c = cuda(inp)
    grads, o, S_T = kda.kda_prefill_backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                             c["conv_state"], c["S0"], do=do.cuda(),
                                             dS_T=None if dST is None else dST.cuda(), chunk=chunk,
                                             scale=scale, l2norm_qk=l2)
    torch.cuda.synchronize()
    n = {k: to_numpy(v) for k, v in inp.items()}
    ref = kda_reference_backward(n["q"], n["k"], n["v"], n["g"], n["beta"], to_numpy(do),
                                 None if dST is None else to_numpy(dST), conv_w=n["conv_w"],
                                 conv_state=n["conv_state"], S0=n["S0"], scale=scale, l2norm_qk=l2)
    tol = TOL[w.io]
    errs = {}
    for name in NAMES:
        if ref.get(name) is None:
            continue
        got = grads[name].cpu().numpy()
        assert np.isfinite(got).all(), name
        errs[name] = rel_l2(got, ref[name])
    print(f"{w.name} C={chunk} conv={conv} l2={l2}: " +
          " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    for name, e in errs.items():
        assert e <= tol, (name, e)


def test_backward_tiny_fp32():
    w = small(B=1, T=64, H=2, D=16, io="fp32", chunk=16, s0=True, conv_state=True)
    check_backward(w, 16)


@pytest.mark.parametrize("io,D,chunk", [("fp32", 16, 16), ("fp32", 32, 32), ("fp32", 64, 64),
                                        ("bf16", 32, 16), ("bf16", 64, 32), ("bf16", 128, 64),
                                        ("bf16", 128, 32), ("bf16", 128, 16), ("bf16", 16, 64),
                                        ("bf16", 32, 64), ("bf16", 64, 64), ("bf16", 16, 16)])
def test_backward_dims_and_chunks(io, D, chunk):
    w = small(B=2, T=77, H=2, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    check_backward(w, chunk, seed=D + chunk)


@pytest.mark.parametrize("T", [1, 3, 16, 17, 64, 65, 130])
def test_backward_lengths(T):
    w = small(B=1, T=T, H=2, D=64, io="fp32", chunk=32, s0=True, conv_state=True)
    check_backward(w, 32, seed=T)


@pytest.mark.parametrize("conv,l2", [(False, True), (True, False), (False, False)])
def test_backward_front_end_modes(conv, l2):
    w = small(B=1, T=50, H=2, D=32, io="fp32", chunk=16, s0=True, conv_state=True)
    check_backward(w, 16, seed=3, conv=conv, l2=l2, scale=0.5 if not l2 else 1.0)


def test_backward_strong_decay_bf16():
    w = small(B=1, T=200, H=2, D=128, io="bf16", chunk=64, strong=True, s0=True, conv_state=True)
    check_backward(w, 64, seed=7)


@pytest.mark.parametrize("io,D,chunk", [("bf16", 128, 64), ("fp32", 64, 32), ("bf16", 32, 16)])
@pytest.mark.parametrize("g0", [-12.0, -5.2])
def test_backward_factored_and_exact_pair_paths(io, D, chunk, g0):
    """Head 0 decays by a constant g0 per token: -12 gives 16-token block spans of
    about 277 log2 units, beyond the factored pair products' limit (the chunks go to
    the exact per-pair kernel); -5.2 gives about 120, just inside it (the widest
    factors the factored kernel meets).  Head 1 keeps its drawn decays."""
    w = small(B=1, T=150, H=2, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    check_backward(w, chunk, seed=17, g_head={0: g0})


def test_backward_without_state_gradients():
    w = small(B=2, T=40, H=2, D=64, io="bf16", chunk=32)
    check_backward(w, 32, seed=8, with_dST=False)


def test_backward_repeated_calls_are_bit_identical():
    w = small(B=1, T=150, H=3, D=128, io="bf16", chunk=64, s0=True, conv_state=True)
    inp = cuda(make(w, 9))
    do = torch.randn(w.B, w.T, w.H, w.D, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).cuda()
    first = None
    for _ in range(5):
        grads, _, _ = kda.kda_prefill_backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                               inp["conv_w"], inp["conv_state"], inp["S0"], do=do,
                                               chunk=64)
        torch.cuda.synchronize()
        if first is None:
            first = {k: v.clone() for k, v in grads.items()}
        else:
            for k, v in grads.items():
                assert torch.equal(v, first[k]), k


def test_backward_empty_sequence():
    """T = 0: dS0 = dS_T, the filter and history gradients are zero."""
    w = small(B=2, T=0, H=2, D=32, io="fp32", chunk=16, s0=True, conv_state=True)
    inp = cuda(make(w, 1))
    dST = torch.randn(2, 2, 32, 32, device="cuda")
    do = torch.empty(2, 0, 2, 32, device="cuda")
    grads, o, S_T = kda.kda_prefill_backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                             inp["conv_w"], inp["conv_state"], inp["S0"], do=do,
                                             dS_T=dST, chunk=16)
    torch.cuda.synchronize()
    assert torch.equal(grads["dS0"], dST)
    assert torch.equal(S_T, inp["S0"])
    assert float(grads["dconv_w"].abs().max()) == 0.0
    assert float(grads["dconv_state"].abs().max()) == 0.0
