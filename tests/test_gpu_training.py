"""The training pair: kda_prefill_forward_saved keeps what its backward needs,
kda_prefill_backward_saved runs the backward without recomputing the forward.

Both run the same kernels on the same data as kda_prefill_backward, so the
forward outputs (o, S_T, the conv hand-over) and every gradient must equal
kda_prefill_backward's bit for bit; o and S_T also match kda_prefill (to the
prefill tolerance: with the output stage at D <= 64 kda_prefill applies it inside
the walk, from unrounded values)."""
import pytest
import torch

import gated_delta_rule_80_amd as kda
from kda_inputs import make_packed_inputs, make_stage_inputs
from kda_testutil import TOL, cuda, make, rel_l2, small

pytestmark = pytest.mark.gpu


def run_both(c, chunk, do, dS_T=None, **kw):
    grads, o, S_T = kda.kda_prefill_backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                             c["conv_state"], c["S0"], do=do, dS_T=dS_T,
                                             chunk=chunk, **kw)
    o2, S2, cs2, saved = kda.kda_prefill_forward_saved(c["q"], c["k"], c["v"], c["g"], c["beta"],
                                                       c["conv_w"], c["conv_state"], c["S0"],
                                                       chunk=chunk, **kw)
    g2 = kda.kda_prefill_backward_saved(saved, do=do, dS_T=dS_T)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S_T, S2)
    assert set(grads) == set(g2)
    for n in grads:
        assert torch.equal(grads[n], g2[n]), n
    return o2, S2, cs2, g2


@pytest.mark.parametrize("io,D,chunk,B,H,T", [
    ("bf16", 128, 64, 2, 2, 300), ("fp32", 64, 32, 1, 3, 200), ("bf16", 32, 16, 2, 2, 77),
    ("bf16", 128, 64, 1, 1, 64 * 70 + 5),  # walks split into segments
])
def test_saved_pair_equals_backward(io, D, chunk, B, H, T):
    w = small(B=B, T=T, H=H, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    c = cuda(make(w, seed=T))
    gen = torch.Generator(device="cuda").manual_seed(3)
    do = torch.randn(B, T, H, D, generator=gen, device="cuda").to(c["q"].dtype)
    dS_T = torch.randn(B, H, D, D, generator=gen, device="cuda")
    o, S_T, cs, _ = run_both(c, chunk, do, dS_T)
    ro, rS, rcs = kda.kda_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                  c["conv_state"], c["S0"], chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(cs, rcs)
    assert rel_l2(o.float().cpu().numpy(), ro.float().cpu().numpy()) <= TOL[io]
    assert rel_l2(S_T.cpu().numpy(), rS.cpu().numpy()) <= TOL[io]


@pytest.mark.parametrize("D", [128, 64])
def test_saved_pair_every_optional_stage(D):
    w = small(B=1, T=260, H=2, D=D, io="bf16", chunk=64, s0=True, conv_state=True)
    c = cuda(make(w, seed=9))
    st = make_stage_inputs(w, seed=9, device="cuda")
    c = dict(c, g=st["f"], beta=st["b_logit"])
    kw = dict(A_log=st["A_log"], dt_bias=st["dt_bias"], beta_logits=True, o_norm_w=st["o_norm_w"],
              o_gate=st["o_gate"])
    do = torch.randn(1, 260, 2, D, device="cuda").to(torch.bfloat16)
    run_both(c, 64, do, **kw)


def test_saved_pair_packed():
    w = small(B=1, T=500, H=2, D=64, io="bf16", chunk=32, s0=True, conv_state=True)
    inp = cuda(make_packed_inputs(w, [200, 0, 37, 263], seed=4))
    do = torch.randn(1, 500, 2, 64, device="cuda").to(torch.bfloat16)
    run_both(inp, 32, do, cu_seqlens=inp["cu_seqlens"])


def test_saved_pair_no_tokens():
    w = small(B=2, T=0, H=2, D=32, io="fp32", chunk=32, s0=True, conv_state=True)
    c = cuda(make(w, seed=2))
    dS_T = torch.randn(2, 2, 32, 32, device="cuda")
    do = torch.empty(2, 0, 2, 32, device="cuda")
    o, S_T, cs, g = run_both(c, 32, do, dS_T)
    assert torch.equal(S_T, c["S0"]) and torch.equal(g["dS0"], dS_T)
    assert not g["dconv_w"].any() and not g["dconv_state"].any()
