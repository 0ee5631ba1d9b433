"""Parity of the optional stages with the fp64 oracle, through the C ABI.

* decay and write strength from raw projections (A_log, dt_bias, beta logits),
  computed inside the chunk preparation (fast and exact paths) and the decode step;
* the output RMSNorm with its gain and the sigmoid output gate, applied inside the
  state walk when one workgroup holds a head's whole output row, by a separate
  in-place pass otherwise, and inside the decode step.

Tolerance as for the plain mixer: relative L2 2e-2 (bf16 inputs), 1e-4 (fp32),
separately for o and S_T; the conv state hand-over exactly.  Sequence lengths are
ragged (not multiples of the chunk) so that masking of the last chunk's tail is
covered: a raw projection of zero does not give a zero decay or write strength."""
import numpy as np
import pytest
import torch

import gated_delta_rule_80_amd as kda
from kda_inputs import make_stage_inputs, to_numpy
from kda_testutil import TOL, cuda, gpu_prefill, make, oracle_prefill, rel_l2, small
from oracle import kda_reference_decode_step

pytestmark = pytest.mark.gpu


def stage_kwargs(w, seed, *, act_g=False, act_b=False, norm=False, gate=False, a_log=None):
    """(modified inputs, GPU kwargs, oracle kwargs) for the chosen stages."""
    inp = make(w, seed)
    st = make_stage_inputs(w, seed)
    if a_log is not None:
        st["A_log"] = torch.full_like(st["A_log"], a_log)
    gk, rk = {}, {}
    if act_g:
        inp = dict(inp, g=st["f"])
        gk.update(A_log=st["A_log"].cuda(), dt_bias=st["dt_bias"].cuda())
        rk.update(A_log=to_numpy(st["A_log"]), dt_bias=to_numpy(st["dt_bias"]))
    if act_b:
        inp = dict(inp, beta=st["b_logit"])
        gk["beta_logits"] = True
        rk["beta_sigmoid"] = True
    if norm:
        gk["o_norm_w"] = st["o_norm_w"].cuda()
        rk["o_norm_w"] = to_numpy(st["o_norm_w"])
    if gate:
        gk["o_gate"] = st["o_gate"].cuda()
        rk["o_gate"] = to_numpy(st["o_gate"])
    return inp, gk, rk


def check(w, seed=0, **stages):
    inp, gk, rk = stage_kwargs(w, seed, **stages)
    o, S, tail = gpu_prefill(inp, w.chunk, **gk)
    ro, rS, rtail = oracle_prefill(inp, **rk)
    tol = TOL[w.io]
    eo, eS = rel_l2(o, ro), rel_l2(S, rS)
    print(f"{w.name} C={w.chunk} {stages}: rel_l2 o={eo:.2e} S_T={eS:.2e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    assert eo <= tol, eo
    assert eS <= tol, eS
    if rtail is not None and tail is not None:
        np.testing.assert_array_equal(tail, rtail)


# ------------------------------------------------- output RMSNorm + sigmoid gate
# (io, D, chunk, B, H): whole rows in the walk for D <= 64, the separate pass at
# D = 128.
OUT_CASES = [
    ("fp32", 16, 16, 2, 2), ("bf16", 32, 32, 2, 2), ("fp32", 64, 32, 1, 3), ("fp32", 64, 64, 1, 2),
    ("bf16", 64, 64, 2, 2), ("bf16", 128, 64, 1, 2), ("fp32", 128, 32, 1, 2), ("bf16", 128, 16, 1, 2),
]


@pytest.mark.parametrize("io,D,chunk,B,H", OUT_CASES)
def test_output_norm_and_gate(io, D, chunk, B, H):
    w = small(B=B, T=77, H=H, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    check(w, seed=D + chunk, norm=True, gate=True)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_output_stage_many_heads_d128(chunk):
    """bf16, D = 128 with B * H = 256 (a full grid of walks)."""
    w = small(B=2, T=70, H=128, D=128, io="bf16", chunk=chunk, s0=True)
    check(w, seed=chunk, norm=True, gate=True)


@pytest.mark.parametrize("io,chunk", [("bf16", 64), ("fp32", 64), ("bf16", 16)])
def test_output_stage_in_walk_long(io, chunk):
    """D = 64 (whole rows in the walk) over many chunks: the double-buffered gate
    tiles alternate correctly."""
    w = small(B=1, T=700, H=2, D=64, io=io, chunk=chunk, s0=True)
    check(w, seed=9, norm=True, gate=True)


@pytest.mark.parametrize("norm,gate", [(True, False), (False, True)])
@pytest.mark.parametrize("io,D,chunk,B,H", [("fp32", 16, 16, 1, 2), ("bf16", 128, 64, 1, 2),
                                            ("bf16", 128, 64, 2, 128)])
def test_output_norm_or_gate_alone(norm, gate, io, D, chunk, B, H):
    w = small(B=B, T=45, H=H, D=D, io=io, chunk=chunk, s0=True)
    check(w, seed=3, norm=norm, gate=gate)


def test_zero_gate_halves_the_output():
    """With a zero gate the GPU output is exactly half the ungated one (the
    sigmoid of 0 is 1/2 in float32 and halving is exact)."""
    w = small(B=1, T=50, H=2, D=64, io="fp32", chunk=32, s0=True)
    inp = make(w, 2)
    o_plain, _, _ = gpu_prefill(inp, 32)
    zero = torch.zeros(w.B, w.T, w.H, w.D, device="cuda")
    o_half, _, _ = gpu_prefill(inp, 32, o_gate=zero)
    np.testing.assert_array_equal(o_half, 0.5 * o_plain)


# ------------------------------------------------- decay and beta from projections
@pytest.mark.parametrize("act_g,act_b", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("io,D,chunk", [("fp32", 16, 16), ("bf16", 128, 64), ("fp32", 64, 32)])
def test_raw_projection_activation(act_g, act_b, io, D, chunk):
    w = small(B=2, T=77, H=2, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    check(w, seed=11, act_g=act_g, act_b=act_b)


@pytest.mark.parametrize("io,D,chunk", [("bf16", 128, 64), ("fp32", 32, 32), ("bf16", 64, 16)])
def test_raw_projection_strong_decay(io, D, chunk):
    """A_log = 3 (rate e^3 ~ 20 per unit of softplus): block spans beyond the fast
    preparation's factoring, so chunks go through the exact preparation."""
    w = small(B=1, T=150, H=2, D=D, io=io, chunk=chunk, s0=True)
    check(w, seed=12, act_g=True, act_b=True, a_log=3.0)


@pytest.mark.parametrize("T", [1, 17, 64, 65])
def test_raw_projection_tail_masking(T):
    """Short and ragged sequences: the activated decay and write strength of the
    padding tokens of the last chunk must be zero, else S_T picks up extra decay."""
    w = small(B=1, T=T, H=2, D=128, io="bf16", chunk=64, s0=True)
    check(w, seed=T, act_g=True, act_b=True)


def test_all_stages_together():
    w = small(B=2, T=200, H=3, D=128, io="bf16", chunk=64, strong=True, s0=True, conv_state=True)
    check(w, seed=21, act_g=True, act_b=True, norm=True, gate=True)


# --------------------------------------------------------------------- decode
@pytest.mark.parametrize("io,D", [("fp32", 16), ("fp32", 64), ("bf16", 32), ("bf16", 128)])
@pytest.mark.parametrize("which", ["all", "norm", "act"])
def test_decode_stages(io, D, which):
    w = small(B=3, T=1, H=4, D=D, io=io, chunk=16, s0=True, conv_state=True)
    w = w.scaled(decode=True)
    stages = dict(act_g=which in ("all", "act"), act_b=which in ("all", "act"),
                  norm=which in ("all", "norm"), gate=which == "all")
    inp, gk, rk = stage_kwargs(w, 5, **stages)
    c = cuda(inp)
    S = c["S0"].clone()
    cs = c["conv_state"].clone()
    o = kda.kda_decode_step(c["q"], c["k"], c["v"], c["g"], c["beta"], S, c["conv_w"], cs, **gk)
    torch.cuda.synchronize()
    n = {k: to_numpy(v) for k, v in inp.items()}
    ro, rS, rcs = kda_reference_decode_step(n["q"], n["k"], n["v"], n["g"], n["beta"], n["S0"],
                                            conv_w=n["conv_w"], conv_state=n["conv_state"], **rk)
    tol = TOL[io]
    eo = rel_l2(o.float().cpu().numpy(), ro)
    eS = rel_l2(S.cpu().numpy(), rS)
    print(f"decode {io} D={D} {which}: rel_l2 o={eo:.2e} S={eS:.2e}", flush=True)
    assert eo <= tol and eS <= tol, (eo, eS)
    np.testing.assert_array_equal(cs.float().cpu().numpy(), rcs)


@pytest.mark.parametrize("D", [64, 128])
def test_stages_compose_with_output_stage(D):
    """Stages 0..3 run one by one equal kda_prefill bit for bit, with the output
    stage applied inside the walk (D = 64) or by the separate pass (D = 128)."""
    w = small(B=1, T=130, H=3, D=D, io="bf16", chunk=64, s0=True, conv_state=True)
    inp, gk, _ = stage_kwargs(w, 7, act_g=True, act_b=True, norm=True, gate=True)
    c = cuda(inp)
    o1, S1, t1 = kda.kda_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                 c["conv_state"], c["S0"], chunk=64, **gk)
    o2, S2, t2 = torch.empty_like(o1), torch.empty_like(S1), torch.empty_like(t1)
    a = kda.prefill_args(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"], c["conv_state"],
                         c["S0"], o2, S2, t2, chunk=64, **gk)
    ws = torch.empty(kda.kda_prefill_workspace_bytes(a), dtype=torch.uint8, device="cuda")
    for stage in (0, 1, 2, 3):
        kda.kda_prefill_stage(a, ws, stage)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(t1, t2)
