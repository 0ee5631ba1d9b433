"""kda_prefill_static, the entry point that allocates nothing (its workspace is the
library's static per-GPU scratch array), against kda_prefill with a workspace of
its own, called through the C ABI.

Two calls in a row, the second with a smaller input: the first needs more than
the scratch (456 MB of records at B=1, T=4096, H=96, D=128, bf16) and runs in
time slices; the second fits and runs as kda_prefill does.  Outputs, final
states and conv hand-overs must equal kda_prefill's bit for bit (slicing hands
the float32 state over exactly and prepares every chunk as the whole-sequence
call does), which is stricter than the oracle tolerance."""
import pytest
import torch

import gated_delta_rule_80_amd as kda
from kda_inputs import WORKLOADS, make_inputs, make_stage_inputs
from kda_testutil import small

pytestmark = pytest.mark.gpu

SCRATCH = 128 << 20


def both(w, seed, stages=False, in_place=False):
    """Run kda_prefill (own workspace) and kda_prefill_static on the same inputs;
    returns ((o, S_T, conv out) of each, static status, whole-sequence workspace bytes)."""
    inp = make_inputs(w, seed=seed, device="cuda")
    st = make_stage_inputs(w, seed=seed, device="cuda") if stages else None
    outs = []
    status = None
    need = None
    for static in (False, True):
        o = torch.empty_like(inp["q"])
        S0 = None if inp["S0"] is None else inp["S0"].clone()
        S_T = S0 if in_place and S0 is not None else torch.empty(
            w.B, w.H, w.D, w.D, dtype=torch.float32, device="cuda")
        cso = torch.empty(w.B, 3, 3, w.H * w.D, dtype=inp["q"].dtype, device="cuda")
        kw = {}
        g, beta = inp["g"], inp["beta"]
        if stages:
            g, beta = st["f"], st["b_logit"]
            kw = dict(A_log=st["A_log"], dt_bias=st["dt_bias"], beta_logits=True,
                      o_norm_w=st["o_norm_w"], o_gate=st["o_gate"])
        a = kda.prefill_args(inp["q"], inp["k"], inp["v"], g, beta, inp["conv_w"],
                             inp["conv_state"], S0, o, S_T, cso, chunk=w.chunk, **kw)
        if static:
            status = kda.kda_prefill_static_raw(a)
        else:
            need = kda.kda_prefill_workspace_bytes(a)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            kda.kda_prefill_raw(a, ws)
        torch.cuda.synchronize()
        outs.append((o, S_T, cso))
    return outs, status, need


def check_equal(outs):
    (o1, s1, c1), (o2, s2, c2) = outs
    assert bool(torch.isfinite(o2.float()).all())
    assert torch.equal(o1, o2)
    assert torch.equal(s1, s2)
    assert torch.equal(c1, c2)


def test_static_scratch_two_calls_second_smaller():
    # first call: larger than the scratch, with an initial state and strong decays
    # (some chunks take the exact preparation) -> time slices
    w1 = WORKLOADS["prefill-b4-8k-s0"].scaled(B=1, T=4096, conv_state_std=1.0)
    outs, status, need = both(w1, seed=3)
    print(f"call 1: B={w1.B} T={w1.T} H={w1.H} D={w1.D} {w1.io}, whole-sequence workspace "
          f"{need / 2**20:.0f} MiB > scratch {SCRATCH >> 20} MiB: status {status}", flush=True)
    assert need > SCRATCH
    assert status == kda.KDA_OK
    check_equal(outs)
    # second call, smaller: fits the scratch
    w2 = small(B=2, T=77, H=2, D=64, io="fp32", chunk=32, s0=True, conv_state=True)
    outs, status, need = both(w2, seed=4)
    print(f"call 2: B={w2.B} T={w2.T} H={w2.H} D={w2.D} {w2.io}, workspace {need} B: status "
          f"{status}", flush=True)
    assert need <= SCRATCH
    assert status == kda.KDA_OK
    check_equal(outs)


def test_static_scratch_sliced_in_place_state():
    """S_T == S0 while slices hand the state over through S_T."""
    w = WORKLOADS["prefill-b4-8k-s0"].scaled(B=2, T=2500, H=48)
    outs, status, need = both(w, seed=5, in_place=True)
    assert need > SCRATCH and status == kda.KDA_OK
    check_equal(outs)


def test_static_scratch_sliced_with_optional_stages():
    """Raw-projection decay and beta, output norm and gate applied inside the walk
    (D = 64): the gate rows of each slice are read at the slice's token offset."""
    w = small(B=1, T=2000, H=200, D=64, io="bf16", chunk=64, s0=True, conv_state=True)
    outs, status, need = both(w, seed=6, stages=True)
    assert need > SCRATCH and status == kda.KDA_OK
    check_equal(outs)


def test_static_scratch_rejects_what_does_not_fit():
    """Nothing is enqueued and KDA_ERR_SCRATCH is returned when not even one chunk
    per (sequence, head) fits, or when packed sequences do not fit whole."""
    w = small(B=1, T=64, H=2000, D=128, io="bf16", chunk=64)
    inp = make_inputs(w, seed=7, device="cuda")
    o = torch.full_like(inp["q"], 7.0)
    S_T = torch.empty(w.B, w.H, w.D, w.D, dtype=torch.float32, device="cuda")
    a = kda.prefill_args(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["conv_w"],
                         None, None, o, S_T, None, chunk=64)
    assert kda.kda_prefill_static_raw(a) == kda.KDA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
    # packed: 8 sequences over T = 12000 tokens at H = 96 need more than the scratch
    from kda_inputs import make_packed_inputs
    wp = WORKLOADS["prefill-4k"]
    lengths = [1500] * 8
    pin = make_packed_inputs(wp, lengths, seed=8, device="cuda")
    op = torch.full_like(pin["q"], 7.0)
    Sp = torch.empty(8, wp.H, wp.D, wp.D, dtype=torch.float32, device="cuda")
    ap = kda.prefill_args(pin["q"], pin["k"], pin["v"], pin["g"], pin["beta"], pin["conv_w"],
                          None, None, op, Sp, None, chunk=64, cu_seqlens=pin["cu_seqlens"])
    assert kda.kda_prefill_workspace_bytes(ap) > SCRATCH
    assert kda.kda_prefill_static_raw(ap) == kda.KDA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((op == 7.0).all())
