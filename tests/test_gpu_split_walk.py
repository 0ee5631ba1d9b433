"""The split state walk against the fp64 oracle, forward and backward.

When a call has few (sequence, head) walks and long sequences, the library cuts
each walk into segments: every segment's affine map (S_end = M S_start + N) is
walked in parallel, the segment start states are composed in order, and each
segment is walked with its outputs from its own start.  These cases are sized so
the split happens (checked through kda_prefill_walk_segments), with several
segment counts, a ragged last chunk and a short last segment, every D, both
element types and the chunk sizes; tolerance as for every prefill: relative L2
2e-2 (bf16) and 1e-4 (fp32) for o and S_T, the conv hand-over exact."""
import numpy as np
import pytest
import torch

import gated_delta_rule_80_amd as kda
from kda_testutil import TOL, cuda, gpu_prefill, make, oracle_prefill, rel_l2, small

pytestmark = pytest.mark.gpu

# (io, D, chunk, B, H, T, strong decay, expected segments)
CASES = [
    ("bf16", 128, 64, 1, 2, 64 * 40 + 17, True, 2),
    ("bf16", 128, 64, 1, 1, 64 * 70 + 1, False, 4),
    ("bf16", 128, 16, 1, 1, 16 * 100 + 5, True, 6),
    ("bf16", 128, 32, 2, 1, 32 * 64, False, 4),
    ("fp32", 128, 32, 1, 1, 32 * 64 + 3, True, 4),
    ("fp32", 128, 16, 1, 1, 16 * 130, False, 8),
    ("fp32", 16, 16, 2, 1, 16 * 50, True, 3),
    ("fp32", 64, 32, 1, 1, 32 * 48 + 31, False, 3),
    ("bf16", 64, 64, 1, 3, 64 * 33, True, 2),
    ("bf16", 32, 32, 1, 2, 32 * 70 + 1, False, 4),
    ("bf16", 16, 16, 1, 2, 16 * 300, True, 18),
]


def args_of(inp, chunk):
    """The call's arguments (host-side plan only: nothing is launched)."""
    c = cuda(inp)
    B, T, H, D = c["q"].shape
    o = torch.empty_like(c["q"])
    S_T = torch.empty(B, H, D, D, device="cuda")
    return kda.prefill_args(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                            c["conv_state"], c["S0"], o, S_T, chunk=chunk)


@pytest.mark.parametrize("io,D,chunk,B,H,T,strong,nseg", CASES)
def test_split_walk_matches_oracle(io, D, chunk, B, H, T, strong, nseg):
    w = small(B=B, T=T, H=H, D=D, io=io, chunk=chunk, strong=strong, s0=True, conv_state=True)
    inp = make(w, seed=D + chunk + T)
    assert kda.kda_prefill_walk_segments(args_of(inp, chunk)) == nseg
    o, S, tail = gpu_prefill(inp, chunk)
    ro, rS, rtail = oracle_prefill(inp)
    tol = TOL[io]
    eo, eS = rel_l2(o, ro), rel_l2(S, rS)
    # the worst 64-token block, so an error confined to one segment cannot hide
    blk = max(rel_l2(o[:, t:t + 64], ro[:, t:t + 64]) for t in range(0, T, 64))
    print(f"{io} D={D} C={chunk} B={B} H={H} T={T} nseg={nseg}: o {eo:.2e} S_T {eS:.2e} "
          f"worst block {blk:.2e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    assert eo <= tol and eS <= tol and blk <= 2.5 * tol, (eo, eS, blk)
    np.testing.assert_array_equal(tail, rtail)


def test_split_walk_in_place_state_and_repeats():
    """S_T may be S0: the segment walks read their starts from the workspace, so
    the in-place call gives the out-of-place result bit for bit; repeated calls
    are bit-identical."""
    w = small(B=1, T=64 * 70 + 9, H=2, D=128, io="bf16", chunk=64, strong=True, s0=True,
              conv_state=True)
    inp = make(w, seed=11)
    assert kda.kda_prefill_walk_segments(args_of(inp, 64)) > 1
    o_ref, S_ref, tail_ref = gpu_prefill(inp, 64)
    for _ in range(3):
        o2, S2, _ = gpu_prefill(inp, 64)
        np.testing.assert_array_equal(o2, o_ref)
        np.testing.assert_array_equal(S2, S_ref)
    c = cuda(inp)
    S = c["S0"].clone()
    cs = c["conv_state"].clone()
    o, _, _ = kda.kda_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"], cs, S,
                              chunk=64, S_T=S, conv_state_out=cs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(S.cpu().numpy(), S_ref)
    np.testing.assert_array_equal(cs.float().cpu().numpy(), tail_ref)
    np.testing.assert_array_equal(o.float().cpu().numpy(), o_ref)


def test_split_walk_without_initial_state():
    w = small(B=2, T=32 * 80 + 5, H=1, D=64, io="bf16", chunk=32, s0=False, conv_state=False)
    inp = make(w, seed=12)
    inp["S0"] = None
    assert kda.kda_prefill_walk_segments(args_of(inp, 32)) > 1
    o, S, _ = gpu_prefill(inp, 32)
    ro, rS, _ = oracle_prefill(inp)
    assert rel_l2(o, ro) <= TOL["bf16"] and rel_l2(S, rS) <= TOL["bf16"]


@pytest.mark.parametrize("io,D,chunk,T", [("fp32", 64, 32, 32 * 96 + 7), ("bf16", 128, 64, 64 * 80),
                                          ("fp32", 128, 16, 16 * 200 + 3)])
def test_split_walk_long_memory(io, D, chunk, T):
    """Slow decay and small write strengths, so the state carries across every
    segment boundary and each segment's start depends on the composed maps M:
    with the initial state removed, the outputs of the last segment change by
    far more than the tolerance, and with it they match the oracle."""
    w = small(B=1, T=T, H=1, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    inp = long_memory(make(w, seed=T))
    nseg = kda.kda_prefill_walk_segments(args_of(inp, chunk))
    assert nseg >= 3
    o, S, _ = gpu_prefill(inp, chunk)
    ro, rS, _ = oracle_prefill(inp)
    ro0, _, _ = oracle_prefill(dict(inp, S0=torch.zeros_like(inp["S0"])))
    last = slice(T - T // nseg, T)
    reach = rel_l2(ro0[:, last], ro[:, last])
    tol = TOL[io]
    eo, eS = rel_l2(o, ro), rel_l2(S, rS)
    el = rel_l2(o[:, last], ro[:, last])
    print(f"{io} D={D} C={chunk} T={T} nseg={nseg}: o {eo:.2e} last segment {el:.2e} S_T {eS:.2e}; "
          f"initial state's share of the last segment's output {reach:.2e}", flush=True)
    assert reach > 20 * tol
    assert eo <= tol and eS <= tol and el <= tol, (eo, eS, el)


def long_memory(inp):
    """Slow decay, small write strengths, a large initial state: the state and
    its gradient carry across every segment boundary."""
    dt = inp["g"].dtype
    return dict(inp, g=(inp["g"].float() * 1e-3).to(dt), beta=(inp["beta"].float() * 0.05).to(dt),
                S0=inp["S0"] * 20.0)


@pytest.mark.parametrize("io,D,chunk,B,H,T,slow", [
    ("bf16", 128, 64, 1, 1, 64 * 70 + 5, False),
    ("bf16", 128, 64, 1, 1, 64 * 70 + 5, True),
    ("fp32", 64, 32, 1, 1, 32 * 96 + 7, True),
    ("fp32", 128, 16, 1, 1, 16 * 130, True),
    ("bf16", 32, 32, 2, 1, 32 * 70 + 1, False),
])
def test_split_backward_matches_oracle(io, D, chunk, B, H, T, slow):
    """kda_prefill_backward splits its forward and reverse walks as the forward
    does; every gradient against the oracle's reverse-mode gradients."""
    from test_gpu_backward import check_backward_inputs
    w = small(B=B, T=T, H=H, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    inp = make(w, seed=T + D)
    if slow:
        inp = long_memory(inp)
    assert kda.kda_prefill_walk_segments(args_of(inp, chunk)) >= 2
    check_backward_inputs(w, chunk, inp, seed=T)


def test_split_walk_stages_static_entry_and_optional_stages():
    """With every optional stage on (decay and beta from raw projections, the
    output norm and gate), a split call's stages (0, 1, 2, 3 and 0, 4, 3) and the
    entry point without a workspace argument (whose scratch holds this call's whole
    workspace, so it splits the same way) give kda_prefill's results bit for bit,
    and kda_prefill matches the oracle."""
    from kda_inputs import make_stage_inputs, to_numpy
    from oracle import kda_reference
    w = small(B=1, T=64 * 70 + 9, H=2, D=128, io="bf16", chunk=64, s0=True, conv_state=True)
    inp = cuda(make(w, seed=21))
    st = make_stage_inputs(w, seed=21, device="cuda")
    kw = dict(A_log=st["A_log"], dt_bias=st["dt_bias"], beta_logits=True,
              o_norm_w=st["o_norm_w"], o_gate=st["o_gate"])

    def call(run):
        o = torch.empty_like(inp["q"])
        S_T = torch.empty(w.B, w.H, w.D, w.D, device="cuda")
        cso = torch.empty(w.B, 3, 3, w.H * w.D, dtype=inp["q"].dtype, device="cuda")
        a = kda.prefill_args(inp["q"], inp["k"], inp["v"], st["f"], st["b_logit"], inp["conv_w"],
                             inp["conv_state"], inp["S0"], o, S_T, cso, chunk=64, **kw)
        assert kda.kda_prefill_walk_segments(a) == 4
        run(a)
        torch.cuda.synchronize()
        return o, S_T, cso

    def with_ws(stages):
        def run(a):
            ws = torch.empty(kda.kda_prefill_workspace_bytes(a), dtype=torch.uint8, device="cuda")
            if stages is None:
                kda.kda_prefill_raw(a, ws)
            else:
                for s in stages:
                    kda.kda_prefill_stage(a, ws, s)
        return run

    ref = call(with_ws(None))
    for got in (call(with_ws((0, 1, 2, 3))), call(with_ws((0, kda.KDA_STAGE_STATE_TAIL, 3))),
                call(lambda a: kda.kda_prefill_static_raw(a))):
        for x, y in zip(ref, got):
            assert torch.equal(x, y)
    n = {k: to_numpy(v) for k, v in inp.items()}
    ns = {k: to_numpy(v) for k, v in st.items()}
    ro, rS, _ = kda_reference(n["q"], n["k"], n["v"], ns["f"], ns["b_logit"], conv_w=n["conv_w"],
                              conv_state=n["conv_state"], S0=n["S0"], A_log=ns["A_log"],
                              dt_bias=ns["dt_bias"], beta_sigmoid=True, o_norm_w=ns["o_norm_w"],
                              o_gate=ns["o_gate"])
    o = ref[0].float().cpu().numpy()
    assert rel_l2(o, ro) <= TOL["bf16"] and rel_l2(ref[1].cpu().numpy(), rS) <= TOL["bf16"]
