"""Packed variable-length sequences (cu_seqlens) on the GPU against the fp64
oracle's packed form: each sequence has its own conv history and initial state,
nothing crosses a boundary.  Lengths mix empty sequences, sequences shorter than
the conv window, exact chunk multiples and ragged tails.

Tolerance as for the plain mixer (relative L2 2e-2 bf16, 1e-4 fp32; o over the
tokens of the sequences, S_T over all sequences); conv hand-over exact."""
import numpy as np
import pytest
import torch

import gated_delta_rule_80_amd as kda
from kda_inputs import make_packed_inputs, make_stage_inputs, to_numpy
from kda_testutil import TOL, rel_l2, small
from oracle import kda_reference_packed

pytestmark = pytest.mark.gpu

MIXED = [0, 1, 2, 3, 5, 64, 65, 130, 0, 17, 40]


def run_gpu(inp, chunk, cu=None, **kw):
    c = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    cu = c["cu_seqlens"] if cu is None else cu.cuda()
    o, S, tail = kda.kda_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                 c["conv_state"], c["S0"], chunk=chunk, cu_seqlens=cu, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), None if tail is None else tail.float().cpu().numpy()


def run_oracle(inp, cu=None, **kw):
    n = {k: to_numpy(v) for k, v in inp.items() if k != "cu_seqlens"}
    cu = inp["cu_seqlens"].tolist() if cu is None else cu
    return kda_reference_packed(n["q"], n["k"], n["v"], n["g"], n["beta"], cu, conv_w=n["conv_w"],
                                conv_state=n["conv_state"], S0=n["S0"], **kw)


def compare(w, o, S, tail, ro, rS, rtail, what):
    tol = TOL[w.io]
    eo, eS = rel_l2(o, ro), rel_l2(S, rS)
    print(f"{what}: rel_l2 o={eo:.2e} S_T={eS:.2e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    assert eo <= tol, eo
    assert eS <= tol, eS
    if rtail is not None:
        np.testing.assert_array_equal(tail, rtail)


@pytest.mark.parametrize("io,D,chunk", [("bf16", 128, 64), ("fp32", 16, 16), ("fp32", 64, 32),
                                        ("bf16", 32, 32), ("bf16", 64, 16)])
def test_packed_mixed_lengths(io, D, chunk):
    w = small(H=2, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    inp = make_packed_inputs(w, MIXED, seed=D + chunk)
    compare(w, *run_gpu(inp, chunk), *run_oracle(inp), f"packed {io} D={D} C={chunk}")


def test_packed_without_history_or_state():
    w = small(H=3, D=128, io="bf16", chunk=64)
    inp = make_packed_inputs(w, [100, 7, 64, 1], seed=2)
    compare(w, *run_gpu(inp, 64), *run_oracle(inp), "packed, zero history and state")


def test_packed_strong_decay_exact_path():
    w = small(H=2, D=128, io="bf16", chunk=64, strong=True, s0=True, conv_state=True)
    inp = make_packed_inputs(w, [150, 3, 90, 0, 200], seed=4)
    compare(w, *run_gpu(inp, 64), *run_oracle(inp), "packed, strong decay")


@pytest.mark.parametrize("D", [64, 128])
def test_packed_with_every_stage(D):
    w = small(H=2, D=D, io="bf16", chunk=64, s0=True, conv_state=True)
    inp = make_packed_inputs(w, MIXED, seed=6)
    st = make_stage_inputs(small(B=1, T=sum(MIXED), H=2, D=D, io="bf16", chunk=64), seed=6)
    inp = dict(inp, g=st["f"], beta=st["b_logit"])
    gk = dict(A_log=st["A_log"].cuda(), dt_bias=st["dt_bias"].cuda(), beta_logits=True,
              o_norm_w=st["o_norm_w"].cuda(), o_gate=st["o_gate"].cuda())
    rk = dict(A_log=to_numpy(st["A_log"]), dt_bias=to_numpy(st["dt_bias"]), beta_sigmoid=True,
              o_norm_w=to_numpy(st["o_norm_w"]), o_gate=to_numpy(st["o_gate"]))
    compare(w, *run_gpu(inp, 64, **gk), *run_oracle(inp, **rk), f"packed, every stage, D={D}")


def test_packed_equal_lengths_match_batch_bitwise():
    """Packed sequences of equal length give exactly the batched call's results."""
    B, L, H, D = 3, 100, 2, 128
    w = small(H=H, D=D, io="bf16", chunk=64, s0=True, conv_state=True)
    inp = make_packed_inputs(w, [L] * B, seed=8)
    o, S, tail = run_gpu(inp, 64)
    c = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    shape = lambda x: x.reshape(B, L, *x.shape[2:])
    ob, Sb, tb = kda.kda_prefill(shape(c["q"]), shape(c["k"]), shape(c["v"]), shape(c["g"]),
                                 shape(c["beta"]), c["conv_w"], c["conv_state"], c["S0"], chunk=64)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o.reshape(B, L, H, D), ob.float().cpu().numpy())
    np.testing.assert_array_equal(S, Sb.cpu().numpy())
    np.testing.assert_array_equal(tail, tb.float().cpu().numpy())


def test_packed_many_sequences():
    """More sequences than one pass of the index kernel (1024 per block)."""
    rng = np.random.default_rng(3)
    lengths = rng.integers(0, 12, size=1500).tolist()
    w = small(H=2, D=16, io="fp32", chunk=16, s0=True, conv_state=True)
    inp = make_packed_inputs(w, lengths, seed=9)
    compare(w, *run_gpu(inp, 16), *run_oracle(inp), "packed, 1500 sequences")


def test_packed_empty_batch_and_all_empty():
    w = small(H=2, D=64, io="fp32", chunk=32, s0=True, conv_state=True)
    inp = make_packed_inputs(w, [0, 0, 0], seed=10)
    o, S, tail = run_gpu(inp, 32)
    np.testing.assert_array_equal(S, inp["S0"].numpy())
    np.testing.assert_array_equal(tail, inp["conv_state"].float().numpy())


def test_packed_malformed_offsets_are_clamped():
    """Offsets that decrease or leave [0, T] are read as their running maximum
    within [0, T]: the call stays inside the buffers and equals the oracle on the
    clamped offsets for the tokens that belong to a sequence."""
    w = small(H=2, D=64, io="bf16", chunk=32, s0=True, conv_state=True)
    T = 150
    inp = make_packed_inputs(w, [T], seed=11)
    N = 5
    S0 = torch.randn(N, 2, 64, 64, generator=torch.Generator().manual_seed(1)) * 0.1
    cs = (torch.randn(N, 3, 3, 128, generator=torch.Generator().manual_seed(2))).to(torch.bfloat16)
    inp = dict(inp, S0=S0, conv_state=cs)
    bad = [-5, 40, 30, 90, 400, 120]
    clamped, m = [], 0
    for x in bad:
        m = max(m, min(max(x, 0), T))
        clamped.append(m)
    o, S, tail = run_gpu(inp, 32, cu=torch.tensor(bad, dtype=torch.int32))
    # the oracle needs offsets from 0 to T: pad with the uncovered tail as one more sequence
    ref_cu = clamped if clamped[-1] == T else clamped + [T]
    extra = len(ref_cu) - 1 - N
    n = {k: to_numpy(v) for k, v in inp.items() if k != "cu_seqlens"}
    S0r = np.concatenate([n["S0"], np.zeros((extra, 2, 64, 64))]) if extra else n["S0"]
    csr = np.concatenate([n["conv_state"], np.zeros((extra, 3, 3, 128))]) if extra else n["conv_state"]
    ro, rS, rt = kda_reference_packed(n["q"], n["k"], n["v"], n["g"], n["beta"], ref_cu,
                                      conv_w=n["conv_w"], conv_state=csr, S0=S0r)
    covered = slice(clamped[0], clamped[-1])
    compare(w, o[:, covered], S, tail, ro[:, covered], rS[:N], rt[:N], "packed, clamped offsets")


def test_packed_stages_compose():
    w = small(H=3, D=128, io="bf16", chunk=64, s0=True, conv_state=True)
    inp = make_packed_inputs(w, MIXED, seed=12)
    c = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    o1, S1, t1 = kda.kda_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                 c["conv_state"], c["S0"], chunk=64, cu_seqlens=c["cu_seqlens"])
    o2, S2, t2 = torch.empty_like(o1), torch.empty_like(S1), torch.empty_like(t1)
    a = kda.prefill_args(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"], c["conv_state"],
                         c["S0"], o2, S2, t2, chunk=64, cu_seqlens=c["cu_seqlens"])
    ws = torch.empty(kda.kda_prefill_workspace_bytes(a), dtype=torch.uint8, device="cuda")
    for stage in (0, 1, 2, 3):
        kda.kda_prefill_stage(a, ws, stage)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"].tolist()
    for i in range(len(cu) - 1):  # o only inside the sequences (here: all tokens)
        assert torch.equal(o1[:, cu[i]:cu[i + 1]], o2[:, cu[i]:cu[i + 1]])
    assert torch.equal(S1, S2) and torch.equal(t1, t2)
