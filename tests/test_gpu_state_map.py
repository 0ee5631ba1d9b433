"""The affine state map of a prefill call (kda_prefill_state_map) against the fp64
oracle, and its use for splitting one sequence over devices, emulated on one GPU.

The oracle gives the map from its own recurrence, which is linear in the state
once the values are taken away: N is the final state from a zero start, and M
the final state from the identity with every value zeroed (the raw v and its
conv history, so the convolved values are exactly zero).  Tolerances as for
every prefill: relative L2 2e-2 for bf16 inputs, 1e-4 for fp32, per tensor."""
import numpy as np
import pytest
import torch

import gated_delta_rule_80_amd as kda
from kda_inputs import to_numpy
from kda_testutil import TOL, cuda, make, rel_l2, small
from oracle import kda_reference

pytestmark = pytest.mark.gpu


def long_memory(inp):
    """Slow decay and small write strengths: M stays far from zero."""
    dt = inp["g"].dtype
    return dict(inp, g=(inp["g"].float() * 1e-3).to(dt), beta=(inp["beta"].float() * 0.05).to(dt))


def oracle_map(inp):
    n = {k: to_numpy(v) for k, v in inp.items()}
    B, T, H, D = n["q"].shape
    _, N, _ = kda_reference(n["q"], n["k"], n["v"], n["g"], n["beta"], conv_w=n["conv_w"],
                            conv_state=n["conv_state"], S0=None)
    cs0 = None
    if n["conv_state"] is not None:
        cs0 = n["conv_state"].copy()
        cs0[:, 2] = 0.0  # the v history
    eye = np.broadcast_to(np.eye(D), (B, H, D, D)).copy()
    _, M, _ = kda_reference(n["q"], n["k"], np.zeros_like(n["v"]), n["g"], n["beta"],
                            conv_w=n["conv_w"], conv_state=cs0, S0=eye)
    return M, N


def gpu_map(inp, chunk):
    c = cuda(inp)
    M, N = kda.kda_prefill_state_map(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                     c["conv_state"], chunk=chunk)
    torch.cuda.synchronize()
    return M.cpu().numpy(), N.cpu().numpy()


# (io, D, chunk, B, H, T): one segment and several, ragged last chunks
CASES = [
    ("fp32", 16, 16, 2, 2, 77),
    ("bf16", 128, 64, 1, 2, 200),
    ("bf16", 128, 64, 1, 1, 64 * 70 + 5),
    ("fp32", 128, 32, 1, 1, 32 * 64 + 3),
    ("fp32", 64, 32, 2, 1, 32 * 48 + 31),
    ("bf16", 32, 16, 1, 2, 16 * 100 + 7),
    ("fp32", 32, 32, 1, 2, 7),      # shorter than one chunk
    ("bf16", 64, 64, 2, 1, 64),     # exactly one chunk
]


@pytest.mark.parametrize("io,D,chunk,B,H,T", CASES)
def test_state_map_matches_oracle(io, D, chunk, B, H, T):
    w = small(B=B, T=T, H=H, D=D, io=io, chunk=chunk, conv_state=True)
    inp = long_memory(make(w, seed=T + D))
    M, N = gpu_map(inp, chunk)
    rM, rN = oracle_map(inp)
    eM, eN = rel_l2(M, rM), rel_l2(N, rN)
    print(f"{io} D={D} C={chunk} B={B} H={H} T={T}: M {eM:.2e} (|M| {np.linalg.norm(rM):.1f}) "
          f"N {eN:.2e}", flush=True)
    assert np.isfinite(M).all() and np.isfinite(N).all()
    assert eM <= TOL[io] and eN <= TOL[io], (eM, eN)


def test_state_map_with_raw_projections():
    """With the decay and beta computed from raw projections the map follows the
    activated values."""
    from kda_inputs import make_stage_inputs
    w = small(B=1, T=64 * 40 + 3, H=2, D=128, io="bf16", chunk=64, conv_state=True)
    inp = make(w, seed=31)
    st = make_stage_inputs(w, seed=31)
    # slow decay (A_log = -7) and small write strengths, so M stays far from zero
    st["A_log"] = torch.full_like(st["A_log"], -7.0)
    inp = dict(inp, g=st["f"], beta=(st["b_logit"].float() - 4.0).to(st["b_logit"].dtype))
    c = cuda(inp)
    M, N = kda.kda_prefill_state_map(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                     c["conv_state"], chunk=64, A_log=st["A_log"].cuda(),
                                     dt_bias=st["dt_bias"].cuda(), beta_logits=True)
    torch.cuda.synchronize()
    n = {k: to_numpy(v) for k, v in inp.items()}
    kw = dict(A_log=to_numpy(st["A_log"]), dt_bias=to_numpy(st["dt_bias"]), beta_sigmoid=True)
    _, rN, _ = kda_reference(n["q"], n["k"], n["v"], n["g"], n["beta"], conv_w=n["conv_w"],
                             conv_state=n["conv_state"], S0=None, **kw)
    cs0 = n["conv_state"].copy()
    cs0[:, 2] = 0.0
    eye = np.broadcast_to(np.eye(128), (1, 2, 128, 128)).copy()
    _, rM, _ = kda_reference(n["q"], n["k"], np.zeros_like(n["v"]), n["g"], n["beta"],
                             conv_w=n["conv_w"], conv_state=cs0, S0=eye, **kw)
    eM, eN = rel_l2(M.cpu().numpy(), rM), rel_l2(N.cpu().numpy(), rN)
    print(f"raw projections: M {eM:.2e} (|M| {np.linalg.norm(rM):.1f}) N {eN:.2e}", flush=True)
    assert np.linalg.norm(rM) > 1.0
    assert eM <= TOL["bf16"] and eN <= TOL["bf16"]


def test_state_map_of_no_tokens_is_the_identity():
    w = small(B=2, T=0, H=3, D=32, io="bf16", chunk=32, conv_state=True)
    M, N = gpu_map(make(w, seed=1), 32)
    assert np.array_equal(M, np.broadcast_to(np.eye(32), M.shape)) and not N.any()


@pytest.mark.parametrize("io,D,chunk,T1,T2,slow", [
    ("bf16", 128, 64, 1000, 64 * 40 + 11, False),
    ("bf16", 128, 64, 1000, 64 * 40 + 11, True),
    ("fp32", 64, 32, 333, 32 * 50, True),
])
def test_sequence_split_over_devices(io, D, chunk, T1, T2, slow):
    """One sequence cut into two shares, as two devices would hold it.  The
    second share computes its map (M, N) from its own tokens and the first
    share's conv hand-over alone; with the first share's final state S_1, S_T =
    M S_1 + N, and the second share's prefill from S_1 gives the rest of the
    outputs.  Both match the prefill of the whole sequence and the oracle."""
    w = small(B=1, T=T1 + T2, H=2, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    inp = make(w, seed=T2)
    if slow:
        inp = dict(long_memory(inp), S0=inp["S0"] * 20.0)
    c = cuda(inp)
    o, S_T, tail = kda.kda_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                   c["conv_state"], c["S0"], chunk=chunk)
    a, b = slice(0, T1), slice(T1, None)
    # each device holds its share in buffers of its own
    part = lambda d, s: {k: (v[:, s].clone() if k in ("q", "k", "v", "g", "beta") else v)
                         for k, v in d.items()}
    c1, c2 = part(c, a), part(c, b)
    o1, S1, tail1 = kda.kda_prefill(c1["q"], c1["k"], c1["v"], c1["g"], c1["beta"], c1["conv_w"],
                                    c1["conv_state"], c1["S0"], chunk=chunk)
    M, N = kda.kda_prefill_state_map(c2["q"], c2["k"], c2["v"], c2["g"], c2["beta"], c2["conv_w"],
                                     tail1, chunk=chunk)
    S_pred = torch.matmul(M, S1) + N
    o2, S2, _ = kda.kda_prefill(c2["q"], c2["k"], c2["v"], c2["g"], c2["beta"], c2["conv_w"],
                                tail1, S1, chunk=chunk)
    torch.cuda.synchronize()
    n = {k: to_numpy(v) for k, v in inp.items()}
    ro, rS, _ = kda_reference(n["q"], n["k"], n["v"], n["g"], n["beta"], conv_w=n["conv_w"],
                              conv_state=n["conv_state"], S0=n["S0"])
    tol = TOL[io]
    e_pred = rel_l2(S_pred.cpu().numpy(), rS)
    e_two = rel_l2(S2.cpu().numpy(), rS)
    e_o = rel_l2(torch.cat([o1, o2], 1).float().cpu().numpy(), ro)
    reach = np.linalg.norm(np.matmul(M.cpu().numpy(), S1.cpu().numpy())) / np.linalg.norm(rS)
    print(f"{io} D={D} T1={T1} T2={T2}: S_T from the map {e_pred:.2e}, from the second share's "
          f"prefill {e_two:.2e}, outputs {e_o:.2e}; first share's part of S_T {reach:.2e}",
          flush=True)
    assert e_pred <= tol and e_two <= tol and e_o <= tol
    assert rel_l2(S_pred.cpu().numpy(), S_T.cpu().numpy()) <= tol
    if slow:
        assert reach > 0.1  # the composition carries a real part of the state
