"""Gradients of the prefill on the GPU against the fp64 oracle's reverse-mode
gradients (kda_reference_backward, itself pinned by finite differences).

Loss L = <o, do> + <S_T, dS_T> with random do, dS_T.  Tolerance: relative L2 per
gradient tensor, 2e-2 for bf16 inputs and 1e-4 for fp32 inputs (the same bar as
the forward), over dq, dk, dv, dg, dbeta, dS0, dconv_w and dconv_state."""
import numpy as np
import pytest
import torch

import gated_delta_rule_80_amd as kda
from kda_inputs import make_packed_inputs, make_stage_inputs, to_numpy
from kda_testutil import TOL, cuda, make, rel_l2, small
from oracle import (kda_reference, kda_reference_backward, kda_reference_backward_packed,
                    output_gate_norm_backward)

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0", "dconv_w", "dconv_state")


def check_backward(w, chunk, seed=0, conv=True, l2=True, scale=1.0, with_dST=True, g_head=None,
                   do_scale=1.0):
    check_backward_inputs(w, chunk, make(w, seed), seed, conv, l2, scale, with_dST, g_head, do_scale)


def check_backward_inputs(w, chunk, inp, seed=0, conv=True, l2=True, scale=1.0, with_dST=True,
                          g_head=None, do_scale=1.0):
    if g_head is not None:
        # constant log-decay per token on the given heads: {head: g}
        g = inp["g"].clone()
        for hh, val in g_head.items():
            g[:, :, hh, :] = val
        inp = dict(inp, g=g)
    if not conv:
        inp = dict(inp, conv_w=None, conv_state=None)
    gen = torch.Generator().manual_seed(seed + 1000)
    do = (torch.randn(w.B, w.T, w.H, w.D, generator=gen) * do_scale).to(inp["q"].dtype)
    dST = torch.randn(w.B, w.H, w.D, w.D, generator=gen) * do_scale if with_dST else None
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
                                        ("bf16", 32, 64), ("bf16", 64, 64), ("bf16", 16, 16),
                                        ("fp32", 128, 32), ("fp32", 128, 16)])
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
@pytest.mark.parametrize("g0", [-12.0, -8.0, -5.2])
def test_backward_factored_and_exact_pair_paths(io, D, chunk, g0):
    """Head 0 decays by a constant g0 per token: -12 gives 16-token block spans of
    about 277 log2 units, beyond the factored pair products' span limit of 240 (the
    chunks go to the exact per-pair kernel); -8 gives about 185 and -5.2 about 120,
    both factored with gradients of ordinary size (factors up to 2^92 and 2^60).
    Head 1 keeps its drawn decays."""
    w = small(B=1, T=150, H=2, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    check_backward(w, chunk, seed=17, g_head={0: g0})


@pytest.mark.parametrize("io,D,chunk", [("bf16", 128, 64), ("fp32", 64, 32)])
def test_backward_pair_path_follows_the_gradient_scale(io, D, chunk):
    """Spans of about 185 log2 units with dO and dS_T scaled by 2^40: the chunk's
    bound on the factored partial sums passes 2^120, so its pair terms go to the
    exact kernel (with unit gradients the same chunks are factored); the
    gradients, 2^40 times larger, still match the oracle."""
    w = small(B=1, T=150, H=2, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    check_backward(w, chunk, seed=17, g_head={0: -8.0}, do_scale=2.0 ** 40)


@pytest.mark.parametrize("io,D,chunk", [("fp32", 64, 32), ("bf16", 128, 64)])
def test_backward_wide_spans_with_free_block_boundaries(io, D, chunk):
    """Head 0 decays by 5.88 nats per token inside every 16-token block but not at
    the first token of a block: each block spans 127.3 log2 units (inside the
    factored pair products' limit), so the pair factor of two adjacent blocks,
    exp(-(s_p + s_q)/2), is a float32 denormal while the products it scales are
    O(1)."""
    w = small(B=1, T=150, H=2, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    inp = make(w, 19)
    g = inp["g"].float()
    t = torch.arange(w.T)
    g[0, :, 0, :] = torch.where(t % 16 == 0, 0.0, -5.88)[:, None]
    inp["g"] = g.to(inp["g"].dtype)
    w2 = w
    check_backward_inputs(w2, chunk, inp, seed=19)


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


@pytest.mark.parametrize("io,D,chunk", [("bf16", 128, 64), ("fp32", 32, 16)])
def test_backward_in_place_states(io, D, chunk):
    """The forward rules allow S_T == S0 and conv_state_out == conv_state_in; the
    backward recomputes the forward, so the hand-over must not overwrite the conv
    history before the gradients have read it.  Called through the C ABI with both
    states in place, the gradients equal those of a call with separate outputs
    (bit for bit), and the recomputed S_T and conv hand-over land in place."""
    w = small(B=2, T=70, H=2, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    inp = cuda(make(w, 21))
    do = torch.randn(w.B, w.T, w.H, w.D, generator=torch.Generator().manual_seed(4)).to(
        inp["q"].dtype).cuda()
    ref, o_ref, S_ref = kda.kda_prefill_backward(inp["q"], inp["k"], inp["v"], inp["g"],
                                                 inp["beta"], inp["conv_w"], inp["conv_state"],
                                                 inp["S0"], do=do, chunk=chunk)
    torch.cuda.synchronize()
    _, _, tail_ref = kda.kda_prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     inp["conv_w"], inp["conv_state"], inp["S0"], chunk=chunk)
    torch.cuda.synchronize()
    S = inp["S0"].clone()
    cs = inp["conv_state"].clone()
    o = torch.empty_like(inp["q"])
    fwd = kda.prefill_args(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["conv_w"],
                           cs, S, o, S, cs, chunk=chunk)
    f32 = dict(dtype=torch.float32, device="cuda")
    shape = (w.B, w.T, w.H, w.D)
    grads = dict(dq=torch.empty(*shape, **f32), dk=torch.empty(*shape, **f32),
                 dv=torch.empty(*shape, **f32), dg=torch.empty(*shape, **f32),
                 dbeta=torch.empty(w.B, w.T, w.H, **f32), dS0=torch.empty(w.B, w.H, w.D, w.D, **f32),
                 dconv_w=torch.empty(3, w.H * w.D, 4, **f32),
                 dconv_state=torch.empty(w.B, 3, 3, w.H * w.D, **f32))
    a = kda.backward_args(fwd, do, None, grads)
    assert kda.kda_validate_backward(a) == kda.KDA_OK
    ws = torch.empty(kda.kda_backward_workspace_bytes(a), dtype=torch.uint8, device="cuda")
    kda.kda_prefill_backward_raw(a, ws)
    torch.cuda.synchronize()
    for name, t in ref.items():
        assert torch.equal(grads[name], t), name
    assert torch.equal(o, o_ref)
    assert torch.equal(S, S_ref)
    assert torch.equal(cs, tail_ref)


# ----------------------------------------------------------- optional stages
STAGES = {
    "norm": dict(norm=True),
    "gate": dict(gate=True),
    "norm+gate": dict(norm=True, gate=True),
    "act": dict(act=True),
    "logits": dict(logits=True),
    "all": dict(norm=True, gate=True, act=True, logits=True),
}
STAGE_GRADS = NAMES + ("dA_log", "ddt_bias", "do_norm_w", "do_gate")


def check_backward_stages(w, chunk, seed, norm=False, gate=False, act=False, logits=False):
    """The backward with optional stages against the oracle's; the recomputed o
    against kda_prefill's with the same stages (bit for bit where both finish o
    with the same separate pass, D = 128; otherwise to the tolerance, since the
    fused walk of D <= 64 keeps the mixer's output in fp32 into the stage)."""
    inp = make(w, seed)
    st = make_stage_inputs(w, seed)
    kw = {}
    if norm:
        kw["o_norm_w"] = st["o_norm_w"]
    if gate:
        kw["o_gate"] = st["o_gate"]
    if act:
        inp = dict(inp, g=st["f"])
        kw["A_log"], kw["dt_bias"] = st["A_log"], st["dt_bias"]
    if logits:
        inp = dict(inp, beta=st["b_logit"])
        kw["beta_logits"] = True
    gen = torch.Generator().manual_seed(seed + 1000)
    do = torch.randn(w.B, w.T, w.H, w.D, generator=gen).to(inp["q"].dtype)
    dST = torch.randn(w.B, w.H, w.D, w.D, generator=gen)
    c = cuda(inp)
    ck = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in kw.items()}
    grads, o, S_T = kda.kda_prefill_backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                             c["conv_state"], c["S0"], do=do.cuda(), dS_T=dST.cuda(),
                                             chunk=chunk, **ck)
    torch.cuda.synchronize()
    o_f, S_f, _ = kda.kda_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                  c["conv_state"], c["S0"], chunk=chunk, **ck)
    torch.cuda.synchronize()
    assert torch.equal(S_T, S_f)
    if w.D == 128 or not (norm or gate):
        assert torch.equal(o, o_f)
    else:
        assert rel_l2(o.float().cpu().numpy(), o_f.float().cpu().numpy()) <= TOL[w.io]
    n = {k: to_numpy(v) for k, v in inp.items()}
    nk = {k: (to_numpy(v) if torch.is_tensor(v) else v) for k, v in kw.items()}
    if "beta_logits" in nk:
        nk["beta_sigmoid"] = nk.pop("beta_logits")
    ref = kda_reference_backward(n["q"], n["k"], n["v"], n["g"], n["beta"], to_numpy(do),
                                 to_numpy(dST), conv_w=n["conv_w"], conv_state=n["conv_state"],
                                 S0=n["S0"], **nk)
    tol = {name: TOL[w.io] for name in STAGE_GRADS}
    if norm and w.io == "bf16":
        # The output norm's backward divides by each row's rms: a row whose mixer
        # output is much smaller than the others passes the forward's own error
        # into the gradients magnified by that ratio.  The bf16 forward's error in
        # the mixer output does not shrink with a row's magnitude (it comes from
        # the rounding of the terms that sum to it), so it is modelled as seeded
        # normal noise of 4e-3 times the output's rms over the call (the forward's
        # measured relative error).  The bar adds twice the change that noise
        # makes in the exact computation's gradients to the plain bar.
        akw = {k: v for k, v in nk.items() if k in ("A_log", "dt_bias", "beta_sigmoid")}
        base = dict(conv_w=n["conv_w"], conv_state=n["conv_state"], S0=n["S0"], **akw)
        o_pre = kda_reference(n["q"], n["k"], n["v"], n["g"], n["beta"], **base)[0]
        noise = np.random.default_rng(seed + 7).standard_normal(o_pre.shape)
        d_pert = output_gate_norm_backward(o_pre + 4e-3 * np.sqrt(np.mean(o_pre ** 2)) * noise,
                                           to_numpy(do), nk.get("o_norm_w"), nk.get("o_gate"))[0]
        pert = kda_reference_backward(n["q"], n["k"], n["v"], n["g"], n["beta"], d_pert,
                                      to_numpy(dST), **base)
        for name in NAMES:
            if ref.get(name) is not None:
                tol[name] += 2.0 * rel_l2(pert[name], ref[name])
    errs = {}
    for name in STAGE_GRADS:
        if ref.get(name) is None:
            assert name not in grads or name in NAMES, name
            continue
        got = grads[name].cpu().numpy()
        assert np.isfinite(got).all(), name
        errs[name] = rel_l2(got, ref[name])
    print(f"{w.name} D={w.D} C={chunk} stages={norm, gate, act, logits}: " +
          " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    for name, e in errs.items():
        assert e <= tol[name], (name, e, tol[name])


@pytest.mark.parametrize("stages", list(STAGES))
@pytest.mark.parametrize("io,D,chunk", [("bf16", 128, 64), ("fp32", 32, 16), ("bf16", 64, 32)])
def test_backward_optional_stages(stages, io, D, chunk):
    w = small(B=2, T=90, H=3, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    check_backward_stages(w, chunk, seed=31 + D, **STAGES[stages])


def test_backward_stages_repeated_calls_are_bit_identical():
    """The parameter gradients are sums over tokens in a fixed order."""
    w = small(B=2, T=300, H=4, D=128, io="bf16", chunk=64, s0=True, conv_state=True)
    inp = cuda(make(w, 12))
    st = {k: v.cuda() for k, v in make_stage_inputs(w, 12).items()}
    do = torch.randn(w.B, w.T, w.H, w.D, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).cuda()
    first = None
    for _ in range(4):
        grads, _, _ = kda.kda_prefill_backward(inp["q"], inp["k"], inp["v"], st["f"], st["b_logit"],
                                               inp["conv_w"], inp["conv_state"], inp["S0"], do=do,
                                               chunk=64, A_log=st["A_log"], dt_bias=st["dt_bias"],
                                               beta_logits=True, o_norm_w=st["o_norm_w"],
                                               o_gate=st["o_gate"])
        torch.cuda.synchronize()
        if first is None:
            first = {k: v.clone() for k, v in grads.items()}
        else:
            for k, v in grads.items():
                assert torch.equal(v, first[k]), k


# ---------------------------------------------------------- packed sequences
PACKED = [0, 1, 2, 3, 5, 64, 65, 130, 0, 17, 40]


def packed_backward(w, lengths, chunk, seed, stages=False):
    """GPU and oracle gradients of a packed batch (each sequence its own S0, conv
    history and dS_T; nothing crosses a boundary)."""
    inp = make_packed_inputs(w, lengths, seed=seed)
    T = sum(lengths)
    N = len(lengths)
    gk, rk = {}, {}
    if stages:
        st = make_stage_inputs(small(B=1, T=T, H=w.H, D=w.D, io=w.io, chunk=chunk), seed=seed)
        inp = dict(inp, g=st["f"], beta=st["b_logit"])
        gk = dict(A_log=st["A_log"].cuda(), dt_bias=st["dt_bias"].cuda(), beta_logits=True,
                  o_norm_w=st["o_norm_w"].cuda(), o_gate=st["o_gate"].cuda())
        rk = dict(A_log=to_numpy(st["A_log"]), dt_bias=to_numpy(st["dt_bias"]), beta_sigmoid=True,
                  o_norm_w=to_numpy(st["o_norm_w"]), o_gate=to_numpy(st["o_gate"]))
    gen = torch.Generator().manual_seed(seed + 1000)
    do = torch.randn(1, T, w.H, w.D, generator=gen).to(inp["q"].dtype)
    dST = torch.randn(N, w.H, w.D, w.D, generator=gen)
    c = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    grads, o, S_T = kda.kda_prefill_backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                             c["conv_state"], c["S0"], do=do.cuda(), dS_T=dST.cuda(),
                                             chunk=chunk, cu_seqlens=c["cu_seqlens"], **gk)
    torch.cuda.synchronize()
    n = {k: to_numpy(v) for k, v in inp.items() if k != "cu_seqlens"}
    ref = kda_reference_backward_packed(n["q"], n["k"], n["v"], n["g"], n["beta"],
                                        inp["cu_seqlens"].tolist(), to_numpy(do), to_numpy(dST),
                                        conv_w=n["conv_w"], conv_state=n["conv_state"], S0=n["S0"], **rk)
    return grads, ref, (inp, c, gk, do, dST)


@pytest.mark.parametrize("io,D,chunk", [("bf16", 128, 64), ("fp32", 32, 16), ("bf16", 64, 32),
                                        ("fp32", 16, 64)])
def test_backward_packed_mixed_lengths(io, D, chunk):
    """Empty sequences, sequences shorter than the conv window, exact chunk
    multiples and ragged tails, against the oracle's packed gradients."""
    w = small(H=2, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    grads, ref, extra = packed_backward(w, PACKED, chunk, seed=D + chunk)
    dST = extra[4]
    errs = {}
    for name in NAMES:
        got = grads[name].cpu().numpy()
        assert np.isfinite(got).all(), name
        errs[name] = rel_l2(got, ref[name])
    print(f"packed backward {io} D={D} C={chunk}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()),
          flush=True)
    for name, e in errs.items():
        assert e <= TOL[io], (name, e)
    # the empty sequences pass their end-state gradient straight through
    for i, L in enumerate(PACKED):
        if L == 0:
            assert torch.equal(grads["dS0"][i].cpu(), dST[i]), i
            assert float(grads["dconv_state"][i].abs().max()) == 0.0, i


def test_backward_packed_every_stage():
    w = small(H=2, D=128, io="bf16", chunk=64, s0=True, conv_state=True)
    grads, ref, _ = packed_backward(w, PACKED, 64, seed=9, stages=True)
    errs = {}
    for name in STAGE_GRADS:
        if ref.get(name) is None:
            continue
        got = grads[name].cpu().numpy()
        assert np.isfinite(got).all(), name
        errs[name] = rel_l2(got, ref[name])
    print("packed backward, every stage: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    # the output norm's backward passes the forward's error on magnified where a
    # row's output is small (see check_backward_stages); at D = 128 with these
    # inputs that stays inside the plain bar
    for name, e in errs.items():
        assert e <= TOL["bf16"], (name, e)


@pytest.mark.parametrize("io,D,chunk", [("bf16", 128, 64), ("fp32", 32, 16)])
def test_backward_packed_equal_lengths_match_batched(io, D, chunk):
    """B equal-length sequences packed into one row give the batched call's
    gradients bit for bit (the same chunks, blocks and summation orders)."""
    B, L = 3, 2 * chunk + 7
    w = small(B=B, T=L, H=2, D=D, io=io, chunk=chunk, s0=True, conv_state=True)
    inp = cuda(make(w, 14))
    gen = torch.Generator().manual_seed(15)
    do = torch.randn(B, L, w.H, w.D, generator=gen).to(inp["q"].dtype).cuda()
    dST = torch.randn(B, w.H, w.D, w.D, generator=gen).cuda()
    ref, o_ref, S_ref = kda.kda_prefill_backward(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                                 inp["conv_w"], inp["conv_state"], inp["S0"], do=do,
                                                 dS_T=dST, chunk=chunk)
    flat = lambda x: x.reshape(1, B * L, *x.shape[2:])
    cu = torch.arange(0, B * L + 1, L, dtype=torch.int32, device="cuda")
    got, o, S = kda.kda_prefill_backward(flat(inp["q"]), flat(inp["k"]), flat(inp["v"]), flat(inp["g"]),
                                         flat(inp["beta"]), inp["conv_w"], inp["conv_state"], inp["S0"],
                                         do=flat(do), dS_T=dST, chunk=chunk, cu_seqlens=cu)
    torch.cuda.synchronize()
    for name, t in ref.items():
        assert torch.equal(got[name].reshape(t.shape), t), name
    assert torch.equal(o.reshape(o_ref.shape), o_ref)
    assert torch.equal(S, S_ref)


def test_backward_packed_many_sequences():
    """1,100 short sequences (more than one pass of the index kernel's 1,024
    threads), many of them empty or shorter than the conv window."""
    rng = np.random.default_rng(16)
    lengths = [int(x) for x in rng.choice([0, 1, 2, 3, 4, 7, 16, 17, 33], size=1100)]
    w = small(H=1, D=64, io="bf16", chunk=16, s0=True, conv_state=True)
    grads, ref, extra = packed_backward(w, lengths, 16, seed=17)
    dST = extra[4]
    for name in NAMES:
        got = grads[name].cpu().numpy()
        assert np.isfinite(got).all(), name
        e = rel_l2(got, ref[name])
        assert e <= TOL["bf16"], (name, e)
    empty = [i for i, L in enumerate(lengths) if L == 0]
    assert torch.equal(grads["dS0"][empty].cpu(), dST[empty])
    assert float(grads["dconv_state"][empty].abs().max()) == 0.0
