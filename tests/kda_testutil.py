"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI and
the fp64 oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import numpy as np
import torch

import gated_delta_rule_80_amd as kda
from kda_inputs import Workload, make_inputs, to_numpy
from oracle import kda_reference

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)


def small(B=1, T=64, H=2, D=16, io="fp32", chunk=16, strong=False, s0=False, conv_state=False):
    return Workload(f"case-B{B}-T{T}-H{H}-D{D}-{io}", B=B, T=T, H=H, D=D, io=io, chunk=chunk,
                    a_lo=-3.0 if strong else -1.0, a_hi=2.0 if strong else 1.0,
                    b_std=1.4142 if strong else 1.0, s0_std=0.1 if s0 else 0.0,
                    conv_state_std=1.0 if conv_state else 0.0)


def cuda(inp: dict) -> dict:
    return {k: (v.cuda() if v is not None else None) for k, v in inp.items()}


def gpu_prefill(inp: dict, chunk: int, **kw):
    c = cuda(inp)
    o, S, tail = kda.kda_prefill(c["q"], c["k"], c["v"], c["g"], c["beta"], c["conv_w"],
                                 c["conv_state"], c["S0"], chunk=chunk, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), (None if tail is None else tail.float().cpu().numpy())


def oracle_prefill(inp: dict, **kw):
    n = {k: to_numpy(v) for k, v in inp.items()}
    return kda_reference(n["q"], n["k"], n["v"], n["g"], n["beta"], conv_w=n["conv_w"],
                         conv_state=n["conv_state"], S0=n["S0"], **kw)


def oracle_heads(inp: dict, heads):
    """Oracle on a few (b, h) slices; each slice is cut on the tensors' own device
    before the copy to the host, so full-size inputs stay on the GPU."""
    out = []
    for b, h in heads:
        D = inp["q"].shape[-1]
        ch = slice(h * D, (h + 1) * D)
        one = lambda x: None if x is None else to_numpy(x[b:b + 1, :, h:h + 1])
        q, k, v, g = (one(inp[n]) for n in ("q", "k", "v", "g"))
        beta = to_numpy(inp["beta"][b:b + 1, :, h:h + 1])
        cw = None if inp["conv_w"] is None else to_numpy(inp["conv_w"][:, ch])
        cs = None if inp["conv_state"] is None else to_numpy(inp["conv_state"][b:b + 1, :, :, ch])
        s0 = None if inp["S0"] is None else to_numpy(inp["S0"][b:b + 1, h:h + 1])
        o, S, _ = kda_reference(q, k, v, g, beta, conv_w=cw, conv_state=cs, S0=s0)
        out.append((o[0, :, 0], S[0, 0]))
    return out


def make(w: Workload, seed=0):
    return make_inputs(w, seed=seed, device="cpu")

