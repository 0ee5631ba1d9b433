"""Seeded synthetic inputs for the KDA mixer (shared by tests, smoke check and bench).

This module only draws random numbers and shapes them into the workloads' value
distributions; it contains none of the mixer's arithmetic (no convolution, norm or
recurrence).  Both the oracle side and the GPU side consume the same tensors.

Workloads (one KDA layer of the released model: 96 heads x head_dim 128, short
conv kernel 4 -- "Kimi-K3 model atlas -- self.layers", linear_attn_config):

* raw q, k, v ~ N(0, 1)
* log-decay g = -exp(a_h) * softplus(z), a_h ~ U(lo, hi) drawn once per head (like
  the per-head ``A_log``), z ~ N(0, 1) per element (one decay per channel, the
  full-rank gate)
* beta = sigmoid(b), b ~ N(0, sigma_b^2)
* conv filters ~ N(0, 0.25) (std 0.5), float32, layout [3 (q,k,v), H*D, 4]
* S0 ~ N(0, 0.01) (std 0.1) float32 where the workload has an initial state
* decode: conv history ~ N(0, 1) in the I/O dtype

The second parameter of every N(., .) is a variance.  bf16 tensors are rounded
from float32 with round-to-nearest-even (torch's conversion).

Optional stages (``make_stage_inputs``, drawn from a generator of their own so the
tensors above do not change):

* output gate pre-activation ~ N(0, 1) in the I/O dtype; output-norm gain
  1 + N(0, 0.01) float32, one per value channel
* raw decay projection f ~ N(0, 1) in the I/O dtype, A_log ~ U(lo, hi) per head
  and dt_bias ~ N(0, 0.25) per channel, both float32; beta logits
  ~ N(0, sigma_b^2) in the I/O dtype
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch
import torch.nn.functional as F


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    D: int
    io: str            # "bf16" | "fp32"
    chunk: int         # 0 for decode
    a_lo: float
    a_hi: float
    b_std: float
    s0_std: float      # 0 => no initial state (S0 = NULL)
    decode: bool = False
    conv_state_std: float = 0.0   # 0 => no conv history (zeros)

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny-fp32": Workload("tiny-fp32", B=1, T=64, H=2, D=16, io="fp32", chunk=16,
                          a_lo=-1.0, a_hi=1.0, b_std=1.0, s0_std=0.0),
    "prefill-4k": Workload("prefill-4k", B=1, T=4096, H=96, D=128, io="bf16", chunk=64,
                           a_lo=-1.0, a_hi=1.0, b_std=1.0, s0_std=0.0),
    "prefill-b4-8k-s0": Workload("prefill-b4-8k-s0", B=4, T=8192, H=96, D=128, io="bf16",
                                 chunk=64, a_lo=-3.0, a_hi=2.0, b_std=math.sqrt(2.0),
                                 s0_std=0.1),
    "decode-b256": Workload("decode-b256", B=256, T=1, H=96, D=128, io="bf16", chunk=0,
                            a_lo=-1.0, a_hi=1.0, b_std=1.0, s0_std=0.1, decode=True,
                            conv_state_std=1.0),
    "prefill-64k": Workload("prefill-64k", B=1, T=65536, H=96, D=128, io="bf16", chunk=64,
                            a_lo=-3.0, a_hi=2.0, b_std=math.sqrt(2.0), s0_std=0.1),
    # one GPU's share of the 64k layer under 8-way tensor parallelism over heads
    "prefill-64k-h12": Workload("prefill-64k-h12", B=1, T=65536, H=12, D=128, io="bf16",
                                chunk=64, a_lo=-3.0, a_hi=2.0, b_std=math.sqrt(2.0), s0_std=0.1),
}
# The same five workloads by position (0: tiny parity case ... 4: long context).
ORDER = ["tiny-fp32", "prefill-4k", "prefill-b4-8k-s0", "decode-b256", "prefill-64k"]

DTYPES = {"bf16": torch.bfloat16, "fp32": torch.float32}


def make_inputs(w: Workload, seed: int = 0, device: str | torch.device = "cpu") -> dict:
    """Draw one set of inputs for workload ``w`` on ``device``.

    Returns a dict of tensors: q, k, v, g [B,T,H,D] (decode: [B,H,D]) in the I/O
    dtype; beta [B,T,H] (decode [B,H]); conv_w [3,H*D,4] fp32; S0 [B,H,D,D] fp32 or
    None; conv_state [B,3,3,H*D] in the I/O dtype or None.
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    io = DTYPES[w.io]
    B, T, H, D = w.B, w.T, w.H, w.D
    shape = (B, H, D) if w.decode else (B, T, H, D)
    bshape = (B, H) if w.decode else (B, T, H)

    def randn(*s, std=1.0):
        x = torch.randn(*s, generator=gen, device=device, dtype=torch.float32)
        return x.mul_(std) if std != 1.0 else x

    q = randn(*shape).to(io)
    k = randn(*shape).to(io)
    v = randn(*shape).to(io)
    a = torch.empty(H, device=device, dtype=torch.float32).uniform_(w.a_lo, w.a_hi, generator=gen)
    z = randn(*shape)
    g = F.softplus(z).mul_(-torch.exp(a).view(*([1] * (len(shape) - 2)), H, 1)).to(io)
    del z
    beta = torch.sigmoid(randn(*bshape, std=w.b_std)).to(io)
    conv_w = randn(3, H * D, 4, std=0.5)
    S0 = randn(B, H, D, D, std=w.s0_std) if w.s0_std > 0 else None
    conv_state = randn(B, 3, 3, H * D, std=w.conv_state_std).to(io) if w.conv_state_std > 0 else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, conv_w=conv_w, S0=S0, conv_state=conv_state)


def make_stage_inputs(w: Workload, seed: int = 0, device: str | torch.device = "cpu") -> dict:
    """Inputs of the optional stages for workload ``w``: o_gate and f [B,T,H,D]
    (decode [B,H,D]) and b_logit [B,T,H] (decode [B,H]) in the I/O dtype; o_norm_w
    [D], A_log [H] and dt_bias [H*D] float32."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 17)
    io = DTYPES[w.io]
    B, T, H, D = w.B, w.T, w.H, w.D
    shape = (B, H, D) if w.decode else (B, T, H, D)
    bshape = (B, H) if w.decode else (B, T, H)

    def randn(*s, std=1.0):
        x = torch.randn(*s, generator=gen, device=device, dtype=torch.float32)
        return x.mul_(std) if std != 1.0 else x

    o_gate = randn(*shape).to(io)
    o_norm_w = randn(D, std=0.1).add_(1.0)
    f = randn(*shape).to(io)
    A_log = torch.empty(H, device=device, dtype=torch.float32).uniform_(w.a_lo, w.a_hi, generator=gen)
    dt_bias = randn(H * D, std=0.5)
    b_logit = randn(*bshape, std=w.b_std).to(io)
    return dict(o_gate=o_gate, o_norm_w=o_norm_w, f=f, A_log=A_log, dt_bias=dt_bias,
                b_logit=b_logit)


def make_packed_inputs(w: Workload, lengths, seed: int = 0,
                       device: str | torch.device = "cpu") -> dict:
    """Packed sequences of the given lengths with workload w's value distributions
    (w.B and w.T are ignored): q, k, v, g [1, T, H, D] and beta [1, T, H] with T =
    sum(lengths); S0 [N, H, D, D] and conv_state [N, 3, 3, H*D] per sequence (when
    w has them); cu_seqlens int32 [N + 1], the running sum of the lengths."""
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    N = len(lengths)
    base = make_inputs(replace(w, B=1, T=T, s0_std=0.0, conv_state_std=0.0), seed=seed, device=device)
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 7919 + 5)
    H, D = w.H, w.D
    S0 = None
    if w.s0_std > 0:
        S0 = torch.randn(N, H, D, D, generator=gen, device=device).mul_(w.s0_std)
    conv_state = None
    if w.conv_state_std > 0:
        conv_state = torch.randn(N, 3, 3, H * D, generator=gen, device=device).mul_(
            w.conv_state_std).to(DTYPES[w.io])
    cu = [0]
    for x in lengths:
        cu.append(cu[-1] + x)
    return dict(base, S0=S0, conv_state=conv_state,
                cu_seqlens=torch.tensor(cu, dtype=torch.int32, device=device))


def to_numpy(t):
    """float64 NumPy copy of a tensor (exact for bf16/fp32 values), or None."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()


def to_storage(t, head_major: bool = False):
    """NumPy copy of a tensor as stored for the oracle's host-process pool: bf16 as
    its raw 16-bit patterns (uint16), float32 as is; a [B, T, H, ...] tensor moved
    to [B, H, T, ...] when head_major, so one (sequence, head) pair is contiguous.
    None stays None."""
    import numpy as np

    if t is None:
        return None
    if head_major:
        t = t.transpose(1, 2)
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
