"""Plain fp64 CPU oracle for the Kimi Delta Attention (KDA) token mixer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
module.  The GPU library never calls it, and it shares no code with the GPU
library: it is a slow, obviously-correct statement of what the mixer computes.

Sources (web pages; cited by title and section):

* "Kimi-K3 model atlas -- self.layers": 69 of the 93 layers are KDA layers whose
  state between calls has a fixed size; the released ``linear_attn_config`` sets
  ``num_heads 96``, ``head_dim 128``, ``short_conv_kernel_size 4`` and a full-rank
  (per-channel) gate.
* "MaxText PR 5548 (Kimi-K3 config, schema, param mapping)", review item 2: the
  KDA tensors ``{q,k,v}_conv1d.weight`` have shape ``[12288, 1, 4]`` and are kept
  in float32, like ``A_log`` and ``dt_bias`` (one decay per channel).
* "Kimi-K3 atlas -- MoE input (decode)", ``KimiRMSNorm``: x / sqrt(mean(x^2) + eps)
  times a per-feature gain, computed in float32 with ``eps = 1e-6``.  Used for the
  identity that ties the L2 norm of q and k to that RMSNorm (see
  ``l2_normalize``) and for the optional output norm (``output_gate_norm``).
* "MaxText PR 5548", review item 2: each KDA layer has an ``o_norm.weight`` of
  shape [128] (one gain per value channel of a head, float32) and a ``g_proj``;
  "MaxText PR 5543", What, item 1: an MLA attention output gated by
  ``g_proj`` is multiplied by the sigmoid of it.

The pages name the mixer and its parameters but do not print its equations.
The definition implemented here is the channel-wise gated delta rule:

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = scale * S_t^T q_t,        alpha_t = exp(g_t)  (one decay per key channel)

preceded by a causal depthwise short convolution (kernel 4) and SiLU on q, k, v
and a per-head L2 normalisation of q and k.  Readings where the pages are silent
(tap order, eps placement, scale, decay axis, ...) are listed in the module-level
constants and in the project design notes; every function says which it uses.

Every function here is pinned by tests that do not re-type it: closed forms,
brute-force matrix products, an independent chunked rewrite, invariants and a
hand-worked example.  No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# Reading: the L2 norm of q and k divides by sqrt(sum(x^2) + eps) with eps inside
# the root.  eps = 1e-6 is the value the pages fix for KimiRMSNorm ("Kimi-K3 atlas
# -- MoE input (decode)", RMSNorm excerpt); the pages give no eps for the L2 norm.
L2_EPS = 1e-6
# Released config, linear_attn_config.short_conv_kernel_size ("Kimi-K3 model
# atlas -- self.layers", config.json).
CONV_K = 4
# eps of the optional output RMSNorm: KimiRMSNorm's default ("Kimi-K3 atlas --
# MoE input (decode)", RMSNorm excerpt).
RMS_EPS = 1e-6


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x * sigmoid(x) = x / (1 + exp(-x)), elementwise, fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def short_conv(x: np.ndarray, w: np.ndarray, history: np.ndarray | None = None) -> np.ndarray:
    """Causal depthwise convolution over time, no bias.

    x:       [T, C] raw inputs of one sequence (fp64)
    w:       [C, K] one K-tap filter per channel; this is the ``[C, 1, K]`` layout
             of the stored ``*_conv1d.weight`` tensors (MaxText PR 5548, review
             item 2) with the singleton middle axis dropped.
    history: [K-1, C] the K-1 raw inputs that precede x, oldest first, or None
             for zeros.

    Reading of the tap order (the pages give only the weight shape): the layout is
    a cross-correlation with K-1 inputs of left padding, so
        y[t, c] = sum_{tau=0}^{K-1} w[c, tau] * x[t - (K-1) + tau, c],
    i.e. the last tap w[c, K-1] multiplies the current input.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, C = x.shape
    K = w.shape[1]
    if history is None:
        history = np.zeros((K - 1, C))
    xe = np.concatenate([np.asarray(history, dtype=np.float64), x], axis=0)  # [K-1+T, C]
    y = np.zeros((T, C))
    for tau in range(K):
        y += w[:, tau][None, :] * xe[tau:tau + T, :]
    return y


def conv_tail(x: np.ndarray, history: np.ndarray | None, K: int = CONV_K) -> np.ndarray:
    """The K-1 most recent raw inputs after consuming x ([T, C]), oldest first.

    This is the convolution's carried state: feeding it back as ``history`` lets a
    later call continue the same sequence.
    """
    x = np.asarray(x, dtype=np.float64)
    C = x.shape[1]
    if history is None:
        history = np.zeros((K - 1, C))
    xe = np.concatenate([np.asarray(history, dtype=np.float64), x], axis=0)
    return xe[xe.shape[0] - (K - 1):, :].copy()


def l2_normalize(x: np.ndarray, eps: float = L2_EPS) -> np.ndarray:
    """x / sqrt(sum_c x_c^2 + eps) over the last axis (one head's channels).

    Reading (pages silent on the L2 norm's eps): eps inside the square root, added
    to the sum of squares.  With eps' = d * eps this equals KimiRMSNorm with unit
    weight divided by sqrt(d), which is how the tests tie it to the pages'
    RMSNorm definition.
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + eps)


def sigmoid(x: np.ndarray) -> np.ndarray:
    """The logistic function 1 / (1 + exp(-x)), elementwise, fp64."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def rms_norm(x: np.ndarray, w: np.ndarray | None = None, eps: float = RMS_EPS) -> np.ndarray:
    """KimiRMSNorm over the last axis: x / sqrt(mean_c x_c^2 + eps), times the gain w.

    ("Kimi-K3 atlas -- MoE input (decode)", RMSNorm excerpt: the mean of squares,
    eps inside the root, one gain per feature.)  The excerpt rounds the normalised
    value to the activation dtype before the gain; here everything is fp64 and the
    GPU rounds once at the end, a difference of one rounding that the parity
    tolerance covers.
    """
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return y if w is None else y * np.asarray(w, dtype=np.float64)


def output_gate_norm(o: np.ndarray, o_norm_w: np.ndarray | None = None,
                     gate: np.ndarray | None = None, eps: float = RMS_EPS) -> np.ndarray:
    """The optional output stage of a head: RMSNorm with the o_norm gain, then the
    sigmoid output gate.

    o:        [..., D] mixer output of one head per row
    o_norm_w: [D] gain shared by the heads (the layer's o_norm.weight has shape
              [head_dim]), or None to skip the norm
    gate:     [..., D] gate pre-activation (the g_proj output), or None to skip
    Reading: norm first, then gate, the order of a gated RMSNorm whose gain is
    o_norm.weight; the pages give the sigmoid gate for the MLA output and no
    formula for KDA's, so the sigmoid is taken by analogy ("MaxText PR 5543",
    What, item 1).
    """
    y = np.asarray(o, dtype=np.float64)
    if o_norm_w is not None:
        y = rms_norm(y, o_norm_w, eps)
    if gate is not None:
        y = y * sigmoid(gate)
    return y


def output_gate_norm_backward(o: np.ndarray, dy: np.ndarray, o_norm_w: np.ndarray | None = None,
                             gate: np.ndarray | None = None, eps: float = RMS_EPS):
    """Reverse of ``output_gate_norm``: given the stage's input o [..., D] and the
    gradient dy of its output, returns (do, do_norm_w [D] or None, dgate or None).

    With r = 1 / sqrt(mean_c o_c^2 + eps), n = o r, a = n w (a = o without the
    norm), s = sigmoid(gate), y = a s (y = a without the gate):
        dgate = dy a s (1 - s),   da = dy s,
        do_norm_w = sum over rows of da n,   dn = da w,
        do = r (dn - n mean_c(dn n))   (the RMSNorm's Jacobian applied to dn).
    """
    o = np.asarray(o, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    if o_norm_w is not None:
        w = np.asarray(o_norm_w, dtype=np.float64)
        r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
        n = o * r
        a = n * w
    else:
        a = o
    dgate = None
    if gate is not None:
        s = sigmoid(gate)
        dgate = dy * a * s * (1.0 - s)
        da = dy * s
    else:
        da = dy
    dw = None
    if o_norm_w is not None:
        dw = np.sum((da * n).reshape(-1, o.shape[-1]), axis=0)
        dn = da * w
        do = r * (dn - n * np.mean(dn * n, axis=-1, keepdims=True))
    else:
        do = da
    return do, dw, dgate


def softplus(x: np.ndarray) -> np.ndarray:
    """softplus(x) = ln(1 + e^x), elementwise, fp64 (as log(e^0 + e^x), which does
    not overflow for large x)."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def kda_gate(f: np.ndarray, A_log: np.ndarray, dt_bias: np.ndarray) -> np.ndarray:
    """Per-channel log-decay from the gate projection: g = -exp(A_log[h]) * softplus(f + dt_bias).

    f:       [..., H, D] gate projection output (the full-rank gate: one value per
             key channel)
    A_log:   [H] float32, one per head; dt_bias: [H*D] float32, one per channel
             ("MaxText PR 5548", review item 2, and the A_log slicing notes: A_log
             is [num_heads], dt_bias [12288], both kept in float32 to avoid decay
             drift over long contexts).
    Reading: the pages give the parameters and their shapes, not the formula; this
    is the plainest form they support (a positive rate exp(A_log) per head times a
    softplus of the biased projection, so g <= 0 always).  The config's
    gate_lower_bound (-5.0, "Kimi-K3 model atlas -- self.layers") is not applied:
    the pages do not say how.
    """
    f = np.asarray(f, dtype=np.float64)
    H, D = f.shape[-2], f.shape[-1]
    rate = np.exp(np.asarray(A_log, dtype=np.float64)).reshape(H, 1)
    bias = np.asarray(dt_bias, dtype=np.float64).reshape(H, D)
    return -rate * softplus(f + bias)


def gated_delta_step(S, q, k, v, g, beta, scale=1.0):
    """One step of the channel-wise gated delta rule for a batch of heads.

    S: [..., dk, dv] state before the step; q, k, g: [..., dk]; v: [..., dv];
    beta: [...].  The decay alpha = exp(g) scales the rows of S (the key axis),
    the reading that matches Diag(alpha) left-multiplying the dk x dv state.

    Written in the rank-one form that the definition expands to:
        S_bar = Diag(alpha) S
        u     = beta * (v - S_bar^T k)
        S'    = S_bar + k u^T            ( = (I - beta k k^T) S_bar + beta k v^T )
        o     = scale * S'^T q           (output reads the updated state)
    """
    alpha = np.exp(g)
    S_bar = alpha[..., :, None] * S
    r = np.matmul(k[..., None, :], S_bar)[..., 0, :]          # S_bar^T k
    u = beta[..., None] * (v - r)
    S_new = S_bar + k[..., :, None] * u[..., None, :]
    o = scale * np.matmul(q[..., None, :], S_new)[..., 0, :]  # S'^T q
    return S_new, o


def _check_decay(g):
    if not np.all(np.isfinite(g)):
        raise ValueError("log-decay g must be finite")
    if np.any(g > 0):
        raise ValueError("log-decay g must be <= 0 (decay factors in (0, 1])")


def kda_reference(q, k, v, g, beta, conv_w=None, conv_state=None, S0=None,
                  scale=1.0, l2norm_qk=True, eps=L2_EPS, o_norm_w=None, o_gate=None,
                  o_norm_eps=RMS_EPS, A_log=None, dt_bias=None, beta_sigmoid=False):
    """The full KDA mixer over a batch of sequences, sequentially in time, fp64.

    q, k, v, g: [B, T, H, D] (raw q, k, v before the convolution; g is the
                per-channel log-decay, finite and <= 0)
    beta:       [B, T, H]
    conv_w:     [3, H*D, K] float32 filters for q, k, v in that order, or None to
                skip the convolution and SiLU (inputs used as given)
    conv_state: [B, 3, K-1, H*D] raw inputs preceding t = 0, or None for zeros
    S0:         [B, H, D, D] initial state, or None for zeros
    o_norm_w, o_gate: the optional output stage (``output_gate_norm``); o_gate is
                [B, T, H, D]
    A_log, dt_bias: if given, g holds the gate projection output f and the decay
                is ``kda_gate(f, A_log, dt_bias)``
    beta_sigmoid: if true, beta holds logits and the write strength is sigmoid(beta)
    Returns (o [B, T, H, D], S_T [B, H, D, D], tail [B, 3, K-1, H*D] or None).

    Steps: (1) short causal conv per channel and SiLU on q, k, v; (2) L2 norm of q
    and k per head; (3) the gated delta rule step by step from S0; (4) if asked,
    the output RMSNorm and sigmoid gate per head.
    """
    q, k, v, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g))
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, D = q.shape
    if A_log is not None:
        g = kda_gate(g, A_log, dt_bias)
    if beta_sigmoid:
        beta = sigmoid(beta)
    _check_decay(g)
    tail = None
    if conv_w is not None:
        conv_w = np.asarray(conv_w, dtype=np.float64)
        K = conv_w.shape[2]
        outs = []
        tails = np.zeros((B, 3, K - 1, H * D))
        for i, x in enumerate((q, k, v)):
            y = np.empty_like(x)
            for b in range(B):
                hist = None if conv_state is None else np.asarray(conv_state[b, i], dtype=np.float64)
                xb = x[b].reshape(T, H * D)
                y[b] = silu(short_conv(xb, conv_w[i], hist)).reshape(T, H, D)
                tails[b, i] = conv_tail(xb, hist, K)
            outs.append(y)
        q, k, v = outs
        tail = tails
    if l2norm_qk:
        q = l2_normalize(q, eps)
        k = l2_normalize(k, eps)
    S = np.zeros((B, H, D, D)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.empty((B, T, H, D))
    for t in range(T):
        S, o[:, t] = gated_delta_step(S, q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], scale)
    if o_norm_w is not None or o_gate is not None:
        o = output_gate_norm(o, o_norm_w, o_gate, o_norm_eps)
    return o, S, tail


def kda_reference_decode_step(q, k, v, g, beta, S, conv_w=None, conv_state=None,
                              scale=1.0, l2norm_qk=True, eps=L2_EPS, o_norm_w=None,
                              o_gate=None, o_norm_eps=RMS_EPS, A_log=None, dt_bias=None,
                              beta_sigmoid=False):
    """One autoregressive KDA step for B sequences: the mixer at T = 1.

    q, k, v, g: [B, H, D] raw inputs of the new token; beta [B, H];
    S [B, H, D, D] cached state; conv_state [B, 3, K-1, H*D] cached raw inputs;
    o_gate [B, H, D] or None.
    Returns (o [B, H, D], S_new, conv_state_new).
    """
    o, S_new, tail = kda_reference(
        np.asarray(q)[:, None], np.asarray(k)[:, None], np.asarray(v)[:, None],
        np.asarray(g)[:, None], np.asarray(beta)[:, None],
        conv_w=conv_w, conv_state=conv_state, S0=S, scale=scale,
        l2norm_qk=l2norm_qk, eps=eps, o_norm_w=o_norm_w,
        o_gate=None if o_gate is None else np.asarray(o_gate)[:, None], o_norm_eps=o_norm_eps,
        A_log=A_log, dt_bias=dt_bias, beta_sigmoid=beta_sigmoid)
    return o[:, 0], S_new, tail


def conv_norm_reference(q, k, v, conv_w, conv_state=None, l2norm_qk=True, eps=L2_EPS):
    """Only the pre-recurrence part: conv + SiLU on q, k, v, then L2 of q and k.

    Same inputs as ``kda_reference``; returns (q_hat, k_hat, v_hat, tail).
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, T, H, D = q.shape
    conv_w = np.asarray(conv_w, dtype=np.float64)
    K = conv_w.shape[2]
    outs = []
    tails = np.zeros((B, 3, K - 1, H * D))
    for i, x in enumerate((q, k, v)):
        y = np.empty_like(x)
        for b in range(B):
            hist = None if conv_state is None else np.asarray(conv_state[b, i], dtype=np.float64)
            xb = x[b].reshape(T, H * D)
            y[b] = silu(short_conv(xb, conv_w[i], hist)).reshape(T, H, D)
            tails[b, i] = conv_tail(xb, hist, K)
        outs.append(y)
    qh, kh, vh = outs
    if l2norm_qk:
        qh = l2_normalize(qh, eps)
        kh = l2_normalize(kh, eps)
    return qh, kh, vh, tails


def kda_reference_backward(q, k, v, g, beta, do, dS_T=None, conv_w=None, conv_state=None,
                           S0=None, scale=1.0, l2norm_qk=True, eps=L2_EPS, o_norm_w=None,
                           o_gate=None, o_norm_eps=RMS_EPS, A_log=None, dt_bias=None,
                           beta_sigmoid=False):
    """Gradients of the mixer by reverse-mode differentiation of its sequential
    definition (``kda_reference``), fp64.

    The scalar differentiated is  L = sum(o * do) + sum(S_T * dS_T)  (dS_T None: 0),
    i.e. do and dS_T are the upstream gradients of o and S_T.  Inputs as
    ``kda_reference``, with its optional stages.  Returns a dict of gradients with the
    inputs' shapes: dq, dk, dv (of the raw inputs), dg, dbeta (of g and beta as given:
    of the gate projection f with A_log, of the logits with beta_sigmoid), dS0
    (zeros-shaped when S0 is None: the gradient of a zero initial state), dconv_w and
    dconv_state (None without the convolution), do_norm_w, do_gate, dA_log and
    ddt_bias (None when their stage is off).

    Reverse of one step (S_bar = Diag(alpha) S, u = beta (v - S_bar^T k),
    S' = S_bar + k u^T, o = scale S'^T q), with G the gradient of S':
        G += scale q do^T;   dq = scale S' do
        dk += G u;   du = G^T k
        dv = beta du;   dbeta = du . (v - S_bar^T k)
        G_bar = G - beta k du^T;   dk -= beta S_bar du
        dalpha = rowsum(G_bar * S);   dg = alpha * dalpha;   G <- Diag(alpha) G_bar
    then the front end in reverse: the L2 norm (z = y / n, n = sqrt(|y|^2 + eps):
    dy = dz / n - y (y . dz) / n^3), SiLU (x sigmoid(x), derivative
    sigmoid(x) (1 + x (1 - sigmoid(x)))) and the convolution (a correlation, whose
    adjoint sends dy[t] back to the inputs t-3 .. t and to the filter taps).
    The optional stages: the output stage first (``output_gate_norm_backward``, on
    the mixer's output before it); the activations last, with g = -exp(A_log) sp,
    sp = softplus(f + dt_bias): df = dg (-exp(A_log)) sigmoid(f + dt_bias),
    dA_log = sum dg g, ddt_bias = sum df; and dbeta_logit = dbeta beta (1 - beta).
    """
    q, k, v, g, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, do))
    beta = np.asarray(beta, dtype=np.float64)
    B, T, H, D = q.shape
    f = None
    if A_log is not None:
        f = g
        g = kda_gate(f, A_log, dt_bias)
    if beta_sigmoid:
        beta = sigmoid(beta)
    _check_decay(g)
    HD = H * D
    raw = (q, k, v)
    pre = ys = None
    if conv_w is not None:
        cw = np.asarray(conv_w, dtype=np.float64)
        K = cw.shape[2]
        hist = np.zeros((B, 3, K - 1, HD)) if conv_state is None else np.asarray(conv_state, dtype=np.float64)
        pre = np.empty((3, B, T, HD))
        for i, x in enumerate(raw):
            for b in range(B):
                pre[i, b] = short_conv(x[b].reshape(T, HD), cw[i], hist[b, i])
        ys = [silu(pre[i]).reshape(B, T, H, D) for i in range(3)]
    else:
        ys = [x.copy() for x in raw]
    yq, yk, yv = ys
    if l2norm_qk:
        nq = np.sqrt(np.sum(yq * yq, axis=-1, keepdims=True) + eps)
        nk = np.sqrt(np.sum(yk * yk, axis=-1, keepdims=True) + eps)
        qh, kh = yq / nq, yk / nk
    else:
        qh, kh = yq, yk
    vh = yv
    # forward, keeping the state before each step
    S = np.zeros((B, H, D, D)) if S0 is None else np.array(S0, dtype=np.float64)
    S_prev = np.empty((T, B, H, D, D))
    o_pre = np.empty((B, T, H, D))
    for t in range(T):
        S_prev[t] = S
        S, o_pre[:, t] = gated_delta_step(S, qh[:, t], kh[:, t], vh[:, t], g[:, t], beta[:, t], scale)
    do_norm_w = do_gate = None
    if o_norm_w is not None or o_gate is not None:
        do, do_norm_w, do_gate = output_gate_norm_backward(o_pre, do, o_norm_w, o_gate, o_norm_eps)
    # reverse
    G = np.zeros((B, H, D, D)) if dS_T is None else np.array(dS_T, dtype=np.float64)
    dqh, dkh, dvh = np.zeros_like(qh), np.zeros_like(kh), np.zeros_like(vh)
    dg, dbeta = np.zeros_like(g), np.zeros_like(beta)
    for t in range(T - 1, -1, -1):
        qt, kt, vt, bt = qh[:, t], kh[:, t], vh[:, t], beta[:, t]
        alpha = np.exp(g[:, t])
        Sp = S_prev[t]
        S_bar = alpha[..., :, None] * Sp
        r = np.einsum("bhcv,bhc->bhv", S_bar, kt)
        u = bt[..., None] * (vt - r)
        S_new = S_bar + kt[..., :, None] * u[..., None, :]
        dot = do[:, t]
        G = G + scale * qt[..., :, None] * dot[..., None, :]
        dqh[:, t] = scale * np.einsum("bhcv,bhv->bhc", S_new, dot)
        dk_t = np.einsum("bhcv,bhv->bhc", G, u)
        du = np.einsum("bhcv,bhc->bhv", G, kt)
        dvh[:, t] = bt[..., None] * du
        dbeta[:, t] = np.sum(du * (vt - r), axis=-1)
        dr = -bt[..., None] * du
        G_bar = G + kt[..., :, None] * dr[..., None, :]
        dk_t += np.einsum("bhcv,bhv->bhc", S_bar, dr)
        dkh[:, t] = dk_t
        dalpha = np.sum(G_bar * Sp, axis=-1)
        dg[:, t] = alpha * dalpha
        G = alpha[..., :, None] * G_bar
    dS0 = G
    # front end in reverse
    if l2norm_qk:
        dyq = dqh / nq - yq * np.sum(yq * dqh, axis=-1, keepdims=True) / nq ** 3
        dyk = dkh / nk - yk * np.sum(yk * dkh, axis=-1, keepdims=True) / nk ** 3
    else:
        dyq, dyk = dqh, dkh
    dys = [dyq, dyk, dvh]
    extra = dict(do_norm_w=do_norm_w, do_gate=do_gate, dA_log=None, ddt_bias=None)
    if A_log is not None:
        rate = np.exp(np.asarray(A_log, dtype=np.float64)).reshape(H, 1)
        z = f + np.asarray(dt_bias, dtype=np.float64).reshape(H, D)
        extra["dA_log"] = np.sum(dg * g, axis=(0, 1, 3))
        dg = dg * (-rate) * sigmoid(z)
        extra["ddt_bias"] = np.sum(dg, axis=(0, 1)).reshape(H * D)
    if beta_sigmoid:
        dbeta = dbeta * beta * (1.0 - beta)
    if conv_w is None:
        dq_, dk_, dv_ = dys
        return dict(dq=dq_, dk=dk_, dv=dv_, dg=dg, dbeta=dbeta, dS0=dS0, dconv_w=None,
                    dconv_state=None, **extra)
    dconv_w = np.zeros_like(cw)
    dhist = np.zeros_like(hist)
    dx = []
    for i in range(3):
        xs = pre[i]
        sg = sigmoid(xs)
        dpre = dys[i].reshape(B, T, HD) * sg * (1.0 + xs * (1.0 - sg))
        dxi = np.zeros((B, T, HD))
        for b in range(B):
            xe = np.concatenate([hist[b, i], raw[i][b].reshape(T, HD)], axis=0)  # [K-1+T, HD]
            dxe = np.zeros_like(xe)
            for tau in range(K):
                dconv_w[i][:, tau] += np.sum(dpre[b] * xe[tau:tau + T], axis=0)
                dxe[tau:tau + T] += cw[i][:, tau][None, :] * dpre[b]
            dhist[b, i] = dxe[:K - 1]
            dxi[b] = dxe[K - 1:]
        dx.append(dxi.reshape(B, T, H, D))
    return dict(dq=dx[0], dk=dx[1], dv=dx[2], dg=dg, dbeta=dbeta, dS0=dS0, dconv_w=dconv_w,
                dconv_state=dhist, **extra)


def kda_reference_packed(q, k, v, g, beta, cu_seqlens, conv_w=None, conv_state=None, S0=None,
                         **kw):
    """The mixer over packed sequences: sequence i is tokens [cu_seqlens[i],
    cu_seqlens[i+1]) of a single row of tokens, with its own conv history and
    initial state; nothing crosses a boundary.

    ("MaxText PR 5550" rejects packed batches for KDA because its layer ignores
    segment ids, i.e. would let state and conv history flow from one sequence
    into the next; "Kimi-K3 model atlas -- self.layers", transformer excerpt:
    the model hands a padding mask to its KDA layers.)

    q, k, v, g: [1, T, H, D]; beta [1, T, H]; cu_seqlens: N + 1 non-decreasing
    offsets from 0 to T; conv_state [N, 3, K-1, H*D] or None; S0 [N, H, D, D] or
    None.  Other keyword arguments as ``kda_reference`` (o_gate is [1, T, H, D]).
    Returns (o [1, T, H, D], S_T [N, H, D, D], tail [N, 3, K-1, H*D] or None).
    """
    cu = [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    if cu[0] != 0 or cu[-1] != np.asarray(q).shape[1] or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must run from 0 to T without decreasing")
    B, T, H, D = np.asarray(q).shape
    if B != 1:
        raise ValueError("packed sequences share one row of tokens (B = 1)")
    o = np.zeros((1, T, H, D))
    S_out = np.zeros((N, H, D, D))
    tails = None if conv_w is None else np.zeros((N, 3, np.asarray(conv_w).shape[2] - 1, H * D))
    o_gate = kw.pop("o_gate", None)
    for i in range(N):
        a, e = cu[i], cu[i + 1]
        sl = slice(a, e)
        cs = None if conv_state is None else np.asarray(conv_state)[i:i + 1]
        s0 = None if S0 is None else np.asarray(S0)[i:i + 1]
        og = None if o_gate is None else np.asarray(o_gate)[:, sl]
        oi, Si, ti = kda_reference(np.asarray(q)[:, sl], np.asarray(k)[:, sl], np.asarray(v)[:, sl],
                                   np.asarray(g)[:, sl], np.asarray(beta)[:, sl], conv_w=conv_w,
                                   conv_state=cs, S0=s0, o_gate=og, **kw)
        o[:, sl] = oi
        S_out[i] = Si[0]
        if tails is not None:
            tails[i] = ti[0]
    return o, S_out, tails


def kda_reference_backward_packed(q, k, v, g, beta, cu_seqlens, do, dS_T=None, conv_w=None,
                                  conv_state=None, S0=None, **kw):
    """Gradients of ``kda_reference_packed``: each sequence's part by
    ``kda_reference_backward`` on its own tokens, conv history and initial state
    (nothing crosses a boundary, so nothing flows across one backwards either).

    Shapes as ``kda_reference_packed``; do [1, T, H, D], dS_T [N, H, D, D] or None.
    Per-token gradients go to their tokens, dS0 [N, H, D, D] and dconv_state
    [N, 3, K-1, H*D] to their sequences; the shared parameters' gradients (dconv_w,
    do_norm_w, dA_log, ddt_bias) are the sums over the sequences.
    """
    cu = [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    B, T, H, D = np.asarray(q).shape
    if B != 1 or cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("packed sequences: B = 1 and offsets from 0 to T without decreasing")
    o_gate = kw.pop("o_gate", None)
    tok = {n: np.zeros((1, T, H, D)) for n in ("dq", "dk", "dv", "dg")}
    tok["dbeta"] = np.zeros((1, T, H))
    if o_gate is not None:
        tok["do_gate"] = np.zeros((1, T, H, D))
    out = dict(tok)
    out["dS0"] = np.zeros((N, H, D, D))
    out["dconv_state"] = None
    shared = {}
    for i in range(N):
        sl = slice(cu[i], cu[i + 1])
        part = lambda x: None if x is None else np.asarray(x)[:, sl]
        one = lambda x: None if x is None else np.asarray(x)[i:i + 1]
        gi = kda_reference_backward(part(q), part(k), part(v), part(g), part(beta), part(do),
                                    one(dS_T), conv_w=conv_w, conv_state=one(conv_state),
                                    S0=one(S0), o_gate=part(o_gate), **kw)
        for n in tok:
            out[n][:, sl] = gi[n]
        out["dS0"][i] = gi["dS0"][0]
        if gi["dconv_state"] is not None:
            if out["dconv_state"] is None:
                out["dconv_state"] = np.zeros((N,) + gi["dconv_state"].shape[1:])
            out["dconv_state"][i] = gi["dconv_state"][0]
        for n in ("dconv_w", "do_norm_w", "dA_log", "ddt_bias"):
            if gi[n] is not None:
                shared[n] = shared.get(n, 0.0) + gi[n]
    for n in ("dconv_w", "do_norm_w", "dA_log", "ddt_bias"):
        out[n] = shared.get(n)
    out.setdefault("do_gate", None)
    return out


def kda_reference_heads(q, k, v, g, beta, heads, conv_w=None, conv_state=None, S0=None,
                        scale=1.0, l2norm_qk=True, eps=L2_EPS, o_norm_w=None, o_gate=None,
                        o_norm_eps=RMS_EPS, A_log=None, dt_bias=None, beta_sigmoid=False):
    """``kda_reference`` restricted to a list of (b, h) pairs.

    Heads are independent (their state, decay and filters are per head/channel),
    so the result for a listed head equals the full call's.  Inputs are the full
    arrays; only the listed slices are read.  Returns a list of (o [T, D], S_T
    [D, D]) in the order of ``heads``.
    """
    out = []
    D = q.shape[3]
    for (b, h) in heads:
        sl = slice(h * D, (h + 1) * D)
        cw = None if conv_w is None else np.asarray(conv_w)[:, sl, :]
        cs = None if conv_state is None else np.asarray(conv_state)[b:b + 1, :, :, sl]
        s0 = None if S0 is None else np.asarray(S0)[b:b + 1, h:h + 1]
        og = None if o_gate is None else np.asarray(o_gate)[b:b + 1, :, h:h + 1]
        o, S, _ = kda_reference(
            np.asarray(q)[b:b + 1, :, h:h + 1], np.asarray(k)[b:b + 1, :, h:h + 1],
            np.asarray(v)[b:b + 1, :, h:h + 1], np.asarray(g)[b:b + 1, :, h:h + 1],
            np.asarray(beta)[b:b + 1, :, h:h + 1], conv_w=cw, conv_state=cs, S0=s0,
            scale=scale, l2norm_qk=l2norm_qk, eps=eps, o_norm_w=o_norm_w, o_gate=og,
            o_norm_eps=o_norm_eps,
            A_log=None if A_log is None else np.asarray(A_log)[h:h + 1],
            dt_bias=None if dt_bias is None else np.asarray(dt_bias)[sl],
            beta_sigmoid=beta_sigmoid)
        out.append((o[0, :, 0], S[0, 0]))
    return out
