"""Pins for the fp64 oracle: values fixed by hand, closed forms, brute force,
invariants and an independent chunked rewrite.  CPU only.

Each pin targets a plausible slip in the oracle: the hand example and the
brute-force matrix form catch a wrong sign, a transposed state, decay on the wrong
axis, a misplaced beta or reading S_{t-1} for the output; the impulse test catches
a reversed tap order; the split tests catch a mishandled conv history or state
hand-over; the norm identity catches eps in the wrong place.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle import (conv_norm_reference, conv_tail, gated_delta_step, kda_reference,
                    kda_reference_backward, kda_reference_backward_packed, kda_reference_decode_step,
                    kda_reference_heads, kda_reference_packed, output_gate_norm_backward,
                    l2_normalize,
                    kda_gate, output_gate_norm, rms_norm, short_conv, sigmoid, silu,
                    softplus)
from chunked_form import chunk_quantities, chunked_head

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, B=1, T=9, H=2, D=4, strong=False, s0=True):
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, H, D))
    v = rng.standard_normal((B, T, H, D))
    scale = 3.0 if strong else 0.5
    g = -scale * np.log1p(np.exp(rng.standard_normal((B, T, H, D))))
    beta = expit(rng.standard_normal((B, T, H)))
    conv_w = 0.5 * rng.standard_normal((3, H * D, 4))
    S0 = 0.1 * rng.standard_normal((B, H, D, D)) if s0 else None
    return q, k, v, g, beta, conv_w, S0


# ---------------------------------------------------------------- P1 hand example
def test_hand_example_t1():
    d = json.load(open(os.path.join(GOLDEN, "hand_t1.json")))
    f = lambda x: np.array(x, dtype=np.float64)
    q, k, v, g = (f(d[n]).reshape(1, 1, 1, 2) for n in ("q", "k", "v", "g"))
    beta = np.full((1, 1, 1), d["beta"])
    S0 = f(d["S0"]).reshape(1, 1, 2, 2)
    o, S, tail = kda_reference(q, k, v, g, beta, conv_w=None, S0=S0, l2norm_qk=False)
    assert tail is None
    np.testing.assert_allclose(S[0, 0], f(d["S1"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[0, 0, 0], f(d["o"]), rtol=0, atol=1e-12)


# ------------------------------------------------- brute force: the matrix form
def test_rank_one_step_equals_matrix_form():
    rng = np.random.default_rng(1)
    dk, dv = 5, 3
    S = rng.standard_normal((dk, dv))
    for _ in range(6):
        q, k, g = rng.standard_normal(dk), rng.standard_normal(dk), -np.abs(rng.standard_normal(dk))
        v = rng.standard_normal(dv)
        beta = float(expit(rng.standard_normal()))
        S_mat = (np.eye(dk) - beta * np.outer(k, k)) @ np.diag(np.exp(g)) @ S + beta * np.outer(k, v)
        o_mat = S_mat.T @ q
        S_new, o = gated_delta_step(S, q, k, v, g, np.float64(beta))
        np.testing.assert_allclose(S_new, S_mat, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(o, o_mat, rtol=1e-13, atol=1e-13)
        S = S_new


def test_full_mixer_brute_force_tiny():
    """Conv + SiLU + L2 + recurrence, each step written with explicit matrices."""
    rng = np.random.default_rng(2)
    B, T, H, D = 1, 5, 1, 3
    q, k, v, g, beta, conv_w, S0 = rand_case(rng, B, T, H, D)
    o, S, tail = kda_reference(q, k, v, g, beta, conv_w=conv_w, S0=S0)
    # brute force: build each conv output as an explicit dot over the 4-tap window
    xs = []
    for i, x in enumerate((q, k, v)):
        xe = np.concatenate([np.zeros((3, D)), x[0, :, 0]], axis=0)
        y = np.array([[np.dot(conv_w[i, c], xe[t:t + 4, c]) for c in range(D)] for t in range(T)])
        xs.append(y * expit(y))
    qh, kh, vh = xs
    qh = qh / np.sqrt((qh ** 2).sum(1, keepdims=True) + 1e-6)
    kh = kh / np.sqrt((kh ** 2).sum(1, keepdims=True) + 1e-6)
    Sm = S0[0, 0].copy()
    for t in range(T):
        b = beta[0, t, 0]
        Sm = (np.eye(D) - b * np.outer(kh[t], kh[t])) @ np.diag(np.exp(g[0, t, 0])) @ Sm + b * np.outer(kh[t], vh[t])
        np.testing.assert_allclose(o[0, t, 0], Sm.T @ qh[t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], Sm, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- closed forms
def test_beta0_alpha1_keeps_state():
    """P2: beta = 0 and g = 0 leave S0 untouched and o_t = S0^T q_t."""
    rng = np.random.default_rng(3)
    q, k, v, _, _, _, S0 = rand_case(rng, B=2, T=7, H=2, D=4)
    g = np.zeros_like(q)
    beta = np.zeros(q.shape[:3])
    o, S, _ = kda_reference(q, k, v, g, beta, S0=S0, l2norm_qk=False)
    np.testing.assert_array_equal(S, S0)
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(o[b, :, h], q[b, :, h] @ S0[b, h], rtol=1e-13, atol=1e-13)


def test_orthonormal_keys_linear_attention():
    """P3: g = 0, S0 = 0, mutually orthonormal keys => S_T = sum_t beta_t k_t v_t^T
    and o_t = sum_{j<=t} beta_j (k_j . q_t) v_j (plain causal linear attention)."""
    rng = np.random.default_rng(4)
    D, T = 6, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((D, D)))
    k = Qm[:, :T].T.reshape(1, T, 1, D)
    q = rng.standard_normal((1, T, 1, D))
    v = rng.standard_normal((1, T, 1, D))
    beta = expit(rng.standard_normal((1, T, 1)))
    o, S, _ = kda_reference(q, k, v, np.zeros_like(q), beta, l2norm_qk=False)
    expect = sum(beta[0, t, 0] * np.outer(k[0, t, 0], v[0, t, 0]) for t in range(T))
    np.testing.assert_allclose(S[0, 0], expect, rtol=1e-12, atol=1e-12)
    for t in range(T):
        ot = sum(beta[0, j, 0] * np.dot(k[0, j, 0], q[0, t, 0]) * v[0, j, 0] for j in range(t + 1))
        np.testing.assert_allclose(o[0, t, 0], ot, rtol=1e-12, atol=1e-12)
    # beta = 1 gives exactly sum k v^T
    o1, S1, _ = kda_reference(q, k, v, np.zeros_like(q), np.ones((1, T, 1)), l2norm_qk=False)
    np.testing.assert_allclose(S1[0, 0], k[0, :, 0].T @ v[0, :, 0], rtol=1e-12, atol=1e-12)


def test_alpha0_resets_state():
    """P4: g = -1000 (alpha = 0) forgets S0: S_t = beta_t k_t v_t^T,
    o_t = beta_t (k_t . q_t) v_t, whatever S0 is."""
    rng = np.random.default_rng(5)
    q, k, v, _, beta, _, S0 = rand_case(rng, B=1, T=6, H=1, D=4)
    g = np.full_like(q, -1000.0)
    o, S, _ = kda_reference(q, k, v, g, beta, S0=S0, l2norm_qk=False)
    T = q.shape[1]
    for t in range(T):
        b = beta[0, t, 0]
        np.testing.assert_allclose(o[0, t, 0], b * np.dot(k[0, t, 0], q[0, t, 0]) * v[0, t, 0],
                                   rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0, 0], beta[0, -1, 0] * np.outer(k[0, -1, 0], v[0, -1, 0]),
                               rtol=1e-12, atol=1e-12)


def test_retrieval_invariant():
    """P5: S_t^T k_t = (1 - beta |k|^2) S_bar^T k_t + beta |k|^2 v_t, with
    S_bar = Diag(exp g_t) S_{t-1}; unit keys and beta = 1 read back v_t exactly."""
    rng = np.random.default_rng(6)
    D = 5
    S = rng.standard_normal((D, D))
    for _ in range(5):
        q, k, v = rng.standard_normal(D), rng.standard_normal(D), rng.standard_normal(D)
        g = -np.abs(rng.standard_normal(D))
        beta = np.float64(expit(rng.standard_normal()))
        S_new, _ = gated_delta_step(S, q, k, v, g, beta)
        S_bar = np.diag(np.exp(g)) @ S
        kk = k @ k
        np.testing.assert_allclose(S_new.T @ k, (1 - beta * kk) * (S_bar.T @ k) + beta * kk * v,
                                   rtol=1e-12, atol=1e-12)
        ku = k / np.linalg.norm(k)
        S_one, _ = gated_delta_step(S, q, ku, v, g, np.float64(1.0))
        np.testing.assert_allclose(S_one.T @ ku, v, rtol=1e-12, atol=1e-12)
        S = S_new


# ----------------------------------------------- P6/P7: chunked == sequential
@pytest.mark.parametrize("C", [7, 16, 64])
@pytest.mark.parametrize("strong", [False, True])
def test_chunked_equals_sequential(C, strong):
    rng = np.random.default_rng(7 + C)
    T, D = 150, 8
    q, k, v, g, beta, _, S0 = rand_case(rng, B=1, T=T, H=1, D=D, strong=strong)
    q = l2_normalize(q)
    k = l2_normalize(k)
    o, S, _ = kda_reference(q, k, v, g, beta, S0=S0, l2norm_qk=False)
    oc, Sc = chunked_head(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], S0[0, 0], C)
    np.testing.assert_allclose(oc, o[0, :, 0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Sc, S[0, 0], rtol=1e-11, atol=1e-12)


def test_chunk_affine_state_map():
    """P7: one chunk maps S0 to M S0 + N with M = Diag(Lam_C) - Ktil^T W, N = Ktil^T Ut."""
    rng = np.random.default_rng(8)
    C, D = 16, 6
    q, k, v, g, beta, _, _ = rand_case(rng, B=1, T=C, H=1, D=D)
    k = l2_normalize(k)
    m = chunk_quantities(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0])
    M = np.diag(m["LamC"]) - m["Ktil"].T @ m["W"]
    N = m["Ktil"].T @ m["Ut"]
    for seed in range(3):
        S0 = np.random.default_rng(seed).standard_normal((1, 1, D, D))
        _, S, _ = kda_reference(q, k, v, g, beta, S0=S0, l2norm_qk=False)
        np.testing.assert_allclose(S[0, 0], M @ S0[0, 0] + N, rtol=1e-11, atol=1e-12)


# ------------------------------------------------------- P8: splitting time
@pytest.mark.parametrize("t0", [1, 2, 3, 17])
def test_time_split_and_decode(t0):
    rng = np.random.default_rng(9)
    B, T, H, D = 2, 24, 2, 4
    q, k, v, g, beta, conv_w, S0 = rand_case(rng, B, T, H, D)
    o, S, tail = kda_reference(q, k, v, g, beta, conv_w=conv_w, S0=S0)
    a = slice(0, t0)
    b = slice(t0, T)
    o1, S1, tail1 = kda_reference(q[:, a], k[:, a], v[:, a], g[:, a], beta[:, a], conv_w=conv_w, S0=S0)
    o2, S2, tail2 = kda_reference(q[:, b], k[:, b], v[:, b], g[:, b], beta[:, b], conv_w=conv_w,
                                  conv_state=tail1, S0=S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(tail2, tail)
    # token-by-token decode reaches the same result
    Sd, cs = S0.copy(), None
    for t in range(T):
        od, Sd, cs = kda_reference_decode_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], Sd,
                                               conv_w=conv_w, conv_state=cs)
        np.testing.assert_allclose(od, o[:, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sd, S, rtol=1e-12, atol=1e-12)


# ------------------------------------------ P9: value columns are independent
def test_value_column_independence():
    rng = np.random.default_rng(10)
    B, T, H, D = 1, 12, 2, 4
    q, k, v, g, beta, conv_w, S0 = rand_case(rng, B, T, H, D)
    o, S, _ = kda_reference(q, k, v, g, beta, conv_w=conv_w, S0=S0)
    v2 = v.copy()
    v2[..., 1] += 3.0
    S02 = S0.copy()
    S02[..., 1] -= 1.0
    o2, S2, _ = kda_reference(q, k, v2, g, beta, conv_w=conv_w, S0=S02)
    keep = [0, 2, 3]
    np.testing.assert_array_equal(o2[..., keep], o[..., keep])
    np.testing.assert_array_equal(S2[..., keep], S[..., keep])
    assert not np.allclose(o2[..., 1], o[..., 1])


def test_heads_are_independent():
    rng = np.random.default_rng(11)
    B, T, H, D = 2, 10, 3, 4
    q, k, v, g, beta, conv_w, S0 = rand_case(rng, B, T, H, D)
    conv_state = rng.standard_normal((B, 3, 3, H * D))
    o, S, _ = kda_reference(q, k, v, g, beta, conv_w=conv_w, conv_state=conv_state, S0=S0)
    heads = [(1, 2), (0, 0), (1, 1)]
    for (b, h), (oh, Sh) in zip(heads, kda_reference_heads(q, k, v, g, beta, heads, conv_w=conv_w,
                                                            conv_state=conv_state, S0=S0)):
        np.testing.assert_array_equal(oh, o[b, :, h])
        np.testing.assert_array_equal(Sh, S[b, h])


# ----------------------------------------- P10: the pages' RMSNorm identity
def kimi_rmsnorm(x, eps=1e-6):
    """KimiRMSNorm with unit weight as printed on "Kimi-K3 atlas -- MoE input
    (decode)": x * rsqrt(mean(x^2) + eps), in float32 there (fp64 here)."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def test_l2_norm_matches_rmsnorm_identity():
    rng = np.random.default_rng(12)
    for d in (16, 128):
        x = rng.standard_normal((50, d)) * np.exp(rng.uniform(-4, 2, size=(50, 1)))
        eps = 1e-6
        np.testing.assert_allclose(l2_normalize(x, d * eps), kimi_rmsnorm(x, eps) / np.sqrt(d),
                                   rtol=1e-13, atol=0)
        # closed form of the norm: |l2(x)| = sqrt(|x|^2 / (|x|^2 + eps)) = 1 - O(eps/|x|^2)
        n2 = (x * x).sum(-1)
        nrm = np.linalg.norm(l2_normalize(x, eps), axis=-1)
        np.testing.assert_allclose(nrm, np.sqrt(n2 / (n2 + eps)), rtol=1e-14, atol=0)
        assert np.all(np.abs(nrm - 1) <= eps / n2)
    np.testing.assert_array_equal(l2_normalize(np.zeros((2, 8))), np.zeros((2, 8)))


# -------------------------------------------------------- P11: convolution
def test_conv_identity_taps_and_impulse():
    rng = np.random.default_rng(13)
    T, C = 11, 5
    x = rng.standard_normal((T, C))
    w_id = np.zeros((C, 4))
    w_id[:, 3] = 1.0
    np.testing.assert_array_equal(short_conv(x, w_id), x)
    w = rng.standard_normal((C, 4))
    imp = np.zeros((T, C))
    imp[4, :] = 1.0
    y = short_conv(imp, w)
    for m in range(4):
        np.testing.assert_array_equal(y[4 + m], w[:, 3 - m])
    assert np.all(y[:4] == 0) and np.all(y[8:] == 0)


def test_conv_matches_numpy_convolve_with_history():
    rng = np.random.default_rng(14)
    T, C = 13, 6
    x = rng.standard_normal((T, C))
    hist = rng.standard_normal((3, C))
    w = rng.standard_normal((C, 4))
    y = short_conv(x, w, hist)
    for c in range(C):
        full = np.convolve(np.concatenate([hist[:, c], x[:, c]]), w[c, ::-1])
        np.testing.assert_allclose(y[:, c], full[3:3 + T], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(conv_tail(x, hist), x[-3:])
    np.testing.assert_array_equal(conv_tail(x[:2], hist), np.concatenate([hist[2:], x[:2]]))


# ------------------------------------------------------------- P12: SiLU
def test_silu_textbook():
    x = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(silu(x), x * expit(x), rtol=1e-14, atol=1e-300)
    assert silu(np.array([0.0]))[0] == 0.0


def test_conv_norm_reference_is_the_mixer_front():
    """The split-out conv/norm stage feeds the recurrence exactly."""
    rng = np.random.default_rng(15)
    q, k, v, g, beta, conv_w, S0 = rand_case(rng, 1, 6, 2, 4)
    qh, kh, vh, tail = conv_norm_reference(q, k, v, conv_w)
    o1, S1, t1 = kda_reference(q, k, v, g, beta, conv_w=conv_w, S0=S0)
    o2, S2, _ = kda_reference(qh, kh, vh, g, beta, conv_w=None, S0=S0, l2norm_qk=False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)
    np.testing.assert_array_equal(tail, t1)


# ------------------------------------------------------- preconditions
def test_decay_preconditions():
    rng = np.random.default_rng(16)
    q, k, v, g, beta, _, _ = rand_case(rng, 1, 3, 1, 2)
    with pytest.raises(ValueError):
        kda_reference(q, k, v, np.abs(g) + 0.1, beta)
    g2 = g.copy()
    g2[0, 0, 0, 0] = np.nan
    with pytest.raises(ValueError):
        kda_reference(q, k, v, g2, beta)


def test_empty_sequence_is_identity():
    rng = np.random.default_rng(17)
    q, k, v, g, beta, conv_w, S0 = rand_case(rng, 1, 0, 2, 4)
    hist = rng.standard_normal((1, 3, 3, 8))
    o, S, tail = kda_reference(q, k, v, g, beta, conv_w=conv_w, conv_state=hist, S0=S0)
    assert o.shape == (1, 0, 2, 4)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_array_equal(tail, hist)


# ------------------------------------------------- output RMSNorm and sigmoid gate
def test_output_gate_norm_hand_example():
    d = json.load(open(os.path.join(GOLDEN, "hand_gate_norm.json")))
    f = lambda x: np.array(x, dtype=np.float64)
    out = output_gate_norm(f(d["o"]), f(d["w"]), f(d["gate"]), eps=d["eps"])
    np.testing.assert_allclose(out, f(d["out"]), rtol=0, atol=1e-14)
    # the same worked numbers in closed form
    np.testing.assert_allclose(out, [3 * np.sqrt(2) / 10, 6 * np.sqrt(2) / 5], rtol=0, atol=1e-14)


def test_rms_norm_closed_forms():
    """Constant and one-hot rows: catches a sum taken for the mean (a factor D) and
    eps outside the root."""
    D, eps = 8, 1e-3
    c = -1.7
    np.testing.assert_allclose(rms_norm(np.full(D, c), eps=eps), np.full(D, c / np.sqrt(c * c + eps)),
                               rtol=1e-15, atol=0)
    x = np.zeros(D)
    x[5] = c
    want = np.zeros(D)
    want[5] = c / np.sqrt(c * c / D + eps)
    np.testing.assert_allclose(rms_norm(x, eps=eps), want, rtol=1e-15, atol=0)
    # with eps = 0 the result has mean square exactly 1 and keeps the direction
    y = rms_norm(np.random.default_rng(3).standard_normal((4, D)), eps=0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14)


def test_rms_norm_and_l2_norm_identity():
    """RMSNorm_eps(x; gain 1) / sqrt(D) = x / sqrt(sum x^2 + D eps): the output norm
    against the (independently pinned) L2 norm of q and k."""
    rng = np.random.default_rng(4)
    for D in (2, 16, 128):
        x = rng.standard_normal((3, 5, D))
        eps = 1e-6
        np.testing.assert_allclose(rms_norm(x, eps=eps) / np.sqrt(D), l2_normalize(x, D * eps),
                                   rtol=1e-13, atol=0)


def test_rms_norm_gain_is_per_channel():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 4))
    w = np.array([0.5, -2.0, 0.0, 3.0])
    np.testing.assert_allclose(rms_norm(x, w), rms_norm(x) * w[None], rtol=1e-15, atol=0)
    assert np.all(rms_norm(x, w)[:, 2] == 0.0)


def test_sigmoid_values():
    np.testing.assert_allclose(sigmoid(np.log([3.0, 1.0 / 3.0, 1.0])), [0.75, 0.25, 0.5],
                               rtol=0, atol=1e-15)
    x = np.linspace(-30, 30, 61)
    np.testing.assert_allclose(sigmoid(x) + sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(sigmoid(x), expit(x), rtol=1e-14, atol=0)


def test_zero_gate_halves_the_output():
    """A gate pre-activation of zero gives exactly half the ungated output (the
    property "MaxText PR 5543" states for its sigmoid gate with zero g_proj)."""
    rng = np.random.default_rng(6)
    o = rng.standard_normal((2, 7, 3, 16))
    w = 1.0 + 0.1 * rng.standard_normal(16)
    np.testing.assert_array_equal(output_gate_norm(o, w, np.zeros_like(o)), 0.5 * output_gate_norm(o, w))
    np.testing.assert_array_equal(output_gate_norm(o, None, np.zeros_like(o)), 0.5 * o)
    np.testing.assert_array_equal(output_gate_norm(o), o)


def test_output_stage_in_the_mixer_is_per_head():
    """The mixer with the output stage equals the plain mixer followed by the stage
    on each head's row; each head normalises over its own D channels only."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, conv_w, S0 = rand_case(rng, B=2, T=11, H=3, D=4)
    gate = rng.standard_normal(q.shape)
    w = rng.standard_normal(4)
    o0, S_plain, _ = kda_reference(q, k, v, g, beta, conv_w=conv_w, S0=S0)
    o1, S1, _ = kda_reference(q, k, v, g, beta, conv_w=conv_w, S0=S0, o_norm_w=w, o_gate=gate)
    np.testing.assert_array_equal(S1, S_plain)  # the state never sees the output stage
    for b in range(2):
        for t in range(11):
            for h in range(3):
                r = o0[b, t, h]
                want = r / np.sqrt(np.mean(r * r) + 1e-6) * w / (1 + np.exp(-gate[b, t, h]))
                np.testing.assert_allclose(o1[b, t, h], want, rtol=1e-13, atol=1e-15)
    # the sampled-head and decode entry points carry the stage the same way
    (oh, _), = kda_reference_heads(q, k, v, g, beta, [(1, 2)], conv_w=conv_w, S0=S0,
                                   o_norm_w=w, o_gate=gate)
    np.testing.assert_allclose(oh, o1[1, :, 2], rtol=1e-13, atol=1e-15)
    od, _, _ = kda_reference_decode_step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0,
                                         conv_w=conv_w, o_norm_w=w, o_gate=gate[:, 0])
    o_first, _, _ = kda_reference(q[:, :1], k[:, :1], v[:, :1], g[:, :1], beta[:, :1],
                                  conv_w=conv_w, S0=S0, o_norm_w=w, o_gate=gate[:, :1])
    np.testing.assert_allclose(od, o_first[:, 0], rtol=1e-13, atol=1e-15)


# ------------------------------------------------- decay and beta from raw projections
def test_gate_activation_hand_example():
    d = json.load(open(os.path.join(GOLDEN, "hand_gate_act.json")))
    f = lambda x: np.array(x, dtype=np.float64)
    g = kda_gate(f(d["f"]), f(d["A_log"]), f(d["dt_bias"]))
    np.testing.assert_allclose(g, f(d["g"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(sigmoid(f(d["b"])), f(d["beta"]), rtol=0, atol=1e-15)


def test_softplus_closed_forms():
    np.testing.assert_allclose(softplus(0.0), np.log(2.0), rtol=1e-15)
    np.testing.assert_allclose(softplus(np.log(np.e - 1.0)), 1.0, rtol=1e-15)
    x = np.linspace(-20, 20, 81)
    np.testing.assert_allclose(softplus(x) - softplus(-x), x, rtol=0, atol=1e-13)
    np.testing.assert_allclose(softplus(x), np.log1p(np.exp(x)), rtol=1e-14)
    assert softplus(800.0) == 800.0 and np.isfinite(softplus(-800.0))


def test_gate_activation_axes():
    """A_log indexes heads and dt_bias indexes channels h*D + c: catches a swapped
    or transposed parameter."""
    H, D = 3, 4
    A_log = np.log(np.array([1.0, 2.0, 4.0]))
    f = np.zeros((2, 5, H, D))
    g = kda_gate(f, A_log, np.zeros(H * D))
    for h in range(H):
        np.testing.assert_allclose(g[..., h, :], -(2.0 ** h) * np.log(2.0), rtol=1e-15)
    bias = np.zeros(H * D)
    bias[2 * D + 1] = np.log(np.e - 1.0)  # head 2, channel 1 only
    g = kda_gate(f, A_log, bias)
    np.testing.assert_allclose(g[..., 2, 1], -4.0, rtol=1e-15)
    np.testing.assert_allclose(g[..., 1, 1], -2.0 * np.log(2.0), rtol=1e-15)
    np.testing.assert_allclose(g[..., 2, 0], -4.0 * np.log(2.0), rtol=1e-15)


def test_gate_activation_is_a_valid_decay():
    rng = np.random.default_rng(8)
    g = kda_gate(4 * rng.standard_normal((2, 50, 3, 8)), rng.uniform(-3, 2, 3),
                 rng.standard_normal(24))
    assert np.all(np.isfinite(g)) and np.all(g <= 0)
    # more negative projections decay less (softplus is increasing)
    f = np.linspace(-5, 5, 11).reshape(1, 11, 1, 1) * np.ones((1, 11, 1, 2))
    g = kda_gate(f, np.zeros(1), np.zeros(2))
    assert np.all(np.diff(g[0, :, 0, 0]) < 0)


def test_raw_projection_inputs_in_the_mixer():
    """The mixer fed raw projections equals the mixer fed the activated values, for
    every entry point."""
    rng = np.random.default_rng(9)
    q, k, v, _, _, conv_w, S0 = rand_case(rng, B=2, T=7, H=3, D=4)
    f = rng.standard_normal(q.shape)
    A_log = rng.uniform(-1, 1, 3)
    dt_bias = 0.5 * rng.standard_normal(12)
    blog = rng.standard_normal(q.shape[:3])
    g = kda_gate(f, A_log, dt_bias)
    beta = sigmoid(blog)
    o0, S0_, _ = kda_reference(q, k, v, g, beta, conv_w=conv_w, S0=S0)
    o1, S1, _ = kda_reference(q, k, v, f, blog, conv_w=conv_w, S0=S0, A_log=A_log,
                              dt_bias=dt_bias, beta_sigmoid=True)
    np.testing.assert_allclose(o1, o0, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S1, S0_, rtol=1e-13, atol=1e-14)
    (oh, Sh), = kda_reference_heads(q, k, v, f, blog, [(1, 2)], conv_w=conv_w, S0=S0,
                                    A_log=A_log, dt_bias=dt_bias, beta_sigmoid=True)
    np.testing.assert_allclose(oh, o0[1, :, 2], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Sh, S0_[1, 2], rtol=1e-13, atol=1e-14)
    od, Sd, _ = kda_reference_decode_step(q[:, 0], k[:, 0], v[:, 0], f[:, 0], blog[:, 0], S0,
                                          conv_w=conv_w, A_log=A_log, dt_bias=dt_bias,
                                          beta_sigmoid=True)
    o_first, S_first, _ = kda_reference(q[:, :1], k[:, :1], v[:, :1], g[:, :1], beta[:, :1],
                                        conv_w=conv_w, S0=S0)
    np.testing.assert_allclose(od, o_first[:, 0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Sd, S_first, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------- packed sequences
def test_packed_equals_reset_in_one_sequence():
    """Packing pinned through the alpha = 0 reset (P4): sequences A and B packed
    give, for B, what one sequence A + B gives when B's first token has g = -1000
    (the state forgets A) and A ends in three zero raw rows (the conv window of
    B's first tokens then sees zeros, B's own empty history)."""
    rng = np.random.default_rng(10)
    La, Lb, H, D = 9, 7, 2, 4
    q, k, v, g, beta, conv_w, _ = rand_case(rng, B=1, T=La + Lb, H=H, D=D)
    for x in (q, k, v):
        x[:, La - 3:La] = 0.0
    S0a = 0.1 * rng.standard_normal((1, H, D, D))
    g_one = g.copy()
    g_one[:, La] = -1000.0
    o_one, S_one, _ = kda_reference(q, k, v, g_one, beta, conv_w=conv_w, S0=S0a)
    S0 = np.concatenate([S0a, np.zeros((1, H, D, D))])
    o_pk, S_pk, tails = kda_reference_packed(q, k, v, g, beta, [0, La, La + Lb], conv_w=conv_w, S0=S0)
    np.testing.assert_allclose(o_pk, o_one, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S_pk[1], S_one[0], rtol=1e-12, atol=1e-13)
    # the tail of each sequence is its own last three raw rows
    HD = H * D
    np.testing.assert_array_equal(tails[1, 0], q[0, La + Lb - 3:].reshape(3, HD))
    np.testing.assert_array_equal(tails[0, 2], v[0, La - 3:La].reshape(3, HD))


def test_packed_empty_and_short_sequences():
    """Empty sequences hand their state and conv history through unchanged; a
    sequence shorter than the conv window mixes its history into the tail."""
    rng = np.random.default_rng(11)
    cu = [0, 0, 5, 5, 6, 6, 8]
    N, H, D = len(cu) - 1, 2, 4
    q, k, v, g, beta, conv_w, _ = rand_case(rng, B=1, T=cu[-1], H=H, D=D)
    S0 = rng.standard_normal((N, H, D, D))
    cs = rng.standard_normal((N, 3, 3, H * D))
    o, S, tails = kda_reference_packed(q, k, v, g, beta, cu, conv_w=conv_w, conv_state=cs, S0=S0)
    for i in (0, 2, 4):
        np.testing.assert_array_equal(S[i], S0[i])
        np.testing.assert_array_equal(tails[i], cs[i])
    # sequence 3 has one token: its tail is the last two history rows, then that token
    np.testing.assert_array_equal(tails[3, 1, :2], cs[3, 1, 1:])
    np.testing.assert_array_equal(tails[3, 1, 2], k[0, 5].reshape(H * D))


def test_packed_equal_lengths_match_batch():
    rng = np.random.default_rng(12)
    B, L, H, D = 3, 6, 2, 4
    q, k, v, g, beta, conv_w, S0 = rand_case(rng, B=B, T=L, H=H, D=D)
    cs = rng.standard_normal((B, 3, 3, H * D))
    ob, Sb, tb = kda_reference(q, k, v, g, beta, conv_w=conv_w, conv_state=cs, S0=S0)
    flat = lambda x: x.reshape(1, B * L, *x.shape[2:])
    op, Sp, tp = kda_reference_packed(flat(q), flat(k), flat(v), flat(g), flat(beta),
                                      [0, L, 2 * L, 3 * L], conv_w=conv_w, conv_state=cs, S0=S0)
    np.testing.assert_allclose(op, flat(ob), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Sp, Sb, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(tp, tb)


def test_packed_rejects_bad_offsets():
    rng = np.random.default_rng(13)
    q, k, v, g, beta, _, _ = rand_case(rng, B=1, T=5, H=1, D=4)
    for cu in ([0, 3, 2, 5], [1, 5], [0, 4], [0, 6]):
        with pytest.raises(ValueError):
            kda_reference_packed(q, k, v, g, beta, cu)


# ------------------------------------------------------------------- backward
def _loss_and_grads(rng, conv, l2, s0=True, B=2, T=7, H=2, D=4, scale=0.7):
    q, k, v, g, beta, conv_w, S0 = rand_case(rng, B=B, T=T, H=H, D=D, s0=s0)
    conv_w = conv_w if conv else None
    cs = rng.standard_normal((B, 3, 3, H * D)) if conv else None
    do = rng.standard_normal(q.shape)
    dST = rng.standard_normal((B, H, D, D))

    def L(q, k, v, g, beta, S0, conv_w, cs):
        o, S, _ = kda_reference(q, k, v, g, beta, conv_w=conv_w, conv_state=cs, S0=S0,
                                scale=scale, l2norm_qk=l2)
        return np.sum(o * do) + np.sum(S * dST)

    gr = kda_reference_backward(q, k, v, g, beta, do, dST, conv_w=conv_w, conv_state=cs, S0=S0,
                                scale=scale, l2norm_qk=l2)
    args = dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, conv_w=conv_w, cs=cs)
    return L, gr, args


@pytest.mark.parametrize("conv,l2", [(True, True), (False, True), (True, False), (False, False)])
def test_backward_matches_finite_differences(conv, l2):
    """Directional derivatives of L = sum(o * do) + sum(S_T * dS_T) by central
    differences of the forward oracle, for every input."""
    rng = np.random.default_rng(20 + 2 * conv + l2)
    L, gr, args = _loss_and_grads(rng, conv, l2)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", S0="dS0", conv_w="dconv_w",
                 cs="dconv_state")
    h = 1e-6
    for n, gn in names.items():
        if args[n] is None:
            assert gr[gn] is None
            continue
        for _ in range(2):
            d = rng.standard_normal(args[n].shape)
            a1, a2 = dict(args), dict(args)
            a1[n] = args[n] + h * d
            a2[n] = args[n] - h * d
            fd = (L(**a1) - L(**a2)) / (2 * h)
            an = np.sum(gr[gn] * d)
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (n, fd, an)


def test_backward_elementwise_tiny():
    """Every element of every gradient on a tiny case, one central difference each."""
    rng = np.random.default_rng(30)
    L, gr, args = _loss_and_grads(rng, True, True, B=1, T=3, H=1, D=2)
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", S0="dS0", conv_w="dconv_w",
                 cs="dconv_state")
    h = 1e-6
    for n, gn in names.items():
        x = args[n]
        for idx in np.ndindex(x.shape):
            a1, a2 = dict(args), dict(args)
            x1, x2 = x.copy(), x.copy()
            x1[idx] += h
            x2[idx] -= h
            a1[n], a2[n] = x1, x2
            fd = (L(**a1) - L(**a2)) / (2 * h)
            assert abs(fd - gr[gn][idx]) <= 1e-7 * max(1.0, abs(fd)), (n, idx, fd, gr[gn][idx])


def test_backward_closed_form_without_writes():
    """beta = 0 and g = 0 (no write, no decay): o_t = scale S0^T q_t, so dq_t = scale
    S0 do_t, dS0 = scale sum_t q_t do_t^T + dS_T, and dk = dv = 0."""
    rng = np.random.default_rng(31)
    B, T, H, D, scale = 1, 5, 2, 3, 0.5
    q, k, v = (rng.standard_normal((B, T, H, D)) for _ in range(3))
    g = np.zeros((B, T, H, D))
    beta = np.zeros((B, T, H))
    S0 = rng.standard_normal((B, H, D, D))
    do = rng.standard_normal((B, T, H, D))
    dST = rng.standard_normal((B, H, D, D))
    gr = kda_reference_backward(q, k, v, g, beta, do, dST, S0=S0, scale=scale, l2norm_qk=False)
    np.testing.assert_allclose(gr["dq"], scale * np.einsum("bhcv,bthv->bthc", S0, do), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(gr["dS0"], scale * np.einsum("bthc,bthv->bhcv", q, do) + dST,
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(gr["dk"], 0.0)
    np.testing.assert_array_equal(gr["dv"], 0.0)


# ------------------------------------------- backward: optional stages, packing
STAGE_SETS = {
    "norm": dict(norm=True),
    "gate": dict(gate=True),
    "norm+gate": dict(norm=True, gate=True),
    "act": dict(act=True),
    "logits": dict(logits=True),
    "all": dict(norm=True, gate=True, act=True, logits=True),
}


def _stage_case(rng, B, T, H, D, norm=False, gate=False, act=False, logits=False):
    """Inputs of a call with the chosen optional stages: with act, g holds the raw
    gate projection; with logits, beta holds logits."""
    q, k, v, g, beta, conv_w, S0 = rand_case(rng, B=B, T=T, H=H, D=D)
    args = dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, conv_w=conv_w,
                cs=rng.standard_normal((B, 3, 3, H * D)))
    kw = {}
    if norm:
        args["o_norm_w"] = 1.0 + 0.3 * rng.standard_normal(D)
    if gate:
        args["o_gate"] = rng.standard_normal((B, T, H, D))
    if act:
        args["g"] = rng.standard_normal((B, T, H, D))
        args["A_log"] = rng.uniform(-1.0, 1.0, H)
        args["dt_bias"] = 0.5 * rng.standard_normal(H * D)
    if logits:
        args["beta"] = rng.standard_normal((B, T, H))
        kw["beta_sigmoid"] = True
    return args, kw


GRAD_OF = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", S0="dS0", conv_w="dconv_w",
               cs="dconv_state", o_norm_w="do_norm_w", o_gate="do_gate", A_log="dA_log",
               dt_bias="ddt_bias")


def _check_fd(rng, L, gr, args, h=1e-6, tol=1e-7, reps=2):
    for n, gn in GRAD_OF.items():
        if args.get(n) is None:
            assert gr.get(gn) is None, n
            continue
        for _ in range(reps):
            d = rng.standard_normal(np.shape(args[n]))
            a1, a2 = dict(args), dict(args)
            a1[n] = args[n] + h * d
            a2[n] = args[n] - h * d
            fd = (L(**a1) - L(**a2)) / (2 * h)
            an = np.sum(gr[gn] * d)
            assert abs(fd - an) <= tol * max(1.0, abs(fd)), (n, fd, an)


@pytest.mark.parametrize("stages", list(STAGE_SETS))
def test_backward_stages_match_finite_differences(stages):
    """The optional stages in the backward: directional derivatives of
    L = sum(o * do) + sum(S_T * dS_T) by central differences of the forward oracle
    with the stages on, for every input, the stage parameters included."""
    rng = np.random.default_rng(40 + list(STAGE_SETS).index(stages))
    B, T, H, D, scale = 2, 6, 2, 4, 0.8
    args, kw = _stage_case(rng, B, T, H, D, **STAGE_SETS[stages])
    do = rng.standard_normal((B, T, H, D))
    dST = rng.standard_normal((B, H, D, D))

    def L(q, k, v, g, beta, S0, conv_w, cs, o_norm_w=None, o_gate=None, A_log=None, dt_bias=None):
        o, S, _ = kda_reference(q, k, v, g, beta, conv_w=conv_w, conv_state=cs, S0=S0, scale=scale,
                                o_norm_w=o_norm_w, o_gate=o_gate, A_log=A_log, dt_bias=dt_bias, **kw)
        return np.sum(o * do) + np.sum(S * dST)

    a = dict(args)
    gr = kda_reference_backward(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("g"), a.pop("beta"), do, dST,
                                conv_w=a.pop("conv_w"), conv_state=a.pop("cs"), S0=a.pop("S0"),
                                scale=scale, **a, **kw)
    _check_fd(rng, L, gr, args)


def test_output_stage_backward_elementwise():
    """Every element of the output stage's three gradients, one central difference
    each of output_gate_norm (norm and gate on, eps 1e-6)."""
    rng = np.random.default_rng(50)
    o = rng.standard_normal((3, 5))
    w = 1.0 + 0.3 * rng.standard_normal(5)
    z = rng.standard_normal((3, 5))
    dy = rng.standard_normal((3, 5))
    do, dw, dz = output_gate_norm_backward(o, dy, w, z)
    L = lambda o, w, z: np.sum(output_gate_norm(o, w, z) * dy)
    h = 1e-6
    for name, x, gx in (("o", o, do), ("w", w, dw), ("z", z, dz)):
        for idx in np.ndindex(x.shape):
            x1, x2 = x.copy(), x.copy()
            x1[idx] += h
            x2[idx] -= h
            a1 = dict(o=o, w=w, z=z); a2 = dict(o=o, w=w, z=z)
            a1[name], a2[name] = x1, x2
            fd = (L(**a1) - L(**a2)) / (2 * h)
            assert abs(fd - gx[idx]) <= 1e-8 * max(1.0, abs(fd)), (name, idx, fd, gx[idx])


def test_output_stage_backward_closed_forms():
    """A zero gate halves everything that flows through it (sigmoid(0) = 1/2, slope
    1/4); the norm's input gradient is orthogonal to its input at eps = 0 (the
    normalised row does not change when o is scaled)."""
    rng = np.random.default_rng(51)
    o = rng.standard_normal((4, 6))
    dy = rng.standard_normal((4, 6))
    do, dw, dz = output_gate_norm_backward(o, dy, None, np.zeros((4, 6)))
    np.testing.assert_allclose(do, dy / 2, rtol=1e-15, atol=0)
    np.testing.assert_allclose(dz, dy * o / 4, rtol=1e-15, atol=0)
    assert dw is None
    w = rng.standard_normal(6)
    do, dw, dz = output_gate_norm_backward(o, dy, w, None, eps=0.0)
    np.testing.assert_allclose(np.sum(do * o, axis=-1), 0.0, atol=1e-12)
    n = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
    np.testing.assert_allclose(dw, np.sum(dy * n, axis=0), rtol=1e-13)
    assert dz is None


def test_activation_backward_closed_form():
    """With A_log = 0 and dt_bias = 0 the decay is g = -softplus(f), whose derivative
    is -sigmoid(f): the gate projection's gradient is the decay's times that, and
    dA_log is sum(dg * g); beta logits scale dbeta by sigmoid'(b)."""
    rng = np.random.default_rng(52)
    B, T, H, D = 1, 4, 2, 3
    q, k, v, f = (rng.standard_normal((B, T, H, D)) for _ in range(4))
    b = rng.standard_normal((B, T, H))
    do = rng.standard_normal((B, T, H, D))
    ref = kda_reference_backward(q, k, v, -softplus(f), sigmoid(b), do)
    gr = kda_reference_backward(q, k, v, f, b, do, A_log=np.zeros(H), dt_bias=np.zeros(H * D),
                                beta_sigmoid=True)
    np.testing.assert_allclose(gr["dg"], -ref["dg"] * sigmoid(f), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(gr["dA_log"], np.sum(ref["dg"] * -softplus(f), axis=(0, 1, 3)),
                               rtol=1e-13)
    np.testing.assert_allclose(gr["ddt_bias"], np.sum(gr["dg"], axis=(0, 1)).reshape(-1), rtol=1e-13)
    np.testing.assert_allclose(gr["dbeta"], ref["dbeta"] * sigmoid(b) * (1 - sigmoid(b)), rtol=1e-13,
                               atol=1e-15)
    for n in ("dq", "dk", "dv", "dS0"):
        np.testing.assert_allclose(gr[n], ref[n], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("stages", ["none", "all"])
def test_backward_packed_matches_finite_differences(stages):
    """Packed sequences (an empty one, one shorter than the conv window, longer
    ones): directional derivatives of the packed forward oracle for every input."""
    rng = np.random.default_rng(60 + (stages == "all"))
    cu = [0, 5, 5, 7, 13]
    N, T, H, D, scale = 4, 13, 2, 4, 0.9
    args, kw = _stage_case(rng, 1, T, H, D, **(STAGE_SETS["all"] if stages == "all" else {}))
    args["S0"] = 0.1 * rng.standard_normal((N, H, D, D))
    args["cs"] = rng.standard_normal((N, 3, 3, H * D))
    do = rng.standard_normal((1, T, H, D))
    dST = rng.standard_normal((N, H, D, D))

    def L(q, k, v, g, beta, S0, conv_w, cs, o_norm_w=None, o_gate=None, A_log=None, dt_bias=None):
        o, S, _ = kda_reference_packed(q, k, v, g, beta, cu, conv_w=conv_w, conv_state=cs, S0=S0,
                                       scale=scale, o_norm_w=o_norm_w, o_gate=o_gate, A_log=A_log,
                                       dt_bias=dt_bias, **kw)
        return np.sum(o * do) + np.sum(S * dST)

    a = dict(args)
    gr = kda_reference_backward_packed(a.pop("q"), a.pop("k"), a.pop("v"), a.pop("g"), a.pop("beta"),
                                       cu, do, dST, conv_w=a.pop("conv_w"), conv_state=a.pop("cs"),
                                       S0=a.pop("S0"), scale=scale, **a, **kw)
    _check_fd(rng, L, gr, args)
    # the empty sequence passes its end-state gradient straight through
    np.testing.assert_array_equal(gr["dS0"][1], dST[1])
    np.testing.assert_array_equal(gr["dconv_state"][1], 0.0)
