"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test names the mistake it is there to catch.  The recurrence under test is
the per-channel gated delta rule S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1}
+ b_t k_t v_t^T, o_t = S_t^T q_t; the gate is g = -exp(A_log) softplus(x +
dt_bias), beta = sigmoid(b).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.chunked import prefill_chunked
from synth import draw_prefill, orthonormal_keys_pm_quarter

HERE = os.path.dirname(os.path.abspath(__file__))
rng = np.random.default_rng


def _unit(a):
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def _rand_case(T, H, dk, dv, seed, g_scale=0.3):
    r = rng(seed)
    q = _unit(r.standard_normal((T, H, dk)))
    k = _unit(r.standard_normal((T, H, dk)))
    v = r.standard_normal((T, H, dv))
    g = -g_scale * r.random((T, H, dk))
    beta = r.random((T, H))
    return q, k, v, g, beta


# ---------------------------------------------------------------- gate pins

def test_gate_golden_exp_alog_table():
    """Audit page §5.1 prints exp(A_log) beside A_log; with softplus(z)=1 the
    gate returns -exp(A_log).  Catches exp missing/negated or a sign error."""
    rows = []
    with open(os.path.join(HERE, "golden", "alog_exp_stats.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, a, ea = line.split()
                rows.append((name, float(a), float(ea)))
    assert len(rows) == 5
    A_log = np.array([r[1] for r in rows])
    H = len(rows)
    z1 = math.log(math.e - 1.0)                      # softplus(z1) == 1
    x = np.full((1, H, 2), z1)
    dt = np.zeros((H, 2))
    g, _ = oracle.gate(x, np.zeros((1, H)), A_log, dt)
    for h, (_, a, ea) in enumerate(rows):
        # printed to 4 decimals: half an ulp of the table plus the input's rounding
        tol = 0.5e-4 + ea * 0.5e-4 + 1e-12
        assert abs(-g[0, h, 0] - ea) <= tol, (a, ea, g[0, h, 0])
        assert abs(g[0, h, 0] - g[0, h, 1]) == 0.0


def test_gate_closed_forms():
    """softplus(0)=ln2, sigmoid(0)=1/2, both asymptotes; catches a dropped
    log1p term, a wrong sigmoid sign, dt_bias indexed by the wrong axis."""
    H, d = 3, 4
    A_log = np.array([0.0, 0.5, -0.75])
    dt = np.arange(H * d, dtype=np.float64).reshape(H, d) * 0.1 - 0.6
    x = -dt[None].copy()                             # x + dt_bias == 0 everywhere
    g, beta = oracle.gate(x, np.zeros((1, H)), A_log, dt)
    assert np.allclose(g[0], -np.exp(A_log)[:, None] * math.log(2.0), rtol=0, atol=1e-15)
    assert np.all(beta == 0.5)
    big = 40.0
    g, beta = oracle.gate(np.full((1, H, d), big) - dt[None], np.full((1, H), big), A_log, dt)
    assert np.allclose(g[0], -np.exp(A_log)[:, None] * big, rtol=1e-15)
    assert np.all(np.abs(beta - 1.0) < 1e-15)
    g, beta = oracle.gate(np.full((1, H, d), -big) - dt[None], np.full((1, H), -big), A_log, dt)
    assert np.allclose(g[0], -np.exp(A_log)[:, None] * math.exp(-big), rtol=1e-12)
    assert np.allclose(beta, math.exp(-big), rtol=1e-12)


def test_gate_matches_library_softplus_and_expit():
    """Random logits against numpy.logaddexp and scipy.special.expit."""
    from scipy.special import expit
    r = rng(7)
    T, H, d = 5, 4, 8
    x = r.standard_normal((T, H, d)) * 6
    b = r.standard_normal((T, H)) * 6
    A_log = r.uniform(-0.75, 2.5, H)
    dt = r.normal(-4.6, 1.2, (H, d))
    g, beta = oracle.gate(x, b, A_log, dt)
    ref = -np.exp(A_log)[None, :, None] * np.logaddexp(0.0, x + dt[None])
    assert np.allclose(g, ref, rtol=1e-14, atol=1e-300)
    assert np.allclose(beta, expit(b), rtol=1e-14)
    assert np.all(g <= 0)


def test_gate_per_channel_alog():
    """A_log given per (head, channel), [H, d] (the variant the audit page's
    §5.2 leaves open, taken only when passed explicitly): channel c of every
    head gets the per-head gate with A_log[:, c], against numpy.logaddexp,
    and a constant row reproduces the per-head result exactly.  H != d with
    distinct values, so a transposed or per-head-only index fails."""
    r = rng(11)
    T, H, d = 4, 3, 5
    x = r.standard_normal((T, H, d)) * 4
    b = r.standard_normal((T, H))
    dt = r.normal(-4.6, 1.2, (H, d))
    A = r.uniform(-0.75, 1.5, (H, d))
    g, beta = oracle.gate(x, b, A, dt)
    ref = -np.exp(A)[None] * np.logaddexp(0.0, x + dt[None])
    assert np.allclose(g, ref, rtol=1e-14, atol=1e-300)
    for c in range(d):
        gc, bc = oracle.gate(x, b, A[:, c].copy(), dt)
        assert np.array_equal(g[:, :, c], gc[:, :, c])
        assert np.array_equal(beta, bc)
    a_head = r.uniform(-0.75, 1.5, H)
    g_pc, _ = oracle.gate(x, b, np.repeat(a_head[:, None], d, axis=1), dt)
    g_ph, _ = oracle.gate(x, b, a_head, dt)
    assert np.array_equal(g_pc, g_ph)
    with pytest.raises(ValueError):
        oracle.gate(x, b, np.zeros(d), dt)       # a bare [d] is not reshaped


# ------------------------------------------------------------ recurrence pins

def test_single_token_closed_form():
    """T=1 from a non-zero state: S1 = (I - b k k^T) Diag(a) S0 + b k v^T,
    o = S1^T q (matrix form).  Catches decay/update order swapped, readout of
    S0 instead of S1, o = S q instead of S^T q, a transposed decay."""
    dk, dv = 8, 6
    r = rng(1)
    q, k, v, g, beta = _rand_case(1, 1, dk, dv, 2)
    S0 = r.standard_normal((1, 1, dk, dv))
    o, S1 = oracle.prefill(q, k, v, g, beta, [0, 1], S0, scale=0.7)
    a, kk, bb = np.exp(g[0, 0]), k[0, 0], beta[0, 0]
    ref = (np.eye(dk) - bb * np.outer(kk, kk)) @ np.diag(a) @ S0[0, 0] + bb * np.outer(kk, v[0, 0])
    assert np.allclose(S1[0, 0], ref, rtol=0, atol=1e-14)
    assert np.allclose(o[0, 0], 0.7 * ref.T @ q[0, 0], rtol=0, atol=1e-14)
    # from zero state: S1 = b k v^T and o = b (q.k) v
    o, S1 = oracle.prefill(q, k, v, g, beta, [0, 1], None)
    assert np.allclose(S1[0, 0], bb * np.outer(kk, v[0, 0]), atol=1e-15)
    assert np.allclose(o[0, 0], bb * (q[0, 0] @ kk) * v[0, 0], atol=1e-15)


def test_matrix_form_brute_force():
    """T=20 steps of the matrix form of the recurrence on a tiny state."""
    T, dk, dv = 20, 5, 3
    q, k, v, g, beta = _rand_case(T, 2, dk, dv, 3, g_scale=1.0)
    S0 = rng(4).standard_normal((1, 2, dk, dv))
    o, Sf = oracle.prefill(q, k, v, g, beta, [0, T], S0)
    for h in range(2):
        S = S0[0, h]
        for t in range(T):
            M = (np.eye(dk) - beta[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(np.exp(g[t, h]))
            S = M @ S + beta[t, h] * np.outer(k[t, h], v[t, h])
            assert np.allclose(o[t, h], S.T @ q[t, h], atol=1e-13)
        assert np.allclose(Sf[0, h], S, atol=1e-13)


def test_beta_zero_is_pure_per_channel_decay():
    """beta=0: S_T = Diag(e^{sum g}) S0, o_t = S0^T (e^{sum_{s<=t} g} * q_t).
    Catches decay applied per value channel (columns) instead of key channel."""
    T, dk, dv = 9, 6, 4
    q, k, v, g, _ = _rand_case(T, 1, dk, dv, 5, g_scale=0.8)
    S0 = rng(6).standard_normal((1, 1, dk, dv))
    o, Sf = oracle.prefill(q, k, v, g, np.zeros((T, 1)), [0, T], S0)
    G = np.cumsum(g[:, 0], axis=0)
    assert np.allclose(Sf[0, 0], np.exp(G[-1])[:, None] * S0[0, 0], rtol=1e-14, atol=0)
    for t in range(T):
        assert np.allclose(o[t, 0], S0[0, 0].T @ (np.exp(G[t]) * q[t, 0]), rtol=1e-13, atol=1e-15)


def test_exact_delta_rule_recall_orthonormal_keys():
    """alpha=1, beta=1, orthonormal keys written in turn into S0=0:
    S = sum_i k_i v_i^T and querying k_i returns v_i.  Catches a sign error in
    the delta correction or a missing beta."""
    m, d = 40, 128
    K = orthonormal_keys_pm_quarter(m, d).double().numpy()
    r = rng(8)
    V = r.standard_normal((m, d))
    q = np.zeros((m, 1, d))
    o, Sf = oracle.prefill(q, K[:, None], V[:, None], np.zeros((m, 1, d)), np.ones((m, 1)),
                           [0, m])
    assert np.allclose(Sf[0, 0], K.T @ V, atol=1e-13)
    assert np.allclose(K @ Sf[0, 0], V, atol=1e-13)   # query k_i -> v_i
    # rewriting key 0 with a new value replaces it and leaves the others
    o2, S2 = oracle.prefill(K[:1, None], K[:1, None], V[5:6, None], np.zeros((1, 1, d)),
                            np.ones((1, 1)), [0, 1], Sf)
    assert np.allclose(o2[0, 0], V[5], atol=1e-13)
    assert np.allclose(K[1:] @ S2[0, 0], V[1:], atol=1e-13)


def test_recall_with_any_decay_and_state():
    """beta=1, |k_t|=1, q_t=k_t gives o_t = v_t exactly for any alpha and S0."""
    T, d = 30, 16
    _, k, v, g, _ = _rand_case(T, 2, d, d, 9, g_scale=2.0)
    S0 = rng(10).standard_normal((1, 2, d, d))
    o, _ = oracle.prefill(k, k, v, g, np.ones((T, 2)), [0, T], S0)
    assert np.allclose(o, v, atol=1e-12)


def test_contraction_and_divergence_control():
    """|k|=1, beta in [0,1]: ||S_t||_2 <= ||S_{t-1}||_2 + beta ||v||.  Negative
    control: beta taken as raw logits > 2 makes the state grow without bound
    (the divergence the Model-Optimizer review reports for an unsquashed beta)."""
    T, d = 200, 8
    q, k, v, _, beta = _rand_case(T, 1, d, d, 11)
    g = np.zeros((T, 1, d))
    S = np.zeros((1, 1, d, d))
    for t in range(T):
        _, S_new = oracle.prefill(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                  beta[t:t + 1], [0, 1], S)
        lhs = np.linalg.norm(S_new[0, 0], 2)
        assert lhs <= np.linalg.norm(S[0, 0], 2) + beta[t, 0] * np.linalg.norm(v[t, 0]) + 1e-12
        S = S_new
    # raw logits instead of sigmoid(logits): |1 - beta| > 1 along k
    k_rep = np.broadcast_to(k[:2], (T // 2, 2, 1, d)).reshape(T, 1, d)
    _, S_bad = oracle.prefill(q, k_rep, v, g, np.full((T, 1), 2.5), [0, T])
    assert not np.isfinite(np.linalg.norm(S_bad)) or np.linalg.norm(S_bad) > 1e12


@pytest.mark.parametrize("C", [1, 2, 3, 5, 7, 16, 64, 10 ** 6])
def test_chunked_form_equals_recurrence(C):
    """The independent chunked fp64 form agrees with the token-by-token
    oracle for every chunk size, on varlen input with an initial state."""
    lengths = [13, 0, 40, 7]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, dk, dv = int(cu[-1]), 2, 8, 4
    q, k, v, g, beta = _rand_case(T, H, dk, dv, 12, g_scale=1.5)
    S0 = rng(13).standard_normal((len(lengths), H, dk, dv))
    o_r, S_r = oracle.prefill(q, k, v, g, beta, cu, S0, scale=0.5)
    o_c, S_c = prefill_chunked(q, k, v, g, beta, cu, S0, scale=0.5, C=C)
    assert np.max(np.abs(o_r - o_c)) <= 1e-12 * max(1.0, np.max(np.abs(o_r)))
    assert np.max(np.abs(S_r - S_c)) <= 1e-12 * max(1.0, np.max(np.abs(S_r)))
    assert np.array_equal(S_r[:, :][1], S0[1])      # zero-length sequence keeps its state


def test_heads_and_value_columns_are_independent():
    """Permuting heads permutes results; a subset of value columns gives the
    same columns of o and S.  Catches cross-head or cross-column mixing."""
    T, H, dk, dv = 17, 3, 8, 6
    q, k, v, g, beta = _rand_case(T, H, dk, dv, 14)
    S0 = rng(15).standard_normal((1, H, dk, dv))
    o, S = oracle.prefill(q, k, v, g, beta, [0, T], S0)
    p = [2, 0, 1]
    o_p, S_p = oracle.prefill(q[:, p], k[:, p], v[:, p], g[:, p], beta[:, p], [0, T], S0[:, p])
    assert np.array_equal(o_p, o[:, p]) and np.array_equal(S_p, S[:, p])
    cols = [1, 4]
    o_c, S_c = oracle.prefill(q, k, v[:, :, cols], g, beta, [0, T], S0[:, :, :, cols])
    assert np.allclose(o_c, o[:, :, cols], atol=1e-14)
    assert np.allclose(S_c, S[:, :, :, cols], atol=1e-14)


def test_split_prefill_and_decode_resume():
    """Prefill [0,T1) then [T1,T) from its final state equals one prefill;
    prefill then a decode step equals prefill over T+1."""
    T, T1, H, d = 50, 21, 2, 8
    q, k, v, g, beta = _rand_case(T + 1, H, d, d, 16)
    o, S = oracle.prefill(q[:T], k[:T], v[:T], g[:T], beta[:T], [0, T])
    o1, S1 = oracle.prefill(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], [0, T1])
    o2, S2 = oracle.prefill(q[T1:T], k[T1:T], v[T1:T], g[T1:T], beta[T1:T], [0, T - T1], S1)
    assert np.allclose(np.concatenate([o1, o2]), o, atol=1e-13)
    assert np.allclose(S2, S, atol=1e-13)
    od, Sd = oracle.decode(q[T:T + 1], k[T:T + 1], v[T:T + 1], g[T:T + 1], beta[T:T + 1], S)
    of, Sf = oracle.prefill(q, k, v, g, beta, [0, T + 1])
    assert np.allclose(od[0], of[T], atol=1e-13)
    assert np.allclose(Sd, Sf, atol=1e-13)


def test_decode_equals_per_sequence_prefill():
    N, H, d = 5, 3, 8
    q, k, v, g, beta = _rand_case(N, H, d, d, 17)
    S0 = rng(18).standard_normal((N, H, d, d))
    od, Sd = oracle.decode(q, k, v, g, beta, S0, scale=0.3)
    cu = np.arange(N + 1, dtype=np.int32)
    op, Sp = oracle.prefill(q, k, v, g, beta, cu, S0, scale=0.3)
    assert np.array_equal(od, op) and np.array_equal(Sd, Sp)


def test_synthetic_recipe_statistics():
    """The generator's draws follow the stated recipe (not method arithmetic):
    unit-norm q/k rows, A_log in [-0.75, 0.5], dt_bias mean near -4.6."""
    dr = draw_prefill([300, 212], H=4, dtype=torch.float32, init_state=True, seed=5)
    assert torch.allclose(torch.linalg.vector_norm(dr.q, dim=-1), torch.ones(512, 4), atol=1e-5)
    assert float(dr.A_log.min()) >= -0.75 and float(dr.A_log.max()) <= 0.5
    assert abs(float(dr.dt_bias.mean()) + 4.6) < 0.15
    assert abs(float(dr.initial_state.std()) - 0.02) < 1e-3
    assert dr.cu_seqlens.tolist() == [0, 300, 512]


# ---- the layer prologue (short causal conv, SiLU, q/k L2 norm)

def _prologue_inputs(T, H, d=8, seed=3):
    rng = np.random.default_rng(seed)
    xs = [rng.standard_normal((T, H, d)) for _ in range(3)]
    ws = [rng.standard_normal((H * d, 4)) for _ in range(3)]
    return xs, ws


def test_prologue_impulse_response():
    """A one-hot input at token t0, channel c returns the conv weights in
    reverse tap order on tokens t0..t0+3 (v has no norm; no activation)."""
    from oracle.prologue import shortconv_l2norm
    T, H, d = 10, 2, 8
    xs, ws = _prologue_inputs(T, H, d)
    xv = np.zeros((T, H, d))
    xv[4, 1, 3] = 1.0
    c = 1 * d + 3
    _, _, yv, _ = shortconv_l2norm(xs[0], xs[1], xv, ws[0], ws[1], ws[2], [0, T], H, d,
                                   activation=None)
    got = yv.reshape(T, H * d)[:, c]
    want = np.zeros(T)
    for i in range(4):
        want[4 + i] = ws[2][c, 3 - i]
    assert np.array_equal(got, want)
    assert np.count_nonzero(yv) == 4


def test_prologue_conv_matches_numpy_convolve():
    """Per channel the conv is numpy.convolve(x, w reversed) cut to the
    sequence (zero state), for every channel of every packed sequence."""
    from oracle.prologue import shortconv_l2norm
    T, H, d = 23, 3, 8
    xs, ws = _prologue_inputs(T, H, d, seed=5)
    cu = [0, 9, 9, 11, 23]
    _, _, yv, _ = shortconv_l2norm(xs[0], xs[1], xs[2], ws[0], ws[1], ws[2], cu, H, d,
                                   activation=None)
    x2 = xs[2].reshape(T, H * d)
    y2 = yv.reshape(T, H * d)
    for n in range(len(cu) - 1):
        b, e = cu[n], cu[n + 1]
        if e == b:
            continue
        for c in range(H * d):
            ref = np.convolve(x2[b:e, c], ws[2][c, ::-1])[:e - b]
            assert np.allclose(y2[b:e, c], ref, rtol=0, atol=1e-13)


def test_prologue_norm_and_silu():
    """q and k rows have unit norm (eps = 0) and point along the activated conv
    output; SiLU matches x * expit(x) and its closed forms."""
    from scipy.special import expit
    from oracle.prologue import shortconv_l2norm, silu, causal_conv
    T, H, d = 7, 2, 8
    xs, ws = _prologue_inputs(T, H, d, seed=8)
    yq, yk, yv, _ = shortconv_l2norm(*xs, *ws, [0, T], H, d, activation="silu", eps=0.0)
    for y in (yq, yk):
        assert np.allclose(np.linalg.norm(y, axis=2), 1.0, atol=1e-14)
    raw = silu(causal_conv(xs[0].reshape(T, H * d), ws[0], np.zeros((3, H * d)))).reshape(T, H, d)
    cos = np.sum(raw * yq, axis=2) / np.linalg.norm(raw, axis=2)
    assert np.allclose(cos, 1.0, atol=1e-14)
    z = np.linspace(-30, 30, 61)
    assert np.allclose(silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert silu(np.array([0.0]))[0] == 0.0
    assert abs(silu(np.array([50.0]))[0] - 50.0) < 1e-15 * 50
    assert abs(silu(np.array([-50.0]))[0]) < 1e-19


def test_prologue_split_with_state_equals_one_shot():
    """Running tokens [0, T1) and then [T1, T) with the conv state handed on
    equals one run over [0, T); one-token steps too; a sequence shorter than 3
    tokens carries the older state entries on."""
    from oracle.prologue import shortconv_l2norm
    T, H, d = 13, 2, 8
    xs, ws = _prologue_inputs(T, H, d, seed=11)
    full = shortconv_l2norm(*xs, *ws, [0, T], H, d)
    T1 = 5
    a = shortconv_l2norm(*[x[:T1] for x in xs], *ws, [0, T1], H, d)
    st = a[3]
    outs = [a[:3]]
    for t in range(T1, T):                      # one-token steps
        r = shortconv_l2norm(*[x[t:t + 1] for x in xs], *ws, [0, 1], H, d, state=st)
        st = r[3]
        outs.append(r[:3])
    for z in range(3):
        got = np.concatenate([o[z] for o in outs], axis=0)
        assert np.allclose(got, full[z], rtol=0, atol=1e-13)
    assert np.allclose(st, full[3], rtol=0, atol=0)
    # a 2-token sequence keeps the last state entry
    r = shortconv_l2norm(*[x[:2] for x in xs], *ws, [0, 2], H, d, state=full[3])
    assert np.array_equal(r[3][0, :, 0], full[3][0, :, 2])
