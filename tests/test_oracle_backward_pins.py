"""Pins of the fp64 oracle's backward (oracle.prefill_backward), CPU only.

The backward is the gradient of the token recurrence S_t = (I - b_t k_t k_t^T)
Diag(exp(g_t)) S_{t-1} + b_t k_t v_t^T, o_t = scale S_t^T q_t (the KDA core of
the Kimi K3 artifact audit's code pages) with respect to q, k, v, g, beta and
the initial state, for the loss sum(d_o * o) + sum(dS_final * S_final).  It is
checked against three things outside itself: central differences of the
forward oracle, torch autograd through an independent plain torch recurrence,
and the closed form of the beta = 0, g = 0 case (a constant state).
"""
import numpy as np
import pytest
import torch

import oracle




def _draw(lengths, H, dk, dv, seed):
    r = np.random.default_rng(seed)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q = r.standard_normal((T, H, dk))
    k = r.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((T, H, dv))
    g = -0.5 * r.random((T, H, dk))
    beta = r.random((T, H))
    S0 = 0.3 * r.standard_normal((len(lengths), H, dk, dv))
    d_o = r.standard_normal((T, H, dv))
    dSf = r.standard_normal((len(lengths), H, dk, dv))
    return q, k, v, g, beta, cu, S0, d_o, dSf


def _loss(inputs, cu, scale, d_o, dSf):
    q, k, v, g, beta, S0 = inputs
    o, Sf = oracle.prefill(q, k, v, g, beta, cu, S0, scale=scale)
    return float(np.sum(o * d_o) + np.sum(Sf * dSf))


def test_backward_matches_central_differences():
    """Every gradient element of a tiny varlen case (an empty sequence, one
    token, several tokens) against a central difference of the forward
    oracle (step 1e-6): catches a dropped term, a wrong sign or index."""
    lengths = [3, 0, 1, 4]
    q, k, v, g, beta, cu, S0, d_o, dSf = _draw(lengths, H=2, dk=3, dv=2, seed=5)
    scale = 0.8
    grads = oracle.prefill_backward(q, k, v, g, beta, cu, S0, scale=scale, d_o=d_o, dS_final=dSf)
    names = ["q", "k", "v", "g", "beta", "S0"]
    inputs = [q, k, v, g, beta, S0]
    h = 1e-6
    for i, name in enumerate(names):
        num = np.zeros_like(inputs[i])
        for idx in np.ndindex(inputs[i].shape):
            plus = [a.copy() for a in inputs]
            minus = [a.copy() for a in inputs]
            plus[i][idx] += h
            minus[i][idx] -= h
            num[idx] = (_loss(plus, cu, scale, d_o, dSf) - _loss(minus, cu, scale, d_o, dSf)) / (2 * h)
        got = grads[i]
        err = np.max(np.abs(got - num)) / max(1.0, np.max(np.abs(num)))
        assert err < 1e-7, (name, err)
    # the empty sequence passes the state gradient straight through
    assert np.array_equal(grads[5][1], dSf[1])


def _torch_recurrence(q, k, v, g, beta, cu, S0, scale):
    outs, finals = [], []
    for n in range(len(cu) - 1):
        S = S0[n]
        for t in range(int(cu[n]), int(cu[n + 1])):
            S = torch.exp(g[t])[..., None] * S                           # [H, dk, dv]
            e = v[t] - torch.einsum("hc,hcj->hj", k[t], S)
            S = S + beta[t][:, None, None] * k[t][..., None] * e[:, None, :]
            outs.append(scale * torch.einsum("hc,hcj->hj", q[t], S))
        finals.append(S)
    return torch.stack(outs), torch.stack(finals)


def test_backward_matches_torch_autograd():
    """Sequences longer than the oracle's 64-token recompute segments (70,
    130), an empty and a one-token sequence, 2 heads, against torch autograd
    (fp64) through a plain torch recurrence."""
    lengths = [70, 0, 130, 1]
    H, dk, dv = 2, 8, 6
    q, k, v, g, beta, cu, S0, d_o, dSf = _draw(lengths, H, dk, dv, seed=9)
    scale = 0.6
    grads = oracle.prefill_backward(q, k, v, g, beta, cu, S0, scale=scale, d_o=d_o, dS_final=dSf)
    ts = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v, g, beta, S0)]
    o, Sf = _torch_recurrence(*ts[:5], cu, ts[5], scale)
    loss = (o * torch.tensor(d_o)).sum() + (Sf * torch.tensor(dSf)).sum()
    loss.backward()
    for name, got, t in zip(["q", "k", "v", "g", "beta", "S0"], grads, ts):
        ref = t.grad.numpy()
        err = np.max(np.abs(got - ref)) / max(1.0, np.max(np.abs(ref)))
        assert err < 1e-11, (name, err)


def test_backward_constant_state_closed_form():
    """beta = 0 and g = 0 keep S_t = S0, so o_t = scale S0^T q_t and, with
    D_t = dS_final + scale sum_{t' >= t} q_t' do_t'^T the gradient reaching
    token t: dq_t = scale S0 do_t, dS0 = D_0, dv = dk = 0,
    dbeta_t = k_t^T D_t (v_t - S0^T k_t), dg_t[c] = sum_j D_t[c, j] S0[c, j]."""
    T, H, dk, dv = 9, 2, 5, 4
    q, k, v, g, beta, cu, S0, d_o, dSf = _draw([T], H, dk, dv, seed=13)
    g[:] = 0.0
    beta[:] = 0.0
    scale = 1.3
    dq, dkk, dvv, dg, db, dS0 = oracle.prefill_backward(q, k, v, g, beta, cu, S0, scale=scale,
                                                        d_o=d_o, dS_final=dSf)
    S = S0[0]
    D = dSf[0].copy()
    for t in range(T - 1, -1, -1):
        D = D + scale * np.einsum("hc,hj->hcj", q[t], d_o[t])
        assert np.allclose(dq[t], scale * np.einsum("hcj,hj->hc", S, d_o[t]), atol=1e-12)
        e = v[t] - np.einsum("hc,hcj->hj", k[t], S)
        assert np.allclose(db[t], np.einsum("hc,hcj,hj->h", k[t], D, e), atol=1e-12)
        assert np.allclose(dg[t], np.sum(D * S, axis=2), atol=1e-12)
    assert np.allclose(dS0[0], D, atol=1e-12)
    assert np.all(dkk == 0) and np.all(dvv == 0)


@pytest.mark.parametrize("per_channel", [False, True])
def test_gate_backward_matches_central_differences(per_channel):
    """oracle.gate_backward against central differences of oracle.gate for
    the loss sum(dg * g) + sum(dbeta * beta), every element of x, b, A_log
    (per head or per channel) and dt_bias."""
    r = np.random.default_rng(21)
    T, H, d = 3, 2, 3
    x = r.standard_normal((T, H, d)) * 3
    b = r.standard_normal((T, H)) * 2
    A = r.uniform(-0.75, 1.0, (H, d) if per_channel else (H,))
    dt = r.normal(-1.0, 1.0, (H, d))
    dg = r.standard_normal((T, H, d))
    dbeta = r.standard_normal((T, H))
    got = oracle.gate_backward(x, b, A, dt, dg, dbeta)

    def loss(xx, bb, AA, dd):
        g, be = oracle.gate(xx, bb, AA, dd)
        return float(np.sum(g * dg) + np.sum(be * dbeta))
    ins = [x, b, A, dt]
    h = 1e-6
    for i, name in enumerate(["x", "b", "A_log", "dt_bias"]):
        num = np.zeros_like(ins[i])
        for idx in np.ndindex(ins[i].shape):
            plus = [a.copy() for a in ins]
            minus = [a.copy() for a in ins]
            plus[i][idx] += h
            minus[i][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        err = np.max(np.abs(got[i] - num)) / max(1.0, np.max(np.abs(num)))
        assert err < 1e-7, (name, err)


def test_gate_backward_closed_form_at_zero():
    """x + dt_bias = 0 and b = 0: sigmoid = 1/2, so dx = -exp(A_log) dg / 2,
    db = dbeta / 4 and dA_log = -ln 2 exp(A_log) sum(dg)."""
    T, H, d = 4, 3, 2
    A = np.array([0.0, 0.5, -0.75])
    dt = np.arange(H * d, dtype=np.float64).reshape(H, d) * 0.3 - 0.5
    x = np.broadcast_to(-dt, (T, H, d)).copy()
    dg = np.random.default_rng(4).standard_normal((T, H, d))
    dbeta = np.random.default_rng(5).standard_normal((T, H))
    dx, db, dA, ddt = oracle.gate_backward(x, np.zeros((T, H)), A, dt, dg, dbeta)
    assert np.allclose(dx, -np.exp(A)[None, :, None] * dg / 2, atol=1e-15)
    assert np.allclose(db, dbeta / 4, atol=1e-15)
    assert np.allclose(dA, -np.log(2.0) * np.exp(A) * dg.sum(axis=(0, 2)), atol=1e-13)
    assert np.allclose(ddt, dx.sum(axis=0), atol=1e-14)
