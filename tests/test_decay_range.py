"""Decay range of the chunked prefill (CPU).

The prefill's prep kernel keeps the cumulative log-decay gamma in log2 units
and forms every decay factor from references inside a 16-row block: with
m = the block's mid row, E_r = 2^(gamma_r - gamma_m) and F_r = 2^(gamma_m -
gamma_r) span at most 8 tokens of one channel's decay, and every other factor
is E or F times a per-(block, channel) constant <= 1.  For fp32 those spans
must stay below 2^126.  The artifact audit's KDA parameter table (§5.1) prints
A_log up to 2.4661 and dt_bias up to 0.1792: with exp(2.4661) = 11.78 a single
token with a gate logit of a few units decays by tens of log2 units, so spans
of 8 tokens reach far past 126.

The kernel floors the per-token log2 decay at -DECAY_FLOOR_LOG2 = -15.5 before
the cumulative sum, so every 8-token span is at most 124 (126 is the limit).
This file checks:
  * a plain fp32 numpy model of the factor construction overflows at the
    printed extremes without the floor and stays finite with it;
  * the floor's effect on the recurrence itself, through the fp64 oracle:
    o and the final state move by far less than the stated tolerances
    (5e-3 x RMS(o), 1e-3 relative Frobenius), because a floored factor
    differs from the exact one by at most 2^-15.5 = 2.2e-5.
"""
import numpy as np
import torch

import oracle
from synth import draw_prefill

DECAY_FLOOR_LOG2 = 15.5
LN2 = np.log(2.0)
A_LOG_MAX = 2.4661      # artifact audit §5.1, the A_log row's maximum
DT_BIAS_MAX = 0.1792    # artifact audit §5.1, the dt_bias row's maximum


def _extreme_g_log2(T, C, seed):
    """Per-token log2 decay [T, C] at the printed extremes (fp64 gate)."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((T, 1, C))
    b = r.standard_normal((T, 1))
    g, _ = oracle.gate(x, b, np.array([A_LOG_MAX]), np.full((1, C), DT_BIAS_MAX))
    return g[:, 0, :] / LN2


def _factor_model(g_log2, k, q, floor):
    """The prep kernel's decay factors of one 64-token chunk, in fp32.

    Returns the arrays the kernel forms (every one must be finite for the
    chunk's image to be finite)."""
    f32 = np.float32
    g = g_log2.astype(f32)
    if floor:
        g = np.where(g < -DECAY_FLOOR_LOG2, f32(-DECAY_FLOOR_LOG2), g)
    gam = np.cumsum(g, axis=0, dtype=f32)            # gamma_r, [64, C]
    ex2 = lambda a: np.exp2(a.astype(f32)).astype(f32)
    out = {}
    gC = gam[63]
    for i in range(4):
        rows = slice(16 * i, 16 * i + 16)
        m = 16 * i + 7
        gm = gam[m]
        gb = gam[16 * i - 1] if i > 0 else np.zeros_like(gm)
        E = ex2(gam[rows] - gm)
        F = ex2(gm - gam[rows])
        ke, qe, kf = k[rows] * E, q[rows] * E, k[rows] * F
        out["E%d" % i], out["F%d" % i] = E, F
        out["Ke%d" % i] = ke * ex2(gm)                  # K e^gamma
        out["Qe%d" % i] = qe * ex2(gm)                  # Q e^gamma
        out["Kd%d" % i] = kf * ex2(gC - gm)             # K e^(gamma_C - gamma)
        out["L%d" % i] = ke * ex2(gm - gb)              # left factor k 2^(gamma_r - gamma_b)
        for j in range(i):                              # right factors of tiles (i, j)
            gmj = gam[16 * j + 7]
            rj = slice(16 * j, 16 * j + 16)
            out["R%d%d" % (i, j)] = k[rj] * ex2(gmj - gam[rj]) * ex2(gb - gmj)
        # diagonal tile entries s <= r: sum_c (k E)_r (k F)_s
        prod = ke[:, None, :] * kf[None, :, :]
        low = np.tril(np.ones((16, 16), bool))
        out["A%d" % i] = prod.sum(-1)[low]
    return out


def test_factor_model_overflows_without_floor_and_stays_finite_with_it():
    r = np.random.default_rng(7)
    C = 128
    over = 0
    for s in range(8):
        g = _extreme_g_log2(64, C, seed=100 + s)
        k = r.standard_normal((64, C)).astype(np.float32)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        q = r.standard_normal((64, C)).astype(np.float32)
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        with np.errstate(over="ignore", invalid="ignore", under="ignore"):
            raw = _factor_model(g, k, q, floor=False)
            fl = _factor_model(g, k, q, floor=True)
        over += sum(not np.isfinite(a).all() for a in raw.values())
        assert all(np.isfinite(a).all() for a in fl.values()), s
        # with the floor every 8-token span, and so every E and F, is in fp32 range
        for i in range(4):
            assert np.abs(np.log2(fl["E%d" % i])).max() <= 126.0
    assert over > 0, "the model should overflow without the floor at the printed extremes"


def test_floor_effect_on_the_recurrence_is_far_below_tolerance():
    """oracle(g) against oracle(max(g, -15.5 ln 2)) with two heads at the
    printed extremes (every channel of head 0, half the channels of head 1)
    beside a head at the printed median A_log."""
    for seed in (1, 2):
        dr = draw_prefill([300, 77], H=3, dtype=torch.bfloat16, init_state=True, seed=seed)
        A = torch.tensor([A_LOG_MAX, A_LOG_MAX, -0.15])
        dt = dr.dt_bias.clone()
        dt[0] = DT_BIAS_MAX
        dt[1, :64] = DT_BIAS_MAX
        g, beta = oracle.gate(dr.x, dr.b, A, dt)
        floored = g < -DECAY_FLOOR_LOG2 * LN2
        assert floored.mean() > 0.1          # the floor is active on these heads
        o, S = oracle.prefill(dr.q, dr.k, dr.v, g, beta, dr.cu_seqlens, dr.initial_state)
        gf = np.where(floored, -DECAY_FLOOR_LOG2 * LN2, g)
        o2, S2 = oracle.prefill(dr.q, dr.k, dr.v, gf, beta, dr.cu_seqlens, dr.initial_state)
        rms = np.sqrt(np.mean(o ** 2))
        eo = np.abs(o - o2).max() / rms
        es = np.linalg.norm(S - S2) / np.linalg.norm(S)
        # measured: about 4e-5 x RMS and 2e-6; the stated bounds are 5e-3 and 1e-3
        assert eo < 2e-4 and es < 2e-5, (eo, es)
