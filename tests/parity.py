"""Shared parity metrics and tolerances for the GPU-vs-oracle tests.

Tolerances (written here, used by every parity test):
  output  : max |o_gpu - o_ref| <= 5e-3 * RMS(o_ref)   (o stored fp32)
            bf16 storage adds its own rounding, at most 2^-8 |o_ref| for
            round-to-nearest-even, so a bf16-stored o is held to
            |o_gpu - o_ref| <= 5e-3 * RMS(o_ref) + 2^-8 |o_ref| elementwise
  state   : ||S_gpu - S_ref||_F / ||S_ref||_F <= 1e-3 over the compared states
            A state stored in bf16 (8 significant bits: round to nearest even
            moves x by at most 2^-8 |x|) against the exact state: 1e-3 + 2^-8.
            Two chains that each round their state to bf16 at the same points
            (the GPU's and the oracle's of the bf16 state mode), where one
            chain's value before rounding is within 1e-3 of the other's:
            1e-3 + 2 * 2^-8, because ||RNE(a) - RNE(b)|| <= ||a - b|| +
            2^-8 (||a|| + ||b||).
  decode o from such a pair of bf16 states: o = scale S'^T w with
            S' = Diag(alpha) S and w = q - beta (q.k) k is linear in the state,
            and each entry of the two states may differ by the two roundings,
            2^-7 |S_cj|, so elementwise
            |o_gpu - o_ref| <= 5e-3 RMS(o_ref) + scale 2^-7 sum_c |S'_cj| |w_c|.
  gate    : |g_gpu - g_ref| <= 1e-5 |g_ref| + 1e-30,  |beta_gpu - beta_ref| <= 1e-6
"""
from __future__ import annotations

import numpy as np
import torch

O_TOL = 5e-3
S_TOL = 1e-3
BF16_U = 2.0 ** -8
S_TOL_BF16 = S_TOL + 2.0 ** -8
S_TOL_BF16_CHAINS = S_TOL + 2.0 ** -7


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def out_err(o_gpu, o_ref) -> float:
    """max-abs error of o as a multiple of RMS(o_ref)."""
    o_gpu, o_ref = to64(o_gpu), to64(o_ref)
    rms = float(np.sqrt(np.mean(o_ref ** 2)))
    return float(np.max(np.abs(o_gpu - o_ref))) / max(rms, 1e-300)


def out_err_bf16(o_gpu, o_ref) -> float:
    """max over elements of |o_gpu - o_ref| / (5e-3 RMS + 2^-8 |o_ref|); <= 1 passes."""
    o_gpu, o_ref = to64(o_gpu), to64(o_ref)
    rms = float(np.sqrt(np.mean(o_ref ** 2)))
    return float(np.max(np.abs(o_gpu - o_ref) / (O_TOL * rms + BF16_U * np.abs(o_ref))))


def out_err_bf16_state(o_gpu, o_ref, S_prev, q, k, beta, alpha, scale=1.0) -> float:
    """max over elements of |o_gpu - o_ref| / (5e-3 RMS(o_ref) + the bf16-state
    term above) for one decode step of N sequences: S_prev [N,H,dk,dv] the
    oracle's bf16 state before the step, q, k [N,H,dk], beta [N,H], alpha
    [N,H,dk] the step's decay; <= 1 passes."""
    o_gpu, o_ref = to64(o_gpu), to64(o_ref)
    S, q, k, beta, alpha = (to64(x) for x in (S_prev, q, k, beta, alpha))
    rms = float(np.sqrt(np.mean(o_ref ** 2)))
    w = q - (beta * np.sum(q * k, -1))[..., None] * k
    term = abs(scale) * 2.0 ** -7 * np.einsum("nhcj,nhc->nhj", np.abs(alpha[..., None] * S),
                                              np.abs(w))
    return float(np.max(np.abs(o_gpu - o_ref) / (O_TOL * rms + term)))


def state_err(S_gpu, S_ref) -> float:
    S_gpu, S_ref = to64(S_gpu), to64(S_ref)
    return float(np.linalg.norm(S_gpu - S_ref) / max(np.linalg.norm(S_ref), 1e-300))


def assert_out(o_gpu, o_ref, what=""):
    e = out_err(o_gpu, o_ref)
    assert e <= O_TOL, "%s output max-abs err %.3e x RMS > %.1e" % (what, e, O_TOL)
    return e


def assert_out_bf16(o_gpu, o_ref, what=""):
    e = out_err_bf16(o_gpu, o_ref)
    assert e <= 1.0, "%s bf16 output err ratio %.3f > 1" % (what, e)
    return e


def assert_state(S_gpu, S_ref, what="", tol=S_TOL):
    e = state_err(S_gpu, S_ref)
    assert e <= tol, "%s state rel-Frobenius err %.3e > %.3e" % (what, e, tol)
    return e
