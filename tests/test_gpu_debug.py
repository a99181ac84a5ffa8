"""GPU: the KDA_DEBUG=1 validation mode.

With KDA_DEBUG=1 each call scans its inputs before its kernels (g <= 0, beta
in [0, 1], q/k/v and states finite, gate logits not NaN) and returns
KDA_ERR_DOMAIN without launching them, and scans its outputs afterwards
(KDA_ERR_NONFINITE for any NaN or inf).  The bad inputs below are finite
buffers of the right sizes holding out-of-domain values: the kernels would
only compute wrong numbers from them, never access memory out of bounds.
"""
import pytest
import torch

from synth import draw_decode_params, draw_decode_step, draw_prefill
from tests.gpu_util import DEV, need_gpu, oracle_gate_f32, say
import gated_delta_rule_58_amd as kda

pytestmark = pytest.mark.gpu

DOMAIN, NONFINITE = 8, 9


def _prefill_inputs():
    dr = draw_prefill([100, 37], H=2, dtype=torch.bfloat16, init_state=True, seed=81)
    g, beta = oracle_gate_f32(dr)
    return dr, g.to(DEV), beta.to(DEV)


def _prefill(dr, g, beta, o):
    cu_h = dr.cu_seqlens
    return kda.chunk_prefill(dr.q.to(DEV), dr.k.to(DEV), dr.v.to(DEV), g, beta, cu_h.to(DEV),
                             dr.initial_state.to(DEV), cu_seqlens_host=cu_h, out=o)


def test_debug_refuses_out_of_domain_prefill_inputs(monkeypatch):
    """NaN beta, beta = 2.5 (an unsquashed logit, the PR review's divergence)
    and a positive g are each refused before launch: o keeps its sentinel."""
    need_gpu()
    say("KDA_DEBUG prefill refusals")
    dr, g, beta = _prefill_inputs()
    monkeypatch.setenv("KDA_DEBUG", "1")
    o = torch.full((137, 2, 128), 7.0, device=DEV)
    _prefill(dr, g, beta, o)                   # in domain: accepted
    torch.cuda.synchronize()
    good = o.clone()
    assert torch.isfinite(good).all()
    def nan_beta(g, b):
        b[5, 1] = float("nan")

    def big_beta(g, b):
        b[17] = 2.5
        b[90] = 2.5

    def positive_g(g, b):
        g[3] = 0.25
    cases = [("NaN beta", nan_beta, "beta outside [0, 1] (1 of"),
             ("beta 2.5", big_beta, "beta outside [0, 1] (4 of"),
             ("g > 0", positive_g, "g not <= 0 (256 of")]
    for name, spoil, text in cases:
        gg, bb = g.clone(), beta.clone()
        spoil(gg, bb)
        o.fill_(7.0)
        with pytest.raises(kda.KdaError) as ei:
            _prefill(dr, gg, bb, o)
        assert ei.value.status == DOMAIN, str(ei.value)
        assert text in str(ei.value) and "nothing was launched" in str(ei.value), str(ei.value)
        torch.cuda.synchronize()
        assert torch.all(o == 7.0), name
    # the same good inputs still give the same result in debug mode
    _prefill(dr, g, beta, o)
    torch.cuda.synchronize()
    assert torch.equal(o, good)


def test_debug_off_lets_bad_beta_through(monkeypatch):
    """Without the mode the library does not scan: beta = 2.5 runs and its
    damage stays silent (finite but wrong here)."""
    need_gpu()
    say("KDA_DEBUG off")
    monkeypatch.delenv("KDA_DEBUG", raising=False)
    dr, g, beta = _prefill_inputs()
    bb = beta.clone()
    bb[17] = 2.5
    o = torch.empty((137, 2, 128), device=DEV)
    _prefill(dr, g, bb, o)          # returns KDA_OK
    torch.cuda.synchronize()


def test_debug_flags_non_finite_outputs(monkeypatch):
    """In-domain inputs whose outputs overflow: a decode state of 3e38 (finite,
    but beyond what the step can hold) with all-positive unit q and k makes
    k^T S overflow, so o and the state become infinite; the call reports
    KDA_ERR_NONFINITE after writing them."""
    need_gpu()
    say("KDA_DEBUG non-finite outputs")
    monkeypatch.setenv("KDA_DEBUG", "1")
    N, H = 3, 2
    A_log, dt_bias, S0 = draw_decode_params(N, H, seed=82)
    st = draw_decode_step(N, H, 0, seed=82, dtype=torch.bfloat16)
    g, beta = kda.gate(st.x.to(DEV), st.b.to(DEV), A_log.to(DEV), dt_bias.to(DEV))
    state = torch.full((N, H, 128, 128), 3e38, device=DEV)
    unit = torch.full((N, H, 128), 128 ** -0.5, device=DEV).to(torch.bfloat16)
    with pytest.raises(kda.KdaError) as ei:
        kda.recurrent_decode(unit, unit, st.v.to(DEV), g, beta, state, o_dtype=torch.float32)
    assert ei.value.status == NONFINITE, str(ei.value)
    assert "o not finite" in str(ei.value), str(ei.value)
    # a sane state passes both scans
    state = S0.to(DEV).contiguous()
    kda.recurrent_decode(st.q.to(DEV), st.k.to(DEV), st.v.to(DEV), g, beta, state)
    torch.cuda.synchronize()


def test_debug_gated_decode_and_gate_logits(monkeypatch):
    """NaN gate logits are refused by the gated decode and by kda_gate; an
    infinite logit is the gate's limit and passes (g = -inf, alpha = 0)."""
    need_gpu()
    say("KDA_DEBUG gated decode and gate")
    monkeypatch.setenv("KDA_DEBUG", "1")
    N, H = 4, 2
    A_log, dt_bias, S0 = draw_decode_params(N, H, seed=83)
    st = draw_decode_step(N, H, 0, seed=83, dtype=torch.bfloat16)
    x = st.x.clone()
    x[1, 0, 5] = float("nan")
    pool = S0.to(DEV).contiguous()
    before = pool.clone()
    with pytest.raises(kda.KdaError) as ei:
        kda.recurrent_decode_gated(st.q.to(DEV), st.k.to(DEV), st.v.to(DEV), x.to(DEV),
                                   st.b.to(DEV), A_log.to(DEV), dt_bias.to(DEV), pool)
    assert ei.value.status == DOMAIN and "x NaN (1 of" in str(ei.value), str(ei.value)
    torch.cuda.synchronize()
    assert torch.equal(pool, before)
    with pytest.raises(kda.KdaError) as ei:
        kda.gate(x.to(DEV), st.b.to(DEV), A_log.to(DEV), dt_bias.to(DEV))
    assert ei.value.status == DOMAIN, str(ei.value)
    x[1, 0, 5] = float("inf")
    g, beta = kda.gate(x.to(DEV), st.b.to(DEV), A_log.to(DEV), dt_bias.to(DEV))
    torch.cuda.synchronize()
    assert g[1, 0, 5].item() == float("-inf")
