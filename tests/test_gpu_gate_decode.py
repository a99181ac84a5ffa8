"""GPU parity of kda_gate and kda_recurrent_decode against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from synth import (CONFIGS, draw_alog_per_channel, draw_decode_params, draw_decode_step,
                   draw_prefill)
from tests.gpu_util import DEV, need_gpu, oracle_gate_f32, say
from tests.parity import (O_TOL, S_TOL_BF16_CHAINS, assert_out, assert_state, out_err,
                          out_err_bf16_state, state_err, to64)
import gated_delta_rule_58_amd as kda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16])
def test_gate_parity(xdt):
    need_gpu()
    say("gate parity", xdt)
    dr = draw_prefill([777], H=96, dtype=torch.bfloat16, seed=21)
    x = dr.x.to(xdt)
    b = dr.b.to(xdt)
    g, beta = kda.gate(x.to(DEV), b.to(DEV), dr.A_log.to(DEV), dr.dt_bias.to(DEV))
    torch.cuda.synchronize()
    g_ref, b_ref = oracle.gate(x, b, dr.A_log, dr.dt_bias)
    g_gpu, b_gpu = to64(g), to64(beta)
    assert np.all(np.abs(g_gpu - g_ref) <= 1e-5 * np.abs(g_ref) + 1e-30)
    assert np.max(np.abs(b_gpu - b_ref)) <= 1e-6
    assert np.all(g_gpu <= 0)


def test_gate_writes_stop_at_the_last_token():
    """A partial last token run (777 = 24 * 32 + 9) writes g and beta for its
    9 tokens only: the memory after them keeps its contents."""
    need_gpu()
    say("gate bounds")
    dr = draw_prefill([777], H=96, dtype=torch.bfloat16, seed=29)
    T, H, d = dr.x.shape
    n, nb = T * H * d, T * H
    sentinel = 7.0
    gbuf = torch.full((n + 2 * H * d,), sentinel, dtype=torch.float32, device=DEV)
    bbuf = torch.full((nb + 2 * H,), sentinel, dtype=torch.float32, device=DEV)
    g, beta = kda.gate(dr.x.to(DEV), dr.b.to(DEV), dr.A_log.to(DEV), dr.dt_bias.to(DEV),
                       g_out=gbuf[:n].view(T, H, d), beta_out=bbuf[:nb].view(T, H))
    torch.cuda.synchronize()
    assert torch.all(gbuf[n:] == sentinel) and torch.all(bbuf[nb:] == sentinel)
    g_ref, b_ref = oracle.gate(dr.x, dr.b, dr.A_log, dr.dt_bias)
    assert np.all(np.abs(to64(g) - g_ref) <= 1e-5 * np.abs(g_ref) + 1e-30)
    assert np.max(np.abs(to64(beta) - b_ref)) <= 1e-6


def test_gate_extreme_logits():
    """Large |x + dt_bias| and |b| stay finite and match the asymptotes."""
    need_gpu()
    say("gate extremes")
    H, d = 4, 128
    x = torch.linspace(-80, 80, 3 * H * d).reshape(3, H, d)
    b = torch.tensor([[-200.0, -20.0, 20.0, 200.0]] * 3)
    A_log = torch.tensor([-0.75, 0.0, 0.5, 2.4661])
    dt = torch.zeros(H, d)
    g, beta = kda.gate(x.to(DEV), b.to(DEV), A_log.to(DEV), dt.to(DEV))
    torch.cuda.synchronize()
    g_ref, b_ref = oracle.gate(x, b, A_log, dt)
    g_gpu = to64(g)
    assert np.all(np.isfinite(g_gpu)) and np.all(np.isfinite(to64(beta)))
    assert np.all(np.abs(g_gpu - g_ref) <= 1e-5 * np.abs(g_ref) + 1e-37)
    assert np.max(np.abs(to64(beta) - b_ref)) <= 1e-6


@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16])
def test_gate_per_channel_alog(xdt):
    """A_log per (head, channel), [H, d]: kda_gate against the oracle gate, and
    far from the per-head gate (so a per-head read of A_log would fail)."""
    need_gpu()
    say("gate per-channel A_log", xdt)
    dr = draw_prefill([300], H=7, dtype=torch.bfloat16, seed=23)
    A = draw_alog_per_channel(7, seed=23)
    x, b = dr.x.to(xdt), dr.b.to(xdt)
    g, beta = kda.gate(x.to(DEV), b.to(DEV), A.to(DEV), dr.dt_bias.to(DEV))
    torch.cuda.synchronize()
    g_ref, b_ref = oracle.gate(x, b, A, dr.dt_bias)
    g_gpu = to64(g)
    assert np.all(np.abs(g_gpu - g_ref) <= 1e-5 * np.abs(g_ref) + 1e-30)
    assert np.max(np.abs(to64(beta) - b_ref)) <= 1e-6
    g_ph, _ = oracle.gate(x, b, dr.A_log, dr.dt_bias)
    assert np.max(np.abs(g_gpu - g_ph)) > 0.1 * np.max(np.abs(g_ph))


@pytest.mark.parametrize("qdt,odt", [(torch.float32, torch.float32),
                                     (torch.bfloat16, torch.float32),
                                     (torch.bfloat16, torch.bfloat16)])
def test_decode_parity_small(qdt, odt):
    need_gpu()
    say("decode small", qdt, odt)
    N, H = 7, 5
    A_log, dt_bias, S0 = draw_decode_params(N, H, seed=31)
    S0 = S0 * 10  # a state of order one, so the update matters
    S_gpu = S0.to(DEV).contiguous()
    S_ref = to64(S0)
    for step in range(6):
        st = draw_decode_step(N, H, step, seed=31, dtype=qdt)
        g, beta = oracle.gate(st.x, st.b, A_log, dt_bias)
        g32, b32 = torch.from_numpy(g).float(), torch.from_numpy(beta).float()
        o = kda.recurrent_decode(st.q.to(DEV), st.k.to(DEV), st.v.to(DEV), g32.to(DEV),
                                 b32.to(DEV), S_gpu, scale=0.8, o_dtype=odt)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.decode(st.q, st.k, st.v, g32, b32, S_ref, scale=0.8)
        if odt == torch.float32:
            assert_out(o, o_ref, "decode step %d" % step)
        else:
            from tests.parity import assert_out_bf16
            assert_out_bf16(o, o_ref, "decode step %d" % step)
        assert_state(S_gpu, S_ref, "decode step %d" % step)


def test_decode_full_config_sampled():
    """256 sequences x 96 heads x 64 steps, fp32 state [256,96,128,128] updated
    in place, HIP gate -> HIP decode; sampled (sequence, head) pairs checked
    against oracle gate -> oracle decode on every step."""
    need_gpu()
    c = CONFIGS[4]
    N, H, steps, seed = c["N"], c["H"], c["steps"], c["seed"]
    say("decode full config N=%d H=%d steps=%d" % (N, H, steps))
    A_log, dt_bias, S0 = draw_decode_params(N, H, seed=seed, device=DEV)
    rng = np.random.default_rng(4)
    pairs = [(int(a), int(b)) for a, b in zip(rng.integers(0, N, 24), rng.integers(0, H, 24))]
    ni = torch.tensor([p[0] for p in pairs])
    hi = torch.tensor([p[1] for p in pairs])
    S_ref = to64(S0[ni, hi])                             # [24, 128, 128]
    state = S0
    for step in range(steps):
        st = draw_decode_step(N, H, step, seed=seed, dtype=c["dtype"], device=DEV)
        g, beta = kda.gate(st.x, st.b, A_log, dt_bias)
        o = kda.recurrent_decode(st.q, st.k, st.v, g, beta, state, o_dtype=torch.float32)
        # oracle gate per sampled pair (each pair has its own head parameters)
        x_s = st.x[ni, hi].cpu()[None]                  # [1, 24, 128] as tokens x "heads"
        b_s = st.b[ni, hi].cpu()[None]
        gr, br = oracle.gate(x_s, b_s, A_log[hi].cpu(), dt_bias[hi].cpu())
        o_ref, S_ref = oracle.decode(st.q[ni, hi].cpu()[None], st.k[ni, hi].cpu()[None],
                                     st.v[ni, hi].cpu()[None], gr, br, S_ref[None])
        S_ref = S_ref[0]
        assert_out(o[ni, hi], o_ref[0], "decode step %d" % step)
    torch.cuda.synchronize()
    assert_state(state[ni, hi], S_ref, "decode after %d steps" % steps)


def test_decode_full_config_every_pair():
    """The same workload (256 sequences x 96 heads x 64 steps, HIP gate -> HIP
    decode, fp32 state in place) with every (sequence, head) pair checked
    against oracle gate -> oracle decode: o on every step against its RMS over
    all pairs, the whole state after the last step by its Frobenius error."""
    need_gpu()
    c = CONFIGS[4]
    N, H, steps, seed = c["N"], c["H"], c["steps"], c["seed"]
    seqs = list(range(N))
    say("decode full config N=%d H=%d steps=%d, every pair" % (N, H, steps))
    A_log, dt_bias, S0 = draw_decode_params(N, H, seed=seed, device=DEV)
    ni = torch.tensor([n for n in seqs for _ in range(H)])
    hi = torch.tensor([h for _ in seqs for h in range(H)])
    S_ref = to64(S0[ni, hi])                             # [pairs, 128, 128]
    state = S0
    o_max, o_ss, o_n = 0.0, 0.0, 0
    for step in range(steps):
        st = draw_decode_step(N, H, step, seed=seed, dtype=c["dtype"], device=DEV)
        g, beta = kda.gate(st.x, st.b, A_log, dt_bias)
        o = kda.recurrent_decode(st.q, st.k, st.v, g, beta, state, o_dtype=torch.float32)
        gr, br = oracle.gate(st.x[ni, hi].cpu()[None], st.b[ni, hi].cpu()[None],
                             A_log[hi].cpu(), dt_bias[hi].cpu())
        o_ref, S_ref = oracle.decode(st.q[ni, hi].cpu()[None], st.k[ni, hi].cpu()[None],
                                     st.v[ni, hi].cpu()[None], gr, br, S_ref[None])
        S_ref = S_ref[0]
        o_max = max(o_max, float(np.max(np.abs(to64(o[ni, hi]) - o_ref[0]))))
        o_ss += float(np.sum(o_ref ** 2))
        o_n += o_ref.size
    torch.cuda.synchronize()
    eo = o_max / max(np.sqrt(o_ss / o_n), 1e-300)
    say("  o err / RMS over %d steps %.3e (bound 5e-3)" % (steps, eo))
    assert eo <= O_TOL, "decode o max-abs err %.3e x RMS" % eo
    es = assert_state(state[ni, hi], S_ref, "decode after %d steps" % steps)
    say("  state rel-F after %d steps %.3e (bound 1e-3)" % (steps, es))


def test_decode_deterministic():
    need_gpu()
    say("decode determinism")
    N, H = 32, 96
    A_log, dt_bias, S0 = draw_decode_params(N, H, seed=5, device=DEV)
    st = draw_decode_step(N, H, 0, seed=5, device=DEV)
    g, beta = kda.gate(st.x, st.b, A_log, dt_bias)
    S1, S2 = S0.clone(), S0.clone()
    o1 = kda.recurrent_decode(st.q, st.k, st.v, g, beta, S1)
    o2 = kda.recurrent_decode(st.q, st.k, st.v, g, beta, S2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16])
def test_decode_gated_matches_gate_then_decode(xdt):
    """kda_recurrent_decode_gated over an fp32 pool with slot n = sequence n
    agrees with kda_gate followed by kda_recurrent_decode (the same gate
    arithmetic, thread layout and summation order) to fp32 rounding, and both
    match the oracle gate followed by the oracle step."""
    need_gpu()
    say("gated decode vs gate + decode", xdt)
    N, H = 9, 5
    A_log, dt_bias, S0 = draw_decode_params(N, H, seed=41)
    S0 = S0 * 10
    S1 = S0.to(DEV).contiguous()
    S2 = S1.clone()
    S_ref = to64(S0)
    Ad, dbd = A_log.to(DEV), dt_bias.to(DEV)
    for step in range(4):
        st = draw_decode_step(N, H, step, seed=41, dtype=torch.bfloat16)
        x, b = st.x.to(xdt), st.b.to(xdt)
        q, k, v = st.q.to(DEV), st.k.to(DEV), st.v.to(DEV)
        g, beta = kda.gate(x.to(DEV), b.to(DEV), Ad, dbd)
        o1 = kda.recurrent_decode(q, k, v, g, beta, S1, scale=0.8, o_dtype=torch.float32)
        o2 = kda.recurrent_decode_gated(q, k, v, x.to(DEV), b.to(DEV), Ad, dbd, S2, scale=0.8,
                                        o_dtype=torch.float32)
        torch.cuda.synchronize()
        assert out_err(o2, o1) <= 1e-5 and state_err(S2, S1) <= 1e-6
        gr, br = oracle.gate(x.float(), b.float(), A_log, dt_bias)
        o_ref, S_ref = oracle.decode(st.q, st.k, st.v, gr, br, S_ref, scale=0.8)
        assert_out(o2, o_ref, "gated decode step %d" % step)
        assert_state(S2, S_ref, "gated decode step %d" % step)


@pytest.mark.parametrize("sdt", [torch.float32, torch.bfloat16])
def test_decode_gated_per_channel_alog(sdt):
    """Gated decode with A_log per (head, channel), [H, d], over an fp32 or
    bf16 pool: 4 steps against the oracle gate and step (the oracle's state
    rounded to bf16 after each step in bf16 mode)."""
    need_gpu()
    say("gated decode per-channel A_log", sdt)
    N, H = 6, 4
    A_log, dt_bias, S0 = draw_decode_params(N, H, seed=47)
    A = draw_alog_per_channel(H, seed=47)
    S0 = (S0 * 10).to(sdt)
    S = S0.to(DEV).contiguous()
    S_ref = to64(S0)
    for step in range(4):
        st = draw_decode_step(N, H, step, seed=47, dtype=torch.bfloat16)
        o = kda.recurrent_decode_gated(st.q.to(DEV), st.k.to(DEV), st.v.to(DEV), st.x.to(DEV),
                                       st.b.to(DEV), A.to(DEV), dt_bias.to(DEV), S, scale=0.9,
                                       o_dtype=torch.float32)
        torch.cuda.synchronize()
        gr, br = oracle.gate(st.x, st.b, A, dt_bias)
        o_ref, S_ref = oracle.decode(st.q, st.k, st.v, gr, br, S_ref, scale=0.9)
        if sdt == torch.bfloat16:
            S_ref = _bf16_round(S_ref)
        assert_out(o, o_ref, "per-channel A_log decode step %d" % step)
    assert_state(S, S_ref, "per-channel A_log decode")


def _bf16_round(S):
    """The bf16 state mode's rounding of an fp64 state: nearest even (torch)."""
    return to64(torch.from_numpy(np.ascontiguousarray(S)).to(torch.bfloat16))


@pytest.mark.parametrize("sdt", [torch.float32, torch.bfloat16])
def test_decode_gated_state_pool(sdt):
    """A pool of 7 slots; 4 sequences mapped to slots [5, -1, 0, 3] (-1 is a
    padding entry); 6 steps against the oracle.  The padding sequence's o is
    zero, the slots no sequence uses stay bit for bit unchanged, and in bf16
    mode the oracle's state is rounded to bf16 after every step, which is what
    that mode computes."""
    need_gpu()
    say("gated decode state pool", sdt)
    N, H, NS = 4, 3, 7
    idx = [5, -1, 0, 3]
    live = [n for n in range(N) if idx[n] >= 0]
    A_log, dt_bias, pool0 = draw_decode_params(NS, H, seed=43)
    pool0 = (pool0 * 10).to(sdt)
    pool = pool0.to(DEV).contiguous()
    S_ref = {n: to64(pool0[idx[n]]) for n in live}
    ind = torch.tensor(idx, dtype=torch.int32, device=DEV)
    for step in range(6):
        st = draw_decode_step(N, H, step, seed=43, dtype=torch.bfloat16)
        o = kda.recurrent_decode_gated(st.q.to(DEV), st.k.to(DEV), st.v.to(DEV), st.x.to(DEV),
                                       st.b.to(DEV), A_log.to(DEV), dt_bias.to(DEV), pool,
                                       state_indices=ind, o_dtype=torch.float32)
        torch.cuda.synchronize()
        gr, br = oracle.gate(st.x, st.b, A_log, dt_bias)
        o_ref, S_new = oracle.decode(st.q[live], st.k[live], st.v[live], gr[live], br[live],
                                     np.stack([S_ref[n] for n in live]))
        if sdt == torch.bfloat16:
            S_new = _bf16_round(S_new)
        for i, n in enumerate(live):
            S_ref[n] = S_new[i]
        assert_out(o[live], o_ref, "pool step %d" % step)
        assert torch.all(o[1] == 0)
    for s in range(NS):
        if s not in idx:
            assert torch.equal(pool[s].cpu(), pool0[s]), s
    for n in live:
        assert_state(pool[idx[n]], S_ref[n], "pool slot %d" % idx[n])


def test_decode_gated_full_size_bf16_every_pair():
    """256 sequences x 96 heads, bf16 state pool of 256 slots addressed through
    a permutation, bf16 logits, 8 steps; every (sequence, head) pair against
    the oracle gate and step with the state rounded to bf16 after each step.
    Both chains round their state to bf16 after every step, so an element
    whose two pre-rounding values straddle a rounding boundary differs by one
    bf16 step between them: o is held to the bound for outputs of such state
    pairs, and the final states to the one for two rounding chains."""
    need_gpu()
    c = CONFIGS[4]
    N, H, seed, steps = c["N"], c["H"], c["seed"], 8
    say("gated decode full size, bf16 pool, %d steps" % steps)
    A_log, dt_bias, S0 = draw_decode_params(N, H, seed=seed, device=DEV)
    pool = S0.to(torch.bfloat16)
    perm = torch.randperm(N, generator=torch.Generator().manual_seed(7)).to(torch.int32)
    ind = perm.to(DEV)
    ni = torch.arange(N).repeat_interleave(H)
    hi = torch.arange(H).repeat(N)
    si = perm[ni].long()
    S_ref = to64(pool[si, hi])                            # [N H, 128, 128]
    for step in range(steps):
        st = draw_decode_step(N, H, step, seed=seed, dtype=torch.bfloat16, device=DEV)
        x, b = st.x.to(torch.bfloat16), st.b.to(torch.bfloat16)
        o = kda.recurrent_decode_gated(st.q, st.k, st.v, x, b, A_log, dt_bias, pool,
                                       state_indices=ind, o_dtype=torch.float32)
        gr, br = oracle.gate(x[ni, hi].cpu()[None].float(), b[ni, hi].cpu()[None].float(),
                             A_log[hi].cpu(), dt_bias[hi].cpu())
        qp, kp = st.q[ni, hi].cpu()[None], st.k[ni, hi].cpu()[None]
        o_ref, S_new = oracle.decode(qp, kp, st.v[ni, hi].cpu()[None], gr, br, S_ref[None])
        e = out_err_bf16_state(o[ni, hi][None], o_ref, S_ref[None], qp, kp, br, np.exp(gr))
        assert e <= 1.0, "bf16 pool step %d: err ratio %.3f" % (step, e)
        S_ref = _bf16_round(S_new[0])
    torch.cuda.synchronize()
    assert_state(pool[si, hi], S_ref, "bf16 pool after %d steps" % steps,
                 tol=S_TOL_BF16_CHAINS)
