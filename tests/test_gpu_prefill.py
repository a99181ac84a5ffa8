"""GPU parity of kda_chunk_prefill against the fp64 oracle.

Small cases feed both sides the same fp32 g/beta (from the oracle gate).  The
full-size workloads run the gated prefill in the one-pass launch
configuration the bench times, and kda_gate then kda_chunk_prefill through
the binding's capped workspace, both with an fp32 output held to the stated
bound, and compare sampled heads (heads are independent) against the oracle
gate then the oracle recurrence; the gated one-pass call is also compared on
every head of each full-size workload.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, draw_alog_per_channel, draw_config, draw_prefill
from tests.gpu_util import DEV, need_gpu, oracle_gate_f32, oracle_gate_f64, sample_heads, say
from tests.parity import (O_TOL, S_TOL, assert_out, assert_out_bf16, assert_state, out_err,
                          state_err, to64)
import gated_delta_rule_58_amd as kda

pytestmark = pytest.mark.gpu


def _run_gpu(dr, g, beta, o_dtype, scale=1.0, S0=None):
    cu = dr.cu_seqlens
    o, Sf = kda.chunk_prefill(dr.q.to(DEV), dr.k.to(DEV), dr.v.to(DEV), g.to(DEV),
                              beta.to(DEV), cu_seqlens=cu.to(DEV), cu_seqlens_host=cu,
                              initial_state=None if S0 is None else S0.to(DEV),
                              scale=scale, o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o, Sf


def _check_small(lengths, H, qdt, init, seed, scale=1.0):
    dr = draw_prefill(lengths, H=H, dtype=qdt, init_state=init, seed=seed)
    g, beta = oracle_gate_f32(dr)
    say("prefill case lengths=%s H=%d dtype=%s init=%s" % (lengths, H, qdt, init))
    o_ref, S_ref = oracle.prefill(dr.q, dr.k, dr.v, g, beta, dr.cu_seqlens, dr.initial_state,
                                  scale=scale)
    o32, S32 = _run_gpu(dr, g, beta, torch.float32, scale, dr.initial_state)
    eo = assert_out(o32, o_ref, str(lengths))
    es = assert_state(S32, S_ref, str(lengths))
    ob, Sb = _run_gpu(dr, g, beta, torch.bfloat16, scale, dr.initial_state)
    assert_out_bf16(ob, o_ref, str(lengths))
    assert torch.equal(ob, o32.to(torch.bfloat16)), "bf16 o is not RNE(fp32 o)"
    assert torch.equal(Sb, S32)
    return eo, es


def test_config0_parity():
    """T=256, H=2, fp32 q/k/v, chunk 64, zero initial state."""
    need_gpu()
    dr = draw_config(0)
    g, beta = oracle_gate_f32(dr)
    say("config 0")
    o_ref, S_ref = oracle.prefill(dr.q, dr.k, dr.v, g, beta, dr.cu_seqlens)
    o, S = _run_gpu(dr, g, beta, torch.float32)
    assert o.shape == (256, 2, 128) and S.shape == (1, 2, 128, 128)
    assert_out(o, o_ref, "config 0")
    assert_state(S, S_ref, "config 0")


# Shapes of the audit page's exact-match table (§7.3): one chunk [16],
# partial tail [17], two chunks [32], multi-chunk/multi-head [65] H=2, the K3
# head count [17] H=96, varlen partial chunks [17,31] H=2; plus the chunk-64
# boundaries and a zero-length sequence.
EDGE = [([16], 1), ([17], 1), ([32], 1), ([65], 2), ([17], 96), ([17, 31], 2),
        ([1], 3), ([63], 2), ([64], 2), ([128], 2), ([129], 2), ([200, 0, 64, 1, 77], 3)]


@pytest.mark.parametrize("lengths,H", EDGE)
def test_edge_shapes(lengths, H):
    need_gpu()
    _check_small(lengths, H, torch.bfloat16, True, seed=100 + sum(lengths) + H, scale=0.7)


@pytest.mark.parametrize("seed", [201, 202, 203, 204, 205, 206])
def test_random_shapes(seed):
    """Random varlen batches (empty, one-token and chunk-boundary lengths among
    them), head counts, q/k/v dtypes, initial states and scales: fp32 o within
    the stated bound, bf16 o the rounding of it, the state within its bound."""
    need_gpu()
    rng = np.random.default_rng(seed)
    nseq = int(rng.integers(1, 7))
    pool = [0, 1, 16, 17, 63, 64, 65, 127, 128, 129]
    lengths = [int(rng.choice(pool)) if rng.random() < 0.4 else int(rng.integers(2, 400))
               for _ in range(nseq)]
    if sum(lengths) == 0:
        lengths[0] = 97
    H = int(rng.choice([1, 2, 3, 5, 8]))
    qdt = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    init = bool(rng.random() < 0.5)
    scale = float(rng.uniform(0.3, 1.5))
    _check_small(lengths, H, qdt, init, seed, scale)


def test_edge_many_sequences():
    """70 packed sequences of 0..39 tokens: more than the 64 that the state
    kernel orders longest first, so workgroups map to sequences in order."""
    need_gpu()
    lengths = np.random.default_rng(5).integers(0, 40, 70).tolist()
    _check_small(lengths, 2, torch.bfloat16, True, seed=170, scale=0.7)


def test_edge_all_sequences_empty():
    """T_tot = 0 with three zero-length sequences: no output rows, and every
    final state is its initial state, bit for bit."""
    need_gpu()
    say("prefill all sequences empty")
    dr = draw_prefill([0, 0, 0], H=2, dtype=torch.bfloat16, init_state=True, seed=171)
    g, beta = oracle_gate_f32(dr)
    o, Sf = _run_gpu(dr, g, beta, torch.float32, 1.0, dr.initial_state)
    assert o.shape == (0, 2, 128)
    assert torch.equal(Sf.cpu(), dr.initial_state)


def test_edge_no_initial_state_fp32_inputs():
    need_gpu()
    _check_small([65, 130], 4, torch.float32, False, seed=7)


def test_delta_rule_recall_on_gpu():
    """alpha=1, beta=1, q_t=k_t with unit keys: o_t = v_t exactly (any state)."""
    need_gpu()
    from synth import orthonormal_keys_pm_quarter
    T, H = 100, 2
    K = orthonormal_keys_pm_quarter(T if T <= 128 else 128)
    k = K[None].repeat(H, 1, 1).permute(1, 0, 2).contiguous().to(torch.bfloat16)
    v = torch.randn(T, H, 128, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    g = torch.zeros(T, H, 128)
    beta = torch.ones(T, H)
    S0 = torch.randn(1, H, 128, 128, generator=torch.Generator().manual_seed(4))
    say("recall on gpu")
    o, S = kda.chunk_prefill(k.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), beta.to(DEV),
                             initial_state=S0.to(DEV), o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(o.cpu() - v.float())) < 2e-3


def test_chunked_equals_decode_loop_and_resume():
    """Prefill over T equals the GPU decode kernel looped token by token, a
    split prefill resumed from the first part's final state, and the oracle."""
    need_gpu()
    T, T1, H = 150, 70, 4
    dr = draw_prefill([T], H=H, dtype=torch.bfloat16, init_state=True, seed=9)
    g, beta = oracle_gate_f32(dr)
    say("prefill vs decode loop vs split")
    o, S = _run_gpu(dr, g, beta, torch.float32, S0=dr.initial_state)
    state = dr.initial_state.to(DEV).clone()
    od = []
    for t in range(T):
        od.append(kda.recurrent_decode(dr.q[t:t + 1].to(DEV), dr.k[t:t + 1].to(DEV),
                                       dr.v[t:t + 1].to(DEV), g[t:t + 1].to(DEV),
                                       beta[t:t + 1].to(DEV), state, o_dtype=torch.float32))
    od = torch.cat(od)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.prefill(dr.q, dr.k, dr.v, g, beta, dr.cu_seqlens, dr.initial_state)
    assert_out(o, o_ref, "prefill")
    assert_out(od, o_ref, "decode loop")
    assert_state(S, S_ref, "prefill")
    assert_state(state, S_ref, "decode loop")
    assert out_err(o, od) <= 5e-3 and state_err(S, state) <= 1e-3
    # split prefill: [0, T1) then [T1, T) from the first part's final state
    d1 = draw_prefill([T1], H=H, dtype=torch.bfloat16, seed=0)
    d1.q, d1.k, d1.v = dr.q[:T1], dr.k[:T1], dr.v[:T1]
    o1, S1 = _run_gpu(d1, g[:T1], beta[:T1], torch.float32, S0=dr.initial_state)
    d2 = draw_prefill([T - T1], H=H, dtype=torch.bfloat16, seed=0)
    d2.q, d2.k, d2.v = dr.q[T1:], dr.k[T1:], dr.v[T1:]
    o2, S2 = _run_gpu(d2, g[T1:], beta[T1:], torch.float32, S0=S1.cpu())
    assert_out(torch.cat([o1, o2]), o_ref, "split")
    assert_state(S2, S_ref, "split")


def test_in_place_state_and_determinism():
    need_gpu()
    dr = draw_prefill([300, 45], H=8, dtype=torch.bfloat16, init_state=True, seed=12)
    g, beta = oracle_gate_f32(dr)
    say("in-place state + determinism")
    q, k, v = dr.q.to(DEV), dr.k.to(DEV), dr.v.to(DEV)
    gg, bb, cu = g.to(DEV), beta.to(DEV), dr.cu_seqlens.to(DEV)
    o1, S1 = kda.chunk_prefill(q, k, v, gg, bb, cu, dr.initial_state.to(DEV))
    o2, S2 = kda.chunk_prefill(q, k, v, gg, bb, cu, dr.initial_state.to(DEV))
    st = dr.initial_state.to(DEV).clone()
    o3, _ = kda.chunk_prefill(q, k, v, gg, bb, cu, st, final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert torch.equal(o1, o3) and torch.equal(S1, st)


def _one_pass_workspace(cu_h, H):
    """Workspace that holds every chunk of the longest sequence: one pass, the
    launch configuration the bench times."""
    lens = (cu_h[1:] - cu_h[:-1]).clamp(min=0)
    chunks = max(1, (int(lens.max()) + 63) // 64)
    nb = kda.chunk_prefill_workspace_bytes(cu_h.numel() - 1, H, 128, 128, chunks)
    return torch.empty(nb, dtype=torch.uint8, device=DEV)


def _full_config(idx, n_heads, seed):
    """Workload idx at full size, on sampled heads against the oracle gate and
    recurrence, at the stated tolerances on an fp32 output:
      (1) kda_chunk_prefill_gated in one pass with the whole workspace (the
          call the bench times), o fp32;
      (2) the same call with o bf16: bit-for-bit the round-to-nearest-even
          rounding of (1), and the same final state;
      (3) kda_gate then kda_chunk_prefill through the binding's default
          workspace (1 GiB cap: several passes at this size), o fp32."""
    c = CONFIGS[idx]
    say("full config %d (%s), sampled heads" % (idx, c["name"]))
    dr = draw_config(idx, device=DEV)
    cu_h = dr.cu_seqlens
    cu = cu_h.to(DEV)
    H = c["H"]
    ws = _one_pass_workspace(cu_h, H)
    say("  gated one pass, fp32 o, workspace %d bytes" % ws.numel())
    o32, S32 = kda.chunk_prefill_gated(dr.q, dr.k, dr.v, dr.x, dr.b, dr.A_log, dr.dt_bias, cu,
                                       dr.initial_state, cu_seqlens_host=cu_h,
                                       o_dtype=torch.float32, workspace=ws)
    say("  gated one pass, bf16 o")
    o16, S16 = kda.chunk_prefill_gated(dr.q, dr.k, dr.v, dr.x, dr.b, dr.A_log, dr.dt_bias, cu,
                                       dr.initial_state, cu_seqlens_host=cu_h,
                                       o_dtype=torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    del ws
    assert torch.equal(o16, o32.to(torch.bfloat16)), "bf16 o is not RNE(fp32 o)"
    assert torch.equal(S16, S32)
    del o16, S16
    say("  kda_gate + kda_chunk_prefill (binding workspace), fp32 o")
    g, beta = kda.gate(dr.x, dr.b, dr.A_log, dr.dt_bias)
    o2, S2 = kda.chunk_prefill(dr.q, dr.k, dr.v, g, beta, cu, dr.initial_state,
                               cu_seqlens_host=cu_h, o_dtype=torch.float32)
    torch.cuda.synchronize()
    del g, beta
    heads = sample_heads(H, n_heads, seed)
    say("  oracle on heads", heads)
    gr, br = oracle_gate_f64(dr, heads)
    S0 = None if dr.initial_state is None else dr.initial_state[:, heads].cpu()
    o_ref, S_ref = oracle.prefill(dr.q[:, heads].cpu(), dr.k[:, heads].cpu(),
                                  dr.v[:, heads].cpu(), gr, br, cu_h, S0)
    e1 = assert_out(o32[:, heads], o_ref, "config %d gated one pass" % idx)
    s1 = assert_state(S32[:, heads], S_ref, "config %d gated one pass" % idx)
    e3 = assert_out(o2[:, heads], o_ref, "config %d gate + prefill" % idx)
    s3 = assert_state(S2[:, heads], S_ref, "config %d gate + prefill" % idx)
    say("  fp32-o err / RMS: gated %.3e, gate+prefill %.3e (bound 5e-3); state rel-F: "
        "gated %.3e, gate+prefill %.3e (bound 1e-3)" % (e1, e3, s1, s3))


def test_config1_full_sampled_heads():
    need_gpu()
    _full_config(1, 8, 1)


def test_config2_full_sampled_heads():
    need_gpu()
    _full_config(2, 4, 2)


def test_config3_full_sampled_heads():
    need_gpu()
    _full_config(3, 3, 3)


def test_strong_decay_heads():
    """Heads whose channels decay by tens of nats per 16-token block (the
    checkpoint's A_log reaches 2.47): exercises the decay-factor references
    and the wide-range path of the diagonal tiles."""
    need_gpu()
    dr = draw_prefill([200, 77], H=4, dtype=torch.bfloat16, init_state=True, seed=41)
    dr.A_log = torch.tensor([1.5, -0.75, 1.0, 0.0])
    dt = dr.dt_bias.clone()
    dt[0] = 0.0                     # head 0: every channel fast (about 3.6 nats per token)
    dt[2, :16] = 1.0                # head 2: a few fast channels among slow ones
    dr.dt_bias = dt
    g, beta = oracle_gate_f32(dr)
    say("strong decay heads")
    o_ref, S_ref = oracle.prefill(dr.q, dr.k, dr.v, g, beta, dr.cu_seqlens, dr.initial_state)
    o, S = _run_gpu(dr, g, beta, torch.float32, S0=dr.initial_state)
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    assert_out(o, o_ref, "strong decay")
    assert_state(S, S_ref, "strong decay")


A_LOG_MAX, DT_BIAS_MAX = 2.4661, 0.1792   # artifact audit §5.1, the printed maxima


@pytest.mark.parametrize("mode", ["g", "gated", "gated_per_channel"])
def test_printed_extreme_decay(mode):
    """Decay at the artifact audit's printed parameter extremes (§5.1: A_log up
    to 2.4661, dt_bias up to 0.1792), where a single token can decay a channel
    by tens of log2 units: every channel of head 0 and half the channels of
    head 1 at both maxima, head 3 at A_log 1.0, head 2 at the median; or, per
    channel, A_log [H, d] ~ U(-0.75, 2.4661) with dt_bias at its maximum on
    every other channel.  Varlen with an initial state; fp32 o at the stated
    bounds, every value finite."""
    need_gpu()
    dr = draw_prefill([300, 77, 129], H=4, dtype=torch.bfloat16, init_state=True, seed=43)
    dt = dr.dt_bias.clone()
    if mode == "gated_per_channel":
        A = torch.rand(4, 128, generator=torch.Generator().manual_seed(44)) * (A_LOG_MAX + 0.75) - 0.75
        A[:, 0] = A_LOG_MAX
        dt[:, ::2] = DT_BIAS_MAX
    else:
        A = torch.tensor([A_LOG_MAX, A_LOG_MAX, -0.1533, 1.0])
        dt[0] = DT_BIAS_MAX
        dt[1, :64] = DT_BIAS_MAX
    dr.A_log, dr.dt_bias = A, dt
    say("printed extreme decay", mode)
    gr, br = oracle.gate(dr.x, dr.b, A, dt)
    o_ref, S_ref = oracle.prefill(dr.q, dr.k, dr.v, gr, br, dr.cu_seqlens, dr.initial_state)
    cu_h = dr.cu_seqlens
    if mode == "g":
        g, beta = oracle_gate_f32(dr)
        o, S = _run_gpu(dr, g, beta, torch.float32, S0=dr.initial_state)
    else:
        o, S = kda.chunk_prefill_gated(dr.q.to(DEV), dr.k.to(DEV), dr.v.to(DEV), dr.x.to(DEV),
                                       dr.b.to(DEV), A.to(DEV), dt.to(DEV), cu_h.to(DEV),
                                       dr.initial_state.to(DEV), cu_seqlens_host=cu_h,
                                       o_dtype=torch.float32)
        torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    eo = assert_out(o, o_ref, "extreme decay " + mode)
    es = assert_state(S, S_ref, "extreme decay " + mode)
    say("  o err / RMS %.3e, state rel-F %.3e" % (eo, es))


def test_multi_pass_workspace():
    """A workspace smaller than the longest sequence's chunk count runs the
    chunk axis in passes (state carried through final_state, or through the
    workspace when no final state is requested): results are bit-identical to
    one pass."""
    need_gpu()
    dr = draw_prefill([200, 0, 64, 1, 77], H=3, dtype=torch.bfloat16, init_state=True, seed=51)
    g, beta = oracle_gate_f32(dr)
    say("multi-pass workspace")
    q, k, v, gg, bb = (t.to(DEV) for t in (dr.q, dr.k, dr.v, g, beta))
    cu_h = dr.cu_seqlens
    cu = cu_h.to(DEV)
    S0 = dr.initial_state.to(DEV)
    o1, S1 = kda.chunk_prefill(q, k, v, gg, bb, cu, S0, cu_seqlens_host=cu_h, o_dtype=torch.float32)
    for cpp in (1, 3):
        nb = kda.chunk_prefill_workspace_bytes(5, 3, 128, 128, cpp)
        ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
        o2, S2 = kda.chunk_prefill(q, k, v, gg, bb, cu, S0, cu_seqlens_host=cu_h,
                                   o_dtype=torch.float32, workspace=ws)
        o3, S3 = kda.chunk_prefill(q, k, v, gg, bb, cu, S0, cu_seqlens_host=cu_h,
                                   o_dtype=torch.float32, workspace=ws, output_final_state=False)
        st = S0.clone()
        o4, _ = kda.chunk_prefill(q, k, v, gg, bb, cu, st, cu_seqlens_host=cu_h,
                                  o_dtype=torch.float32, workspace=ws, final_state=st)
        torch.cuda.synchronize()
        assert S3 is None
        assert torch.equal(o1, o2) and torch.equal(S1, S2), cpp
        assert torch.equal(o1, o3) and torch.equal(o1, o4) and torch.equal(S1, st), cpp
    o_ref, S_ref = oracle.prefill(dr.q, dr.k, dr.v, g, beta, cu_h, dr.initial_state)
    assert_out(o1, o_ref, "multi-pass")
    assert_state(S1, S_ref, "multi-pass")


@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16])
def test_gated_matches_gate_then_prefill(xdt):
    """kda_chunk_prefill_gated matches the oracle gate followed by the oracle
    recurrence, and kda_gate followed by kda_chunk_prefill within the same
    tolerances, on varlen input with empty and one-token sequences, initial
    state and scale.  The two GPU paths are not bit-identical: the in-register
    gate skips kda_gate's last-ulp corrections (g differs by about
    exp(A_log) 2^-23), which moves the fp16 rounding of some decayed
    operands, so their difference is of the size of either path's own
    rounding error (about 1e-3 x RMS(o) here)."""
    need_gpu()
    dr = draw_prefill([200, 0, 64, 1, 77], H=3, dtype=torch.bfloat16, init_state=True, seed=61)
    say("gated prefill vs gate + prefill", xdt)
    x, b = dr.x.to(xdt), dr.b.to(xdt)
    q, k, v = dr.q.to(DEV), dr.k.to(DEV), dr.v.to(DEV)
    xd, bd, A, dtb = x.to(DEV), b.to(DEV), dr.A_log.to(DEV), dr.dt_bias.to(DEV)
    cu_h = dr.cu_seqlens
    cu = cu_h.to(DEV)
    S0 = dr.initial_state.to(DEV)
    g, beta = kda.gate(xd, bd, A, dtb)
    o1, S1 = kda.chunk_prefill(q, k, v, g, beta, cu, S0, cu_seqlens_host=cu_h, scale=0.7,
                               o_dtype=torch.float32)
    o2, S2 = kda.chunk_prefill_gated(q, k, v, xd, bd, A, dtb, cu, S0, cu_seqlens_host=cu_h,
                                     scale=0.7, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert out_err(o2, o1) <= O_TOL and state_err(S2, S1) <= S_TOL
    gr, br = oracle.gate(x.float(), b.float(), dr.A_log, dr.dt_bias)
    o_ref, S_ref = oracle.prefill(dr.q, dr.k, dr.v, gr, br, cu_h, dr.initial_state, scale=0.7)
    assert_out(o2, o_ref, "gated")
    assert_state(S2, S_ref, "gated")


@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16])
def test_gated_per_channel_alog(xdt):
    """kda_chunk_prefill_gated with A_log per (head, channel), [H, dk], on
    varlen input with empty and one-token sequences and an initial state,
    against the oracle gate (per-channel) followed by the oracle recurrence."""
    need_gpu()
    dr = draw_prefill([200, 0, 64, 1, 77], H=3, dtype=torch.bfloat16, init_state=True, seed=63)
    A = draw_alog_per_channel(3, seed=63)
    say("gated prefill per-channel A_log", xdt)
    x, b = dr.x.to(xdt), dr.b.to(xdt)
    cu_h = dr.cu_seqlens
    o, S = kda.chunk_prefill_gated(dr.q.to(DEV), dr.k.to(DEV), dr.v.to(DEV), x.to(DEV),
                                   b.to(DEV), A.to(DEV), dr.dt_bias.to(DEV), cu_h.to(DEV),
                                   dr.initial_state.to(DEV), cu_seqlens_host=cu_h, scale=0.7,
                                   o_dtype=torch.float32)
    torch.cuda.synchronize()
    gr, br = oracle.gate(x.float(), b.float(), A, dr.dt_bias)
    o_ref, S_ref = oracle.prefill(dr.q, dr.k, dr.v, gr, br, cu_h, dr.initial_state, scale=0.7)
    assert_out(o, o_ref, "gated per-channel A_log")
    assert_state(S, S_ref, "gated per-channel A_log")


class _WholeTensor:
    """The output and state metrics of the tolerances over every compared
    head, accumulated over head groups: max |o_gpu - o_ref| over all of them
    against their common RMS(o_ref), and the relative Frobenius error of all
    their final states, as if the groups were one tensor."""

    def __init__(self):
        self.o_max, self.o_ss, self.o_n = 0.0, 0.0, 0
        self.s_dd, self.s_rr = 0.0, 0.0

    def add(self, o_gpu, o_ref, S_gpu, S_ref):
        self.o_max = max(self.o_max, float(np.max(np.abs(to64(o_gpu) - o_ref))))
        self.o_ss += float(np.sum(o_ref ** 2))
        self.o_n += o_ref.size
        self.s_dd += float(np.sum((to64(S_gpu) - S_ref) ** 2))
        self.s_rr += float(np.sum(S_ref ** 2))

    def errs(self):
        rms = np.sqrt(self.o_ss / max(self.o_n, 1))
        return self.o_max / max(rms, 1e-300), float(np.sqrt(self.s_dd / max(self.s_rr, 1e-300)))


def _full_config_heads(idx, heads, group):
    """Workload idx at full size through kda_chunk_prefill_gated in one pass
    (the call the bench times, o fp32), compared on the given heads (groups
    of `group` heads at a time against the oracle gate and recurrence) at the
    stated bounds over all of them."""
    c = CONFIGS[idx]
    say("full config %d (%s), %d heads" % (idx, c["name"], len(heads)))
    dr = draw_config(idx, device=DEV)
    cu_h = dr.cu_seqlens
    ws = _one_pass_workspace(cu_h, c["H"])
    o, S = kda.chunk_prefill_gated(dr.q, dr.k, dr.v, dr.x, dr.b, dr.A_log, dr.dt_bias,
                                   cu_h.to(DEV), dr.initial_state, cu_seqlens_host=cu_h,
                                   o_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    del ws
    acc = _WholeTensor()
    for i in range(0, len(heads), group):
        hs = heads[i:i + group]
        say("  oracle on heads %s .. %s" % (hs[0], hs[-1]))
        gr, br = oracle_gate_f64(dr, hs)
        S0 = None if dr.initial_state is None else dr.initial_state[:, hs].cpu()
        o_ref, S_ref = oracle.prefill(dr.q[:, hs].cpu(), dr.k[:, hs].cpu(), dr.v[:, hs].cpu(),
                                      gr, br, cu_h, S0)
        acc.add(o[:, hs], o_ref, S[:, hs], S_ref)
        del gr, br, o_ref, S_ref
    eo, es = acc.errs()
    say("  %d heads: fp32-o err / RMS %.3e (bound 5e-3), state rel-F %.3e (bound 1e-3)"
        % (len(heads), eo, es))
    assert eo <= O_TOL, "config %d output max-abs err %.3e x RMS" % (idx, eo)
    assert es <= S_TOL, "config %d state rel-Frobenius err %.3e" % (idx, es)


def test_config1_full_every_head():
    need_gpu()
    _full_config_heads(1, list(range(CONFIGS[1]["H"])), 96)


def test_config2_full_every_head():
    need_gpu()
    _full_config_heads(2, list(range(CONFIGS[2]["H"])), 24)


def test_config3_full_every_head():
    """131,072 tokens (2,048 chunks a head), eight heads at a time."""
    need_gpu()
    _full_config_heads(3, list(range(CONFIGS[3]["H"])), 8)
