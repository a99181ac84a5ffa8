"""GPU: the gated prefill reading and writing states in a slot pool (fp32 or
bf16) and handing them to the gated decode, against the fp64 oracle.

Serving keeps every sequence's recurrent state in one preallocated pool
[num_slots, H, 128, 128]: the prefill takes its entry states from slots
state_indices[n] and writes its exit states back there, and the one-token
decode steps from the same slots.  In bf16 mode the state is stored rounded
to bf16 (nearest even) at the prefill's exit and after every decode step, which
is what that mode computes, so the oracle's state is rounded at the same
points.  The prefill's bf16 exit state is held to the exact (unrounded)
oracle state within 1e-3 + 2^-8 (its own rounding added), the two rounded
chains after the decode steps within 1e-3 + 2 * 2^-8 (both roundings), and
each decode step's o to 5e-3 RMS plus the effect of one rounding of each
chain on every state entry (tests/parity.py derives the bounds).
"""
import numpy as np
import pytest
import torch

import oracle
from synth import draw_decode_step, draw_prefill
from tests.gpu_util import DEV, need_gpu, say
from tests.parity import (S_TOL, S_TOL_BF16, S_TOL_BF16_CHAINS, assert_out, assert_state,
                          out_err_bf16_state, to64)
import gated_delta_rule_58_amd as kda

pytestmark = pytest.mark.gpu


def _round_bf16(S):
    return to64(torch.from_numpy(np.ascontiguousarray(S)).float().to(torch.bfloat16))


@pytest.mark.parametrize("sdt", [torch.float32, torch.bfloat16])
def test_prefill_into_pool_then_decode(sdt):
    """Four sequences of 150, 0, 64 and 77 tokens mapped to slots [5, 2, -1, 0]
    of a 7-slot pool updated in place: the third is a padding entry (zero entry
    state, no exit state, o still computed), the second is empty (its slot is
    carried through unchanged).  Then 3 gated decode steps from the same slots
    (the padding sequence's o is zero).  Slots no sequence names stay bit for
    bit unchanged."""
    need_gpu()
    say("prefill into a state pool then decode", sdt)
    lengths, idx, NS, H = [150, 0, 64, 77], [5, 2, -1, 0], 7, 3
    N = len(lengths)
    dr = draw_prefill(lengths, H=H, dtype=torch.bfloat16, seed=71)
    pool0 = (torch.randn((NS, H, 128, 128), generator=torch.Generator().manual_seed(72)) *
             0.05).to(sdt)
    pool = pool0.to(DEV).contiguous()
    ind = torch.tensor(idx, dtype=torch.int32, device=DEV)
    cu_h = dr.cu_seqlens
    o, fin = kda.chunk_prefill_gated(dr.q.to(DEV), dr.k.to(DEV), dr.v.to(DEV), dr.x.to(DEV),
                                     dr.b.to(DEV), dr.A_log.to(DEV), dr.dt_bias.to(DEV),
                                     cu_h.to(DEV), pool, final_state=pool, state_indices=ind,
                                     cu_seqlens_host=cu_h, scale=0.8, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert fin is pool
    S0 = np.stack([to64(pool0[s]) if s >= 0 else np.zeros((H, 128, 128)) for s in idx])
    gr, br = oracle.gate(dr.x, dr.b, dr.A_log, dr.dt_bias)
    o_ref, S_ref = oracle.prefill(dr.q, dr.k, dr.v, gr, br, cu_h, S0, scale=0.8)
    assert_out(o, o_ref, "pooled prefill")
    bf = sdt == torch.bfloat16
    state = {}
    for n, s in enumerate(idx):
        if s < 0:
            continue
        if lengths[n] == 0:
            assert torch.equal(pool[s].cpu(), pool0[s]), "empty sequence's slot changed"
        else:
            assert_state(pool[s], S_ref[n], "pooled prefill slot %d" % s,
                         tol=S_TOL_BF16 if bf else S_TOL)
        state[n] = _round_bf16(S_ref[n]) if bf else S_ref[n]
    for s in range(NS):
        if s not in idx:
            assert torch.equal(pool[s].cpu(), pool0[s]), s
    live = [n for n in range(N) if idx[n] >= 0]
    for step in range(3):
        st = draw_decode_step(N, H, step, seed=73, dtype=torch.bfloat16)
        od = kda.recurrent_decode_gated(st.q.to(DEV), st.k.to(DEV), st.v.to(DEV), st.x.to(DEV),
                                        st.b.to(DEV), dr.A_log.to(DEV), dr.dt_bias.to(DEV), pool,
                                        state_indices=ind, scale=0.8, o_dtype=torch.float32)
        torch.cuda.synchronize()
        g, b = oracle.gate(st.x, st.b, dr.A_log, dr.dt_bias)
        S_prev = np.stack([state[n] for n in live])
        o_r, S_new = oracle.decode(st.q[live], st.k[live], st.v[live], g[live], b[live], S_prev,
                                   scale=0.8)
        if bf:
            S_new = _round_bf16(S_new)
            e = out_err_bf16_state(od[live], o_r, S_prev, st.q[live], st.k[live], b[live],
                                   np.exp(g[live]), scale=0.8)
            assert e <= 1.0, "decode step %d from bf16 states: err ratio %.3f" % (step, e)
        else:
            assert_out(od[live], o_r, "decode step %d" % step)
        for i, n in enumerate(live):
            state[n] = S_new[i]
        assert torch.all(od[2] == 0)
    for n in live:
        assert_state(pool[idx[n]], state[n], "after decode, slot %d" % idx[n],
                     tol=S_TOL_BF16_CHAINS if bf else S_TOL)
    for s in range(NS):
        if s not in idx:
            assert torch.equal(pool[s].cpu(), pool0[s]), s


def test_pool_matches_plain_states_and_multi_pass():
    """An fp32 pool with a permutation of slots gives bit for bit the results of
    the plain [N, H, 128, 128] states, also when the workspace runs the chunk
    axis in passes (the state between passes stays fp32); a bf16 pool's exit
    state is the round-to-nearest-even rounding of the fp32 one."""
    need_gpu()
    say("pool vs plain states, passes")
    lengths, H = [200, 64, 1, 130], 2
    N = len(lengths)
    dr = draw_prefill(lengths, H=H, dtype=torch.bfloat16, init_state=True, seed=74)
    cu_h = dr.cu_seqlens
    args = (dr.q.to(DEV), dr.k.to(DEV), dr.v.to(DEV), dr.x.to(DEV), dr.b.to(DEV),
            dr.A_log.to(DEV), dr.dt_bias.to(DEV), cu_h.to(DEV))
    S0 = dr.initial_state.to(DEV)
    o1, S1 = kda.chunk_prefill_gated(*args, S0, cu_seqlens_host=cu_h, o_dtype=torch.float32)
    perm = [3, 0, 2, 1]
    ind = torch.tensor(perm, dtype=torch.int32, device=DEV)
    for cpp in (1, 2, 4):
        ws = torch.empty(kda.chunk_prefill_workspace_bytes(N, H, 128, 128, cpp), dtype=torch.uint8,
                         device=DEV)
        pool = torch.empty((N, H, 128, 128), device=DEV)
        for n in range(N):
            pool[perm[n]] = S0[n]
        o2, _ = kda.chunk_prefill_gated(*args, pool, final_state=pool, state_indices=ind,
                                        cu_seqlens_host=cu_h, o_dtype=torch.float32,
                                        workspace=ws)
        pb = pool.new_empty(pool.shape, dtype=torch.bfloat16)
        for n in range(N):
            pb[perm[n]] = S0[n].to(torch.bfloat16)
        o3, _ = kda.chunk_prefill_gated(*args, pb, final_state=pb, state_indices=ind,
                                        cu_seqlens_host=cu_h, o_dtype=torch.float32,
                                        workspace=ws)
        o4, S4 = kda.chunk_prefill_gated(*args, S0.to(torch.bfloat16), cu_seqlens_host=cu_h,
                                         o_dtype=torch.float32, workspace=ws,
                                         state_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), cpp
        for n in range(N):
            assert torch.equal(pool[perm[n]], S1[n]), (cpp, n)
        assert torch.equal(o3, o4), cpp
        for n in range(N):
            assert torch.equal(pb[perm[n]], S4[n]), (cpp, n)
    # the bf16 exit state rounds the fp32 walk state: from the same (bf16) entry
    # states the fp32-state call's exit state rounds to the bf16 one
    o5, S5 = kda.chunk_prefill_gated(*args, S0.to(torch.bfloat16).float(), cu_seqlens_host=cu_h,
                                     o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o5, o4)
    assert torch.equal(S5.to(torch.bfloat16), S4)
