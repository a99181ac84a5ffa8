"""GPU: kda_chunk_prefill_gated_static, the gated prefill over the library's own
device scratch (no workspace, no allocation), against kda_chunk_prefill_gated
with a caller's workspace: bit for bit the same outputs and states, on calls in
a row that shrink (the scratch keeps the previous call's contents, which no
call reads), including one that runs the chunk axis in several passes."""
import pytest
import torch

from synth import draw_prefill
from tests.gpu_util import DEV, need_gpu, say
import gated_delta_rule_58_amd as kda

pytestmark = pytest.mark.gpu


def _compare(lengths, H, seed, sdt=torch.float32, pool_perm=None, odt=torch.bfloat16):
    dr = draw_prefill(lengths, H=H, dtype=torch.bfloat16, init_state=True, seed=seed)
    cu_h = dr.cu_seqlens
    N = len(lengths)
    args = (dr.q.to(DEV), dr.k.to(DEV), dr.v.to(DEV), dr.x.to(DEV), dr.b.to(DEV),
            dr.A_log.to(DEV), dr.dt_bias.to(DEV), cu_h.to(DEV))
    S0 = dr.initial_state.to(DEV).to(sdt)
    ind = None
    if pool_perm is not None:
        ind = torch.tensor(pool_perm, dtype=torch.int32, device=DEV)
        pool = torch.zeros((max(pool_perm) + 2,) + tuple(S0.shape[1:]), dtype=sdt, device=DEV)
        for n, s in enumerate(pool_perm):
            if s >= 0:
                pool[s] = S0[n]
        S0 = pool
    f_ref = S0.clone() if ind is not None else torch.empty_like(S0)
    o_ref, _ = kda.chunk_prefill_gated(*args, S0, final_state=f_ref, cu_seqlens_host=cu_h,
                                       o_dtype=odt, state_indices=ind)
    o = torch.empty_like(o_ref)
    f = S0.clone() if ind is not None else torch.empty_like(S0)
    kda.chunk_prefill_gated_static(*args, initial_state=S0, final_state=f, out=o,
                                   cu_seqlens_host=cu_h, state_indices=ind)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), lengths
    assert torch.equal(f, f_ref), lengths
    return N * H


def test_static_scratch_matches_the_workspace_call():
    need_gpu()
    say("static scratch: multi-pass call (T=3200, H=96)")
    _compare([3200], 96, seed=91)                      # 50 chunks: two passes of the scratch
    say("static scratch: smaller varlen call, bf16 pool with indices")
    _compare([300, 0, 77, 129], 4, seed=92, sdt=torch.bfloat16, pool_perm=[2, 0, -1, 4],
             odt=torch.float32)
    say("static scratch: smallest call")
    _compare([17], 1, seed=93)


def test_static_scratch_refuses_more_pairs_than_it_holds():
    """More (sequence, head) pairs than one chunk per pass fits in the scratch:
    refused on the host with KDA_ERR_WORKSPACE, nothing launched."""
    need_gpu()
    say("static scratch refusal")
    N, H = 23, 96                                      # 2,208 pairs > 2,131
    cu = torch.arange(N + 1, dtype=torch.int32)
    T = N
    q = torch.zeros((T, H, 128), dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((T, H, 128), device=DEV)
    b = torch.zeros((T, H), device=DEV)
    o = torch.full((T, H, 128), 3.0, device=DEV)
    with pytest.raises(kda.KdaError) as ei:
        kda.chunk_prefill_gated_static(q, q, q, x, b, torch.zeros(H, device=DEV),
                                       torch.zeros(H, 128, device=DEV), cu.to(DEV), out=o,
                                       cu_seqlens_host=cu)
    assert ei.value.status == 6 and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)
