"""GPU parity of kda_shortconv_l2norm (the layer prologue: short causal conv,
SiLU, q/k L2 norm) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import DEV, need_gpu, say
from tests.parity import to64
import gated_delta_rule_58_amd as kda

pytestmark = pytest.mark.gpu


def _draw(T, H, dtype, seed, n_seq_state=None):
    g = torch.Generator().manual_seed(seed)
    xs = [torch.randn((T, H, 128), generator=g).to(dtype) for _ in range(3)]
    ws = [torch.randn((H * 128, 4), generator=g) * 0.5 for _ in range(3)]
    st = None
    if n_seq_state is not None:
        st = torch.randn((n_seq_state, 3, 3, H * 128), generator=g)
        st = st.to(dtype).float()  # the state holds earlier inputs, so input precision
    return xs, ws, st


def _check(y, y_ref, out_dtype, what):
    """fp32 arithmetic: 1e-5 relative plus 1e-6 of the tensor's RMS (a few ulp
    through the 4-term conv, SiLU and the 128-channel norm); a bf16 output
    adds its own rounding, 2^-8 relative."""
    y, y_ref = to64(y), to64(y_ref)
    scale = np.sqrt(np.mean(y_ref ** 2)) + 1e-30
    rel = 1e-5 + (2.0 ** -8 if out_dtype == torch.bfloat16 else 0.0)
    tol = 1e-6 * scale + rel * np.abs(y_ref)
    err = np.abs(y - y_ref)
    assert np.all(err <= tol), "%s: max err %.3e (scale %.3e)" % (what, err.max(), scale)


@pytest.mark.parametrize("dtype,act", [(torch.bfloat16, "silu"), (torch.float32, "silu"),
                                       (torch.bfloat16, None)])
def test_prologue_parity_varlen(dtype, act):
    """Packed sequences of 200, 0, 64, 1, 77, 130 tokens (runs of 64 with
    ragged tails, an empty and a one-token sequence), H = 5, initial conv
    state, against the oracle; the state out is the inputs themselves."""
    need_gpu()
    say("prologue parity", dtype, act)
    lengths = [200, 0, 64, 1, 77, 130]
    T, H = sum(lengths), 5
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    xs, ws, st = _draw(T, H, dtype, 71, len(lengths))
    cu_t = torch.from_numpy(cu)
    yq, yk, yv, so = kda.shortconv_l2norm(*[x.to(DEV) for x in xs], *[w.to(DEV) for w in ws],
                                          cu_seqlens=cu_t.to(DEV), conv_state=st.to(DEV),
                                          activation=act, cu_seqlens_host=cu_t)
    torch.cuda.synchronize()
    rq, rk, rv, rs = oracle.shortconv_l2norm(*xs, *ws, cu, H, activation=act, state=st)
    for y, r, nm in ((yq, rq, "q"), (yk, rk, "k"), (yv, rv, "v")):
        _check(y, r, dtype, nm)
    assert np.array_equal(to64(so), rs)


def test_prologue_prefill_then_steps_equals_one_shot():
    """A prefill of T1 tokens per sequence, then one-token calls that update the
    conv state in place, reproduce one prefill over all tokens bit for bit."""
    need_gpu()
    say("prologue prefill + steps")
    N, H, T1, steps = 3, 4, 70, 3
    T = T1 + steps
    xs, ws, _ = _draw(N * T, H, torch.bfloat16, 73)
    xs = [x.reshape(N, T, H, 128) for x in xs]
    wd = [w.to(DEV) for w in ws]
    cu_all = torch.arange(0, N * T + 1, T, dtype=torch.int32)
    full = kda.shortconv_l2norm(*[x.reshape(N * T, H, 128).to(DEV) for x in xs], *wd,
                                cu_seqlens=cu_all.to(DEV), cu_seqlens_host=cu_all)
    cu1 = torch.arange(0, N * T1 + 1, T1, dtype=torch.int32)
    pre = kda.shortconv_l2norm(*[x[:, :T1].reshape(N * T1, H, 128).to(DEV) for x in xs], *wd,
                               cu_seqlens=cu1.to(DEV), cu_seqlens_host=cu1)
    state = pre[3]
    cu_s = torch.arange(0, N + 1, dtype=torch.int32)
    got = [[p.reshape(N, T1, H, 128)] for p in pre[:3]]
    for s in range(steps):
        r = kda.shortconv_l2norm(*[x[:, T1 + s].contiguous().to(DEV) for x in xs], *wd,
                                 cu_seqlens=cu_s.to(DEV), cu_seqlens_host=cu_s,
                                 conv_state=state, state_out=state)
        for z in range(3):
            got[z].append(r[z].reshape(N, 1, H, 128))
    torch.cuda.synchronize()
    for z in range(3):
        assert torch.equal(torch.cat(got[z], dim=1).reshape(N * T, H, 128), full[z])
    assert torch.equal(state, full[3])


def test_prologue_full_layer_shape_every_head():
    """T = 4096, H = 96, bf16 projections (the K3 layer's prefill shape): every
    output of every head against the oracle."""
    need_gpu()
    say("prologue full shape")
    T, H = 4096, 96
    xs, ws, _ = _draw(T, H, torch.bfloat16, 75)
    cu = torch.tensor([0, T], dtype=torch.int32)
    ys = kda.shortconv_l2norm(*[x.to(DEV) for x in xs], *[w.to(DEV) for w in ws],
                              cu_seqlens=cu.to(DEV), cu_seqlens_host=cu)
    torch.cuda.synchronize()
    heads = list(range(H))
    cols = np.concatenate([np.arange(h * 128, h * 128 + 128) for h in heads])
    r = oracle.shortconv_l2norm(*[x[:, heads] for x in xs], *[w[cols] for w in ws],
                                [0, T], len(heads))
    for z in range(3):
        _check(ys[z][:, heads], r[z], torch.bfloat16, "full shape %d" % z)
