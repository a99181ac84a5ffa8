#!/usr/bin/env python3
"""KDA core benchmark on one MI355X.

A step is one pass of the prefill hot path over one batch, from the raw
gate/beta logits to o and the final state: kda_chunk_prefill_gated (the gate
formed in registers inside the chunked prefill), on the K3-layer prefill
workload (one sequence, T=4096, H=96, d=128, bf16 q/k/v, fp32 gate logits,
zero initial state, bf16 o, fp32 final state).  `value` is sequence tokens/s
of that step, inputs already resident in HBM.  The same step as two calls
(kda_gate, then kda_chunk_prefill on g and beta) is timed beside it.

The same JSON line carries
  roofline      the gated prefill call: algorithmic HBM bytes per call / its
                average time (HIP events on the launch stream), against
                8 TB/s; plus its algorithmic MFMA rate
  decode        kda_recurrent_decode on 256 sequences x 96 heads (fp32 state
                [256,96,128,128] updated in place), 64 steps: state-update GB/s
  cpu_baseline  the fp64 oracle (gate + token-by-token recurrence) on a
                bounded sample of the same workload, on this host's cores.
Timing follows the audit page's protocol shape (warmup, repeated timed
launches, event timing, output buffers reused).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s (H=96,d=128) + decode state-update HBM GB/s"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0

T, H, D, C = 4096, 96, 128, 64
# algorithmic bytes of one gated chunk-prefill call: per token q,k,v bf16 +
# gate logits f32 + beta logit f32 + o bf16, plus the fp32 final state written
# once (zero initial state) and the per-head A_log and dt_bias read once
PREFILL_TOKEN_BYTES = H * (3 * D * 2 + D * 4 + 4 + D * 2)            # 147,840
PREFILL_BYTES = T * PREFILL_TOKEN_BYTES + H * D * D * 4 + H * 4 + H * D * 4   # 611,893,632
# algorithmic MACs per (chunk, head) at C=64: A 258,048, P 266,240, solve 41,664,
# U 258,048, W 258,048, W.S / Qt.S / Khat^T.Delta 1,048,576 each, P.Delta 266,240
MAC_PER_CHUNK_HEAD = 4_494_016
PREFILL_FLOPS = 2 * MAC_PER_CHUNK_HEAD * (T // C) * H                 # 5.52e10
# backward, algorithmic MACs per (chunk, head) at C=64 (triangular factors
# counted by their nonzeros, products the kernels form densely counted dense):
#   prep   At 258,048, P 266,240, (I + A)^-1 41,664, W / U / Qt 266,240 each
#   walks  forward and backward, 3 products of 1,048,576 each per direction
#   grad   X, K_D dS, dK_E, dQ_E, dK_D 1,048,576 each; Delta, P^T dO, dY, dM, dP
#          266,240 each; dM M^T, dA 262,144 each; the pairwise At / P terms
#          (4 sums over the lower pairs x 128 channels) 1,048,576
BWD_MAC_PER_CHUNK_HEAD = 1_364_672 + 6_291_456 + 8_146_944            # 15,803,072
BWD_FLOPS = 2 * BWD_MAC_PER_CHUNK_HEAD * (T // C) * H                 # 1.94e11
MFMA_F32_PEAK_TFLOPS = 157.3
# decode: per (sequence, head, step) state read + write, q/k/v bf16, g f32, beta, o bf16
DEC_N, DEC_STEPS = 256, 64
DEC_PAIR_BYTES = 2 * D * D * 4 + 3 * D * 2 + D * 4 + 4 + D * 2       # 132,612
DEC_STEP_BYTES = DEC_N * H * DEC_PAIR_BYTES                           # 3,259,072,512


# HBM traffic of one kda_chunk_prefill call, from the committed rocprofv3
# FETCH_SIZE / WRITE_SIZE summary; valid only while the kernel sources hash to
# the value recorded with the counters.
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "chunk_prefill_T4096_H96_hbm_traffic.md")
CHUNK_SOURCES = ["gated_delta_rule_58_amd/csrc/prep.hip", "gated_delta_rule_58_amd/csrc/prep_chunk.hpp",
                 "gated_delta_rule_58_amd/csrc/state.hip",
                 "gated_delta_rule_58_amd/csrc/chunk_common.hpp",
                 "gated_delta_rule_58_amd/csrc/gate_math.hpp"]


def measured_traffic():
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(l.split(": ", 1) for l in text.splitlines()
                  if l.startswith(("traffic_bytes_per_launch: ", "source_sha256: ")))
    if fields.get("source_sha256", "").strip() != chunk_source_digest():
        return None
    return int(fields["traffic_bytes_per_launch"])


def chunk_source_digest():
    """sha256 of the prefill kernels' code lines: comments and blank lines
    are dropped, so a comment edit keeps the recorded traffic valid."""
    h = hashlib.sha256()
    for f in CHUNK_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--repeats", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=96,
                    help="heads of the workload the CPU oracle runs (sample)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle sample until this much time is spent")
    ap.add_argument("--ws-chunks", type=int, default=T // C,
                    help="chunks per pass the prefill workspace holds (T/64 = one pass)")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "prologue", "workloads",
                                       "backward", "copy", "states", "sweep"],
                    default="all",
                    help="profiling aid: run one part only (prints a diagnostic line, "
                         "not the bench line)")
    return ap.parse_args()


def bench_length_sweep(args, torch, kda, synth):
    """kda_chunk_prefill_gated (o bf16, fp32 final state) and
    kda_chunk_prefill_backward (bf16 d_o) on one sequence of T tokens, H = 96,
    for T = 1,024 .. 131,072 (the T=4096 recipe at other lengths).  Each point
    first runs its call for 0.3 s so the clocks have settled, then times about
    300 ms of calls (at least 2) with events."""
    dev = "cuda:0"
    import time

    def timeit(fn, reps):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            fn()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    points = []
    for Tn in (1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072):
        dr = synth.draw_prefill([Tn], H, torch.bfloat16, False, 7, dev)
        cu_h = dr.cu_seqlens
        cu_d = cu_h.to(dev)
        ws = torch.empty(kda.chunk_prefill_workspace_bytes(1, H, D, D, (Tn + C - 1) // C),
                         dtype=torch.uint8, device=dev)
        o = torch.empty((Tn, H, D), dtype=torch.bfloat16, device=dev)
        Sf = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)

        def fwd():
            kda.chunk_prefill_gated(dr.q, dr.k, dr.v, dr.x, dr.b, dr.A_log, dr.dt_bias, cu_d,
                                    None, out=o, final_state=Sf, cu_seqlens_host=cu_h,
                                    workspace=ws)
        ms = timeit(fwd, max(5, 4_000_000 // Tn))
        del ws, o, Sf
        g, beta = kda.gate(dr.x, dr.b, dr.A_log, dr.dt_bias)
        d_o = torch.randn((Tn, H, D), device=dev,
                          generator=torch.Generator(device=dev).manual_seed(5)).to(torch.bfloat16)
        wsb = torch.empty(kda.chunk_prefill_backward_workspace_bytes(Tn, 1, H), dtype=torch.uint8,
                          device=dev)

        def bwd():
            kda.chunk_prefill_backward(dr.q, dr.k, dr.v, g, beta, d_o, cu_d, None,
                                       want_d_initial_state=False, cu_seqlens_host=cu_h,
                                       workspace=wsb)
        bms = timeit(bwd, max(2, 400_000 // Tn))
        points.append(dict(T=Tn, prefill_ms=ms, prefill_tokens_per_s=Tn / (ms * 1e-3),
                           backward_ms=bms, backward_tokens_per_s=Tn / (bms * 1e-3)))
        del dr, g, beta, d_o, wsb
        torch.cuda.empty_cache()
    return dict(workload="one sequence of T tokens, H=96, bf16 q/k/v, fp32 gate logits",
                points=points)


def bench_copy(args, torch):
    """A plain device copy of known size (1 GiB read + 1 GiB written per launch),
    used to calibrate the FETCH_SIZE / WRITE_SIZE counters."""
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(max(1, args.warmup)):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    return dict(bytes_read=4 * n, bytes_written=4 * n, ms=ms, GBps=8 * n / (ms * 1e-3) / 1e9)


def bench_prefill(args, torch, kda, synth):
    dev = "cuda:0"
    dr = synth.draw_config(1, device=dev)
    cu_h = dr.cu_seqlens
    cu_d = cu_h.to(dev)
    g = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    beta = torch.empty((T, H), dtype=torch.float32, device=dev)
    o = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    Sf = torch.empty((1, H, D, D), dtype=torch.float32, device=dev)

    def gate():
        kda.gate(dr.x, dr.b, dr.A_log, dr.dt_bias, g_out=g, beta_out=beta)

    def fused():
        kda.chunk_prefill_gated(dr.q, dr.k, dr.v, dr.x, dr.b, dr.A_log, dr.dt_bias, cu_d, None,
                                out=o, final_state=Sf, cu_seqlens_host=cu_h, workspace=ws)

    ws = torch.empty(kda.chunk_prefill_workspace_bytes(1, H, D, D, args.ws_chunks),
                     dtype=torch.uint8, device=dev)

    def prefill():
        kda.chunk_prefill(dr.q, dr.k, dr.v, g, beta, cu_d, None, out=o, final_state=Sf,
                          cu_seqlens_host=cu_h, workspace=ws)

    def timed(fns):
        """Per-step event times of the calls in fns (in order), over repeats x steps."""
        for _ in range(args.warmup):
            for f in fns:
                f()
        torch.cuda.synchronize()
        per = [[] for _ in fns]
        for _ in range(args.repeats):
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
                  for _ in range(args.steps)]
            torch.cuda.synchronize()
            for i in range(args.steps):
                ev[i][0].record()
                for j, f in enumerate(fns):
                    f()
                    ev[i][j + 1].record()
            torch.cuda.synchronize()
            for i in range(args.steps):
                for j in range(len(fns)):
                    per[j].append(ev[i][j].elapsed_time(ev[i][j + 1]))
        steps = [sum(x) for x in zip(*per)]
        return per, steps

    (fz,), fsteps = timed([fused])
    (gt, ch), ssteps = timed([gate, prefill])
    mean = lambda x: sum(x) / len(x)
    p95 = lambda x: sorted(x)[int(0.95 * (len(x) - 1))]
    return dict(step_ms=mean(fsteps), p95_step_ms=p95(fsteps), fused_ms=mean(fz),
                sep_step_ms=mean(ssteps), chunk_ms=mean(ch), gate_ms=mean(gt))


def bench_prefill_states(args, torch, kda, synth):
    """kda_chunk_prefill_gated on the T=4096, H=96 workload with the three state
    modes a serving stack uses: no state (neither initial nor final), fp32
    initial and final states, bf16 initial and final states (the initial ones
    drawn N(0, 0.02) per sequence and head)."""
    dev = "cuda:0"
    dr = synth.draw_config(1, device=dev)
    cu_h = dr.cu_seqlens
    cu_d = cu_h.to(dev)
    ws = torch.empty(kda.chunk_prefill_workspace_bytes(1, H, D, D, args.ws_chunks),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    S0 = torch.randn((1, H, D, D), generator=torch.Generator(device=dev).manual_seed(11),
                     device=dev) * 0.02
    modes = {"none": (None, None),
             "fp32": (S0, torch.empty_like(S0)),
             "bf16": (S0.to(torch.bfloat16), torch.empty_like(S0, dtype=torch.bfloat16))}
    out = {}
    for name, (si, sf) in modes.items():
        def call():
            kda.chunk_prefill_gated(dr.q, dr.k, dr.v, dr.x, dr.b, dr.A_log, dr.dt_bias, cu_d, si,
                                    output_final_state=sf is not None, out=o, final_state=sf,
                                    cu_seqlens_host=cu_h, workspace=ws)
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        times = []
        for _ in range(args.repeats):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            ev[0].record()
            for i in range(args.steps):
                call()
                ev[i + 1].record()
            torch.cuda.synchronize()
            times += [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
        ms = sum(times) / len(times)
        es = 0 if si is None else si.element_size()
        nbytes = T * PREFILL_TOKEN_BYTES + 2 * H * D * D * es + H * 4 + H * D * 4
        out[name] = dict(ms=ms, tokens_per_s=T / (ms * 1e-3), alg_bytes=nbytes,
                         alg_GBps=nbytes / (ms * 1e-3) / 1e9)
    return out


def bench_prefill_workload(args, torch, kda, synth, idx):
    """kda_chunk_prefill_gated on prefill workload idx at its full size (2: 8 packed
    sequences of 32,768 tokens with initial states; 3: one sequence of 131,072
    tokens), one pass (the workspace holds every chunk of the longest sequence)."""
    dev = "cuda:0"
    c = synth.CONFIGS[idx]
    dr = synth.draw_config(idx, device=dev)
    cu_h = dr.cu_seqlens
    cu_d = cu_h.to(dev)
    Tw = int(cu_h[-1])
    Nw = cu_h.numel() - 1
    max_len = int((cu_h[1:] - cu_h[:-1]).max())
    ws = torch.empty(kda.chunk_prefill_workspace_bytes(Nw, H, D, D, (max_len + C - 1) // C),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((Tw, H, D), dtype=torch.bfloat16, device=dev)
    Sf = torch.empty((Nw, H, D, D), dtype=torch.float32, device=dev)

    def call():
        kda.chunk_prefill_gated(dr.q, dr.k, dr.v, dr.x, dr.b, dr.A_log, dr.dt_bias, cu_d,
                                dr.initial_state, out=o, final_state=Sf, cu_seqlens_host=cu_h,
                                workspace=ws)
    reps = max(1, min(args.steps, 10))
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    times = []
    for _ in range(args.repeats):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            call()
            ev[i + 1].record()
        torch.cuda.synchronize()
        times += [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    ms = sum(times) / len(times)
    nbytes = (Tw * PREFILL_TOKEN_BYTES + Nw * H * D * D * 4 * (2 if dr.initial_state is not None else 1)
              + H * 4 + H * D * 4)
    del ws, dr
    gbs = nbytes / (ms * 1e-3) / 1e9
    return dict(workload=c["name"], tokens=Tw,
                sequences=Nw, ms=ms, tokens_per_s=Tw / (ms * 1e-3), alg_GBps=gbs,
                frac=gbs / HBM_PEAK_GBS)


def bench_decode(args, torch, kda, synth):
    dev = "cuda:0"
    c = synth.CONFIGS[4]
    A_log, dt_bias, state = synth.draw_decode_params(DEC_N, H, seed=c["seed"], device=dev)
    steps = []
    for s in range(DEC_STEPS):
        st = synth.draw_decode_step(DEC_N, H, s, seed=c["seed"], device=dev)
        g, beta = kda.gate(st.x, st.b, A_log, dt_bias)
        steps.append((st.q, st.k, st.v, g, beta))
        del st
    o = torch.empty((DEC_N, H, D), dtype=torch.bfloat16, device=dev)
    for s in range(min(args.warmup, DEC_STEPS)):
        q, k, v, g, beta = steps[s]
        kda.recurrent_decode(q, k, v, g, beta, state, out=o)
    torch.cuda.synchronize()
    times = []
    for _ in range(args.repeats):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(DEC_STEPS + 1)]
        ev[0].record()
        for s in range(DEC_STEPS):
            q, k, v, g, beta = steps[s]
            kda.recurrent_decode(q, k, v, g, beta, state, out=o)
            ev[s + 1].record()
        torch.cuda.synchronize()
        times += [ev[s].elapsed_time(ev[s + 1]) for s in range(DEC_STEPS)]
    ms = sum(times) / len(times)
    gbs = DEC_STEP_BYTES / (ms * 1e-3) / 1e9
    return dict(ms_per_step=ms, GBps=gbs, frac=gbs / HBM_PEAK_GBS, steps=DEC_STEPS,
                bytes_per_step=DEC_STEP_BYTES)


def bench_decode_gated(args, torch, kda, synth, state_dtype):
    """kda_recurrent_decode_gated on the decode workload's shape: fp32 gate and
    beta logits in, a pool of 256 states (fp32 or bf16) addressed through a
    permutation of the slots, updated in place."""
    dev = "cuda:0"
    c = synth.CONFIGS[4]
    A_log, dt_bias, S0 = synth.draw_decode_params(DEC_N, H, seed=c["seed"], device=dev)
    pool = S0.to(state_dtype).contiguous()
    del S0
    perm = torch.randperm(DEC_N, generator=torch.Generator().manual_seed(3))
    ind = perm.to(torch.int32).to(dev)
    steps = [synth.draw_decode_step(DEC_N, H, s, seed=c["seed"], device=dev)
             for s in range(DEC_STEPS)]
    steps = [(st.q, st.k, st.v, st.x.float(), st.b.float()) for st in steps]
    o = torch.empty((DEC_N, H, D), dtype=torch.bfloat16, device=dev)

    def step(s):
        q, k, v, x, b = steps[s]
        kda.recurrent_decode_gated(q, k, v, x, b, A_log, dt_bias, pool, state_indices=ind,
                                   out=o)
    for s in range(min(args.warmup, DEC_STEPS)):
        step(s)
    torch.cuda.synchronize()
    times = []
    for _ in range(args.repeats):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(DEC_STEPS + 1)]
        ev[0].record()
        for s in range(DEC_STEPS):
            step(s)
            ev[s + 1].record()
        torch.cuda.synchronize()
        times += [ev[s].elapsed_time(ev[s + 1]) for s in range(DEC_STEPS)]
    ms = sum(times) / len(times)
    es = 2 if state_dtype == torch.bfloat16 else 4
    # per (sequence, head): state in + out, q/k/v bf16, x fp32, b fp32, o bf16;
    # per step: the slot indices and the per-head A_log and dt_bias
    pair = 2 * D * D * es + 3 * D * 2 + D * 4 + 4 + D * 2
    nbytes = DEC_N * H * pair + DEC_N * 4 + H * 4 + H * D * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return dict(ms_per_step=ms, GBps=gbs, frac=gbs / HBM_PEAK_GBS, bytes_per_step=nbytes,
                tokens_per_s=DEC_N / (ms * 1e-3))


def bench_prologue(args, torch, kda):
    """kda_shortconv_l2norm at the K3 layer's prefill shape: T=4096, H=96, bf16
    q/k/v projections in and out, SiLU, conv state out."""
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(5)
    xs = [torch.randn((T, H, D), generator=g, device=dev).to(torch.bfloat16) for _ in range(3)]
    ws = [torch.randn((H * D, 4), generator=g, device=dev) * 0.5 for _ in range(3)]
    cu = torch.tensor([0, T], dtype=torch.int32)
    cud = cu.to(dev)
    st = torch.empty((1, 3, 3, H * D), dtype=torch.float32, device=dev)

    def call():
        kda.shortconv_l2norm(*xs, *ws, cu_seqlens=cud, cu_seqlens_host=cu, state_out=st)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    times = []
    for _ in range(args.repeats):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record()
        for i in range(args.steps):
            call()
            ev[i + 1].record()
        torch.cuda.synchronize()
        times += [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = sum(times) / len(times)
    nbytes = 2 * 3 * T * H * D * 2 + 3 * H * D * 4 * 4 + 9 * H * D * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return dict(ms=ms, GBps=gbs, frac=gbs / HBM_PEAK_GBS, bytes=nbytes,
                tokens_per_s=T / (ms * 1e-3))


def bench_backward(args, torch, kda, synth):
    """kda_chunk_prefill_backward at the benchmarked prefill shape: T=4096, H=96,
    bf16 q/k/v and d_o, fp32 g/beta (from kda_gate), zero initial state,
    gradients of q, k, v, g, beta (fp32 out)."""
    dev = "cuda:0"
    dr = synth.draw_config(1, device=dev)
    cu_h = dr.cu_seqlens
    cu_d = cu_h.to(dev)
    g, beta = kda.gate(dr.x, dr.b, dr.A_log, dr.dt_bias)
    d_o = torch.randn((T, H, D), generator=torch.Generator(device=dev).manual_seed(9),
                      device=dev).to(torch.bfloat16)
    ws = torch.empty(kda.chunk_prefill_backward_workspace_bytes(T, 1, H), dtype=torch.uint8,
                     device=dev)

    def call():
        kda.chunk_prefill_backward(dr.q, dr.k, dr.v, g, beta, d_o, cu_d, None,
                                   want_d_initial_state=False, cu_seqlens_host=cu_h,
                                   workspace=ws)
    for _ in range(max(1, args.warmup)):
        call()
    torch.cuda.synchronize()
    nsteps = max(1, args.steps // 4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(nsteps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / nsteps
    # q, k, v, d_o bf16 + g fp32 + beta in; dq, dk, dv, dg fp32 + dbeta out
    nbytes = T * H * (D * (3 * 2 + 2 + 4 + 4 * 4) + 4 + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tf = BWD_FLOPS / (ms * 1e-3) / 1e12
    return dict(ms=ms, tokens_per_s=T / (ms * 1e-3), GBps=gbs, frac=gbs / HBM_PEAK_GBS,
                bytes=nbytes, workspace_bytes=ws.numel(),
                roofline={"bound": "mfma", "achieved": tf, "peak": MFMA_F32_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": tf / MFMA_F32_PEAK_TFLOPS,
                          "alg_flops_per_call": BWD_FLOPS,
                          "alg_mac_per_chunk_head": BWD_MAC_PER_CHUNK_HEAD,
                          "precision": "fp32 products on fp32 16x16x4 MFMA, except the walk's "
                                       "(its state update, and Z = A1 R with bf16 d_o): bf16 "
                                       "16x16x32 MFMA on three-term bf16 splits (fp32-exact; "
                                       "with bf16 d_o, Qt^T dO takes d_o as is), priced at "
                                       "the fp32 peak"})


def cpu_baseline(args, synth):
    """fp64 oracle on `cpu_heads` of the 96 heads of the same T=4096 workload."""
    import numpy as np
    import torch
    import oracle
    nh = max(1, min(args.cpu_heads, H))
    dr = synth.draw_config(1, device="cpu")
    heads = list(range(nh))
    x = dr.x[:, heads].contiguous()
    b = dr.b[:, heads].contiguous()
    q = dr.q[:, heads].double().numpy()
    k = dr.k[:, heads].double().numpy()
    v = dr.v[:, heads].double().numpy()
    # the whole call is about a second on 16 cores: repeat it for ~10 s of CPU
    # work and report the mean of the repeats
    reps, total = 0, 0.0
    while reps < 30 and (reps == 0 or total < args.cpu_seconds):
        t0 = time.perf_counter()
        g, beta = oracle.gate(x, b, dr.A_log[heads], dr.dt_bias[heads])
        o, S, threads = oracle.prefill(q, k, v, g, beta, dr.cu_seqlens, return_threads=True)
        total += time.perf_counter() - t0
        reps += 1
    full_s = total / reps * H / nh
    return {"value": T / full_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": "T=4096 tokens on %d of 96 heads (fp64 gate + token-by-token recurrence), "
                      "%d runs, %.1f s in all, scaled to 96 heads" % (nh, reps, total)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import gated_delta_rule_58_amd as kda
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    kda.lib()
    if args.only != "all":
        fn = {"prefill": lambda: bench_prefill(args, torch, kda, synth),
              "decode": lambda: dict(plain=bench_decode(args, torch, kda, synth),
                                     gated_f32_pool=bench_decode_gated(args, torch, kda, synth,
                                                                       torch.float32),
                                     gated_bf16_pool=bench_decode_gated(args, torch, kda, synth,
                                                                        torch.bfloat16)),
              "prologue": lambda: bench_prologue(args, torch, kda),
              "states": lambda: bench_prefill_states(args, torch, kda, synth),
              "backward": lambda: bench_backward(args, torch, kda, synth),
              "workloads": lambda: {str(i): bench_prefill_workload(args, torch, kda, synth, i)
                                    for i in (2, 3)},
              "copy": lambda: bench_copy(args, torch),
              "sweep": lambda: bench_length_sweep(args, torch, kda, synth)}[args.only]
        print(json.dumps({"diagnostic": args.only, **fn()}), flush=True)
        return
    pre = bench_prefill(args, torch, kda, synth)
    print("prefill: step (gated prefill) %.4f ms, p95 %.4f ms; gate + prefill %.4f ms "
          "(gate %.4f, chunk %.4f)" % (pre["step_ms"], pre["p95_step_ms"], pre["sep_step_ms"],
                                      pre["gate_ms"], pre["chunk_ms"]),
          file=sys.stderr, flush=True)
    stm = bench_prefill_states(args, torch, kda, synth)
    print("prefill state modes: " + ", ".join("%s %.4f ms" % (k, v["ms"]) for k, v in stm.items()),
          file=sys.stderr, flush=True)
    dec = bench_decode(args, torch, kda, synth)
    print("decode: %.4f ms/step, %.1f GB/s" % (dec["ms_per_step"], dec["GBps"]),
          file=sys.stderr, flush=True)
    dg = {}
    for name, sdt in (("gated_f32_pool", torch.float32), ("gated_bf16_pool", torch.bfloat16)):
        dg[name] = bench_decode_gated(args, torch, kda, synth, sdt)
        print("decode %s: %.4f ms/step, %.1f GB/s" % (name, dg[name]["ms_per_step"],
                                                     dg[name]["GBps"]),
              file=sys.stderr, flush=True)
    wl = {}
    for i, name in ((2, "varlen_8seq_32768"), (3, "long_131072")):
        wl[name] = bench_prefill_workload(args, torch, kda, synth, i)
        print("prefill workload %s: %.3f ms, %.2f M tokens/s" % (name, wl[name]["ms"],
                                                                 wl[name]["tokens_per_s"] / 1e6),
              file=sys.stderr, flush=True)
    pro = bench_prologue(args, torch, kda)
    print("prologue (short conv + SiLU + q/k L2 norm): %.4f ms, %.1f GB/s"
          % (pro["ms"], pro["GBps"]), file=sys.stderr, flush=True)
    cp = bench_copy(argparse.Namespace(steps=8, warmup=2), torch)
    print("copy (1 GiB read + 1 GiB written): %.1f GB/s" % cp["GBps"], file=sys.stderr,
          flush=True)
    bwd = bench_backward(args, torch, kda, synth)
    print("prefill backward: %.3f ms, %.2f M tokens/s" % (bwd["ms"], bwd["tokens_per_s"] / 1e6),
          file=sys.stderr, flush=True)
    step_s = pre["fused_ms"] * 1e-3
    ach = PREFILL_BYTES / step_s / 1e9
    mfma = PREFILL_FLOPS / step_s / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args, synth)
    line = {
        "metric": METRIC,
        "value": T / (pre["step_ms"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma/f32-acc (bf16 q/k/v/o, f32 g/beta/state)",
        "data": "synthetic",
        "config": {"workload": "k3-layer-prefill T=4096 H=96 d=128: kda_chunk_prefill_gated "
                               "(gate logits -> o and final state, one call)",
                   "T": T, "H": H, "d": D, "chunk": C, "qkv": "bf16", "o": "bf16",
                   "gate_logits": "f32", "initial_state": "zero", "repeats": args.repeats},
        "prefill": {"step_ms": pre["step_ms"], "p95_step_ms": pre["p95_step_ms"],
                    "gate_then_prefill_ms": pre["sep_step_ms"],
                    "gate_kernel_ms": pre["gate_ms"], "chunk_prefill_ms": pre["chunk_ms"],
                    "chunk_prefill_tokens_per_s": T / (pre["chunk_ms"] * 1e-3)},
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "frac_of_measured_copy": ach / cp["GBps"],
                     "kernel": "kda_chunk_prefill_gated (prep_kernel + state_kernel, one pass)",
                     "alg_bytes_per_launch": PREFILL_BYTES},
        "roofline_mfma": {"achieved": mfma, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": mfma / MFMA_F16_PEAK_TFLOPS,
                          "alg_flops_per_launch": PREFILL_FLOPS},
        "decode": {"workload": "256 seqs x 96 heads x 1 token, 64 steps, fp32 state in place",
                   "ms_per_step": dec["ms_per_step"], "GBps": dec["GBps"], "frac": dec["frac"],
                   "frac_of_measured_copy": dec["GBps"] / cp["GBps"],
                   "bytes_per_step": DEC_STEP_BYTES,
                   "gated": {"workload": "kda_recurrent_decode_gated: fp32 gate/beta logits, "
                                         "state pool of 256 slots addressed by a permutation",
                             **{k: {kk: dg[k][kk] for kk in ("ms_per_step", "GBps", "frac",
                                                             "tokens_per_s", "bytes_per_step")}
                                for k in dg}}},
        "prefill_state_modes": {"workload": "kda_chunk_prefill_gated T=4096 H=96: no state / "
                                            "fp32 initial+final / bf16 initial+final",
                                **stm},
        "prefill_workloads": wl,
        "prologue": {"workload": "kda_shortconv_l2norm T=4096 H=96 bf16 q/k/v in and out, "
                                 "SiLU, conv state out",
                     "ms": pro["ms"], "GBps": pro["GBps"], "frac": pro["frac"],
                     "bytes_per_call": pro["bytes"], "tokens_per_s": pro["tokens_per_s"]},
        "copy": {"workload": "device copy of 1 GiB (read + write), the measured bandwidth "
                             "ceiling the fractions of_measured_copy use",
                 "GBps": cp["GBps"], "ms": cp["ms"]},
        "prefill_backward": {"workload": "kda_chunk_prefill_backward T=4096 H=96, bf16 "
                                         "q/k/v and d_o, fp32 g/beta, zero initial state",
                             **bwd},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
