// C ABI of libkda: argument validation, error reporting and launches.
//
// Every entry point validates all of its arguments before touching the HIP
// runtime, so a refused call launches nothing, writes nothing and makes no
// HIP call at all (which also lets the refusals be tested on a machine with
// no GPU).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "kda_internal.hpp"

namespace {

thread_local char g_err[512] = "";

kda_status fail(kda_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

kda_status ok() {
  g_err[0] = '\0';
  return KDA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool known_dtype(kda_dtype d) { return d == KDA_F32 || d == KDA_BF16; }

// A_log is one value per head ([H]) or, given explicitly, one per (head,
// channel) ([H, d]); any other length, the checkpoint's [128] among them, is
// refused rather than reshaped (Kimi K3 artifact audit, §5.2).
kda_status check_alog(const char* fn, int64_t len, int32_t H, int32_t d, bool* per_channel) {
  *per_channel = len != H && len == (int64_t)H * d;
  if (len == H || *per_channel) return KDA_OK;
  return fail(KDA_ERR_SHAPE,
              "%s: A_log has %lld values but H = %d, d = %d; A_log must be [H] (per head) or "
              "[H, d] (per head and channel); other shapes are refused, not reshaped",
              fn, (long long)len, H, d);
}

kda_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KDA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// Runs a call's launches (`run`).  With KDA_DEBUG=1 `pre` first adds the scans
// of its inputs (a failure returns KDA_ERR_DOMAIN before `run`), and `post`
// the scans of its outputs after it (KDA_ERR_NONFINITE); the call then waits
// for its stream.
template <class Pre, class Run, class Post>
kda_status run_checked(const char* fn, hipStream_t s, Pre pre, Run run, Post post) {
  if (!kda::dbg::enabled()) return launched(run(), fn);
  std::lock_guard<std::mutex> lock(kda::dbg::mutex());
  kda::dbg::Session ses(s);
  std::string rep;
  hipError_t e = ses.begin();
  if (e == hipSuccess) {
    pre(ses);
    e = ses.finish(&rep);
  }
  if (e != hipSuccess)
    return fail(KDA_ERR_LAUNCH, "%s (KDA_DEBUG): input scan failed: %s", fn, hipGetErrorString(e));
  if (!rep.empty())
    return fail(KDA_ERR_DOMAIN, "%s (KDA_DEBUG): %s; nothing was launched", fn, rep.c_str());
  e = run();
  if (e != hipSuccess) return launched(e, fn);
  e = ses.begin();
  if (e == hipSuccess) {
    post(ses);
    e = ses.finish(&rep);
  }
  if (e != hipSuccess)
    return fail(KDA_ERR_LAUNCH, "%s (KDA_DEBUG): output scan failed: %s", fn,
                hipGetErrorString(e));
  if (!rep.empty()) return fail(KDA_ERR_NONFINITE, "%s (KDA_DEBUG): %s", fn, rep.c_str());
  return ok();
}

using kda::dbg::kFinite;
using kda::dbg::kNonPositive;
using kda::dbg::kNotNaN;
using kda::dbg::kUnit;

}  // namespace

extern "C" {

const char* kda_last_error(void) { return g_err; }

const char* kda_version(void) { return "kda-gfx950 0.1"; }

kda_status kda_gate(const void* x, kda_dtype x_dt, const void* b, kda_dtype b_dt,
                    const float* A_log, int64_t A_log_len, const float* dt_bias,
                    int64_t dt_bias_len, float* g_out, float* beta_out, int64_t n_tok,
                    int32_t H, int32_t d, void* stream) {
  if (n_tok < 0 || H <= 0 || d <= 0)
    return fail(KDA_ERR_INVALID_ARG, "kda_gate: need n_tok >= 0, H > 0, d > 0 (got %lld, %d, %d)",
                (long long)n_tok, H, d);
  if (!known_dtype(x_dt) || !known_dtype(b_dt))
    return fail(KDA_ERR_DTYPE, "kda_gate: x_dt and b_dt must be KDA_F32 or KDA_BF16");
  bool alog_pc = false;
  if (const kda_status st = check_alog("kda_gate", A_log_len, H, d, &alog_pc)) return st;
  if (dt_bias_len != (int64_t)H * d)
    return fail(KDA_ERR_SHAPE, "kda_gate: dt_bias has %lld values, need H*d = %lld",
                (long long)dt_bias_len, (long long)H * d);
  if (d % 4 != 0 || d > 1024)
    return fail(KDA_ERR_UNSUPPORTED, "kda_gate: d must be a multiple of 4 and at most 1024 (got %d)",
                d);
  if ((H + 256 / (d / 4) - 1) / (256 / (d / 4)) > 65535)
    return fail(KDA_ERR_UNSUPPORTED, "kda_gate: H = %d is too large for d = %d", H, d);
  if (!A_log || !dt_bias) return fail(KDA_ERR_INVALID_ARG, "kda_gate: A_log/dt_bias is NULL");
  if (n_tok == 0) return ok();
  if (!x || !b || !g_out || !beta_out)
    return fail(KDA_ERR_INVALID_ARG, "kda_gate: x, b, g_out and beta_out must be non-NULL");
  if (!aligned(x, x_dt == KDA_BF16 ? 8 : 16) || !aligned(g_out, 16) || !aligned(dt_bias, 16))
    return fail(KDA_ERR_ALIGNMENT, "kda_gate: x, g_out and dt_bias must be 16-byte aligned "
                                   "(8-byte for bf16 x)");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nx = n_tok * H * d, nb = n_tok * H;
  const int64_t na = alog_pc ? (int64_t)H * d : H;
  return run_checked(
      "kda_gate", s,
      [&](kda::dbg::Session& c) {
        c.add("x", x, nx, x_dt == KDA_BF16, kNotNaN);
        c.add("b", b, nb, b_dt == KDA_BF16, kNotNaN);
        c.add("A_log", A_log, na, false, kFinite);
        c.add("dt_bias", dt_bias, (int64_t)H * d, false, kFinite);
      },
      [&] {
        return kda::launch_gate(x, x_dt == KDA_BF16, b, b_dt == KDA_BF16, A_log, alog_pc,
                                dt_bias, g_out, beta_out, n_tok, H, d, s);
      },
      [&](kda::dbg::Session& c) {
        c.add("g", g_out, nx, false, kNotNaN);
        c.add("beta", beta_out, nb, false, kNotNaN);
      });
}

size_t kda_gate_backward_workspace_bytes(int64_t n_tok, int32_t H, int32_t d) {
  if (n_tok < 0 || H <= 0 || d <= 0) return 0;
  return kda::gate_bwd_workspace_bytes(n_tok, H, d);
}

kda_status kda_gate_backward(const void* x, kda_dtype x_dt, const void* b, kda_dtype b_dt,
                             const float* A_log, int64_t A_log_len, const float* dt_bias,
                             int64_t dt_bias_len, const float* dg, const float* dbeta, float* dx,
                             float* db, float* dA_log, float* ddt_bias, int64_t n_tok,
                             int32_t H, int32_t d, void* workspace, size_t workspace_bytes,
                             void* stream) {
  const char* fn = "kda_gate_backward";
  if (n_tok < 0 || H <= 0 || d <= 0)
    return fail(KDA_ERR_INVALID_ARG, "%s: need n_tok >= 0, H > 0, d > 0 (got %lld, %d, %d)", fn,
                (long long)n_tok, H, d);
  if (!known_dtype(x_dt) || !known_dtype(b_dt))
    return fail(KDA_ERR_DTYPE, "%s: x_dt and b_dt must be KDA_F32 or KDA_BF16", fn);
  bool alog_pc = false;
  if (const kda_status st = check_alog(fn, A_log_len, H, d, &alog_pc)) return st;
  if (dt_bias_len != (int64_t)H * d)
    return fail(KDA_ERR_SHAPE, "%s: dt_bias has %lld values, need H*d = %lld", fn,
                (long long)dt_bias_len, (long long)H * d);
  if (d % 4 != 0 || d > 1024)
    return fail(KDA_ERR_UNSUPPORTED, "%s: d must be a multiple of 4 and at most 1024 (got %d)", fn,
                d);
  if ((H + 256 / (d / 4) - 1) / (256 / (d / 4)) > 65535 || n_tok > ((int64_t)1 << 31) - 1)
    return fail(KDA_ERR_UNSUPPORTED, "%s: H = %d or n_tok = %lld is too large", fn, H,
                (long long)n_tok);
  if (!A_log || !dt_bias || !dA_log || !ddt_bias)
    return fail(KDA_ERR_INVALID_ARG, "%s: A_log, dt_bias, dA_log and ddt_bias must be non-NULL",
                fn);
  if (n_tok > 0 && (!x || !b || !dg || !dbeta || !dx || !db))
    return fail(KDA_ERR_INVALID_ARG, "%s: x, b, dg, dbeta, dx and db must be non-NULL", fn);
  if (!aligned(x, x_dt == KDA_BF16 ? 8 : 16) || !aligned(dg, 16) || !aligned(dx, 16) ||
      !aligned(dt_bias, 16) || !aligned(A_log, 4) || !aligned(b, b_dt == KDA_BF16 ? 2 : 4) ||
      !aligned(dbeta, 4) || !aligned(db, 4) || !aligned(dA_log, 4) || !aligned(ddt_bias, 4))
    return fail(KDA_ERR_ALIGNMENT, "%s: x, dg, dx and dt_bias must be 16-byte aligned (8 for "
                                   "bf16 x), the rest aligned to their element size", fn);
  const size_t need = kda::gate_bwd_workspace_bytes(n_tok, H, d);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(KDA_ERR_WORKSPACE, "%s: need a workspace of at least %zu bytes (got %zu)", fn,
                need, workspace_bytes);
  if (!aligned(workspace, 16))
    return fail(KDA_ERR_ALIGNMENT, "%s: workspace must be 16-byte aligned", fn);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nx = n_tok * H * d, nb = n_tok * H;
  const int64_t na = alog_pc ? (int64_t)H * d : H;
  return run_checked(
      fn, s,
      [&](kda::dbg::Session& c) {
        c.add("x", x, nx, x_dt == KDA_BF16, kNotNaN);
        c.add("b", b, nb, b_dt == KDA_BF16, kNotNaN);
        c.add("A_log", A_log, na, false, kFinite);
        c.add("dt_bias", dt_bias, (int64_t)H * d, false, kFinite);
        c.add("dg", dg, nx, false, kFinite);
        c.add("dbeta", dbeta, nb, false, kFinite);
      },
      [&] {
        return kda::launch_gate_backward(x, x_dt == KDA_BF16, b, b_dt == KDA_BF16, A_log,
                                         alog_pc, dt_bias, dg, dbeta, dx, db, dA_log, ddt_bias,
                                         n_tok, H, d, workspace, s);
      },
      [&](kda::dbg::Session& c) {
        c.add("dx", dx, nx, false, kFinite);
        c.add("db", db, nb, false, kFinite);
        c.add("dA_log", dA_log, na, false, kFinite);
        c.add("ddt_bias", ddt_bias, (int64_t)H * d, false, kFinite);
      });
}

}  // extern "C"

namespace {

// Checks shared by both prefill entry points; `fn` names the caller.
// decay / decay_al: g (or x) and its alignment; bb / bb_al: beta (or its logits).
kda_status check_prefill(const char* fn, const void* q, const void* k, const void* v,
                         kda_dtype qkv_dt, const void* decay, size_t decay_al, const void* bb,
                         size_t bb_al, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                         int32_t N, const void* initial_state, const void* final_state,
                         const void* o, kda_dtype o_dt, int64_t T_tot, int32_t H, int32_t dk,
                         int32_t dv, float scale, const void* workspace, size_t workspace_bytes,
                         bool backward = false) {
  if (N <= 0 || H <= 0 || T_tot < 0)
    return fail(KDA_ERR_INVALID_ARG, "%s: need N > 0, H > 0, T_tot >= 0 (got %d, %d, %lld)", fn,
                N, H, (long long)T_tot);
  if (!known_dtype(qkv_dt) || !known_dtype(o_dt))
    return fail(KDA_ERR_DTYPE, "%s: qkv_dt and o_dt must be KDA_F32 or KDA_BF16", fn);
  if (dk != 128 || dv != 128)
    return fail(KDA_ERR_UNSUPPORTED, "%s: only dk = dv = 128 is implemented (got %d, %d)", fn,
                dk, dv);
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f)
    return fail(KDA_ERR_INVALID_ARG, "%s: scale must be finite", fn);
  if (T_tot > ((int64_t)1 << 31) - 1)
    return fail(KDA_ERR_UNSUPPORTED, "%s: T_tot must fit in int32", fn);
  if (!cu_seqlens) return fail(KDA_ERR_INVALID_ARG, "%s: cu_seqlens is NULL", fn);
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] != 0 || cu_seqlens_host[N] != T_tot)
      return fail(KDA_ERR_SHAPE, "%s: cu_seqlens must start at 0 and end at T_tot = %lld "
                                 "(got %d .. %d)", fn, (long long)T_tot, cu_seqlens_host[0],
                  cu_seqlens_host[N]);
    for (int32_t n = 0; n < N; ++n)
      if (cu_seqlens_host[n + 1] < cu_seqlens_host[n])
        return fail(KDA_ERR_SHAPE, "%s: cu_seqlens decreases at index %d", fn, n);
  }
  if (T_tot > 0 && (!q || !k || !v || !decay || !bb || !o))
    return fail(KDA_ERR_INVALID_ARG, "%s: q, k, v, the decay input, beta and o must be non-NULL",
                fn);
  const void* ptrs[] = {q, k, v, o, initial_state, final_state};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16))
      return fail(KDA_ERR_ALIGNMENT, "%s: tensors must be 16-byte aligned", fn);
  if (!aligned(decay, decay_al) || !aligned(bb, bb_al) || !aligned(cu_seqlens, 4))
    return fail(KDA_ERR_ALIGNMENT, "%s: the decay input must be %zu-byte aligned, beta %zu-byte, "
                                   "cu_seqlens 4-byte", fn, decay_al, bb_al);
  const size_t ws_min = backward ? kda::bwd::workspace_bytes(T_tot, N, H)
                                 : kda::chunk_workspace_bytes(N, H, 1);
  if (!workspace || workspace_bytes < ws_min)
    return fail(KDA_ERR_WORKSPACE, "%s: need a workspace of at least %zu bytes (got %zu at %p)",
                fn, ws_min, workspace_bytes, workspace);
  if (!aligned(workspace, 256))
    return fail(KDA_ERR_ALIGNMENT, "%s: workspace must be 256-byte aligned", fn);
  if ((int64_t)N * H > ((int64_t)1 << 24) || H > 16384)
    return fail(KDA_ERR_UNSUPPORTED, "%s: need H <= 16384 and N*H <= 2^24", fn);
  return KDA_OK;
}

// The gated prefill's arguments (kda_chunk_prefill_gated without the
// workspace and stream).
struct GatedPrefill {
  const void *q, *k, *v;
  kda_dtype qkv_dt;
  const void* x;
  kda_dtype x_dt;
  const void* b;
  kda_dtype b_dt;
  const float* A_log;
  int64_t A_log_len;
  const float* dt_bias;
  int64_t dt_bias_len;
  const int32_t *cu_seqlens, *cu_seqlens_host;
  int32_t N;
  const void* initial_state;
  void* final_state;
  kda_dtype state_dt;
  int64_t num_slots;
  const int32_t* state_indices;
  void* o;
  kda_dtype o_dt;
  int64_t T_tot;
  int32_t H, dk, dv;
  float scale;
};

// Host-side validation of a gated prefill; `user_ws` says whether the
// workspace is the caller's (then a final-state pool must not overlap it).
kda_status check_gated(const char* fn, const GatedPrefill& a, const void* workspace,
                       size_t workspace_bytes, bool user_ws, bool* alog_pc) {
  if (!known_dtype(a.x_dt) || !known_dtype(a.b_dt) || !known_dtype(a.state_dt))
    return fail(KDA_ERR_DTYPE, "%s: x_dt, b_dt and state_dt must be KDA_F32 or KDA_BF16", fn);
  if (a.num_slots < 0)
    return fail(KDA_ERR_INVALID_ARG, "%s: num_slots must be >= 0 (got %lld)", fn,
                (long long)a.num_slots);
  if ((a.initial_state || a.final_state) && !a.state_indices && a.num_slots < a.N)
    return fail(KDA_ERR_SHAPE, "%s: without state_indices sequence n uses slot n, so num_slots "
                               "must be >= N (got %lld < %d)", fn, (long long)a.num_slots, a.N);
  if (!aligned(a.state_indices, 4))
    return fail(KDA_ERR_ALIGNMENT, "%s: state_indices must be 4-byte aligned", fn);
  *alog_pc = false;
  if (a.H > 0)
    if (const kda_status st = check_alog(fn, a.A_log_len, a.H, a.dk, alog_pc)) return st;
  if (a.H > 0 && a.dt_bias_len != (int64_t)a.H * a.dk)
    return fail(KDA_ERR_SHAPE, "%s: dt_bias has %lld values, need H*dk = %lld", fn,
                (long long)a.dt_bias_len, (long long)a.H * a.dk);
  if (!a.A_log || !a.dt_bias) return fail(KDA_ERR_INVALID_ARG, "%s: A_log/dt_bias is NULL", fn);
  if (!aligned(a.dt_bias, 16) || (*alog_pc && !aligned(a.A_log, 16)))
    return fail(KDA_ERR_ALIGNMENT, "%s: dt_bias (and a per-channel A_log) must be 16-byte "
                                   "aligned", fn);
  const kda_status st = check_prefill(fn, a.q, a.k, a.v, a.qkv_dt, a.x, 16, a.b,
                                      a.b_dt == KDA_BF16 ? 2 : 4, a.cu_seqlens,
                                      a.cu_seqlens_host, a.N, a.initial_state, a.final_state,
                                      a.o, a.o_dt, a.T_tot, a.H, a.dk, a.dv, a.scale, workspace,
                                      workspace_bytes);
  if (st != KDA_OK) return st;
  // the final-state pool must not overlap what the call reads or writes besides
  // the initial-state pool (which it may equal: an in-place update)
  if (a.final_state) {
    const size_t s_es = a.state_dt == KDA_BF16 ? 2 : 4;
    const char* sb = static_cast<const char*>(a.final_state);
    const char* se = sb + (size_t)a.num_slots * a.H * a.dk * a.dv * s_es;
    const size_t qkv_es = a.qkv_dt == KDA_BF16 ? 2 : 4;
    const size_t T = (size_t)a.T_tot;
    struct { const void* p; size_t n; } others[] = {
        {a.q, T * a.H * a.dk * qkv_es}, {a.k, T * a.H * a.dk * qkv_es},
        {a.v, T * a.H * a.dv * qkv_es}, {a.o, T * a.H * a.dv * (a.o_dt == KDA_BF16 ? 2 : 4)},
        {workspace, user_ws ? workspace_bytes : 0},
        {a.state_indices, a.state_indices ? (size_t)a.N * 4 : 0}};
    for (auto& r : others) {
      const char* b0 = static_cast<const char*>(r.p);
      if (r.n && b0 && b0 < se && sb < b0 + r.n)
        return fail(KDA_ERR_INVALID_ARG, "%s: the final-state pool overlaps another tensor", fn);
    }
  }
  return KDA_OK;
}

// Launches a validated gated prefill (under KDA_DEBUG's scans when that is on).
kda_status run_gated(const char* fn, const GatedPrefill& a, bool alog_pc, void* workspace,
                     size_t workspace_bytes, hipStream_t s) {
  const int g_mode = (a.x_dt == KDA_BF16 ? 2 : 1) | (alog_pc ? 4 : 0);
  kda::StatePool pool;
  pool.in = a.initial_state;
  pool.out = a.final_state;
  pool.idx = a.state_indices;
  pool.slots = a.state_indices ? a.num_slots : (a.num_slots < a.N ? a.num_slots : a.N);
  pool.bf16 = a.state_dt == KDA_BF16;
  const bool qb = a.qkv_dt == KDA_BF16;
  const int64_t nt = a.T_tot * a.H * 128;
  const int N = a.N, H = a.H;
  return run_checked(
      fn, s,
      [&](kda::dbg::Session& c) {
        c.add("q", a.q, nt, qb, kFinite);
        c.add("k", a.k, nt, qb, kFinite);
        c.add("v", a.v, nt, qb, kFinite);
        c.add("x", a.x, nt, a.x_dt == KDA_BF16, kNotNaN);
        c.add("b", a.b, a.T_tot * H, a.b_dt == KDA_BF16, kNotNaN);
        c.add("A_log", a.A_log, alog_pc ? (int64_t)H * 128 : H, false, kFinite);
        c.add("dt_bias", a.dt_bias, (int64_t)H * 128, false, kFinite);
        c.add_states("initial_state", a.initial_state, pool.bf16, a.state_indices, pool.slots,
                     N, H);
      },
      [&] {
        return kda::launch_chunk_prefill(a.q, a.k, a.v, qb, a.x, g_mode, a.b, a.b_dt == KDA_BF16,
                                         a.A_log, a.dt_bias, a.cu_seqlens, a.cu_seqlens_host, N,
                                         pool, a.o, a.o_dt == KDA_BF16, a.T_tot, H, a.scale,
                                         workspace, workspace_bytes, s);
      },
      [&](kda::dbg::Session& c) {
        c.add("o", a.o, nt, a.o_dt == KDA_BF16, kFinite);
        c.add_states("final_state", a.final_state, pool.bf16, a.state_indices, pool.slots, N, H);
      });
}

}  // namespace

extern "C" {

kda_status kda_chunk_prefill(const void* q, const void* k, const void* v, kda_dtype qkv_dt,
                             const float* g, const float* beta, const int32_t* cu_seqlens,
                             const int32_t* cu_seqlens_host, int32_t N,
                             const float* initial_state, float* final_state, void* o,
                             kda_dtype o_dt, int64_t T_tot, int32_t H, int32_t dk,
                             int32_t dv, float scale, void* workspace, size_t workspace_bytes,
                             void* stream) {
  const kda_status st = check_prefill("kda_chunk_prefill", q, k, v, qkv_dt, g, 16, beta, 4,
                                      cu_seqlens, cu_seqlens_host, N, initial_state, final_state,
                                      o, o_dt, T_tot, H, dk, dv, scale, workspace,
                                      workspace_bytes);
  if (st != KDA_OK) return st;
  kda::StatePool pool;
  pool.in = initial_state;
  pool.out = final_state;
  pool.slots = N;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool qb = qkv_dt == KDA_BF16;
  const int64_t nt = T_tot * H * 128;
  return run_checked(
      "kda_chunk_prefill", s,
      [&](kda::dbg::Session& c) {
        c.add("q", q, nt, qb, kFinite);
        c.add("k", k, nt, qb, kFinite);
        c.add("v", v, nt, qb, kFinite);
        c.add("g", g, nt, false, kNonPositive);
        c.add("beta", beta, T_tot * H, false, kUnit);
        c.add_states("initial_state", initial_state, false, nullptr, N, N, H);
      },
      [&] {
        return kda::launch_chunk_prefill(q, k, v, qb, g, 0, beta, false, nullptr, nullptr,
                                         cu_seqlens, cu_seqlens_host, N, pool, o,
                                         o_dt == KDA_BF16, T_tot, H, scale, workspace,
                                         workspace_bytes, s);
      },
      [&](kda::dbg::Session& c) {
        c.add("o", o, nt, o_dt == KDA_BF16, kFinite);
        c.add_states("final_state", final_state, false, nullptr, N, N, H);
      });
}

kda_status kda_chunk_prefill_gated(const void* q, const void* k, const void* v, kda_dtype qkv_dt,
                                   const void* x, kda_dtype x_dt, const void* b, kda_dtype b_dt,
                                   const float* A_log, int64_t A_log_len, const float* dt_bias,
                                   int64_t dt_bias_len, const int32_t* cu_seqlens,
                                   const int32_t* cu_seqlens_host, int32_t N,
                                   const void* initial_state, void* final_state,
                                   kda_dtype state_dt, int64_t num_slots,
                                   const int32_t* state_indices, void* o, kda_dtype o_dt,
                                   int64_t T_tot, int32_t H, int32_t dk, int32_t dv, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "kda_chunk_prefill_gated";
  const GatedPrefill a{q, k, v, qkv_dt, x, x_dt, b, b_dt, A_log, A_log_len, dt_bias,
                       dt_bias_len, cu_seqlens, cu_seqlens_host, N, initial_state, final_state,
                       state_dt, num_slots, state_indices, o, o_dt, T_tot, H, dk, dv, scale};
  bool alog_pc = false;
  if (const kda_status st = check_gated(fn, a, workspace, workspace_bytes, true, &alog_pc))
    return st;
  return run_gated(fn, a, alog_pc, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---- kda_chunk_prefill_gated_static: the gated prefill over a workspace that
// lives in this file as a device array, for callers that cannot allocate.
namespace {

constexpr size_t kStaticScratchBytes = size_t(KDA_PREFILL_STATIC_SCRATCH_BYTES);
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];  // per device: device address of `scratch`

// The device address of this device's `scratch` (looked up once per device,
// with that device current).  Host code uses only this address: the array's
// own name in host code is a host-side stand-in, not device memory.
kda_status scratch_for_current_device(const char* fn, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(KDA_ERR_LAUNCH, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(KDA_ERR_UNSUPPORTED, "%s: device %d is beyond the %d the library tracks", fn, dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(KDA_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) failed: %s", fn,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

// (sequence, head) pairs the static scratch holds at one chunk per pass
size_t static_scratch_max_pairs() {
  const size_t per_pair = kda::chunk_workspace_bytes(2, 1, 1) - kda::chunk_workspace_bytes(1, 1, 1);
  const size_t fixed = kda::chunk_workspace_bytes(1, 1, 1) - per_pair;
  return (kStaticScratchBytes - fixed) / per_pair;
}

}  // namespace

extern "C" {

kda_status kda_chunk_prefill_gated_static(
    const void* q, const void* k, const void* v, kda_dtype qkv_dt, const void* x, kda_dtype x_dt,
    const void* b, kda_dtype b_dt, const float* A_log, int64_t A_log_len, const float* dt_bias,
    int64_t dt_bias_len, const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t N,
    const void* initial_state, void* final_state, kda_dtype state_dt, int64_t num_slots,
    const int32_t* state_indices, void* o, kda_dtype o_dt, int64_t T_tot, int32_t H, int32_t dk,
    int32_t dv, float scale, void* stream) {
  const char* fn = "kda_chunk_prefill_gated_static";
  if (N > 0 && H > 0 && dk == 128 && dv == 128 && (int64_t)N * H <= ((int64_t)1 << 24)) {
    const size_t need = kda::chunk_workspace_bytes(N, H, 1);
    if (need > kStaticScratchBytes)
      return fail(KDA_ERR_WORKSPACE,
                  "%s: N * H = %lld (sequence, head) pairs need %zu bytes of scratch for one "
                  "chunk per pass, more than the static scratch's %zu (at most %zu pairs); use "
                  "kda_chunk_prefill_gated with a workspace",
                  fn, (long long)N * H, need, kStaticScratchBytes, static_scratch_max_pairs());
  }
  const GatedPrefill a{q, k, v, qkv_dt, x, x_dt, b, b_dt, A_log, A_log_len, dt_bias,
                       dt_bias_len, cu_seqlens, cu_seqlens_host, N, initial_state, final_state,
                       state_dt, num_slots, state_indices, o, o_dt, T_tot, H, dk, dv, scale};
  // every check before the first HIP call: the workspace argument is a
  // non-null, aligned stand-in of the scratch's size (the scratch is the
  // library's own memory, so it overlaps no argument)
  bool alog_pc = false;
  if (const kda_status st = check_gated(fn, a, reinterpret_cast<const void*>(uintptr_t(256)),
                                        kStaticScratchBytes, false, &alog_pc))
    return st;
  void* ws = nullptr;
  if (const kda_status st = scratch_for_current_device(fn, &ws)) return st;
  return run_gated(fn, a, alog_pc, ws, kStaticScratchBytes, static_cast<hipStream_t>(stream));
}

size_t kda_chunk_prefill_backward_workspace_bytes(int64_t T_tot, int32_t N, int32_t H,
                                                  int32_t dk, int32_t dv) {
  if (dk != 128 || dv != 128 || T_tot < 0 || N <= 0 || H <= 0) return 0;
  return kda::bwd::workspace_bytes(T_tot, N, H);
}

kda_status kda_chunk_prefill_backward(const void* q, const void* k, const void* v,
                                      kda_dtype qkv_dt, const float* g, const float* beta,
                                      const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                                      int32_t N, const float* initial_state, const void* d_o,
                                      kda_dtype do_dt, const float* d_final_state, float* dq,
                                      float* dk, float* dv, float* dg, float* dbeta,
                                      float* d_initial_state, int64_t T_tot, int32_t H,
                                      int32_t dk_dim, int32_t dv_dim, float scale,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "kda_chunk_prefill_backward";
  const kda_status st = check_prefill(fn, q, k, v, qkv_dt, g, 16, beta, 4, cu_seqlens,
                                      cu_seqlens_host, N, initial_state, d_final_state, dq, do_dt,
                                      T_tot, H, dk_dim, dv_dim, scale, workspace, workspace_bytes,
                                      true);
  if (st != KDA_OK) return st;
  if (T_tot > 0 && (!dk || !dv || !dg || !dbeta))
    return fail(KDA_ERR_INVALID_ARG, "%s: dq, dk, dv, dg and dbeta must be non-NULL", fn);
  const void* outs[] = {d_o, dk, dv, dg, d_initial_state};
  for (const void* p : outs)
    if (p && !aligned(p, 16))
      return fail(KDA_ERR_ALIGNMENT, "%s: d_o and the gradients must be 16-byte aligned", fn);
  if (!aligned(dbeta, 4))
    return fail(KDA_ERR_ALIGNMENT, "%s: dbeta must be 4-byte aligned", fn);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool qb = qkv_dt == KDA_BF16;
  const int64_t nt = T_tot * H * 128;
  return run_checked(
      fn, s,
      [&](kda::dbg::Session& c) {
        c.add("q", q, nt, qb, kFinite);
        c.add("k", k, nt, qb, kFinite);
        c.add("v", v, nt, qb, kFinite);
        c.add("g", g, nt, false, kNonPositive);
        c.add("beta", beta, T_tot * H, false, kUnit);
        c.add("d_o", d_o, nt, do_dt == KDA_BF16, kFinite);
        c.add_states("initial_state", initial_state, false, nullptr, N, N, H);
        c.add_states("d_final_state", d_final_state, false, nullptr, N, N, H);
      },
      [&] {
        return kda::bwd::launch(q, k, v, qb, g, beta, cu_seqlens, cu_seqlens_host, N,
                                initial_state, d_o, do_dt == KDA_BF16, d_final_state, dq, dk,
                                dv, dg, dbeta, d_initial_state, T_tot, H, scale, workspace, s);
      },
      [&](kda::dbg::Session& c) {
        c.add("dq", dq, nt, false, kFinite);
        c.add("dk", dk, nt, false, kFinite);
        c.add("dv", dv, nt, false, kFinite);
        c.add("dg", dg, nt, false, kFinite);
        c.add("dbeta", dbeta, T_tot * H, false, kFinite);
        c.add_states("d_initial_state", d_initial_state, false, nullptr, N, N, H);
      });
}

size_t kda_chunk_prefill_workspace_bytes(int32_t N, int32_t H, int32_t dk, int32_t dv,
                                         int32_t chunks_per_pass) {
  if (dk != 128 || dv != 128) return 0;
  return kda::chunk_workspace_bytes(N, H, chunks_per_pass);
}

kda_status kda_recurrent_decode(const void* q, const void* k, const void* v, kda_dtype qkv_dt,
                                const float* g, const float* beta, float* state, void* o,
                                kda_dtype o_dt, int32_t N, int32_t H, int32_t dk, int32_t dv,
                                float scale, void* stream) {
  if (N < 0 || H <= 0)
    return fail(KDA_ERR_INVALID_ARG, "kda_recurrent_decode: need N >= 0, H > 0 (got %d, %d)", N, H);
  if (!known_dtype(qkv_dt) || !known_dtype(o_dt))
    return fail(KDA_ERR_DTYPE, "kda_recurrent_decode: qkv_dt and o_dt must be KDA_F32 or KDA_BF16");
  if (dk != 128 || dv != 128)
    return fail(KDA_ERR_UNSUPPORTED, "kda_recurrent_decode: only dk = dv = 128 is implemented "
                                     "(got %d, %d)", dk, dv);
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f)
    return fail(KDA_ERR_INVALID_ARG, "kda_recurrent_decode: scale must be finite");
  if (N == 0) return ok();
  if (!q || !k || !v || !g || !beta || !state || !o)
    return fail(KDA_ERR_INVALID_ARG, "kda_recurrent_decode: all tensor pointers must be non-NULL");
  const void* ptrs[] = {q, k, v, g, state, o};
  for (const void* p : ptrs)
    if (!aligned(p, 16))
      return fail(KDA_ERR_ALIGNMENT, "kda_recurrent_decode: tensors must be 16-byte aligned");
  const char* sb = reinterpret_cast<const char*>(state);
  const char* se = sb + (size_t)N * H * dk * dv * sizeof(float);
  const size_t qkv_es = qkv_dt == KDA_BF16 ? 2 : 4;
  const size_t o_es = o_dt == KDA_BF16 ? 2 : 4;
  struct { const void* p; size_t n; } others[] = {
      {q, (size_t)N * H * dk * qkv_es}, {k, (size_t)N * H * dk * qkv_es},
      {v, (size_t)N * H * dv * qkv_es}, {g, (size_t)N * H * dk * 4},
      {beta, (size_t)N * H * 4},        {o, (size_t)N * H * dv * o_es}};
  for (auto& r : others) {
    const char* b0 = static_cast<const char*>(r.p);
    if (b0 < se && sb < b0 + r.n)
      return fail(KDA_ERR_INVALID_ARG, "kda_recurrent_decode: state overlaps another tensor");
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool qb = qkv_dt == KDA_BF16;
  const int64_t nt = (int64_t)N * H * 128;
  return run_checked(
      "kda_recurrent_decode", s,
      [&](kda::dbg::Session& c) {
        c.add("q", q, nt, qb, kFinite);
        c.add("k", k, nt, qb, kFinite);
        c.add("v", v, nt, qb, kFinite);
        c.add("g", g, nt, false, kNonPositive);
        c.add("beta", beta, (int64_t)N * H, false, kUnit);
        c.add_states("state", state, false, nullptr, N, N, H);
      },
      [&] {
        return kda::launch_decode(q, k, v, qb, g, beta, state, o, o_dt == KDA_BF16, N, H, scale,
                                  s);
      },
      [&](kda::dbg::Session& c) {
        c.add("o", o, nt, o_dt == KDA_BF16, kFinite);
        c.add_states("state", state, false, nullptr, N, N, H);
      });
}

kda_status kda_recurrent_decode_gated(const void* q, const void* k, const void* v,
                                      kda_dtype qkv_dt, const void* x, kda_dtype x_dt,
                                      const void* b, kda_dtype b_dt, const float* A_log,
                                      int64_t A_log_len, const float* dt_bias,
                                      int64_t dt_bias_len, void* state, kda_dtype state_dt,
                                      int64_t num_slots, const int32_t* state_indices, void* o,
                                      kda_dtype o_dt, int32_t N, int32_t H, int32_t dk,
                                      int32_t dv, float scale, void* stream) {
  const char* fn = "kda_recurrent_decode_gated";
  if (N < 0 || H <= 0)
    return fail(KDA_ERR_INVALID_ARG, "%s: need N >= 0, H > 0 (got %d, %d)", fn, N, H);
  if (!known_dtype(qkv_dt) || !known_dtype(x_dt) || !known_dtype(b_dt) ||
      !known_dtype(state_dt) || !known_dtype(o_dt))
    return fail(KDA_ERR_DTYPE, "%s: qkv_dt, x_dt, b_dt, state_dt and o_dt must be KDA_F32 or "
                               "KDA_BF16", fn);
  if (dk != 128 || dv != 128)
    return fail(KDA_ERR_UNSUPPORTED, "%s: only dk = dv = 128 is implemented (got %d, %d)", fn,
                dk, dv);
  bool alog_pc = false;
  if (const kda_status st = check_alog(fn, A_log_len, H, dk, &alog_pc)) return st;
  if (dt_bias_len != (int64_t)H * dk)
    return fail(KDA_ERR_SHAPE, "%s: dt_bias has %lld values, need H*dk = %lld", fn,
                (long long)dt_bias_len, (long long)H * dk);
  if (num_slots < 0)
    return fail(KDA_ERR_INVALID_ARG, "%s: num_slots must be >= 0 (got %lld)", fn,
                (long long)num_slots);
  if (!state_indices && num_slots < N)
    return fail(KDA_ERR_SHAPE, "%s: without state_indices sequence n uses slot n, so num_slots "
                               "must be >= N (got %lld < %d)", fn, (long long)num_slots, N);
  if (!(scale == scale) || scale > 3.0e38f || scale < -3.0e38f)
    return fail(KDA_ERR_INVALID_ARG, "%s: scale must be finite", fn);
  if (N == 0) return ok();
  if (!q || !k || !v || !x || !b || !A_log || !dt_bias || !o || (num_slots > 0 && !state))
    return fail(KDA_ERR_INVALID_ARG, "%s: all tensor pointers must be non-NULL", fn);
  const void* ptrs[] = {q, k, v, x, o, state};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16))
      return fail(KDA_ERR_ALIGNMENT, "%s: q, k, v, x, o and state must be 16-byte aligned", fn);
  if (!aligned(b, b_dt == KDA_BF16 ? 2 : 4) || !aligned(A_log, 4) || !aligned(dt_bias, 4) ||
      !aligned(state_indices, 4))
    return fail(KDA_ERR_ALIGNMENT, "%s: b, A_log, dt_bias and state_indices must be aligned to "
                                   "their element size", fn);
  const size_t s_es = state_dt == KDA_BF16 ? 2 : 4;
  const char* sb = reinterpret_cast<const char*>(state);
  const char* se = sb + (size_t)num_slots * H * dk * dv * s_es;
  const size_t qkv_es = qkv_dt == KDA_BF16 ? 2 : 4;
  const size_t x_es = x_dt == KDA_BF16 ? 2 : 4;
  const size_t o_es = o_dt == KDA_BF16 ? 2 : 4;
  struct { const void* p; size_t n; } others[] = {
      {q, (size_t)N * H * dk * qkv_es},  {k, (size_t)N * H * dk * qkv_es},
      {v, (size_t)N * H * dv * qkv_es},  {x, (size_t)N * H * dk * x_es},
      {b, (size_t)N * H * (b_dt == KDA_BF16 ? 2 : 4)}, {o, (size_t)N * H * dv * o_es},
      {state_indices, state_indices ? (size_t)N * 4 : 0}};
  for (auto& r : others) {
    const char* b0 = static_cast<const char*>(r.p);
    if (r.n && b0 < se && sb < b0 + r.n)
      return fail(KDA_ERR_INVALID_ARG, "%s: the state pool overlaps another tensor", fn);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool qb = qkv_dt == KDA_BF16, sb16 = state_dt == KDA_BF16;
  const int64_t nt = (int64_t)N * H * 128;
  return run_checked(
      fn, s,
      [&](kda::dbg::Session& c) {
        c.add("q", q, nt, qb, kFinite);
        c.add("k", k, nt, qb, kFinite);
        c.add("v", v, nt, qb, kFinite);
        c.add("x", x, nt, x_dt == KDA_BF16, kNotNaN);
        c.add("b", b, (int64_t)N * H, b_dt == KDA_BF16, kNotNaN);
        c.add("A_log", A_log, alog_pc ? (int64_t)H * 128 : H, false, kFinite);
        c.add("dt_bias", dt_bias, (int64_t)H * 128, false, kFinite);
        c.add_states("state", state, sb16, state_indices, num_slots, N, H);
      },
      [&] {
        return kda::launch_decode_gated(q, k, v, qb, x, x_dt == KDA_BF16, b, b_dt == KDA_BF16,
                                        A_log, alog_pc, dt_bias, state, sb16, num_slots,
                                        state_indices, o, o_dt == KDA_BF16, N, H, scale, s);
      },
      [&](kda::dbg::Session& c) {
        c.add("o", o, nt, o_dt == KDA_BF16, kFinite);
        c.add_states("state", state, sb16, state_indices, num_slots, N, H);
      });
}

kda_status kda_shortconv_l2norm(const void* xq, const void* xk, const void* xv, kda_dtype in_dt,
                                const float* wq, const float* wk, const float* wv, int64_t w_len,
                                int32_t activation, float eps, const int32_t* cu_seqlens,
                                const int32_t* cu_seqlens_host, int32_t N,
                                const float* conv_state_in, float* conv_state_out, void* yq,
                                void* yk, void* yv, kda_dtype out_dt, int64_t T_tot, int32_t H,
                                int32_t d, void* stream) {
  const char* fn = "kda_shortconv_l2norm";
  if (N < 0 || H <= 0 || T_tot < 0)
    return fail(KDA_ERR_INVALID_ARG, "%s: need N >= 0, H > 0, T_tot >= 0 (got %d, %d, %lld)", fn,
                N, H, (long long)T_tot);
  if (!known_dtype(in_dt) || !known_dtype(out_dt))
    return fail(KDA_ERR_DTYPE, "%s: in_dt and out_dt must be KDA_F32 or KDA_BF16", fn);
  if (d != 128)
    return fail(KDA_ERR_UNSUPPORTED, "%s: only d = 128 is implemented (got %d)", fn, d);
  if (w_len != (int64_t)H * d * 4)
    return fail(KDA_ERR_SHAPE, "%s: each conv weight has %lld values, need H*d*4 = %lld (the "
                               "checkpoint's [H*d, 1, 4])", fn, (long long)w_len,
                (long long)H * d * 4);
  if (activation != KDA_ACT_NONE && activation != KDA_ACT_SILU)
    return fail(KDA_ERR_INVALID_ARG, "%s: activation must be KDA_ACT_NONE or KDA_ACT_SILU", fn);
  if (!(eps >= 0.0f) || eps > 3.0e38f)
    return fail(KDA_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  if (T_tot > ((int64_t)1 << 31) - 1 || H > 16384)
    return fail(KDA_ERR_UNSUPPORTED, "%s: need T_tot < 2^31 and H <= 16384", fn);
  if (N == 0) {
    if (T_tot != 0) return fail(KDA_ERR_SHAPE, "%s: N = 0 needs T_tot = 0", fn);
    return ok();
  }
  if (!cu_seqlens) return fail(KDA_ERR_INVALID_ARG, "%s: cu_seqlens is NULL", fn);
  int64_t max_len = T_tot, min_len = 0;  // bounds when the lengths are unknown on the host
  if (cu_seqlens_host) {
    if (cu_seqlens_host[0] != 0 || cu_seqlens_host[N] != T_tot)
      return fail(KDA_ERR_SHAPE, "%s: cu_seqlens must start at 0 and end at T_tot = %lld "
                                 "(got %d .. %d)", fn, (long long)T_tot, cu_seqlens_host[0],
                  cu_seqlens_host[N]);
    max_len = 0;
    min_len = T_tot;
    for (int32_t n = 0; n < N; ++n) {
      if (cu_seqlens_host[n + 1] < cu_seqlens_host[n])
        return fail(KDA_ERR_SHAPE, "%s: cu_seqlens decreases at index %d", fn, n);
      const int64_t l = (int64_t)cu_seqlens_host[n + 1] - cu_seqlens_host[n];
      if (l > max_len) max_len = l;
      if (l < min_len) min_len = l;
    }
  }
  if (!wq || !wk || !wv || (T_tot > 0 && (!xq || !xk || !xv || !yq || !yk || !yv)))
    return fail(KDA_ERR_INVALID_ARG, "%s: inputs, weights and outputs must be non-NULL", fn);
  const void* ptrs[] = {xq, xk, xv, wq, wk, wv, conv_state_in, conv_state_out, yq, yk, yv};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16))
      return fail(KDA_ERR_ALIGNMENT, "%s: tensors must be 16-byte aligned", fn);
  if (!aligned(cu_seqlens, 4)) return fail(KDA_ERR_ALIGNMENT, "%s: cu_seqlens must be 4-byte aligned", fn);
  // outputs must not overlap inputs (runs read 3 rows of their neighbours);
  // the state may be updated in place only when every sequence is one run
  const size_t in_b = (size_t)T_tot * H * d * (in_dt == KDA_BF16 ? 2 : 4);
  const size_t out_b = (size_t)T_tot * H * d * (out_dt == KDA_BF16 ? 2 : 4);
  const void* ins[] = {xq, xk, xv};
  const void* outs[] = {yq, yk, yv};
  for (const void* a : ins)
    for (const void* b : outs) {
      const char* a0 = static_cast<const char*>(a);
      const char* b0 = static_cast<const char*>(b);
      if (in_b && out_b && a0 < b0 + out_b && b0 < a0 + in_b)
        return fail(KDA_ERR_INVALID_ARG, "%s: an output overlaps an input", fn);
    }
  if (conv_state_in && conv_state_out) {
    const size_t sb = (size_t)N * 9 * H * d * 4;
    const char* a0 = reinterpret_cast<const char*>(conv_state_in);
    const char* b0 = reinterpret_cast<const char*>(conv_state_out);
    if (a0 < b0 + sb && b0 < a0 + sb && (a0 != b0 || max_len > 1))
      return fail(KDA_ERR_INVALID_ARG, "%s: the conv state may be updated in place only when "
                                       "every sequence has at most one token", fn);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool ib = in_dt == KDA_BF16, ob = out_dt == KDA_BF16;
  const int64_t nt = T_tot * H * d, ns = (int64_t)N * 9 * H * d;
  return run_checked(
      fn, s,
      [&](kda::dbg::Session& c) {
        c.add("xq", xq, nt, ib, kFinite);
        c.add("xk", xk, nt, ib, kFinite);
        c.add("xv", xv, nt, ib, kFinite);
        c.add("wq", wq, w_len, false, kFinite);
        c.add("wk", wk, w_len, false, kFinite);
        c.add("wv", wv, w_len, false, kFinite);
        c.add("conv_state_in", conv_state_in, ns, false, kFinite);
      },
      [&] {
        return kda::launch_shortconv(xq, xk, xv, ib, wq, wk, wv, activation == KDA_ACT_SILU, eps,
                                     cu_seqlens, N, min_len, max_len, T_tot, H, conv_state_in,
                                     conv_state_out, yq, yk, yv, ob, s);
      },
      [&](kda::dbg::Session& c) {
        c.add("yq", yq, nt, ob, kFinite);
        c.add("yk", yk, nt, ob, kFinite);
        c.add("yv", yv, nt, ob, kFinite);
        c.add("conv_state_out", conv_state_out, ns, false, kFinite);
      });
}

}  // extern "C"
