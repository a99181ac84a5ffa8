// Internal declarations shared by the HIP translation units of libkda.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <string>

#include "kda.h"

namespace kda {

// KDA_DEBUG=1 scans (debug.hip): input-domain scans before a call's kernels,
// non-finite scans of its outputs after them.
namespace dbg {
enum Rule { kFinite = 0, kNotNaN = 1, kNonPositive = 2, kUnit = 3 };
bool enabled();          // KDA_DEBUG is "1" (read on every call)
std::mutex& mutex();     // held for a whole debug call
class Session {
 public:
  explicit Session(hipStream_t s);
  hipError_t begin();    // clears the counters (a kernel on the stream)
  // count the values of p[0 .. n) (fp32 or bf16) that break `rule`
  void add(const char* what, const void* p, int64_t n, bool bf16, int rule);
  // count non-finite values of the 128 x 128 states of slot idx[n] (n when idx is
  // null) for every (sequence n < N, head), skipping slots outside [0, slots)
  void add_states(const char* what, const void* p, bool bf16, const int32_t* idx, int64_t slots,
                  int N, int H);
  // waits for the stream; report lists every scan that found values ("" if none)
  hipError_t finish(std::string* report);

 private:
  hipStream_t stream_;
  uint32_t* words_ = nullptr;
  int count_ = 0;
  const char* what_[16];
  int rule_[16];
  int64_t n_[16];
};
}  // namespace dbg

// ---- launchers (one per kernel family); return hipSuccess or the launch error
// A_log per head [H], or per (head, channel) [H, d] when alog_pc.
hipError_t launch_gate(const void* x, bool x_bf16, const void* b, bool b_bf16, const float* A_log,
                       bool alog_pc, const float* dt_bias, float* g, float* beta, int64_t n_tok,
                       int H, int d, hipStream_t s);

// Gradient of the gate: dx, db elementwise; dA_log and ddt_bias summed over
// the tokens through ws (gate_bwd_workspace_bytes) in a fixed order.
size_t gate_bwd_workspace_bytes(int64_t n_tok, int H, int d);
hipError_t launch_gate_backward(const void* x, bool x_bf16, const void* b, bool b_bf16,
                                const float* A_log, bool alog_pc, const float* dt_bias,
                                const float* dg, const float* dbeta, float* dx, float* db,
                                float* dA_log, float* ddt_bias, int64_t n_tok, int H, int d,
                                void* ws, hipStream_t s);

hipError_t launch_decode(const void* q, const void* k, const void* v, bool qkv_bf16,
                         const float* g, const float* beta, float* state, void* o, bool o_bf16,
                         int N, int H, float scale, hipStream_t s);

// One-token decode from the gate's raw inputs (x [N,H,128] fp32 or bf16, beta
// logits b [N,H]) over a pool of num_slots x H states (fp32 or bf16); sequence
// n uses slot slots[n] (n when slots is null), and a slot outside the pool
// skips it (o = 0).
hipError_t launch_decode_gated(const void* q, const void* k, const void* v, bool qkv_bf16,
                               const void* gx, bool x_bf16, const void* b, bool b_bf16,
                               const float* A_log, bool alog_pc, const float* dt_bias, void* pool,
                               bool state_bf16, int64_t num_slots, const int32_t* slots, void* o,
                               bool o_bf16, int N, int H, float scale, hipStream_t s);

// The layer's prologue: causal depthwise conv (kernel 4) of q, k, v, optional
// SiLU, L2 norm of q and k per (token, head); conv state [N][3][3][H*128] fp32.
// min_len / max_len: the shortest / longest sequence (0 / T_tot when unknown):
// a zero-length sequence needs its state copied by a second launch.
hipError_t launch_shortconv(const void* xq, const void* xk, const void* xv, bool in_bf16,
                            const float* wq, const float* wk, const float* wv, bool silu,
                            float eps, const int32_t* cu, int N, int64_t min_len,
                            int64_t max_len, int64_t T_tot, int H, const float* state_in,
                            float* state_out, void* yq, void* yk, void* yv, bool out_bf16,
                            hipStream_t s);

// Entry or exit states of the chunked prefill: fp32 or bf16 [slots, H, 128, 128];
// sequence n uses slot idx[n] (n when idx is null).  A slot outside
// [0, slots) means a zero entry state / no exit state.
struct StatePool {
  const void* in = nullptr;       // null: zero entry states
  void* out = nullptr;            // null: no exit states written
  const int32_t* idx = nullptr;   // slot per sequence, or null
  int64_t slots = 0;
  bool bf16 = false;
};

// Chunked prefill: prep + state kernel per pass over the chunks (prefill.hip).
// The decay input is either g (g_mode 0, fp32) with post-sigmoid beta in b,
// or raw gate logits x (g_mode 1 fp32, 2 bf16) with beta logits in b and the
// gate parameters A_log [H], dt_bias [H, 128]; g_mode | 4: A_log [H, 128].
hipError_t launch_chunk_prefill(const void* q, const void* k, const void* v, bool qkv_bf16,
                                const void* g, int g_mode, const void* b, bool b_bf16,
                                const float* A_log, const float* dt_bias, const int32_t* cu,
                                const int32_t* cu_host, int N, const StatePool& st,
                                void* o, bool o_bf16, int64_t T_tot, int H, float scale,
                                void* ws, size_t ws_bytes, hipStream_t s);
size_t chunk_workspace_bytes(int N, int H, int chunks_per_pass);

// Chunked prefill backward (backward.hip): gradients of q, k, v, g, beta and
// the initial state from d_o (bf16 or fp32, NULL = 0) and dS_final (NULL = 0).
namespace bwd {
size_t workspace_bytes(int64_t T_tot, int N, int H);
hipError_t launch(const void* q, const void* k, const void* v, bool qkv_bf16, const float* g,
                  const float* beta, const int32_t* cu, const int32_t* cu_host, int N,
                  const float* S0, const void* d_o, bool do_bf16, const float* dS_final,
                  float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dS0,
                  int64_t T_tot, int H, float scale, void* ws, hipStream_t s);
}  // namespace bwd

namespace chunk {
// Entry and exit states of one state-kernel pass (each fp32 or bf16, each
// addressed by slot index or by sequence): the pool, or the workspace's fp32
// carry between passes.  A slot outside [0, slots) reads zeros / is not written.
struct StateIO {
  const void* in;
  const int32_t* in_idx;
  void* out;
  const int32_t* out_idx;
  int64_t in_slots, out_slots;
  bool in_bf16, out_bf16;
};
// One pass: chunks [c_lo, c_lo + S_len) of every sequence (prep.hip, state.hip).
hipError_t launch_prep(const void* q, const void* k, bool qkv_bf16, const void* g, int g_mode,
                       const void* b, bool b_bf16, const float* A_log, const float* dt_bias,
                       const int32_t* cu, int N, int T_tot, int H, int c_lo, int S_len, char* ws,
                       hipStream_t s);
hipError_t launch_state(const void* v, bool qkv_bf16, const int32_t* cu, int N, int T_tot,
                        int H, const StateIO& sio, void* o, bool o_bf16,
                        float scale, int c_lo, int S_len, const char* ws, hipStream_t s);
}  // namespace chunk

}  // namespace kda
