// Host side of kda_chunk_prefill: passes over the chunk axis.
//
// The workspace holds a state carry [N, H, 128, 128] fp32 followed by the
// images of S_len chunks of every (sequence, head).  Each pass launches the
// prep kernel on chunks [c_lo, c_lo + S_len) of every sequence, then the
// state kernel, which walks those chunks from the carried state.  One pass
// covers the whole batch when S_len reaches the longest sequence's chunk
// count.
#include "chunk_common.hpp"
#include "kda_internal.hpp"

namespace kda {

size_t chunk_workspace_bytes(int N, int H, int chunks_per_pass) {
  if (N <= 0 || H <= 0 || chunks_per_pass <= 0) return 0;
  const size_t pairs = (size_t)N * H;
  return pairs * chunk::D * chunk::D * sizeof(float) +
         pairs * (size_t)chunks_per_pass * chunk::Ws::bytes;
}

hipError_t launch_chunk_prefill(const void* q, const void* k, const void* v, bool qkv_bf16,
                                const void* g, int g_mode, const void* b, bool b_bf16,
                                const float* A_log, const float* dt_bias, const int32_t* cu,
                                const int32_t* cu_host, int N, const StatePool& st,
                                void* o, bool o_bf16, int64_t T_tot, int H, float scale,
                                void* ws, size_t ws_bytes, hipStream_t s) {
  using namespace chunk;
  int64_t max_nch = (T_tot + C - 1) / C;
  if (cu_host) {
    max_nch = 0;
    for (int n = 0; n < N; ++n) {
      const int64_t nc = ((int64_t)cu_host[n + 1] - cu_host[n] + C - 1) / C;
      if (nc > max_nch) max_nch = nc;
    }
  }
  const size_t pairs = (size_t)N * H;
  const size_t carry_bytes = pairs * D * D * sizeof(float);
  int64_t S_len = (int64_t)((ws_bytes - carry_bytes) / (pairs * Ws::bytes));  // >= 1 (checked)
  if (S_len > max_nch) S_len = max_nch > 0 ? max_nch : 1;
  // The state carried between passes stays fp32 and is addressed by sequence:
  // in the final-state buffer when that is an fp32 [N, H, 128, 128] array,
  // else in the workspace.
  const bool out_plain = st.out && !st.bf16 && !st.idx;
  float* carry = out_plain ? static_cast<float*>(st.out) : static_cast<float*>(ws);
  char* images = static_cast<char*>(ws) + carry_bytes;
  const int T = static_cast<int>(T_tot);
  for (int64_t c_lo = 0;; c_lo += S_len) {
    const bool last = c_lo + S_len >= max_nch;
    hipError_t e = chunk::launch_prep(q, k, qkv_bf16, g, g_mode, b, b_bf16, A_log, dt_bias, cu,
                                      N, T, H, (int)c_lo, (int)S_len, images, s);
    if (e != hipSuccess) return e;
    chunk::StateIO sio;
    if (c_lo == 0) {
      sio.in = st.in;
      sio.in_idx = st.idx;
      sio.in_slots = st.slots;
      sio.in_bf16 = st.bf16;
    } else {
      sio.in = carry;
      sio.in_idx = nullptr;
      sio.in_slots = N;
      sio.in_bf16 = false;
    }
    if (last) {
      sio.out = st.out;
      sio.out_idx = st.idx;
      sio.out_slots = st.slots;
      sio.out_bf16 = st.bf16;
    } else {
      sio.out = carry;
      sio.out_idx = nullptr;
      sio.out_slots = N;
      sio.out_bf16 = false;
    }
    e = chunk::launch_state(v, qkv_bf16, cu, N, T, H, sio, o, o_bf16, scale, (int)c_lo,
                            (int)S_len, images, s);
    if (e != hipSuccess) return e;
    if (last) return hipSuccess;
  }
}

}  // namespace kda
