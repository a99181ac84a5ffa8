// Prep kernel of kda_chunk_prefill: one workgroup (one prep_chunk unit) per
// (chunk, head), for all chunks of a pass at once (prep_chunk.hpp holds the
// computation).
#include "prep_chunk.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace chunk {
namespace {

template <bool QKV_BF16, int GIN>
__global__ void __launch_bounds__(NTHR, 3) prep_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ g,
    GateArgs ga, const int32_t* __restrict__ cu, int T_tot, int H, int Hp,
    int c_lo, int S_len, char* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) char lds[PrepLds::total];
  // ---- block -> (chunk slot, head); head % 8 == block % 8, so every chunk of
  // a head is prepared on the XCD that later runs that head's state walk.
  const int hx = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int hgroups = Hp >> 3;
  const int h = (rest % hgroups) * 8 + hx;
  const int slot = rest / hgroups;
  if (h >= H) return;
  const int n = slot / S_len;
  const int cidx = c_lo + slot % S_len;
  int bos = cu[n], eos = cu[n + 1];
  bos = bos < 0 ? 0 : (bos > T_tot ? T_tot : bos);
  eos = eos < bos ? bos : (eos > T_tot ? T_tot : eos);
  if ((int64_t)cidx * C >= eos - bos) return;  // this sequence has no such chunk
  const int t0 = bos + cidx * C;
  const int Lc = (eos - t0) < C ? (eos - t0) : C;
  char* img = ws + ((int64_t)slot * H + h) * Ws::bytes;
  prep_chunk<QKV_BF16, GIN>(q, k, g, ga, H, h, t0, Lc, img, lds, threadIdx.x);
}

}  // namespace

hipError_t launch_prep(const void* q, const void* k, bool qkv_bf16, const void* g, int g_mode,
                       const void* b, bool b_bf16, const float* A_log, const float* dt_bias,
                       const int32_t* cu, int N, int T_tot, int H, int c_lo, int S_len, char* ws,
                       hipStream_t s) {
  const int Hp = (H + 7) & ~7;
  const int64_t blocks = (int64_t)N * S_len * Hp;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const GateArgs ga{b, b_bf16, A_log, dt_bias};
  const dim3 grid((unsigned)blocks);
#define KDA_PREP(QB, GM) \
  prep_kernel<QB, GM><<<grid, NTHR, 0, s>>>(q, k, g, ga, cu, T_tot, H, Hp, c_lo, S_len, ws)
  if (qkv_bf16) {
    if (g_mode == kG) KDA_PREP(true, kG);
    else if (g_mode == kX32) KDA_PREP(true, kX32);
    else if (g_mode == kX16) KDA_PREP(true, kX16);
    else if (g_mode == (kX32 | kPC)) KDA_PREP(true, kX32 | kPC);
    else KDA_PREP(true, kX16 | kPC);
  } else {
    if (g_mode == kG) KDA_PREP(false, kG);
    else if (g_mode == kX32) KDA_PREP(false, kX32);
    else if (g_mode == kX16) KDA_PREP(false, kX16);
    else if (g_mode == (kX32 | kPC)) KDA_PREP(false, kX32 | kPC);
    else KDA_PREP(false, kX16 | kPC);
  }
#undef KDA_PREP
  return hipGetLastError();
}

}  // namespace chunk
}  // namespace kda
