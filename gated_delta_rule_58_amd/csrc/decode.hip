// kda_recurrent_decode: one token per sequence, fused recurrent KDA step.
//
// For one (sequence, head) with fp32 state S [128 x 128] (S[c][j]):
//   S' = Diag(exp(g)) S
//   o  = scale * (S'^T q + (q.k) * delta),   delta = beta * (v - S'^T k)
//   S  = S' + k delta^T                       (written back in place)
// which is S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T with
// o = S_t^T q expanded so that S is read once and written once (the code
// audit's fused recurrent one-token decode regime).
//
// The kernel is HBM-bound: 64 KiB of state in and out per (sequence, head).
// One 256-thread workgroup owns one state tile.  Thread t holds 4 value
// columns (4*(t%32) ..) of the 16 key rows t/32 + 8*i, i = 0..15, as 16
// float4 registers; every wave-wide load/store covers two adjacent 512-byte
// rows (1 KiB contiguous).  The two column reductions (k^T S' and q^T S')
// run over the 8 row slots: lane pairs (l, l^32) by cross-lane shuffle, then
// the 4 waves through LDS.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int D = 128;

template <bool QKV_BF16, bool O_BF16>
__global__ void __launch_bounds__(256) decode_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    void* __restrict__ o, float scale) {
  const int t = threadIdx.x;
  const int cg = t & 31;   // column group: columns 4*cg .. 4*cg+3
  const int rs = t >> 5;   // row slot: rows rs + 8*i
  const int w = t >> 6;    // wave
  const int64_t pair = blockIdx.x;
  float* S = state + pair * (D * D);

  __shared__ float s_k[D], s_q[D], s_a[D];
  __shared__ f32x4 s_red[4][32][2];
  __shared__ float s_qk[2];

  // Issue the state loads first: they are the bulk of the traffic.
  f32x4 st[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (rs + 8 * i) * D) + cg);

  if (t < D) {
    const float kk = load1(k, pair * D + t, QKV_BF16);
    const float qq = load1(q, pair * D + t, QKV_BF16);
    s_k[t] = kk;
    s_q[t] = qq;
    s_a[t] = expf(g[pair * D + t]);
    float p = kk * qq;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
    if ((t & 63) == 0) s_qk[t >> 6] = p;
  }
  const f32x4 vv = load4(v, pair * D + 4 * cg, QKV_BF16);
  const float b = beta[pair];
  __syncthreads();

  f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = rs + 8 * i;
    st[i] *= s_a[r];
    pk += s_k[r] * st[i];
    pq += s_q[r] * st[i];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pk[e] += __shfl_xor(pk[e], 32);
    pq[e] += __shfl_xor(pq[e], 32);
  }
  if ((t & 32) == 0) {
    s_red[w][cg][0] = pk;
    s_red[w][cg][1] = pq;
  }
  __syncthreads();
  f32x4 kS = s_red[0][cg][0] + s_red[1][cg][0] + s_red[2][cg][0] + s_red[3][cg][0];
  f32x4 qS = s_red[0][cg][1] + s_red[1][cg][1] + s_red[2][cg][1] + s_red[3][cg][1];
  const float qk = s_qk[0] + s_qk[1];
  const f32x4 delta = b * (vv - kS);

#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = rs + 8 * i;
    st[i] += s_k[r] * delta;
    __builtin_nontemporal_store(st[i], reinterpret_cast<f32x4*>(S + r * D) + cg);
  }
  if (rs == 0) store4(o, pair * D + 4 * cg, scale * (qS + qk * delta), O_BF16);
}

}  // namespace

hipError_t launch_decode(const void* q, const void* k, const void* v, bool qkv_bf16,
                         const float* g, const float* beta, float* state, void* o, bool o_bf16,
                         int N, int H, float scale, hipStream_t s) {
  const int64_t pairs = (int64_t)N * H;
  if (pairs == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(pairs));
  if (qkv_bf16 && o_bf16)
    decode_kernel<true, true><<<grid, 256, 0, s>>>(q, k, v, g, beta, state, o, scale);
  else if (qkv_bf16)
    decode_kernel<true, false><<<grid, 256, 0, s>>>(q, k, v, g, beta, state, o, scale);
  else if (o_bf16)
    decode_kernel<false, true><<<grid, 256, 0, s>>>(q, k, v, g, beta, state, o, scale);
  else
    decode_kernel<false, false><<<grid, 256, 0, s>>>(q, k, v, g, beta, state, o, scale);
  return hipGetLastError();
}

}  // namespace kda
