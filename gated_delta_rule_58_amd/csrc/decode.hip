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
// One 512-thread workgroup handles two consecutive (sequence, head) pairs.
// Thread t holds 4 value columns (4*(t%32) ..) of the 8 key rows t/32 + 16*i,
// i = 0..7, as 8 float4 registers; every wave-wide load/store covers two
// adjacent 512-byte rows (1 KiB contiguous).  The second pair's state loads
// are issued before the first pair's stores, so each CU keeps reads in flight
// while it writes.  The two column reductions (k^T S' and q^T S') run over
// the 8 row slots of a thread, then lane pairs (l, l^32) by cross-lane
// shuffle, then the 8 waves through LDS.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int D = 128;
constexpr int NTHR = 512;
constexpr int PAIRS_PER_BLOCK = 2;

template <bool QKV_BF16, bool O_BF16>
__global__ void __launch_bounds__(NTHR) decode_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    void* __restrict__ o, float scale, int64_t pairs) {
  const int t = threadIdx.x;
  const int cg = t & 31;   // column group: columns 4*cg .. 4*cg+3
  const int rs = t >> 5;   // row slot: rows rs + 16*i
  const int w = t >> 6;    // wave

  __shared__ float s_k[2][D], s_q[2][D], s_a[2][D];
  __shared__ f32x4 s_red[NTHR / 64][32][2];
  __shared__ float s_qk[2][2];

  // Small inputs of a pair in two halves: fetch issues the loads (before the
  // previous pair's stores) and keeps the raw bits, commit widens and uses
  // them (after those stores): q, k, decay and q.k into LDS buffer buf; v and
  // beta stay in registers.  Every thread loads (threads past the 128
  // channels repeat the first ones), so no load sits inside a branch.
  struct Small {
    typename Raw<QKV_BF16>::T1 kk, qq;
    float gg, b;
    typename Raw<QKV_BF16>::T4 vv;
  };
  auto fetch_small = [&](int64_t p, Small& sm) {
    const int c = t & (D - 1);
    sm.kk = load1_raw<QKV_BF16>(k, p * D + c);
    sm.qq = load1_raw<QKV_BF16>(q, p * D + c);
    sm.gg = g[p * D + c];
    sm.vv = load4_raw<QKV_BF16>(v, p * D + 4 * cg);
    sm.b = beta[p];
  };
  auto commit_small = [&](int buf, Small& sm) {
    hold(sm.kk);
    hold(sm.qq);
    hold(sm.gg);
    hold(sm.vv);
    if (t < D) {
      const float kk = widen1<QKV_BF16>(sm.kk), qq = widen1<QKV_BF16>(sm.qq);
      s_k[buf][t] = kk;
      s_q[buf][t] = qq;
      s_a[buf][t] = expf(sm.gg);
      float pr = kk * qq;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) pr += __shfl_xor(pr, off);
      if ((t & 63) == 0) s_qk[buf][t >> 6] = pr;
    }
  };
  auto load_state = [&](int64_t p, f32x4* st) {
    const float* S = state + p * (D * D);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (rs + 16 * i) * D) + cg);
  };

  int64_t pair = (int64_t)blockIdx.x * PAIRS_PER_BLOCK;
  f32x4 st[8], nx[8];
  Small cur, nxt;
  fetch_small(pair, cur);
  load_state(pair, st);
  commit_small(0, cur);
#pragma unroll
  for (int j = 0; j < PAIRS_PER_BLOCK; ++j, ++pair) {
    const int buf = j & 1;
    barrier_lds();
    f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = rs + 16 * i;
      st[i] *= s_a[buf][r];
      pk += s_k[buf][r] * st[i];
      pq += s_q[buf][r] * st[i];
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
    barrier_lds();
    f32x4 kS = s_red[0][cg][0], qS = s_red[0][cg][1];
#pragma unroll
    for (int jj = 1; jj < NTHR / 64; ++jj) {
      kS += s_red[jj][cg][0];
      qS += s_red[jj][cg][1];
    }
    const float qk = s_qk[buf][0] + s_qk[buf][1];
    const f32x4 delta = cur.b * (widen4<QKV_BF16>(cur.vv) - kS);
    // next pair's loads go out before this pair's stores
    const bool more = j + 1 < PAIRS_PER_BLOCK && pair + 1 < pairs;
    if (more) {
      fetch_small(pair + 1, nxt);
      load_state(pair + 1, nx);
    }
    float* S = state + pair * (D * D);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = rs + 16 * i;
      st[i] += s_k[buf][r] * delta;
      __builtin_nontemporal_store(st[i], reinterpret_cast<f32x4*>(S + r * D) + cg);
    }
    if (rs == 0) store4(o, pair * D + 4 * cg, scale * (qS + qk * delta), O_BF16);
    if (!more) break;
    commit_small(buf ^ 1, nxt);
    cur = nxt;
#pragma unroll
    for (int i = 0; i < 8; ++i) st[i] = nx[i];
  }
}

}  // namespace

hipError_t launch_decode(const void* q, const void* k, const void* v, bool qkv_bf16,
                         const float* g, const float* beta, float* state, void* o, bool o_bf16,
                         int N, int H, float scale, hipStream_t s) {
  const int64_t pairs = (int64_t)N * H;
  if (pairs == 0) return hipSuccess;
  const int64_t blocks = (pairs + PAIRS_PER_BLOCK - 1) / PAIRS_PER_BLOCK;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks));
  if (qkv_bf16 && o_bf16)
    decode_kernel<true, true><<<grid, NTHR, 0, s>>>(q, k, v, g, beta, state, o, scale, pairs);
  else if (qkv_bf16)
    decode_kernel<true, false><<<grid, NTHR, 0, s>>>(q, k, v, g, beta, state, o, scale, pairs);
  else if (o_bf16)
    decode_kernel<false, true><<<grid, NTHR, 0, s>>>(q, k, v, g, beta, state, o, scale, pairs);
  else
    decode_kernel<false, false><<<grid, NTHR, 0, s>>>(q, k, v, g, beta, state, o, scale, pairs);
  return hipGetLastError();
}

}  // namespace kda
