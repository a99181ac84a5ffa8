// kda_gate: log-decay g = -exp(A_log) * softplus(x + dt_bias[h,c]) and
// beta = sigmoid(b), one elementwise HBM-bound pass.
//
// Shapes per the Kimi K3 artifact audit (§4.1 KDA tensor table; §5.2 shape
// table): A_log one value per head (or, explicitly, one per (head, channel)),
// dt_bias one per (head, channel).  beta is squashed here in fp32
// (Model-Optimizer PR #2749 review, KDA beta fix).
//
// Work split: blockIdx.y picks a group of R = 256 / (d/4) heads, blockIdx.x a
// run of tokens.  A thread owns one (head, 4-channel) slot for the whole run,
// so its -exp(A_log) and dt_bias quads are formed once and every token costs
// one 16-byte load of x and one 16-byte store of g.  A wave covers 256
// consecutive channels of one token: fully coalesced.  beta for the block's
// (token, head) pairs is one extra pass by one lane per pair.
//
// Arithmetic: gate_math.hpp.
#include "gate_math.hpp"
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kTokUnroll = 4;   // x loads in flight per thread
constexpr int kTokPerBlock = 32;

// 4 consecutive logits as fp32, read once: non-temporal, so the stream of x
// does not displace the cached lines of g that the prefill reads next.
template <bool BF16>
__device__ __forceinline__ f32x4 load4_stream(const void* base, int64_t idx) {
  if constexpr (BF16) {
    const u16x4 r = __builtin_nontemporal_load(reinterpret_cast<const u16x4*>(
        static_cast<const uint16_t*>(base) + idx));
    return f32x4{bf16_bits_to_f32(r[0]), bf16_bits_to_f32(r[1]), bf16_bits_to_f32(r[2]),
                 bf16_bits_to_f32(r[3])};
  }
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx));
}

template <bool XBF16, bool BBF16>
__global__ void __launch_bounds__(kThreads) gate_kernel(
    const void* __restrict__ x, const void* __restrict__ b, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, float* __restrict__ g, float* __restrict__ beta,
    int n_tok, int H, int d, int rows_per_block, int alog_pc) {
  const int qpr = d >> 2;
  const int tid = threadIdx.x;
  const int hh = tid / qpr;
  const int h = blockIdx.y * rows_per_block + hh;
  const int c = (tid - hh * qpr) << 2;
  const int tok0 = blockIdx.x * kTokPerBlock;
  const int ntk = min(kTokPerBlock, n_tok - tok0);
  const int64_t tok_stride = (int64_t)H * d;

  if (hh < rows_per_block && h < H) {
    f32x4 a;  // -exp(A_log) for the thread's 4 channels
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = -expf(alog_pc ? A_log[(int64_t)h * d + c + e] : A_log[h]);
    const f32x4 db = *reinterpret_cast<const f32x4*>(dt_bias + (int64_t)h * d + c);
    const int64_t base = (int64_t)tok0 * tok_stride + (int64_t)h * d + c;
    for (int t = 0; t < ntk; t += kTokUnroll) {
      f32x4 xv[kTokUnroll];
#pragma unroll
      for (int u = 0; u < kTokUnroll; ++u)
        if (t + u < ntk) xv[u] = load4_stream<XBF16>(x, base + (t + u) * tok_stride);
#pragma unroll
      for (int u = 0; u < kTokUnroll; ++u) {
        if (t + u < ntk) {
          f32x4 out;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float z = gate_input(xv[u][e], db[e]);
            out[e] = gate_log_decay(a[e], z);
          }
          *reinterpret_cast<f32x4*>(g + base + (t + u) * tok_stride) = out;
        }
      }
    }
  }

  // beta = sigmoid(b) for the block's (token, head) pairs.
  const int hbase = blockIdx.y * rows_per_block;
  const int nh = min(rows_per_block, H - hbase);
  for (int i = tid; i < ntk * nh; i += kThreads) {
    const int tk = i / nh;
    const int64_t row = (int64_t)(tok0 + tk) * H + hbase + (i - tk * nh);
    const float bl = load1(b, row, BBF16);
    beta[row] = gate_beta(bl);
  }
}

}  // namespace

hipError_t launch_gate(const void* x, bool x_bf16, const void* b, bool b_bf16, const float* A_log,
                       bool alog_pc, const float* dt_bias, float* g, float* beta, int64_t n_tok,
                       int H, int d, hipStream_t s) {
  if (n_tok == 0) return hipSuccess;
  // d is a multiple of 4 with d/4 <= 256 (checked by the caller).
  const int rows_per_block = kThreads / (d >> 2);
  const int head_groups = (H + rows_per_block - 1) / rows_per_block;
  // One launch covers at most 2^30 tokens so the block index stays in range.
  const int64_t max_tok = (int64_t)1 << 30;
  for (int64_t t0 = 0; t0 < n_tok; t0 += max_tok) {
    const int nt = static_cast<int>(n_tok - t0 < max_tok ? n_tok - t0 : max_tok);
    const int64_t off = t0 * H;
    const void* xs = static_cast<const char*>(x) + off * d * (x_bf16 ? 2 : 4);
    const void* bs = static_cast<const char*>(b) + off * (b_bf16 ? 2 : 4);
    float* gs = g + off * d;
    float* betas = beta + off;
    const dim3 grid((nt + kTokPerBlock - 1) / kTokPerBlock, head_groups);
    if (x_bf16 && b_bf16)
      gate_kernel<true, true><<<grid, kThreads, 0, s>>>(xs, bs, A_log, dt_bias, gs, betas, nt, H,
                                                        d, rows_per_block, alog_pc ? 1 : 0);
    else if (x_bf16)
      gate_kernel<true, false><<<grid, kThreads, 0, s>>>(xs, bs, A_log, dt_bias, gs, betas, nt, H,
                                                         d, rows_per_block, alog_pc ? 1 : 0);
    else if (b_bf16)
      gate_kernel<false, true><<<grid, kThreads, 0, s>>>(xs, bs, A_log, dt_bias, gs, betas, nt, H,
                                                         d, rows_per_block, alog_pc ? 1 : 0);
    else
      gate_kernel<false, false><<<grid, kThreads, 0, s>>>(xs, bs, A_log, dt_bias, gs, betas, nt,
                                                          H, d, rows_per_block, alog_pc ? 1 : 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kda
