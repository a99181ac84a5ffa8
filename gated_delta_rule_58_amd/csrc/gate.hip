// kda_gate: log-decay g = -exp(A_log) * softplus(x + dt_bias[h,c]) and
// beta = sigmoid(b), one elementwise HBM-bound pass.
//
// Shapes per the Kimi K3 artifact audit (§4.1 KDA tensor table; §5.2 shape
// table): A_log one value per head (or, explicitly, one per (head, channel)),
// dt_bias one per (head, channel).  beta is squashed here in fp32
// (Model-Optimizer PR #2749 review, KDA beta fix).
//
// Work split: blockIdx.y picks a group of R = 256 / (d/4) heads, blockIdx.x a
// run of 32 tokens.  A thread owns one (head, 4-channel) slot for the whole run,
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
constexpr int kTokUnroll = 8;   // x loads per group; two groups in flight per thread
constexpr int kTokPerBlock = 32;

// 4 consecutive logits of token t of the run through the run's buffer (rows
// past the run read 0), as raw bits: widened only where used.
template <bool BF16>
struct X4 {
  typedef typename Raw<BF16>::T4 T;
};
template <bool BF16>
__device__ __forceinline__ typename X4<BF16>::T load_x4(__amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (BF16)
    return __builtin_bit_cast(u16x4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kBufNT));
  else
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufNT));
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
    // The run's x and g as buffers over its ntk tokens: every load and store
    // runs on every path (x past the run reads 0, g past it is dropped), so
    // the loads of a group stay in flight together and the next group's go
    // out before this group's arithmetic (a branch per token made each load
    // wait for the one before it).  x is read once: non-temporal.
    // (the buffers start at the run's first token, the same for every lane, so
    // the resource stays in scalar registers; a lane's channels are an offset)
    constexpr int XS = XBF16 ? 2 : 4;
    const int stride_b = static_cast<int>(tok_stride);  // elements per token
    const int lane_off = h * d + c;
    const uint32_t span = static_cast<uint32_t>((int64_t)ntk * tok_stride);
    const auto rx = buffer_over(static_cast<const char*>(x) + (int64_t)tok0 * tok_stride * XS,
                                span * XS);
    const auto rg = buffer_over(g + (int64_t)tok0 * tok_stride, span * 4);
    typename X4<XBF16>::T xa[kTokUnroll], xb[kTokUnroll];
    auto load_group = [&](int t0, typename X4<XBF16>::T* xv) {
#pragma unroll
      for (int u = 0; u < kTokUnroll; ++u)
        xv[u] = load_x4<XBF16>(rx, ((t0 + u) * stride_b + lane_off) * XS);
    };
    auto run_group = [&](int t0, typename X4<XBF16>::T* xv) {
#pragma unroll
      for (int u = 0; u < kTokUnroll; ++u) {
        const f32x4 xf = widen4<XBF16>(xv[u]);
        f32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = gate_log_decay(a[e], gate_input(xf[e], db[e]));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, out), rg,
                                               ((t0 + u) * stride_b + lane_off) * 4, 0, 0);
      }
    };
    load_group(0, xa);
#pragma unroll
    for (int t = 0; t < kTokPerBlock; t += 2 * kTokUnroll) {
      load_group(t + kTokUnroll, xb);
      run_group(t, xa);
      if (t + 2 * kTokUnroll < kTokPerBlock) load_group(t + 2 * kTokUnroll, xa);
      run_group(t + kTokUnroll, xb);
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

// Gradient of the gate, per token run (same thread layout as gate_kernel):
//   dx = dg (-exp(A_log) sigmoid(z)),  db = dbeta beta (1 - beta),
// plus, per thread, the run's partial sums of dx (for dt_bias) and dg g (for
// A_log) into part[0 / 1][run][h][c]; gate_bwd_reduce adds the runs.
template <bool XBF16, bool BBF16>
__global__ void __launch_bounds__(kThreads) gate_bwd_kernel(
    const void* __restrict__ x, const void* __restrict__ b, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, const float* __restrict__ dg,
    const float* __restrict__ dbeta, float* __restrict__ dx, float* __restrict__ db,
    float* __restrict__ part, int n_tok, int H, int d, int rows_per_block, int alog_pc) {
  const int qpr = d >> 2;
  const int tid = threadIdx.x;
  const int hh = tid / qpr;
  const int h = blockIdx.y * rows_per_block + hh;
  const int c = (tid - hh * qpr) << 2;
  const int tok0 = blockIdx.x * kTokPerBlock;
  const int ntk = min(kTokPerBlock, n_tok - tok0);
  const int64_t tok_stride = (int64_t)H * d;
  if (hh < rows_per_block && h < H) {
    f32x4 a;
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = -expf(alog_pc ? A_log[(int64_t)h * d + c + e] : A_log[h]);
    const f32x4 dtb = *reinterpret_cast<const f32x4*>(dt_bias + (int64_t)h * d + c);
    const int64_t base = (int64_t)tok0 * tok_stride + (int64_t)h * d + c;
    f32x4 sdx = {0.0f, 0.0f, 0.0f, 0.0f}, sda = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int t = 0; t < ntk; ++t) {
      const int64_t i = base + t * tok_stride;
      const f32x4 xv = load4(x, i, XBF16);
      const f32x4 gv = *reinterpret_cast<const f32x4*>(dg + i);
      f32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float z = gate_input(xv[e], dtb[e]);
        out[e] = gv[e] * (a[e] * gate_beta(z));
        sdx[e] += out[e];
        sda[e] = fmaf(gv[e], gate_log_decay(a[e], z), sda[e]);
      }
      *reinterpret_cast<f32x4*>(dx + i) = out;
    }
    const int64_t pbase = ((int64_t)blockIdx.x * H + h) * d + c;
    const int64_t half = (int64_t)gridDim.x * H * d;
    *reinterpret_cast<f32x4*>(part + pbase) = sdx;
    *reinterpret_cast<f32x4*>(part + half + pbase) = sda;
  }
  const int hbase = blockIdx.y * rows_per_block;
  const int nh = min(rows_per_block, H - hbase);
  for (int i = tid; i < ntk * nh; i += kThreads) {
    const int tk = i / nh;
    const int64_t row = (int64_t)(tok0 + tk) * H + hbase + (i - tk * nh);
    const float be = gate_beta(load1(b, row, BBF16));
    db[row] = dbeta[row] * be * (1.0f - be);
  }
}

// ddt_bias[h][c] and dA_log (per channel, or summed over the head's
// channels) from the runs' partial sums; one workgroup per head.
__global__ void __launch_bounds__(1024) gate_bwd_reduce(const float* __restrict__ part, int nrun,
                                                        int H, int d, int alog_pc,
                                                        float* __restrict__ ddt_bias,
                                                        float* __restrict__ dA_log) {
  __shared__ float red[32];
  const int h = blockIdx.x, c = threadIdx.x;
  const int64_t half = (int64_t)nrun * H * d;
  float sdt = 0.0f, sda = 0.0f;
  if (c < d) {
    for (int r = 0; r < nrun; ++r) {
      sdt += part[((int64_t)r * H + h) * d + c];
      sda += part[half + ((int64_t)r * H + h) * d + c];
    }
    ddt_bias[(int64_t)h * d + c] = sdt;
    if (alog_pc) dA_log[(int64_t)h * d + c] = sda;
  }
  if (alog_pc) return;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sda += __shfl_xor(sda, off);
  if ((c & 63) == 0) red[c >> 6] = sda;
  __syncthreads();
  if (c == 0) {
    float s2 = 0.0f;
    for (int w = 0; w < (int)((blockDim.x + 63) / 64); ++w) s2 += red[w];
    dA_log[h] = s2;
  }
}

}  // namespace

size_t gate_bwd_workspace_bytes(int64_t n_tok, int H, int d) {
  return (size_t)2 * (size_t)((n_tok + kTokPerBlock - 1) / kTokPerBlock) * (size_t)H *
         (size_t)d * sizeof(float);
}

hipError_t launch_gate_backward(const void* x, bool x_bf16, const void* b, bool b_bf16,
                                const float* A_log, bool alog_pc, const float* dt_bias,
                                const float* dg, const float* dbeta, float* dx, float* db,
                                float* dA_log, float* ddt_bias, int64_t n_tok, int H, int d,
                                void* ws, hipStream_t s) {
  const int rows_per_block = kThreads / (d >> 2);
  const int head_groups = (H + rows_per_block - 1) / rows_per_block;
  const int64_t nrun = (n_tok + kTokPerBlock - 1) / kTokPerBlock;
  float* part = static_cast<float*>(ws);
  if (nrun > 0) {
    const dim3 grid((unsigned)nrun, head_groups);
    const int nt = static_cast<int>(n_tok);
    const int pc = alog_pc ? 1 : 0;
#define KDA_GB(XB, BB)                                                                        \
  gate_bwd_kernel<XB, BB><<<grid, kThreads, 0, s>>>(x, b, A_log, dt_bias, dg, dbeta, dx, db, \
                                                    part, nt, H, d, rows_per_block, pc)
    if (x_bf16 && b_bf16) KDA_GB(true, true);
    else if (x_bf16) KDA_GB(true, false);
    else if (b_bf16) KDA_GB(false, true);
    else KDA_GB(false, false);
#undef KDA_GB
  }
  const int rthreads = ((d + 63) / 64) * 64;
  gate_bwd_reduce<<<dim3((unsigned)H), rthreads, 0, s>>>(part, (int)nrun, H, d, alog_pc ? 1 : 0,
                                                          ddt_bias, dA_log);
  return hipGetLastError();
}

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
