// kda_gate: log-decay g = -exp(A_log[h]) * softplus(x + dt_bias[h,c]) and
// beta = sigmoid(b), one elementwise HBM-bound pass.
//
// Shapes per the Kimi K3 artifact audit (§4.1 KDA tensor table; §5.2 shape
// table): A_log one value per head, dt_bias one per (head, channel).  beta is
// squashed here in fp32 (Model-Optimizer PR #2749 review, KDA beta fix).
//
// Each thread handles 4 consecutive channels (one 16-byte fp32 load of x, one
// 16-byte store of g); the thread that owns channel 0 of a (token, head) row
// also writes beta.  Grid-stride loop, launched with enough blocks to fill
// every CU several times over.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

__device__ __forceinline__ float softplus_f32(float z) {
  // max(z,0) + log1p(exp(-|z|)): no overflow, accurate for large |z|.
  return fmaxf(z, 0.0f) + log1pf(expf(-fabsf(z)));
}

template <bool XBF16, bool BBF16>
__global__ void __launch_bounds__(256) gate_kernel(const void* __restrict__ x,
                                                   const void* __restrict__ b,
                                                   const float* __restrict__ A_log,
                                                   const float* __restrict__ dt_bias,
                                                   float* __restrict__ g,
                                                   float* __restrict__ beta, int64_t n_quads,
                                                   int H, int d) {
  const int quads_per_row = d >> 2;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n_quads;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / quads_per_row;  // (token, head) row
    const int c = static_cast<int>(i - row * quads_per_row) << 2;
    const int h = static_cast<int>(row % H);
    const f32x4 xv = load4(x, i << 2, XBF16);
    const f32x4 db = *reinterpret_cast<const f32x4*>(dt_bias + (int64_t)h * d + c);
    const float a = -expf(A_log[h]);
    f32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = a * softplus_f32(xv[e] + db[e]);
    *reinterpret_cast<f32x4*>(g + (i << 2)) = out;
    if (c == 0) {
      const float bl = load1(b, row, BBF16);
      beta[row] = 1.0f / (1.0f + expf(-bl));
    }
  }
}

}  // namespace

hipError_t launch_gate(const void* x, bool x_bf16, const void* b, bool b_bf16, const float* A_log,
                       const float* dt_bias, float* g, float* beta, int64_t n_tok, int H, int d,
                       hipStream_t s) {
  const int64_t n_quads = n_tok * H * (d / 4);
  if (n_quads == 0) return hipSuccess;
  const int threads = 256;
  int64_t blocks = (n_quads + threads - 1) / threads;
  const int64_t cap = 256 * 32;  // 32 blocks per CU on 256 CUs, then grid-stride
  if (blocks > cap) blocks = cap;
  if (x_bf16 && b_bf16)
    gate_kernel<true, true><<<blocks, threads, 0, s>>>(x, b, A_log, dt_bias, g, beta, n_quads, H, d);
  else if (x_bf16)
    gate_kernel<true, false><<<blocks, threads, 0, s>>>(x, b, A_log, dt_bias, g, beta, n_quads, H, d);
  else if (b_bf16)
    gate_kernel<false, true><<<blocks, threads, 0, s>>>(x, b, A_log, dt_bias, g, beta, n_quads, H, d);
  else
    gate_kernel<false, false><<<blocks, threads, 0, s>>>(x, b, A_log, dt_bias, g, beta, n_quads, H, d);
  return hipGetLastError();
}

}  // namespace kda
