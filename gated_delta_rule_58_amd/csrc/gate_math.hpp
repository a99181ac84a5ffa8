// The KDA gate, elementwise (Kimi K3 artifact audit, §4.1 KDA tensor table:
// per-head A_log, per-(head, channel) dt_bias; beta squashed once in fp32,
// Model-Optimizer PR #2749 review):
//   g    = -exp(A_log[h]) * softplus(x + dt_bias[h, c])
//   beta = sigmoid(b)
// softplus(z) = max(z, 0) + log1p(exp(-|z|)).
//
// kda_gate writes g to memory, so it keeps every digit: the tail
// log1p(exp(-|z|)) uses the hardware exp2/log2 with two corrections that keep
// it within a few ulp of the exact value, where a plain log2(1 + e) would lose
// up to all of the digits of a small e:
//   e = 2^(-t) with t = |z| log2(e) rounded; the product's residual (an fma)
//       and the fp32 constant's own error are folded back in to first order;
//   log1p(e) = log(u) * e / (u - 1) with u = fl(1 + e) (exact when u = 1).
// The gated prefill only sums g into the cumulative decay, where an absolute
// error of a few 2^-24 per token is far below the fp16 rounding of the
// decayed operands; it uses the plain form in log2 units (gate_log2_decay_fast).
#pragma once

#include <hip/hip_runtime.h>

namespace kda {

constexpr float kGateLog2e = 1.4426950216293335f;     // fp32 nearest of log2(e)
constexpr float kGateLog2eLo = 1.92596298909109e-08f;  // log2(e) - kGateLog2e
constexpr float kGateLn2 = 0.6931471824645996f;

// log1p(exp(-az)) for az = |z| >= 0; beyond 200 the value is below fp32's
// range (and an infinite az must not reach the residual product).
__device__ __forceinline__ float softplus_tail(float az) {
#pragma clang fp contract(off)
  az = fminf(az, 200.0f);
  const float t = az * kGateLog2e;
  const float r = fmaf(az, kGateLog2e, -t) + az * kGateLog2eLo;  // az*log2(e) - t
  const float e = __builtin_amdgcn_exp2f(-t) * fmaf(-r, kGateLn2, 1.0f);
  const float u = 1.0f + e;
  const float d = u - 1.0f;
  const float l = __builtin_amdgcn_logf(u) * kGateLn2 * (e * __builtin_amdgcn_rcpf(d));
  return d == 0.0f ? e : l;
}

// Every function here turns floating-point contraction off, so that the gate
// kernel and the gated prefill execute exactly the same operations.
// neg_a = -exp(A_log[h]); z = x + dt_bias
__device__ __forceinline__ float gate_log_decay(float neg_a, float z) {
#pragma clang fp contract(off)
  return neg_a * (fmaxf(z, 0.0f) + softplus_tail(fabsf(z)));
}

// g log2(e) with the plain hardware exp2 / log2: -a log2(e) max(z, 0) -
// a log2(1 + 2^(-|z| log2 e)).  Absolute error about a 2^-23; the relative
// error grows where softplus(z) is tiny (z << 0), which the cumulative decay
// does not feel.
__device__ __forceinline__ float gate_log2_decay_fast(float neg_a, float z) {
  const float e = __builtin_amdgcn_exp2f(-fabsf(z) * kGateLog2e);
  const float l2 = __builtin_amdgcn_logf(1.0f + e);
  return fmaf(neg_a * kGateLog2e, fmaxf(z, 0.0f), neg_a * l2);
}

__device__ __forceinline__ float gate_beta(float b_logit) {
#pragma clang fp contract(off)
  return 1.0f / (1.0f + expf(-b_logit));
}

// z = x + dt_bias, rounded on its own (no contraction into a neighbour)
__device__ __forceinline__ float gate_input(float x, float dt_bias) {
#pragma clang fp contract(off)
  return x + dt_bias;
}

}  // namespace kda
