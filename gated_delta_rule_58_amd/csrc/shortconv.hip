// kda_shortconv_l2norm: the KDA layer's prologue to the core.  The q, k and v
// projections each go through a causal depthwise convolution of kernel 4 per
// channel (the checkpoint's q/k/v_conv1d.weight, fp32 [H*128, 1, 4]: Kimi K3
// artifact audit, §4.1), an optional SiLU, and q and k are then L2-normalised
// over the 128 channels of each (token, head):
//   y[t, c] = sum_{i=0..3} w[c, i] x[t - 3 + i, c]     (x before the sequence
//             start comes from the conv state, or is 0)
//   y = silu(y) if requested;   q, k: y / sqrt(sum_c y^2 + eps)
// Sequences are packed (cu_seqlens) and never mix; the conv state of a
// sequence is its last 3 inputs per channel, oldest first, in and out, so a
// prefill followed by one-token steps equals one longer prefill.
//
// HBM-bound elementwise work with a 16-lane reduction.  A thread owns one
// (head, 8-channel octet) of one tensor (q, k or v: blockIdx.z) and 8
// consecutive tokens of one sequence: it keeps its 32 conv weights in
// registers and issues the 11 input rows of its window (3 before, 8 own) at
// once.  A wave covers 4 heads (1 KiB of each row), a workgroup 4 consecutive
// 8-token groups of those heads; workgroups tile each sequence (blockIdx.x =
// sequence x 32-token block), so a group never crosses a sequence start.
// Rows before the start come from the conv state (or are 0), the thread that
// holds a sequence's last token writes the state out, and the 16 lanes of a
// head reduce the L2 norm with shuffles.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int D = 128;
constexpr int TPT = 8;             // tokens per thread
constexpr int GPB = 4;             // token groups per workgroup (one per wave)
constexpr int TPB = TPT * GPB;     // tokens per workgroup
constexpr int HPW = 4;             // heads per wave
constexpr int NTHR = GPB * HPW * 16;
constexpr int NW = TPT + 3;        // window rows per thread

struct Row8f {
  f32x4 a, b;
};

__device__ __forceinline__ Row8f load_row8(const void* base, int64_t idx, bool bf16) {
  if (bf16) {
    const u16x8 r = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(base) + idx);
    return Row8f{f32x4{bf16_bits_to_f32(r[0]), bf16_bits_to_f32(r[1]), bf16_bits_to_f32(r[2]),
                       bf16_bits_to_f32(r[3])},
                 f32x4{bf16_bits_to_f32(r[4]), bf16_bits_to_f32(r[5]), bf16_bits_to_f32(r[6]),
                       bf16_bits_to_f32(r[7])}};
  }
  const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
  return Row8f{p[0], p[1]};
}

__device__ __forceinline__ void store_row8(void* base, int64_t idx, const Row8f& y, bool bf16) {
  if (bf16) {
    u16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = f32_to_bf16_bits(y.a[e]);
      r[4 + e] = f32_to_bf16_bits(y.b[e]);
    }
    *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(base) + idx) = r;
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx);
    p[0] = y.a;
    p[1] = y.b;
  }
}

// SiLU and the norm's reciprocal square root on the hardware exp2 / rcp / rsq
// (about 1 ulp each): the IEEE division and expf made this kernel VALU-bound.
__device__ __forceinline__ float silu(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y * 1.4426950408889634f));
}

template <bool IN_BF16>
struct RawRow;
template <>
struct RawRow<true> {
  u16x8 v;
  __device__ __forceinline__ float at(int e) const { return bf16_bits_to_f32(v[e]); }
};
template <>
struct RawRow<false> {
  f32x4 a, b;
  __device__ __forceinline__ float at(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

template <bool IN_BF16, bool OUT_BF16>
__global__ void __launch_bounds__(NTHR) shortconv_kernel(
    const void* __restrict__ xq, const void* __restrict__ xk, const void* __restrict__ xv,
    const float* __restrict__ wq, const float* __restrict__ wk, const float* __restrict__ wv,
    int silu_on, float eps, const int32_t* __restrict__ cu, int N, int64_t T_tot, int H,
    int nblk, const float* state_in, float* state_out, void* __restrict__ yq,
    void* __restrict__ yk, void* __restrict__ yv) {
  const int z = blockIdx.z;  // 0 q, 1 k, 2 v
  const void* x = z == 0 ? xq : (z == 1 ? xk : xv);
  const float* w = z == 0 ? wq : (z == 1 ? wk : wv);
  void* y = z == 0 ? yq : (z == 1 ? yk : yv);
  const int t = threadIdx.x;
  const int n = blockIdx.x / nblk;
  const int64_t t0 = (int64_t)(blockIdx.x % nblk) * TPB + (int64_t)(t / 64) * TPT;
  const int h = blockIdx.y * HPW + (t % 64) / 16;
  const int oct = t % 16;
  if (n >= N || h >= H) return;  // whole 16-lane groups leave together
  auto clampi = [&](int64_t v) { return v < 0 ? (int64_t)0 : (v > T_tot ? T_tot : v); };
  const int64_t bos = clampi(cu[n]);
  const int64_t eos = clampi(cu[n + 1]) < bos ? bos : clampi(cu[n + 1]);
  const int64_t L = eos - bos;
  if (t0 >= L) return;
  const int64_t HD = (int64_t)H * D;
  const int64_t c0 = (int64_t)h * D + 8 * oct;
  // conv state layout [N][3 tensors][3 taps, oldest first][H*128] fp32
  const int64_t sbase = ((int64_t)n * 3 + z) * 3 * HD + c0;
  // the conv weights first (the first token needs them all), then the window:
  // row j = token t0 - 3 + j of the sequence; all loads issued up front
  f32x4 wc[8];  // wc[e][i] = w[c0 + e, i]
#pragma unroll
  for (int e = 0; e < 8; ++e) wc[e] = *reinterpret_cast<const f32x4*>(w + (c0 + e) * 4);
  RawRow<IN_BF16> win[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int64_t r = t0 - 3 + j;
    if (r >= 0 && r < L) {
      const int64_t e = (bos + r) * HD + c0;
      if constexpr (IN_BF16) {
        win[j].v = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(x) + e);
      } else {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + e);
        win[j].a = p[0];
        win[j].b = p[1];
      }
    }
  }
  // rows before the sequence start: the conv state (fp32), or 0
  float pre[3][8];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int64_t r = t0 - 3 + j;
    if (r < 0 && state_in) {
      const f32x4* p = reinterpret_cast<const f32x4*>(state_in + sbase + (3 + r) * HD);
      const f32x4 a = p[0], b = p[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pre[j][e] = a[e];
        pre[j][4 + e] = b[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) pre[j][e] = 0.f;
    }
  }
  auto val = [&](int j, int e) -> float {  // window row j, channel e (fp32)
    return (j < 3 && t0 - 3 + j < 0) ? pre[j][e] : win[j].at(e);
  };
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    if (t0 + k >= L) break;
    Row8f o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc += wc[e][i] * val(k + i, e);
      if (silu_on) acc = silu(acc);
      if (e < 4) o.a[e] = acc;
      else o.b[e - 4] = acc;
    }
    if (z < 2) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += o.a[e] * o.a[e] + o.b[e] * o.b[e];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) ss += __shfl_xor(ss, off);
      const float inv = __builtin_amdgcn_rsqf(ss + eps);
      o.a *= inv;
      o.b *= inv;
    }
    store_row8(y, (bos + t0 + k) * HD + c0, o, OUT_BF16);
  }
  // the thread holding the sequence's last token passes the last 3 inputs on:
  // window rows L - t0 .. L - t0 + 2
  if (state_out && t0 + TPT >= L) {
    const int j0 = static_cast<int>(L - t0);  // 1..8
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      if (j >= j0 && j <= j0 + 2) {
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = val(j, e);
          b[e] = val(j, 4 + e);
        }
        f32x4* p = reinterpret_cast<f32x4*>(state_out + sbase + (j - j0) * HD);
        p[0] = a;
        p[1] = b;
      }
    }
  }
}

// Sequences with no tokens pass their state on unchanged (zeros without one).
__global__ void __launch_bounds__(256) shortconv_empty_kernel(const int32_t* __restrict__ cu, int N,
                                                              int64_t T_tot, int64_t HD,
                                                              const float* state_in,
                                                              float* state_out) {
  const int n = blockIdx.x;
  auto clampi = [&](int64_t v) { return v < 0 ? (int64_t)0 : (v > T_tot ? T_tot : v); };
  if (n >= N || clampi(cu[n + 1]) > clampi(cu[n])) return;
  const int64_t base = (int64_t)n * 9 * HD;
  for (int64_t i = threadIdx.x; i < 9 * HD; i += blockDim.x)
    state_out[base + i] = state_in ? state_in[base + i] : 0.0f;
}

}  // namespace

hipError_t launch_shortconv(const void* xq, const void* xk, const void* xv, bool in_bf16,
                            const float* wq, const float* wk, const float* wv, bool silu,
                            float eps, const int32_t* cu, int N, int64_t min_len,
                            int64_t max_len, int64_t T_tot, int H, const float* state_in,
                            float* state_out, void* yq, void* yk, void* yv, bool out_bf16,
                            hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (T_tot > 0 && max_len > 0) {
    const int64_t nblk = (max_len + TPB - 1) / TPB;
    if ((int64_t)N * nblk > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(N * nblk), static_cast<unsigned>((H + HPW - 1) / HPW),
                    3);
#define KDA_SC(IB, OB)                                                                         \
  shortconv_kernel<IB, OB><<<grid, NTHR, 0, s>>>(xq, xk, xv, wq, wk, wv, silu ? 1 : 0, eps, cu, \
                                                 N, T_tot, H, (int)nblk, state_in, state_out,  \
                                                 yq, yk, yv)
    if (in_bf16 && out_bf16) KDA_SC(true, true);
    else if (in_bf16) KDA_SC(true, false);
    else if (out_bf16) KDA_SC(false, true);
    else KDA_SC(false, false);
#undef KDA_SC
  }
  if (state_out && min_len == 0)
    shortconv_empty_kernel<<<dim3(static_cast<unsigned>(N)), 256, 0, s>>>(
        cu, N, T_tot, (int64_t)H * D, state_in, state_out);
  return hipGetLastError();
}

}  // namespace kda
