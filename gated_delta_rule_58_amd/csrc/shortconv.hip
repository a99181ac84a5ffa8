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
// (head, 8-channel octet) of one tensor (q, k or v: blockIdx.z) and 16
// consecutive tokens of one sequence: it keeps its 32 conv weights in
// registers and issues the 19 input rows of its window (3 before, 16 own) at
// once.  A wave covers 4 heads (1 KiB of each row), a workgroup 4 consecutive
// 16-token groups of those heads; workgroups tile each sequence (blockIdx.x =
// (sequence x 64-token block) x head group, head groups fastest), so a group
// never crosses a sequence start.  Rows before the start come from the conv
// state (or are 0), the wave that holds a sequence's last token writes the
// state out, and the 16 lanes of a head reduce the L2 norm with DPP
// operations.  Outputs are written once and not read back: non-temporal
// stores.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int D = 128;
constexpr int TPT = 16;            // tokens per thread
constexpr int GPB = 4;             // token groups per workgroup (one per wave)
constexpr int TPB = TPT * GPB;     // tokens per workgroup
constexpr int HPW = 4;             // heads per wave
constexpr int NTHR = GPB * HPW * 16;
constexpr int NW = TPT + 3;        // window rows per thread

struct Row8f {
  f32x4 a, b;
};

// SiLU and the norm's reciprocal square root on the hardware exp2 / rcp / rsq
// (about 1 ulp each): the IEEE division and expf made this kernel VALU-bound.
__device__ __forceinline__ float silu(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y * 1.4426950408889634f));
}

// Sum over the 16 lanes of a row (one head's 128 channels), in every lane:
// DPP swaps within quads, then rotations by 4 and 8 inside the row (VALU
// operations; a shuffle through LDS would wait on LDS four times per token).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float sum16(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_add<0x124>(v);  // row_ror 4
  return dpp_add<0x128>(v);  // row_ror 8
}

template <bool IN_BF16>
struct RawRow;
template <>
struct RawRow<true> {
  u16x8 v;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int off) {
    v = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  }
  __device__ __forceinline__ float at(int e) const { return bf16_bits_to_f32(v[e]); }
};
template <>
struct RawRow<false> {
  f32x4 a, b;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int off) {
    a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16, 0, 0));
  }
  __device__ __forceinline__ float at(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// The window rows and the output rows go through buffer resources: rows
// before the sequence start or at or past its end read 0 (the offset wraps or
// passes the range) and stores past the end are dropped, so the main path has
// no per-row branch or select.  Each window row is widened to fp32 once and
// added into the (at most four) outputs it feeds as soon as it is used, which
// keeps at most four output rows open; an output row is finished (SiLU, norm,
// store) once its last row has gone in.  The conv sum keeps its order (tap 0
// first), so the results do not depend on this arrangement.
template <bool IN_BF16, bool OUT_BF16, bool SILU>
__global__ void __launch_bounds__(NTHR) shortconv_kernel(
    const void* __restrict__ xq, const void* __restrict__ xk, const void* __restrict__ xv,
    const float* __restrict__ wq, const float* __restrict__ wk, const float* __restrict__ wv,
    float eps, const int32_t* __restrict__ cu, int N, int64_t T_tot, int H,
    int nblk, const float* state_in, float* state_out, void* __restrict__ yq,
    void* __restrict__ yk, void* __restrict__ yv) {
  constexpr int ES = IN_BF16 ? 2 : 4, EO = OUT_BF16 ? 2 : 4;
  // window rows in flight ahead of the one in use: all of them for bf16 input,
  // 10 (80 registers) for fp32
  constexpr int LOOKAHEAD = IN_BF16 ? NW : 10;
  const int z = blockIdx.z;  // 0 q, 1 k, 2 v
  const char* x = static_cast<const char*>(z == 0 ? xq : (z == 1 ? xk : xv));
  const float* w = z == 0 ? wq : (z == 1 ? wk : wv);
  char* y = static_cast<char*>(z == 0 ? yq : (z == 1 ? yk : yv));
  const int t = threadIdx.x;
  // head groups vary fastest: consecutive workgroups read adjacent 1 KiB pieces
  // of the same token rows
  const int HG = (H + HPW - 1) / HPW;
  const int hg = static_cast<int>(blockIdx.x % HG);
  const int64_t sbk = blockIdx.x / HG;
  const int n = static_cast<int>(sbk / nblk);
  const int64_t tblk = (sbk % nblk) * TPB;
  const int64_t t0 = tblk + (int64_t)(t / 64) * TPT;
  const int h = hg * HPW + (t % 64) / 16;
  const int oct = t % 16;
  if (n >= N || h >= H) return;  // whole 16-lane groups leave together
  auto clampi = [&](int64_t v) { return v < 0 ? (int64_t)0 : (v > T_tot ? T_tot : v); };
  const int64_t bos = clampi(cu[n]);
  const int64_t eos = clampi(cu[n + 1]) < bos ? bos : clampi(cu[n + 1]);
  const int64_t L = eos - bos;
  if (t0 >= L) return;  // whole waves
  const int64_t HD = (int64_t)H * D;
  const int64_t c0 = (int64_t)h * D + 8 * oct;
  // conv state layout [N][3 tensors][3 taps, oldest first][H*128] fp32
  const int64_t sbase = ((int64_t)n * 3 + z) * 3 * HD + c0;
  // the workgroup's rows [B, rows_end) of the sequence, B = max(tblk - 3, 0)
  const int64_t B = tblk >= 3 ? tblk - 3 : 0;
  const int64_t rows_end = L < tblk + TPB ? L : tblk + TPB;
  const auto rx = buffer_over(x + ((bos + B) * HD) * ES, (uint32_t)((rows_end - B) * HD * ES));
  const auto ry = buffer_over(y + ((bos + tblk) * HD) * EO, (uint32_t)((rows_end - tblk) * HD * EO));
  // the conv weights first (the first token needs them all), then the window:
  // row j = token t0 - 3 + j of the sequence; all loads issued up front
  f32x4 wc[8];  // wc[e][i] = w[c0 + e, i]
#pragma unroll
  for (int e = 0; e < 8; ++e) wc[e] = *reinterpret_cast<const f32x4*>(w + (c0 + e) * 4);
  RawRow<IN_BF16> win[NW];
  const int r0 = static_cast<int>(t0 - 3 - B);  // row of window row 0, from B (>= -3)
  auto load_row = [&](int j) { win[j].load(rx, static_cast<int>(((r0 + j) * HD + c0) * ES)); };
#pragma unroll
  for (int j = 0; j < (LOOKAHEAD < NW ? LOOKAHEAD : NW); ++j) load_row(j);
  float o[TPT][8];
#pragma unroll
  for (int k = 0; k < TPT; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[k][e] = 0.0f;
  if (t0 == 0 && state_in) {  // rows -3..-1 from the conv state (their loads read 0)
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const f32x4* p = reinterpret_cast<const f32x4*>(state_in + sbase + j * HD);
      const f32x4 a = p[0], b = p[1];
#pragma unroll
      for (int k = 0; k <= j; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[k][e] = fmaf(wc[e][j - k], e < 4 ? a[e] : b[e - 4], o[k][e]);
    }
  }
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    if (j + LOOKAHEAD < NW) load_row(j + LOOKAHEAD);
    float xf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) xf[e] = win[j].at(e);
#pragma unroll
    for (int k = (j - 3 > 0 ? j - 3 : 0); k <= (j < TPT - 1 ? j : TPT - 1); ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[k][e] = fmaf(wc[e][j - k], xf[e], o[k][e]);
    if (j >= 3) {  // output row k = j - 3 is complete
      const int k = j - 3;
      Row8f r;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = SILU ? silu(o[k][e]) : o[k][e];
        if (e < 4) r.a[e] = v;
        else r.b[e - 4] = v;
      }
      if (z < 2) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += r.a[e] * r.a[e] + r.b[e] * r.b[e];
        const float inv = __builtin_amdgcn_rsqf(sum16(ss) + eps);
        r.a *= inv;
        r.b *= inv;
      }
      const int oo = static_cast<int>(((t0 - tblk + k) * HD + c0) * EO);
      if constexpr (OUT_BF16) {
        u16x8 b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          b[e] = f32_to_bf16_bits(r.a[e]);
          b[4 + e] = f32_to_bf16_bits(r.b[e]);
        }
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, b), ry, oo, 0, kBufNT);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, r.a), ry, oo, 0, kBufNT);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, r.b), ry, oo + 16, 0,
                                               kBufNT);
      }
    }
  }
  // the wave holding the sequence's last token passes the last 3 inputs on:
  // tokens L - 3 .. L - 1, from the window (reloaded) or, before the
  // sequence start, from the conv state (or 0)
  if (state_out && t0 + TPT >= L) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int64_t r = L - 3 + i;
      f32x4 a, b;
      if (r >= 0) {
        RawRow<IN_BF16> row;
        row.load(rx, static_cast<int>(((r - B) * HD + c0) * ES));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = row.at(e);
          b[e] = row.at(4 + e);
        }
      } else if (state_in) {
        const f32x4* p = reinterpret_cast<const f32x4*>(state_in + sbase + (3 + r) * HD);
        a = p[0];
        b = p[1];
      } else {
        a = f32x4{0.f, 0.f, 0.f, 0.f};
        b = a;
      }
      f32x4* p = reinterpret_cast<f32x4*>(state_out + sbase + i * HD);
      p[0] = a;
      p[1] = b;
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
    const int64_t nwg = (int64_t)N * nblk * ((H + HPW - 1) / HPW);
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(nwg), 1, 3);
#define KDA_SC(IB, OB)                                                                   \
  do {                                                                                   \
    if (silu)                                                                            \
      shortconv_kernel<IB, OB, true><<<grid, NTHR, 0, s>>>(xq, xk, xv, wq, wk, wv, eps, cu,  \
                                                           N, T_tot, H, (int)nblk,           \
                                                           state_in, state_out, yq, yk, yv); \
    else                                                                                 \
      shortconv_kernel<IB, OB, false><<<grid, NTHR, 0, s>>>(xq, xk, xv, wq, wk, wv, eps, cu, \
                                                            N, T_tot, H, (int)nblk,          \
                                                            state_in, state_out, yq, yk, yv);\
  } while (0)
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
