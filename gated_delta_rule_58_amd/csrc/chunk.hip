// kda_chunk_prefill: chunked KDA prefill over packed variable-length batches.
//
// Math (one sequence, one head; chunk of C=64 tokens, entry state S, d=128).
// The recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
// o_t = S_t^T q_t (the code audit's chunked training/prefill regime) unrolls
// over a chunk into, with gamma_r = sum_{s<=r} g_s per key channel:
//   A[r,s] = b_r sum_c k_rc k_sc e^(gamma_rc - gamma_sc)   (s < r)
//   P[r,s] =     sum_c q_rc k_sc e^(gamma_rc - gamma_sc)   (s <= r)
//   X      = V - (K * e^gamma) S
//   (I + A) Delta = diag(b) X                                (forward substitution)
//   O      = scale * ((Q * e^gamma) S + P Delta)
//   S     <- Diag(e^gamma_C) S + (K * e^(gamma_C - gamma))^T Delta
// Every term is independent across value columns, so one workgroup owns one
// (sequence, head, 64-column value tile) and walks the chunks of its sequence
// in order.
//
// Work split inside a workgroup (4 waves), per chunk:
//  * chunk operands (phases P0..P2, independent of the state): wave i owns
//    chunk rows 16i..16i+15 (block i).  It forms e^gamma-scaled Q and K, the
//    decay-scaled K^T, the tiles (i, j<=i) of A and P, and the inverse T_ii of
//    its diagonal block (I + A_ii).  All land in LDS as fp16 MFMA operands.
//  * state products (phase P3, no barriers inside): wave w owns value
//    columns 16w..16w+15 of the tile and keeps its 128x16 slice of S, and its
//    64x16 slices of X, Delta and O, in MFMA accumulators for the whole
//    sequence.  Delta is solved block by block,
//        Delta_i = T_ii (b_i X_i - sum_{j<i} A_ij Delta_j),
//    with 16x16x16 MFMAs whose accumulator layout is their B-operand layout.
//    The contraction index of every 16x16x32 product whose B operand comes
//    from an accumulator is stored permuted in LDS (see `pperm`), so an
//    accumulator tile pair is directly the B fragment of the next product:
//    the state never round-trips through LDS.
//
// Decay factors.  gamma is kept in log2 units and every exponential is a
// hardware exp2.  Inside a chunk gamma can fall far below -126, so factors
// are built relative to references: for block i with mid row m_i = 16i+7,
//   E_r = 2^(gamma_r - gamma_m),  F_r = 2^(gamma_m - gamma_r)
// span at most 8 tokens of decay (2 exp2 per element), and every other factor
// is E or F times a per-(block, channel) constant that is <= 1, e.g.
//   2^gamma_r = E_r 2^gamma_m,  2^(gamma_C - gamma_r) = F_r 2^(gamma_C - gamma_m).
// An off-diagonal tile (i, j) multiplies k_r 2^(gamma_r - gamma_b) by
// k_s 2^(gamma_b - gamma_s), b = last row of block j: both <= 1 (fp16).  The
// diagonal tiles multiply E and F, bounded by 8 tokens of decay, as hi+lo
// bf16 pairs, which keep fp32 range.  Requirement: no channel decays by more
// than 126 (log2 units) over 8 consecutive tokens.
//
// Precision.  MFMA operands are fp16 (bf16 inputs convert exactly); the state
// S, X, Delta and P are split into hi+lo fp16 pairs, so their rounding does
// not reach the result; accumulation is fp32.
#include <type_traits>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int C = 64;     // chunk length
constexpr int D = 128;    // dk = dv
constexpr int DV = 64;    // value columns per workgroup
constexpr int NT = D / DV;
constexpr int NTHR = 256; // 4 waves
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f16_k16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Orders this wave's LDS writes before its later LDS reads (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Contraction-index permutation inside a group of 32.  For the 16x16x32 MFMA,
// lane (lr, lg) supplies contraction elements 8lg..8lg+7; an accumulator tile
// pair (t, t+1) holds rows 16t+4lg+i and 16(t+1)+4lg+i in lane (lr, lg).  So
// logical index L = 16a + 4b + c (a<2, b<4, c<4) is stored at position
// 8b + 4a + c, and fragment element e of lane group lg is logical
// 16(e>>2) + 4lg + (e&3).
__device__ __forceinline__ int pperm(int L) { return ((L >> 2) & 3) * 8 + (L >> 4) * 4 + (L & 3); }
__device__ __forceinline__ int ppos64(int s) { return (s & 32) + pperm(s & 31); }

__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

// 16x16x32 B fragment (hi and lo fp16) from an accumulator tile pair.
__device__ __forceinline__ void bfrag_split(const f32x4& t0, const f32x4& t1, f16x8& hi,
                                            f16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    _Float16 a, b;
    split_f16(e < 4 ? t0[e] : t1[e - 4], a, b);
    hi[e] = a;
    lo[e] = b;
  }
}
// 16x16x16 B fragment (hi and lo fp16) from one accumulator tile.
__device__ __forceinline__ void bfrag16_split(const f32x4& t, f16x4& hi, f16x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    _Float16 a, b;
    split_f16(t[e], a, b);
    hi[e] = a;
    lo[e] = b;
  }
}

// LDS layout (bytes).
struct Lds {
  static constexpr int GAM_LD = 132;   // fp32 [64][132]   half-local gamma (log2 units)
  static constexpr int OP_LD = 136;    // fp16 [64][136]   Kt, Qt (channel-permuted); R [48][136]
  static constexpr int TT_LD = 72;     // fp16 [..][72]    Khat^T, P hi/lo (token-permuted)
  static constexpr int AT_LD = 72;     // fp16 [64][72]    -A_ij below the diagonal blocks, T_ii on them
  static constexpr int SC_LD = 17;     // fp32 [4][16][17] per-wave A_ii scratch

  static constexpr int off_gam = 0;                       // P0..P1a
  static constexpr int off_R = 0;                         // P1b..P2 (aliases gam)
  static constexpr int end_gamR = C * GAM_LD * 4;
  static constexpr int off_Kt = end_gamR;
  static constexpr int off_Qt = off_Kt + C * OP_LD * 2;
  static constexpr int off_KhT = off_Qt + C * OP_LD * 2;
  static constexpr int off_Ph = off_KhT + D * TT_LD * 2;
  static constexpr int off_Pl = off_Ph + C * TT_LD * 2;
  static constexpr int off_AT = off_Pl + C * TT_LD * 2;
  static constexpr int off_scr = off_AT + C * AT_LD * 2;
  static constexpr int off_cst = off_scr + 4 * 16 * SC_LD * 4;
  static constexpr int off_beta = off_cst + 18 * D * 4;
  static constexpr int off_tot = off_beta + C * 4;
  static constexpr int off_seq = off_tot + D * 4;
  static constexpr int total = off_seq + 16;
};
static_assert(Lds::total <= 160 * 1024, "LDS budget");
static_assert(3 * 16 * Lds::OP_LD * 2 <= Lds::end_gamR, "R fits in the gamma region");

// Per-channel constant slots (after exp2, all <= 1):
//  0..3   em_i = 2^gamma_{m_i}
//  4..7   eL_i = 2^(gamma_C - gamma_{m_i})
//  8..13  c(i,j) = 2^(gamma_{m_i} - gamma_{b_{j+1}}), b_{j+1} = last row of block j:
//         (1,0),(2,1),(3,2) at 8,9,10; (2,0) 11; (3,1) 12; (3,0) 13
//  14..16 eR_j = 2^(gamma_{b_{j+1}} - gamma_{m_j}), j = 0..2
//  17     eC = 2^gamma_C
__device__ __forceinline__ int cij_slot(int i, int j) {
  return (j == i - 1) ? 7 + i : (i == 2 ? 11 : (j == 1 ? 12 : 13));
}

template <bool BF16>
struct QKRaw;  // raw prefetched q or k values of one lane: 4 k-steps x 2 halves x 4
template <>
struct QKRaw<true> {
  u16x4 v[4][2];
};
template <>
struct QKRaw<false> {
  f32x4 v[4][2];
};

template <bool BF16>
__device__ __forceinline__ void load_qk(QKRaw<BF16>& R, const void* base, int64_t tok, int lg) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int c = 32 * kk + 16 * a + 4 * lg;
      if constexpr (BF16)
        R.v[kk][a] = *reinterpret_cast<const u16x4*>(static_cast<const uint16_t*>(base) + tok + c);
      else
        R.v[kk][a] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + tok + c);
    }
}

template <bool BF16>
__device__ __forceinline__ float qk_at(const QKRaw<BF16>& R, int kk, int a, int e) {
  if constexpr (BF16) return bf16_bits_to_f32(R.v[kk][a][e]);
  else return R.v[kk][a][e];
}

template <bool QKV_BF16, bool O_BF16>
__global__ void __launch_bounds__(NTHR, 1) chunk_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int N, const float* __restrict__ S0,
    float* __restrict__ Sf, void* __restrict__ o, int T_tot, int H, float scale) {
  __shared__ __attribute__((aligned(16))) char lds[Lds::total];
  float* gam = reinterpret_cast<float*>(lds + Lds::off_gam);
  _Float16* Rb = reinterpret_cast<_Float16*>(lds + Lds::off_R);
  _Float16* Kt = reinterpret_cast<_Float16*>(lds + Lds::off_Kt);
  _Float16* Qt = reinterpret_cast<_Float16*>(lds + Lds::off_Qt);
  _Float16* KhT = reinterpret_cast<_Float16*>(lds + Lds::off_KhT);
  _Float16* Ph = reinterpret_cast<_Float16*>(lds + Lds::off_Ph);
  _Float16* Pl = reinterpret_cast<_Float16*>(lds + Lds::off_Pl);
  _Float16* AT = reinterpret_cast<_Float16*>(lds + Lds::off_AT);
  float* cst = reinterpret_cast<float*>(lds + Lds::off_cst);
  float* s_beta = reinterpret_cast<float*>(lds + Lds::off_beta);
  float* s_tot = reinterpret_cast<float*>(lds + Lds::off_tot);
  int* s_seq = reinterpret_cast<int*>(lds + Lds::off_seq);

  const int tid = threadIdx.x;
  const int w = tid >> 6;          // wave
  const int lane = tid & 63;
  const int lr = lane & 15;        // MFMA row/column within a 16x16 tile
  const int lg = lane >> 4;        // MFMA k-group
  float* scr = reinterpret_cast<float*>(lds + Lds::off_scr) + w * 16 * Lds::SC_LD;

  // ---- workgroup -> (sequence, head, value tile).  Both tiles of one
  // (sequence, head) land on the same XCD (blockIdx % 8) and share its L2.
  const int P = N * H;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int p = (slot / NT) * 8 + xcd;
  const int tile = slot % NT;
  if (p >= P) return;
  const int h = p % H;
  const int seq_rank = p / H;
  int n = seq_rank;
  if (N > 1 && N <= 64) {
    // Longest sequences first: rank sequences by length (ties by index).
    if (tid < N) {
      auto clampi = [&](int x) { return x < 0 ? 0 : (x > T_tot ? T_tot : x); };
      const int li = clampi(cu[tid + 1]) - clampi(cu[tid]);
      int rank = 0;
      for (int j = 0; j < N; ++j) {
        const int lj = clampi(cu[j + 1]) - clampi(cu[j]);
        rank += (lj > li) || (lj == li && j < tid);
      }
      if (rank == seq_rank) s_seq[0] = tid;
    }
    __syncthreads();
    n = s_seq[0];
  }
  int bos = cu[n], eos = cu[n + 1];
  bos = bos < 0 ? 0 : (bos > T_tot ? T_tot : bos);
  eos = eos < bos ? bos : (eos > T_tot ? T_tot : eos);
  const int64_t HD = (int64_t)H * D;
  const int64_t hD = (int64_t)h * D;
  const int col0 = tile * DV;
  const int jcol = col0 + 16 * w + lr;   // value column owned by this lane (state products)

  // ---- state slice: wave w, tile t: key rows 16t + 4lg + i, value column jcol.
  f32x4 Sacc[8];
  const int64_t sbase = ((int64_t)n * H + h) * D * D;
  if (S0) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) Sacc[t][i] = S0[sbase + (int64_t)(16 * t + 4 * lg + i) * D + jcol];
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) Sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- prefetch registers for the next chunk.  Loads are unconditional,
  // from rows clamped into the chunk (a partial chunk re-reads its last row);
  // rows past the end are zeroed where the values are used, so no load sits
  // behind a branch and none forces an early wait.
  using VRaw = typename std::conditional<QKV_BF16, uint32_t, float>::type;
  const int gc = tid & 127, ghf = tid >> 7;  // gamma pass: channel, half
  const int rA = 16 * w + lr;                // chunk row of this lane in the operand phases
  float gpf[32];
  QKRaw<QKV_BF16> kpf, qpf;
  VRaw vraw[16];
  float bpf = 0.0f;
  auto prefetch_gkq = [&](int t0n) {
    const int rmax = ((eos - t0n) < C ? (eos - t0n) : C) - 1;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int rr = (32 * ghf + i) < rmax ? (32 * ghf + i) : rmax;
      gpf[i] = g[(int64_t)(t0n + rr) * HD + hD + gc];
    }
    const int rr = rA < rmax ? rA : rmax;
    const int64_t tok = (int64_t)(t0n + rr) * HD + hD;
    load_qk<QKV_BF16>(kpf, k, tok, lg);
    load_qk<QKV_BF16>(qpf, q, tok, lg);
    if (tid < C) bpf = beta[(int64_t)(t0n + (tid < rmax ? tid : rmax)) * H + h];
  };
  auto prefetch_v = [&](int t0n) {
    const int rmax = ((eos - t0n) < C ? (eos - t0n) : C) - 1;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int rr = 16 * rt + 4 * lg + i;
        rr = rr < rmax ? rr : rmax;
        const int64_t vi = (int64_t)(t0n + rr) * HD + hD + jcol;
        if constexpr (QKV_BF16) vraw[4 * rt + i] = static_cast<const uint16_t*>(v)[vi];
        else vraw[4 * rt + i] = static_cast<const float*>(v)[vi];
      }
  };
  auto vval = [&](int idx) -> float {
    if constexpr (QKV_BF16) return __uint_as_float(vraw[idx] << 16);
    else return vraw[idx];
  };
  if (bos < eos) {
    prefetch_gkq(bos);
    prefetch_v(bos);
  }

  for (int t0 = bos; t0 < eos; t0 += C) {
    const int Lc = (eos - t0) < C ? (eos - t0) : C;

    // ================= P0: gamma, cumsum of g within each 32-row half (log2 units)
    // Blocks never straddle a half, so E/F (differences inside a block) need no
    // offset; the constants add the first half's total to rows >= 32.
    {
      float gv[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) gv[i] = (32 * ghf + i < Lc) ? gpf[i] * LOG2E : 0.0f;
#pragma unroll
      for (int i = 1; i < 32; ++i) gv[i] += gv[i - 1];
#pragma unroll
      for (int i = 0; i < 32; ++i) gam[(32 * ghf + i) * Lds::GAM_LD + gc] = gv[i];
      if (ghf == 0) s_tot[gc] = gv[31];
      if (tid < C) s_beta[tid] = (tid < Lc) ? bpf : 0.0f;
    }
    __syncthreads();

    // ================= P1a: constants, decay factors, diagonal tiles and T_ii
    // Lane (lr, lg) of wave i handles chunk row r = 16i + lr and, in k-step kk,
    // the 8 channels 32kk + 16a + 4lg + j (a < 2, j < 4), fragment element 4a + j.
    const int bi = w;
    const int r = rA;
    const bool rvalid = r < Lc;
    float kE[4][8], qE[4][8], kF[4][8];
    {
      // per-channel constants: half 0 does slots 0..8, half 1 slots 9..17
      {
        const int c = gc;
        const float off = s_tot[c];
        const float gm0 = gam[7 * Lds::GAM_LD + c], gm1 = gam[23 * Lds::GAM_LD + c];
        const float gm2 = gam[39 * Lds::GAM_LD + c] + off, gm3 = gam[55 * Lds::GAM_LD + c] + off;
        const float gb1 = gam[15 * Lds::GAM_LD + c], gb2 = off;
        const float gb3 = gam[47 * Lds::GAM_LD + c] + off, gl = gam[63 * Lds::GAM_LD + c] + off;
        if (ghf == 0) {
          cst[0 * D + c] = ex2(gm0);
          cst[1 * D + c] = ex2(gm1);
          cst[2 * D + c] = ex2(gm2);
          cst[3 * D + c] = ex2(gm3);
          cst[4 * D + c] = ex2(gl - gm0);
          cst[5 * D + c] = ex2(gl - gm1);
          cst[6 * D + c] = ex2(gl - gm2);
          cst[7 * D + c] = ex2(gl - gm3);
          cst[8 * D + c] = ex2(gm1 - gb1);
        } else {
          cst[9 * D + c] = ex2(gm2 - gb2);
          cst[10 * D + c] = ex2(gm3 - gb3);
          cst[11 * D + c] = ex2(gm2 - gb1);
          cst[12 * D + c] = ex2(gm3 - gb2);
          cst[13 * D + c] = ex2(gm3 - gb1);
          cst[14 * D + c] = ex2(gb1 - gm0);
          cst[15 * D + c] = ex2(gb2 - gm1);
          cst[16 * D + c] = ex2(gb3 - gm2);
          cst[17 * D + c] = ex2(gl);
        }
      }
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
      const int mrow = 16 * bi + 7;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8 ekh, ekl, eqh, eql, fkh, fkl;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int c = 32 * kk + 16 * a + 4 * lg;
          const f32x4 gr = *reinterpret_cast<const f32x4*>(gam + r * Lds::GAM_LD + c);
          const f32x4 gm = *reinterpret_cast<const f32x4*>(gam + mrow * Lds::GAM_LD + c);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = 4 * a + j;
            const float kv = rvalid ? qk_at<QKV_BF16>(kpf, kk, a, j) : 0.0f;
            const float qv = rvalid ? qk_at<QKV_BF16>(qpf, kk, a, j) : 0.0f;
            const float dg = gr[j] - gm[j];
            const float E = ex2(dg), F = ex2(-dg);
            kE[kk][e] = kv * E;
            qE[kk][e] = qv * E;
            kF[kk][e] = kv * F;
            __bf16 x0, x1;
            split_bf16(kE[kk][e], x0, x1); ekh[e] = x0; ekl[e] = x1;
            split_bf16(qE[kk][e], x0, x1); eqh[e] = x0; eql[e] = x1;
            split_bf16(kF[kk][e], x0, x1); fkh[e] = x0; fkl[e] = x1;
          }
        }
        accA = mma_bf16(ekh, fkh, accA);
        accA = mma_bf16(ekh, fkl, accA);
        accA = mma_bf16(ekl, fkh, accA);
        accP = mma_bf16(eqh, fkh, accP);
        accP = mma_bf16(eqh, fkl, accP);
        accP = mma_bf16(eql, fkh, accP);
      }
      // diagonal tile (bi, bi): lane holds rows 16bi + 4lg + i, column s = 16bi + lr
      const int sp = ppos64(16 * bi + lr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 4 * lg + i, row = 16 * bi + rr;
        scr[rr * Lds::SC_LD + lr] = (lr < rr) ? accA[i] * s_beta[row] : 0.0f;
        _Float16 x0, x1;
        split_f16((lr <= rr) ? accP[i] : 0.0f, x0, x1);
        Ph[row * Lds::TT_LD + sp] = x0;
        Pl[row * Lds::TT_LD + sp] = x1;
        if ((bi & 1) == 0) {  // upper tile (bi, bi+1) of P lies inside a 32-wide k-step
          const int su = ppos64(16 * bi + 16 + lr);
          Ph[row * Lds::TT_LD + su] = static_cast<_Float16>(0.0f);
          Pl[row * Lds::TT_LD + su] = static_cast<_Float16>(0.0f);
        }
      }
      // T_ii = (I + A_ii)^-1 by forward substitution, one column per lane
      wave_lds_sync();
      if (lane < 16) {
        const int jj = lane;
        float tc[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          float acc = (rr == jj) ? 1.0f : 0.0f;
#pragma unroll
          for (int s = 0; s < rr; ++s) acc -= scr[rr * Lds::SC_LD + s] * tc[s];
          tc[rr] = acc;
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          AT[(16 * bi + rr) * Lds::AT_LD + 16 * bi + jj] = static_cast<_Float16>(tc[rr]);
      }
    }
    __syncthreads();

    // the chunk's q/k/g/beta are consumed: fetch the next chunk's
    if (t0 + C < eos) prefetch_gkq(t0 + C);

    // ================= P1b: operands that need the constants
    {
      const int kpos = ppos64(r);  // token-permuted column of this row in Khat^T
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        f16x8 kt, qt, rr8;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int c = 32 * kk + 16 * a + 4 * lg;
          const f32x4 em = *reinterpret_cast<const f32x4*>(cst + bi * D + c);
          const f32x4 eL = *reinterpret_cast<const f32x4*>(cst + (4 + bi) * D + c);
          const f32x4 eR = *reinterpret_cast<const f32x4*>(cst + (14 + (bi < 3 ? bi : 0)) * D + c);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = 4 * a + j;
            kt[e] = static_cast<_Float16>(kE[kk][e] * em[j]);
            qt[e] = static_cast<_Float16>(qE[kk][e] * em[j]);
            KhT[(c + j) * Lds::TT_LD + kpos] = static_cast<_Float16>(kF[kk][e] * eL[j]);
            rr8[e] = static_cast<_Float16>(kF[kk][e] * eR[j]);
          }
        }
        *reinterpret_cast<f16x8*>(Kt + r * Lds::OP_LD + 32 * kk + 8 * lg) = kt;
        *reinterpret_cast<f16x8*>(Qt + r * Lds::OP_LD + 32 * kk + 8 * lg) = qt;
        if (bi < 3) *reinterpret_cast<f16x8*>(Rb + r * Lds::OP_LD + 32 * kk + 8 * lg) = rr8;
      }
    }
    __syncthreads();

    // ================= P2: off-diagonal tiles (i, j<i), i = this wave's block
#pragma unroll
    for (int bj = 0; bj < 3; ++bj) {
      if (bj >= bi) continue;
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
      const int slotc = cij_slot(bi, bj);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        f16x8 lk, lq;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const f32x4 cc = *reinterpret_cast<const f32x4*>(cst + slotc * D + 32 * kk + 16 * a + 4 * lg);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            lk[4 * a + j] = static_cast<_Float16>(kE[kk][4 * a + j] * cc[j]);
            lq[4 * a + j] = static_cast<_Float16>(qE[kk][4 * a + j] * cc[j]);
          }
        }
        const f16x8 rb = *reinterpret_cast<const f16x8*>(Rb + (16 * bj + lr) * Lds::OP_LD + 32 * kk + 8 * lg);
        accA = mma_f16(lk, rb, accA);
        accP = mma_f16(lq, rb, accP);
      }
      const int sp = ppos64(16 * bj + lr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * bi + 4 * lg + i;
        AT[row * Lds::AT_LD + 16 * bj + lr] = static_cast<_Float16>(-accA[i] * s_beta[row]);
        _Float16 x0, x1;
        split_f16(accP[i], x0, x1);
        Ph[row * Lds::TT_LD + sp] = x0;
        Pl[row * Lds::TT_LD + sp] = x1;
      }
    }
    __syncthreads();

    // ================= P3: state products for value column jcol (no barriers)
    {
      // S as B fragments (hi/lo), contraction over key channels
      f16x8 sbh[4], sbl[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) bfrag_split(Sacc[2 * kk], Sacc[2 * kk + 1], sbh[kk], sbl[kk]);
      // X = V - Kt S ;  O = Qt S
      f32x4 Xacc[4], Oacc[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 ax = {0.f, 0.f, 0.f, 0.f}, ao = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const f16x8 ak = *reinterpret_cast<const f16x8*>(Kt + (16 * rt + lr) * Lds::OP_LD + 32 * kk + 8 * lg);
          const f16x8 aq = *reinterpret_cast<const f16x8*>(Qt + (16 * rt + lr) * Lds::OP_LD + 32 * kk + 8 * lg);
          ax = mma_f16(ak, sbh[kk], ax);
          ax = mma_f16(ak, sbl[kk], ax);
          ao = mma_f16(aq, sbh[kk], ao);
          ao = mma_f16(aq, sbl[kk], ao);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ax[i] = ((16 * rt + 4 * lg + i < Lc) ? vval(4 * rt + i) : 0.0f) - ax[i];
        Xacc[rt] = ax;
        Oacc[rt] = ao;
      }
      // the chunk's v is consumed: fetch the next chunk's
      if (t0 + C < eos) prefetch_v(t0 + C);
      // -- P3b: Delta_i = T_ii (b_i X_i - sum_{j<i} A_ij Delta_j), 16-row blocks
      f32x4 Dacc[4];
#pragma unroll
      for (int bi4 = 0; bi4 < 4; ++bi4) {
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = s_beta[16 * bi4 + 4 * lg + i] * Xacc[bi4][i];
#pragma unroll
        for (int bj4 = 0; bj4 < 3; ++bj4) {
          if (bj4 >= bi4) continue;
          const f16x4 na = *reinterpret_cast<const f16x4*>(AT + (16 * bi4 + lr) * Lds::AT_LD + 16 * bj4 + 4 * lg);
          f16x4 dh, dl;
          bfrag16_split(Dacc[bj4], dh, dl);
          acc = mma_f16_k16(na, dh, acc);
          acc = mma_f16_k16(na, dl, acc);
        }
        const f16x4 ti = *reinterpret_cast<const f16x4*>(AT + (16 * bi4 + lr) * Lds::AT_LD + 16 * bi4 + 4 * lg);
        f16x4 xh, xl;
        bfrag16_split(acc, xh, xl);
        f32x4 d = mma_f16_k16(ti, xh, f32x4{0.f, 0.f, 0.f, 0.f});
        Dacc[bi4] = mma_f16_k16(ti, xl, d);
      }
      f16x8 dbh[2], dbl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bfrag_split(Dacc[2 * ks], Dacc[2 * ks + 1], dbh[ks], dbl[ks]);
      // -- P3c: O += P Delta ; store o
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 ao = Oacc[rt];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks > (rt >> 1)) continue;
          const f16x8 ph = *reinterpret_cast<const f16x8*>(Ph + (16 * rt + lr) * Lds::TT_LD + 32 * ks + 8 * lg);
          const f16x8 pl = *reinterpret_cast<const f16x8*>(Pl + (16 * rt + lr) * Lds::TT_LD + 32 * ks + 8 * lg);
          ao = mma_f16(ph, dbh[ks], ao);
          ao = mma_f16(pl, dbh[ks], ao);
          ao = mma_f16(ph, dbl[ks], ao);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 16 * rt + 4 * lg + i;
          if (rr < Lc) {
            const int64_t oi = (int64_t)(t0 + rr) * HD + hD + jcol;
            const float val = scale * ao[i];
            if (O_BF16) static_cast<uint16_t*>(o)[oi] = f32_to_bf16_bits(val);
            else static_cast<float*>(o)[oi] = val;
          }
        }
      }
      // -- P3d: S <- e^gamma_C S + Khat^T Delta
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const f32x4 dec = *reinterpret_cast<const f32x4*>(cst + 17 * D + 16 * t + 4 * lg);
        f32x4 s = Sacc[t] * dec;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const f16x8 a = *reinterpret_cast<const f16x8*>(KhT + (16 * t + lr) * Lds::TT_LD + 32 * ks + 8 * lg);
          s = mma_f16(a, dbh[ks], s);
          s = mma_f16(a, dbl[ks], s);
        }
        Sacc[t] = s;
      }
    }
    __syncthreads();
  }

  if (Sf) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Sf[sbase + (int64_t)(16 * t + 4 * lg + i) * D + jcol] = Sacc[t][i];
  }
}

}  // namespace

hipError_t launch_chunk_prefill(const void* q, const void* k, const void* v, bool qkv_bf16,
                                const float* g, const float* beta, const int32_t* cu, int N,
                                const float* S0, float* S_final, void* o, bool o_bf16,
                                int64_t T_tot, int H, float scale, hipStream_t s) {
  const int64_t P = (int64_t)N * H;
  const int64_t blocks = 8 * NT * ((P + 7) / 8);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks));
  const int T = static_cast<int>(T_tot);
#define KDA_LAUNCH(QB, OB)                                                                   \
  chunk_kernel<QB, OB><<<grid, NTHR, 0, s>>>(q, k, v, g, beta, cu, N, S0, S_final, o, T, H, \
                                             scale)
  if (qkv_bf16 && o_bf16) KDA_LAUNCH(true, true);
  else if (qkv_bf16) KDA_LAUNCH(true, false);
  else if (o_bf16) KDA_LAUNCH(false, true);
  else KDA_LAUNCH(false, false);
#undef KDA_LAUNCH
  return hipGetLastError();
}

}  // namespace kda
