// Prep kernel of kda_chunk_prefill: everything about one (chunk, head) that
// does not depend on the state, for all chunks at once.
//
// One workgroup (4 waves) per (chunk, head).  It writes that chunk's
// workspace image (layout in chunk_common.hpp): K e^gamma, Q e^gamma,
// (K e^(gamma_C - gamma))^T, the decay-weighted P, the diagonal-block
// inverses T_ii with the off-diagonal blocks -A_ij of the triangular system
// (I + A) Delta = diag(beta) X, e^gamma_C and beta.
//
// Phases:
//  P0  gamma = cumsum(g) per channel (lanes 2c, 2c+1 own channel c, rows
//      0..31 and 32..63), the per-(block, channel) decay constants, and the
//      transposed K e^(gamma_C - gamma) straight from that layout.
//  P1  wave i owns chunk rows 16i..16i+15 (block i): decay factors, the
//      row-major operands (written to the image), the diagonal tiles A_ii and
//      P_ii, and T_ii = (I + A_ii)^-1 by repeated squaring.
//  P2  off-diagonal tiles (i, j < i) of A and P, two per wave at most.
//
// Decay factors.  gamma is kept in log2 units and every exponential is a
// hardware exp2.  Inside a chunk gamma can fall far below -126, so factors
// are built relative to references: for block i with mid row m_i = 16i+7,
//   E_r = 2^(gamma_r - gamma_m),  F_r = 2^(gamma_m - gamma_r)
// span at most 8 tokens of decay (2 exp2 per element), and every other factor
// is E or F times a per-(block, channel) constant that is <= 1, e.g.
//   2^gamma_r = E_r 2^gamma_m.
// An off-diagonal tile (i, j) multiplies k_r 2^(gamma_r - gamma_b) by
// k_s 2^(gamma_b - gamma_s), b = last row of block j: both <= 1 (fp16).  The
// diagonal tiles multiply E and F, bounded by 8 tokens of decay: plain fp16
// when every |gamma_r - gamma_m| of the block is <= 7, otherwise hi+lo bf16
// pairs, which keep fp32 range.  Requirement: no channel decays by more than
// 126 (log2 units) over 8 consecutive tokens.
#include "chunk_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace chunk {
namespace {

struct PrepLds {
  static constexpr int SC_LD = 17;  // fp32 [4][16][17] per-wave transpose scratch
  static constexpr int off_gam = 0;                       // fp32 [64][128], gidx swizzle
  static constexpr int off_R = off_gam + C * D * 4;       // fp16 [48][128], ke_off layout
  static constexpr int off_L3 = off_R + 48 * D * 2;       // fp16 [32][128], ke_off layout
  static constexpr int off_PM = off_L3 + 32 * D * 2;      // image of Ws::PM
  static constexpr int off_AT = off_PM + Ws::PM_BYTES;    // image of Ws::AT (follows PM)
  static constexpr int off_scr = off_AT + Ws::AT_BYTES;
  static constexpr int off_cst = off_scr + 4 * 16 * SC_LD * 4;
  static constexpr int off_beta = off_cst + 14 * D * 4;
  static constexpr int total = off_beta + C * 4;
};
static_assert(PrepLds::total <= 80 * 1024, "two prep workgroups per CU");

// float index of element (row, c) of the swizzled gamma buffer
__device__ __forceinline__ int gidx(int row, int c) {
  return row * 128 + ((((c >> 2) ^ (row & 15))) << 2) + (c & 3);
}

// Per-channel constant slots (after exp2, all <= 1):
//  0..3   em_i = 2^gamma_{m_i}
//  4..9   c(i,j) = 2^(gamma_{m_i} - gamma_{b_{j+1}}), b_{j+1} = last row of block j:
//         (1,0),(2,1),(3,2) at 4,5,6; (2,0) 7; (3,1) 8; (3,0) 9
//  10..12 eR_j = 2^(gamma_{b_{j+1}} - gamma_{m_j}), j = 0..2
//  13     eC = 2^gamma_C
__device__ __forceinline__ int cij_slot(int i, int j) {
  return (j == i - 1) ? 3 + i : (i == 2 ? 7 : (j == 1 ? 8 : 9));
}

template <bool BF16>
struct QKRaw;  // raw q or k values of one lane: 4 k-steps x 2 halves x 4
template <>
struct QKRaw<true> {
  u16x4 v[4][2];
};
template <>
struct QKRaw<false> {
  f32x4 v[4][2];
};

template <bool BF16>
__device__ __forceinline__ void load_qk(QKRaw<BF16>& R, __amdgpu_buffer_rsrc_t rs, int off0) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int c = 32 * kk + 16 * a;  // plus 4lg, folded into off0
      if constexpr (BF16) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, off0 + 2 * c, 0, 0);
        R.v[kk][a] = __builtin_bit_cast(u16x4, x);
      } else {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off0 + 4 * c, 0, 0);
        R.v[kk][a] = __builtin_bit_cast(f32x4, x);
      }
    }
}

template <bool BF16>
__device__ __forceinline__ float qk_at(const QKRaw<BF16>& R, int kk, int a, int e) {
  if constexpr (BF16) return bf16_bits_to_f32(R.v[kk][a][e]);
  else return R.v[kk][a][e];
}

template <bool QKV_BF16>
__global__ void __launch_bounds__(NTHR, 2) prep_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, const int32_t* __restrict__ cu, int T_tot, int H, int Hp,
    int c_lo, int S_len, char* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) char lds[PrepLds::total];
  float* gam = reinterpret_cast<float*>(lds + PrepLds::off_gam);
  char* Rb = lds + PrepLds::off_R;
  char* L3 = lds + PrepLds::off_L3;
  char* ATi = lds + PrepLds::off_AT;
  char* PMi = lds + PrepLds::off_PM;
  float* cst = reinterpret_cast<float*>(lds + PrepLds::off_cst);
  float* s_beta = reinterpret_cast<float*>(lds + PrepLds::off_beta);

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

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave (uniform)
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  float* scr = reinterpret_cast<float*>(lds + PrepLds::off_scr) + w * 16 * PrepLds::SC_LD;
  const int HD = H * D;
  constexpr int QS = QKV_BF16 ? 2 : 4;

  // chunk buffers: rows [t0, t0 + Lc) of head h; loads past Lc return 0
  auto buf_tok = [&](const void* base, int esz) {
    const char* b = static_cast<const char*>(base) + ((int64_t)t0 * HD + (int64_t)h * D) * esz;
    return make_buf(b, (uint32_t)(Lc * HD * esz - h * D * esz));
  };

  // ---- loads: g straight to LDS (16-byte rows chunks, swizzled), k and q in
  // row layout (P1), k in column layout (P0), beta.
  const int gc = tid >> 1, ghf = tid & 1;  // P0: channel, half
  const int rA = 16 * w + lr;              // P1: chunk row of this lane
  {
    const auto rg = buf_tok(g, 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // rows 16w + 2j + (lane >> 5): lane writes chunk lane & 31
      const int row0 = 16 * w + 2 * j;
      const int hi = lane >> 5;
      const int lchunk = (lane & 31) ^ ((2 * j + hi) & 15);
      buf_to_lds16(rg, (lds_ptr_t)(gam + row0 * D), hi * HD * 4 + lchunk * 16, row0 * HD * 4);
    }
  }
  QKRaw<QKV_BF16> kpf, qpf;
  const auto rk = buf_tok(k, QS);
  load_qk<QKV_BF16>(kpf, rk, rA * HD * QS + 4 * lg * QS);
  load_qk<QKV_BF16>(qpf, buf_tok(q, QS), rA * HD * QS + 4 * lg * QS);
  uint32_t kcol[32];  // k[32 ghf + i][gc]
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if constexpr (QKV_BF16)
      kcol[i] = __builtin_amdgcn_raw_buffer_load_b16(rk, (32 * ghf * HD + gc) * QS, i * HD * QS, 0);
    else
      kcol[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, (32 * ghf * HD + gc) * QS, i * HD * QS, 0);
  }
  float bval = 0.0f;
  if (tid < C) {
    const char* bb = reinterpret_cast<const char*>(beta) + ((int64_t)t0 * H + h) * 4;
    bval = buf_f32(make_buf(bb, (uint32_t)(Lc * H * 4 - h * 4)), tid * H * 4);
  }
  wait_vmem();
  __syncthreads();

  // ================= P0: gamma (cumsum of g, log2 units), decay constants,
  // (K e^(gamma_C - gamma))^T.
  {
    float gv[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) gv[i] = gam[gidx(32 * ghf + i, gc)] * LOG2E;
#pragma unroll
    for (int i = 1; i < 32; ++i) gv[i] += gv[i - 1];
    const float tot0 = __shfl_xor(gv[31], 1);
    if (ghf) {
#pragma unroll
      for (int i = 0; i < 32; ++i) gv[i] += tot0;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) gam[gidx(32 * ghf + i, gc)] = gv[i];
    // key rows: block mids 7,23,39,55 and block ends 15,31,47,63
    const float o7 = __shfl_xor(gv[7], 1), o15 = __shfl_xor(gv[15], 1);
    const float o23 = __shfl_xor(gv[23], 1), o31 = __shfl_xor(gv[31], 1);
    const float gm0 = ghf ? o7 : gv[7], gm1 = ghf ? o23 : gv[23];
    const float gm2 = ghf ? gv[7] : o7, gm3 = ghf ? gv[23] : o23;
    const float gb1 = ghf ? o15 : gv[15], gb2 = ghf ? o31 : gv[31];
    const float gb3 = ghf ? gv[15] : o15, gl = ghf ? gv[31] : o31;
    const int c = gc;
    if (ghf == 0) {
      cst[0 * D + c] = ex2(gm0);
      cst[1 * D + c] = ex2(gm1);
      cst[2 * D + c] = ex2(gm2);
      cst[3 * D + c] = ex2(gm3);
      cst[4 * D + c] = ex2(gm1 - gb1);
      cst[5 * D + c] = ex2(gm2 - gb2);
      cst[6 * D + c] = ex2(gm3 - gb3);
    } else {
      cst[7 * D + c] = ex2(gm2 - gb1);
      cst[8 * D + c] = ex2(gm3 - gb2);
      cst[9 * D + c] = ex2(gm3 - gb1);
      cst[10 * D + c] = ex2(gb1 - gm0);
      cst[11 * D + c] = ex2(gb2 - gm1);
      cst[12 * D + c] = ex2(gb3 - gm2);
      cst[13 * D + c] = ex2(gl);
    }
    if (tid < C) s_beta[tid] = bval;
    // Khat^T row c, tokens 32 ghf + i at positions 32 ghf + pperm(i): chunk b
    // of this half holds tokens 16(e>>2) + 4b + (e&3), e = 0..7.
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f16x8 kd;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 16 * (e >> 2) + 4 * b + (e & 3);
        const float kv = QKV_BF16 ? __uint_as_float(kcol[i] << 16) : __uint_as_float(kcol[i]);
        kd[e] = static_cast<_Float16>(kv * ex2(gl - gv[i]));
      }
      const int chunk = (4 * ghf + b) ^ ((c >> 1) & 7);
      *reinterpret_cast<f16x8*>(img + Ws::KDT + c * 128 + chunk * 16) = kd;  // kdt_off layout
    }
  }
  __syncthreads();

  // ================= P1: decay factors, operands, diagonal tiles and T_ii.
  // Lane (lr, lg) of wave i handles chunk row r = 16i + lr and, in k-step kk,
  // the 8 channels 32kk + 16a + 4lg + j (a < 2, j < 4), fragment element 4a + j.
  const int bi = w;
  const int r = rA;
  float kE[4][8], qE[4][8];
  {
    const int mrow = 16 * bi + 7;
    float kF[4][8];
    float dgmax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f16x8 kt, qt, rr8, l3k, l3q;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int c = 32 * kk + 16 * a + 4 * lg;
        const f32x4 gr = *reinterpret_cast<const f32x4*>(gam + gidx(r, c));
        const f32x4 gm = *reinterpret_cast<const f32x4*>(gam + gidx(mrow, c));
        const f32x4 em = *reinterpret_cast<const f32x4*>(cst + bi * D + c);
        const f32x4 eR = *reinterpret_cast<const f32x4*>(cst + (10 + (bi < 3 ? bi : 0)) * D + c);
        const f32x4 c30 = *reinterpret_cast<const f32x4*>(cst + 9 * D + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * a + j;
          const float kv = qk_at<QKV_BF16>(kpf, kk, a, j);
          const float qv = qk_at<QKV_BF16>(qpf, kk, a, j);
          const float dg = gr[j] - gm[j];
          dgmax = fmaxf(dgmax, fabsf(dg));
          const float E = ex2(dg), F = ex2(-dg);
          const float ke = kv * E, qe = qv * E, kf = kv * F;
          kE[kk][e] = ke;
          qE[kk][e] = qe;
          kF[kk][e] = kf;
          kt[e] = static_cast<_Float16>(ke * em[j]);
          qt[e] = static_cast<_Float16>(qe * em[j]);
          if (bi < 3) rr8[e] = static_cast<_Float16>(kf * eR[j]);
          if (bi == 3) {
            l3k[e] = static_cast<_Float16>(ke * c30[j]);
            l3q[e] = static_cast<_Float16>(qe * c30[j]);
          }
        }
      }
      const int po = ke_off(r, 32 * kk + 8 * lg);
      *reinterpret_cast<f16x8*>(img + Ws::KE + po) = kt;
      *reinterpret_cast<f16x8*>(img + Ws::QE + po) = qt;
      if (bi < 3) *reinterpret_cast<f16x8*>(Rb + po) = rr8;
      if (bi == 3) {  // left factors of tile (3,0), which wave 0 multiplies
        *reinterpret_cast<f16x8*>(L3 + ke_off(lr, 32 * kk + 8 * lg)) = l3k;
        *reinterpret_cast<f16x8*>(L3 + ke_off(16 + lr, 32 * kk + 8 * lg)) = l3q;
      }
    }
    // Diagonal tiles A_ii = (k E)(k F)^T and P_ii = (q E)(k F)^T.
    f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
    if (!__any(dgmax > 7.0f)) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        f16x8 ek, eq, fk;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ek[e] = static_cast<_Float16>(kE[kk][e]);
          eq[e] = static_cast<_Float16>(qE[kk][e]);
          fk[e] = static_cast<_Float16>(kF[kk][e]);
        }
        accA = mma_f16(ek, fk, accA);
        accP = mma_f16(eq, fk, accP);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8 ekh, ekl, eqh, eql, fkh, fkl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 x0, x1;
          split_bf16(kE[kk][e], x0, x1); ekh[e] = x0; ekl[e] = x1;
          split_bf16(qE[kk][e], x0, x1); eqh[e] = x0; eql[e] = x1;
          split_bf16(kF[kk][e], x0, x1); fkh[e] = x0; fkl[e] = x1;
        }
        accA = mma_bf16(ekh, fkh, accA);
        accA = mma_bf16(ekh, fkl, accA);
        accA = mma_bf16(ekl, fkh, accA);
        accP = mma_bf16(eqh, fkh, accP);
        accP = mma_bf16(eqh, fkl, accP);
        accP = mma_bf16(eql, fkh, accP);
      }
    }
    // -- diagonal tile (bi, bi): lane holds rows 16bi + 4lg + i, column s = 16bi + lr
    const int sp = ppos64(16 * bi + lr);
    f32x4 nB;  // N = A_ii (strictly lower, beta-scaled rows) in accumulator layout
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * lg + i, row = 16 * bi + rr;
      nB[i] = (lr < rr) ? accA[i] * s_beta[row] : 0.0f;
      *reinterpret_cast<_Float16*>(PMi + pm_off(row, sp)) =
          static_cast<_Float16>((lr <= rr) ? accP[i] : 0.0f);
      if ((bi & 1) == 0)  // upper tile (bi, bi+1) of P lies inside a 32-wide k-step
        *reinterpret_cast<_Float16*>(PMi + pm_off(row, ppos64(16 * bi + 16 + lr))) =
            static_cast<_Float16>(0.0f);
    }
    // -- T_ii = (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8), exact since
    // N^16 = 0.  Products are 16x16x16 MFMAs: the left factor is read in operand
    // layout through a wave-private LDS transpose, the right factor is an
    // accumulator (hi+lo fp16).
    auto to_a = [&](const f32x4& xb) -> f32x4 {  // accumulator layout -> A-operand layout
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < 4; ++i) scr[(4 * lg + i) * PrepLds::SC_LD + lr] = xb[i];
      wave_lds_sync();
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = scr[lr * PrepLds::SC_LD + 4 * lg + e];
      return x;
    };
    auto mul = [&](const f32x4& xa, const f32x4& yb) -> f32x4 {
      f16x4 a, bh, bl;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = static_cast<_Float16>(xa[e]);
      bfrag16_split(yb, bh, bl);
      f32x4 d = mma_f16_k16(a, bh, f32x4{0.f, 0.f, 0.f, 0.f});
      return mma_f16_k16(a, bl, d);
    };
    f32x4 eye;
#pragma unroll
    for (int i = 0; i < 4; ++i) eye[i] = (4 * lg + i == lr) ? 1.0f : 0.0f;  // same in both layouts
    const f32x4 nA = to_a(nB);
    const f32x4 n2B = mul(nA, nB);
    const f32x4 n4B = mul(to_a(n2B), n2B);
    const f32x4 n8B = mul(to_a(n4B), n4B);
    const f32x4 m2B = mul(eye - nA, eye + n2B);
    const f32x4 m3B = mul(to_a(m2B), eye + n4B);
    const f32x4 tB = mul(to_a(m3B), eye + n8B);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<_Float16*>(ATi + at_off(16 * bi + 4 * lg + i, 16 * bi + lr)) =
          static_cast<_Float16>(tB[i]);
  }
  __syncthreads();

  // ================= P2: off-diagonal tiles (i, j<i): two per wave at most.
  // Wave w multiplies its own left factors (rows of block w) except wave 0,
  // which takes tile (3,0) with the left factors wave 3 left in LDS.
  {
    auto offdiag = [&](int ti, int tj) {
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
      const int slotc = cij_slot(ti, tj);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        f16x8 lk, lq;
        if (ti == bi) {
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            const f32x4 cc = *reinterpret_cast<const f32x4*>(cst + slotc * D + 32 * kk + 16 * a + 4 * lg);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              lk[4 * a + j] = static_cast<_Float16>(kE[kk][4 * a + j] * cc[j]);
              lq[4 * a + j] = static_cast<_Float16>(qE[kk][4 * a + j] * cc[j]);
            }
          }
        } else {
          lk = *reinterpret_cast<const f16x8*>(L3 + ke_off(lr, 32 * kk + 8 * lg));
          lq = *reinterpret_cast<const f16x8*>(L3 + ke_off(16 + lr, 32 * kk + 8 * lg));
        }
        const f16x8 rb = *reinterpret_cast<const f16x8*>(Rb + ke_off(16 * tj + lr, 32 * kk + 8 * lg));
        accA = mma_f16(lk, rb, accA);
        accP = mma_f16(lq, rb, accP);
      }
      const int sp = ppos64(16 * tj + lr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * ti + 4 * lg + i;
        *reinterpret_cast<_Float16*>(ATi + at_off(row, 16 * tj + lr)) =
            static_cast<_Float16>(-accA[i] * s_beta[row]);
        *reinterpret_cast<_Float16*>(PMi + pm_off(row, sp)) = static_cast<_Float16>(accP[i]);
      }
    };
    if (bi == 0) {
      offdiag(3, 0);
    } else if (bi == 1) {
      offdiag(1, 0);
    } else if (bi == 2) {
      offdiag(2, 0);
      offdiag(2, 1);
    } else {
      offdiag(3, 1);
      offdiag(3, 2);
    }
  }
  __syncthreads();

  // ---- copy the LDS-built parts of the image: PM and AT (contiguous in both),
  // EC, BETA
  {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    constexpr int units = (Ws::PM_BYTES + Ws::AT_BYTES) / 16;
    static_assert(Ws::AT == Ws::PM + Ws::PM_BYTES, "PM and AT adjacent");
    for (int u = tid; u < units; u += NTHR)
      *reinterpret_cast<u32x4*>(img + Ws::PM + 16 * u) =
          *reinterpret_cast<const u32x4*>(lds + PrepLds::off_PM + 16 * u);
    if (tid < 32)
      *reinterpret_cast<u32x4*>(img + Ws::EC + 16 * tid) =
          *reinterpret_cast<const u32x4*>(cst + 13 * D + 4 * tid);
    else if (tid < 48)
      *reinterpret_cast<u32x4*>(img + Ws::BETA + 16 * (tid - 32)) =
          *reinterpret_cast<const u32x4*>(s_beta + 4 * (tid - 32));
  }
}

}  // namespace

hipError_t launch_prep(const void* q, const void* k, bool qkv_bf16, const float* g,
                       const float* beta, const int32_t* cu, int N, int T_tot, int H, int c_lo,
                       int S_len, char* ws, hipStream_t s) {
  const int Hp = (H + 7) & ~7;
  const int64_t blocks = (int64_t)N * S_len * Hp;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (qkv_bf16)
    prep_kernel<true><<<dim3((unsigned)blocks), NTHR, 0, s>>>(q, k, g, beta, cu, T_tot, H, Hp,
                                                              c_lo, S_len, ws);
  else
    prep_kernel<false><<<dim3((unsigned)blocks), NTHR, 0, s>>>(q, k, g, beta, cu, T_tot, H, Hp,
                                                               c_lo, S_len, ws);
  return hipGetLastError();
}

}  // namespace chunk
}  // namespace kda
