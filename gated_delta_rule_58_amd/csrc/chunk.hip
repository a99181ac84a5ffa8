// kda_chunk_prefill: chunked KDA prefill over packed variable-length batches.
//
// Math (one sequence, one head; chunk of C=64 tokens, entry state S, d=128).
// The recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
// o_t = S_t^T q_t (the code audit's chunked training/prefill regime) unrolls
// over a chunk into, with gamma_r = sum_{s<=r} g_s per key channel:
//   A[r,s] = b_r sum_c k_rc k_sc e^(gamma_rc - gamma_sc)   (s < r)
//   P[r,s] =     sum_c q_rc k_sc e^(gamma_rc - gamma_sc)   (s <= r)
//   T      = (I + A)^-1                                     (unit lower triangular)
//   X      = V - (K * e^gamma) S
//   Delta  = T diag(b) X
//   O      = scale * ((Q * e^gamma) S + P Delta)
//   S     <- Diag(e^gamma_C) S + (K * e^(gamma_C - gamma))^T Delta
// Every term is independent across value columns, so one workgroup owns one
// (sequence, head, 64-column value tile) and walks the chunks of its sequence
// in order, carrying its 128x64 slice of S in MFMA accumulators.
//
// Decay factors.  Inside a chunk gamma can fall below -88, so e^gamma and
// e^-gamma cannot be formed directly in fp32.  Rows are grouped in 16-row
// blocks; for block i with mid row m_i = 16i+7,
//   E_r = e^(gamma_r - gamma_m),  F_r = e^(gamma_m - gamma_r)
// span at most 8 tokens of decay (2 exps per element), and every factor above
// is E or F times a per-(block, channel) constant that is <= 1:
//   e^gamma_r              = E_r e^gamma_m
//   e^(gamma_C - gamma_r)  = F_r e^(gamma_C - gamma_m)
//   e^(gamma_r - gamma_b)  = E_r e^(gamma_m - gamma_b)     b = last row of block i-1
//   e^(gamma_b - gamma_s)  = F_s e^(gamma_b - gamma_m')    s in an earlier block
// so the products of the off-diagonal 16x16 blocks of A and P use operands
// <= 1 (fp16), and the diagonal blocks use E and F (bounded by 8 tokens of
// decay) as hi+lo bf16 pairs, which keep fp32 range.  The requirement is that
// no channel decays by more than 88 (in log space) over 8 consecutive tokens.
//
// Precision.  MFMA operands are fp16 (bf16 inputs convert exactly); the
// state S, X, Delta and P are split into hi+lo fp16 pairs, so the rounding of
// those operands does not reach the result; accumulation is fp32.
//
// Wave roles (4 waves): wave i owns rows 16i..16i+15 of the chunk for A/P,
// X, Delta and O, and key rows 32i..32i+31 of the state update.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int C = 64;     // chunk length
constexpr int D = 128;    // dk = dv
constexpr int NTHR = 256; // 4 waves

__device__ __forceinline__ f32x4 mma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f16_k16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// LDS layout (bytes).  Region X is live from the gamma pass to the A/P
// products, region Y from the triangular inverse to the state update; they
// alias.
template <int DV>
struct Lds {
  static constexpr int GAM_LD = 132;   // fp32 [64][132]
  static constexpr int L_LD = 136;     // fp16 [2][48][136]
  static constexpr int M_LD = 68;      // fp32 [64][68] (A, P, T)
  static constexpr int ST_LD = 136;    // fp16 [2][DV][136]  S^T hi/lo
  static constexpr int TT_LD = 72;     // fp16 [2][DV][72]   (bX)^T, Delta^T hi/lo ; [128][72] Khat^T

  static constexpr int off_gam = 0;
  static constexpr int off_L = off_gam + C * GAM_LD * 4;
  static constexpr int end_X = off_L + 2 * 48 * L_LD * 2;
  static constexpr int off_T = 0;
  static constexpr int off_bx = off_T + C * M_LD * 4;
  static constexpr int off_dl = off_bx + 2 * DV * TT_LD * 2;
  static constexpr int end_Y = off_dl + 2 * DV * TT_LD * 2;
  static constexpr int off_persist = (end_X > end_Y ? end_X : end_Y);
  static constexpr int off_ST = off_persist;
  static constexpr int off_KhT = off_ST + 2 * DV * ST_LD * 2;
  static constexpr int off_A = off_KhT + D * TT_LD * 2;
  static constexpr int off_P = off_A + C * M_LD * 4;
  static constexpr int off_cst = off_P + C * M_LD * 4;
  static constexpr int off_beta = off_cst + 18 * D * 4;
  static constexpr int off_tot = off_beta + C * 4;
  static constexpr int off_seq = off_tot + D * 4;
  static constexpr int total = off_seq + 16;
};

// Constant slots (per channel): em[4] e^gamma_m, eL[4] e^(gamma_C-gamma_m),
// eB[1..3] e^(gamma_m - gamma_b), eR[6] e^(gamma_b(i) - gamma_m(j)) for
// (i,j) = (1,0),(2,0),(2,1),(3,0),(3,1),(3,2), eT e^gamma_C.
__device__ __forceinline__ int eR_slot(int i, int j) { return 11 + (i * (i - 1)) / 2 + j; }

__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

template <int DV, bool QKV_BF16, bool O_BF16>
__global__ void __launch_bounds__(NTHR, 1) chunk_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int N, const float* __restrict__ S0,
    float* __restrict__ Sf, void* __restrict__ o, int T_tot, int H, float scale) {
  using L = Lds<DV>;
  constexpr int NT = D / DV;   // value tiles per head
  constexpr int NCT = DV / 16; // 16-column tiles per value tile
  __shared__ __attribute__((aligned(16))) char lds[L::total];

  float* gam = reinterpret_cast<float*>(lds + L::off_gam);
  _Float16* Lbuf = reinterpret_cast<_Float16*>(lds + L::off_L);
  float* Tb = reinterpret_cast<float*>(lds + L::off_T);
  _Float16* bxT = reinterpret_cast<_Float16*>(lds + L::off_bx);
  _Float16* dlT = reinterpret_cast<_Float16*>(lds + L::off_dl);
  _Float16* sT = reinterpret_cast<_Float16*>(lds + L::off_ST);
  _Float16* KhT = reinterpret_cast<_Float16*>(lds + L::off_KhT);
  float* Ab = reinterpret_cast<float*>(lds + L::off_A);
  float* Pb = reinterpret_cast<float*>(lds + L::off_P);
  float* cst = reinterpret_cast<float*>(lds + L::off_cst);
  float* s_beta = reinterpret_cast<float*>(lds + L::off_beta);
  float* s_tot = reinterpret_cast<float*>(lds + L::off_tot);
  int* s_seq = reinterpret_cast<int*>(lds + L::off_seq);

  const int tid = threadIdx.x;
  const int w = tid >> 6;          // wave
  const int lane = tid & 63;
  const int lr = lane & 15;        // MFMA row/col within a 16x16 tile
  const int lg = lane >> 4;        // MFMA k-group

  // ---- workgroup -> (sequence, head, value tile).  All tiles of one
  // (sequence, head) land on the same XCD (blockIdx % 8) so they share its L2.
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
  const int col0 = tile * DV;

  // ---- state slice in accumulators: wave w holds key rows 32w + 16rt +
  // 4lg + i (i = 0..3) and value column col0 + 16ct + lr.
  f32x4 sacc[2][NCT];
  const int64_t sbase = ((int64_t)n * H + h) * D * D;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 32 * w + 16 * rt + 4 * lg + i;
        sacc[rt][ct][i] = S0 ? S0[sbase + (int64_t)row * D + col0 + 16 * ct + lr] : 0.0f;
      }

  auto write_sT = [&]() {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f16x4 hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          _Float16 a, b;
          split_f16(sacc[rt][ct][i], a, b);
          hi[i] = a;
          lo[i] = b;
        }
        const int j = 16 * ct + lr, c = 32 * w + 16 * rt + 4 * lg;
        *reinterpret_cast<f16x4*>(sT + j * L::ST_LD + c) = hi;
        *reinterpret_cast<f16x4*>(sT + (DV + j) * L::ST_LD + c) = lo;
      }
  };
  write_sT();

  for (int t0 = bos; t0 < eos; t0 += C) {
    const int Lc = (eos - t0) < C ? (eos - t0) : C;

    // ================= P0: gamma = inclusive cumsum of g over the chunk
    {
      const int c = tid & 127, hf = tid >> 7;
      float gv[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int r = 32 * hf + i;
        gv[i] = (r < Lc) ? g[(int64_t)(t0 + r) * HD + (int64_t)h * D + c] : 0.0f;
      }
#pragma unroll
      for (int i = 1; i < 32; ++i) gv[i] += gv[i - 1];
      if (hf == 0) s_tot[c] = gv[31];
      if (tid < C) s_beta[tid] = (tid < Lc) ? beta[(int64_t)(t0 + tid) * H + h] : 0.0f;
      __syncthreads();
      const float add = hf ? s_tot[c] : 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) gam[(32 * hf + i) * L::GAM_LD + c] = gv[i] + add;
      __syncthreads();
      if (tid < D) {
        const float gm0 = gam[7 * L::GAM_LD + c], gm1 = gam[23 * L::GAM_LD + c];
        const float gm2 = gam[39 * L::GAM_LD + c], gm3 = gam[55 * L::GAM_LD + c];
        const float gb1 = gam[15 * L::GAM_LD + c], gb2 = gam[31 * L::GAM_LD + c];
        const float gb3 = gam[47 * L::GAM_LD + c], gl = gam[63 * L::GAM_LD + c];
        cst[0 * D + c] = expf(gm0);
        cst[1 * D + c] = expf(gm1);
        cst[2 * D + c] = expf(gm2);
        cst[3 * D + c] = expf(gm3);
        cst[4 * D + c] = expf(gl - gm0);
        cst[5 * D + c] = expf(gl - gm1);
        cst[6 * D + c] = expf(gl - gm2);
        cst[7 * D + c] = expf(gl - gm3);
        cst[8 * D + c] = expf(gm1 - gb1);
        cst[9 * D + c] = expf(gm2 - gb2);
        cst[10 * D + c] = expf(gm3 - gb3);
        cst[eR_slot(1, 0) * D + c] = expf(gb1 - gm0);
        cst[eR_slot(2, 0) * D + c] = expf(gb2 - gm0);
        cst[eR_slot(2, 1) * D + c] = expf(gb2 - gm1);
        cst[eR_slot(3, 0) * D + c] = expf(gb3 - gm0);
        cst[eR_slot(3, 1) * D + c] = expf(gb3 - gm1);
        cst[eR_slot(3, 2) * D + c] = expf(gb3 - gm2);
        cst[17 * D + c] = expf(gl);
      }
      __syncthreads();
    }

    // ================= P1: decay factors, operands, diagonal blocks of A/P
    const int bi = w;                    // row block of this wave
    const int r = 16 * bi + lr;          // chunk row held by this lane
    const bool rvalid = r < Lc;
    const int64_t tok = (int64_t)(t0 + r) * HD + (int64_t)h * D;
    float kreg[4][8], freg[4][8];
    f16x8 Kt[4], Qt[4];
    {
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
      const int mrow = 16 * bi + 7;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int c0 = 32 * kk + 8 * lg;
        float kv[8], qv[8];
        if (rvalid) {
          const f32x4 k0 = load4(k, tok + c0, QKV_BF16), k1 = load4(k, tok + c0 + 4, QKV_BF16);
          const f32x4 q0 = load4(q, tok + c0, QKV_BF16), q1 = load4(q, tok + c0 + 4, QKV_BF16);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kv[e] = k0[e]; kv[4 + e] = k1[e];
            qv[e] = q0[e]; qv[4 + e] = q1[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) kv[e] = qv[e] = 0.0f;
        }
        const f32x4 gr0 = *reinterpret_cast<const f32x4*>(gam + r * L::GAM_LD + c0);
        const f32x4 gr1 = *reinterpret_cast<const f32x4*>(gam + r * L::GAM_LD + c0 + 4);
        const f32x4 gm0 = *reinterpret_cast<const f32x4*>(gam + mrow * L::GAM_LD + c0);
        const f32x4 gm1 = *reinterpret_cast<const f32x4*>(gam + mrow * L::GAM_LD + c0 + 4);
        f16x8 lk, lq;
        bf16x8 ekh, ekl, eqh, eql, fkh, fkl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float dg = (e < 4 ? gr0[e] : gr1[e - 4]) - (e < 4 ? gm0[e] : gm1[e - 4]);
          const float E = expf(dg), F = expf(-dg);
          const int c = c0 + e;
          const float em = cst[bi * D + c], eL = cst[(4 + bi) * D + c];
          const float kE = kv[e] * E, qE = qv[e] * E, kF = kv[e] * F;
          kreg[kk][e] = kv[e];
          freg[kk][e] = F;
          Kt[kk][e] = static_cast<_Float16>(kE * em);
          Qt[kk][e] = static_cast<_Float16>(qE * em);
          KhT[c * L::TT_LD + r] = static_cast<_Float16>(kF * eL);
          if (bi > 0) {
            const float eB = cst[(7 + bi) * D + c];
            lk[e] = static_cast<_Float16>(kE * eB);
            lq[e] = static_cast<_Float16>(qE * eB);
          }
          __bf16 a, b;
          split_bf16(kE, a, b); ekh[e] = a; ekl[e] = b;
          split_bf16(qE, a, b); eqh[e] = a; eql[e] = b;
          split_bf16(kF, a, b); fkh[e] = a; fkl[e] = b;
        }
        if (bi > 0) {
          *reinterpret_cast<f16x8*>(Lbuf + (r - 16) * L::L_LD + c0) = lk;
          *reinterpret_cast<f16x8*>(Lbuf + (48 + r - 16) * L::L_LD + c0) = lq;
        }
        accA = mma_bf16(ekh, fkh, accA);
        accA = mma_bf16(ekh, fkl, accA);
        accA = mma_bf16(ekl, fkh, accA);
        accP = mma_bf16(eqh, fkh, accP);
        accP = mma_bf16(eqh, fkl, accP);
        accP = mma_bf16(eql, fkh, accP);
      }
      // diagonal tile (bi, bi): rows 16bi + 4lg + i, column 16bi + lr
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 4 * lg + i;
        const float a = (lr < rr) ? accA[i] * s_beta[16 * bi + rr] : 0.0f;
        const float pp = (lr <= rr) ? accP[i] : 0.0f;
        Ab[(16 * bi + rr) * L::M_LD + 16 * bi + lr] = a;
        Pb[(16 * bi + rr) * L::M_LD + 16 * bi + lr] = pp;
        if ((bi & 1) == 0) {  // zero the upper tile (bi, bi+1) of P: products read it
          Pb[(16 * bi + rr) * L::M_LD + 16 * bi + 16 + lr] = 0.0f;
        }
      }
    }
    __syncthreads();

    // ================= P2: off-diagonal tiles (i, j), j = this wave's block
    {
      const int bj = w;
#pragma unroll
      for (int bi2 = 1; bi2 < 4; ++bi2) {
        if (bi2 <= bj) continue;
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int c0 = 32 * kk + 8 * lg;
          f16x8 R;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            R[e] = static_cast<_Float16>(kreg[kk][e] * freg[kk][e] * cst[eR_slot(bi2, bj) * D + c0 + e]);
          const f16x8 lk = *reinterpret_cast<const f16x8*>(Lbuf + (16 * bi2 - 16 + lr) * L::L_LD + c0);
          const f16x8 lq = *reinterpret_cast<const f16x8*>(Lbuf + (48 + 16 * bi2 - 16 + lr) * L::L_LD + c0);
          accA = mma_f16(lk, R, accA);
          accP = mma_f16(lq, R, accP);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 16 * bi2 + 4 * lg + i;
          Ab[rr * L::M_LD + 16 * bj + lr] = accA[i] * s_beta[rr];
          Pb[rr * L::M_LD + 16 * bj + lr] = accP[i];
        }
      }
    }
    __syncthreads();

    // ================= P3: T = (I + A)^-1
    // (a) diagonal 16x16 blocks by forward substitution, one column per lane
    if (lane < 16) {
      const int jj = lane, b0 = 16 * w;
      float tc[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float acc = (rr == jj) ? 1.0f : 0.0f;
#pragma unroll
        for (int s = 0; s < rr; ++s) acc -= Ab[(b0 + rr) * L::M_LD + b0 + s] * tc[s];
        tc[rr] = acc;
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        Tb[(b0 + rr) * L::M_LD + b0 + jj] = tc[rr];
        if ((w & 1) == 0) Tb[(b0 + rr) * L::M_LD + b0 + 16 + jj] = 0.0f;  // upper tile
      }
    }
    __syncthreads();
    // (b) off-diagonal blocks, by distance from the diagonal:
    //     T_ij = -T_ii * sum_{k=j}^{i-1} A_ik T_kj
#pragma unroll
    for (int dist = 1; dist < 4; ++dist) {
      const int bi3 = w, bj3 = w - dist;
      if (bj3 >= 0) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int kb = bj3; kb < bi3; ++kb) {
          f16x4 a, b;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = static_cast<_Float16>(Ab[(16 * bi3 + lr) * L::M_LD + 16 * kb + 4 * lg + e]);
            b[e] = static_cast<_Float16>(Tb[(16 * kb + 4 * lg + e) * L::M_LD + 16 * bj3 + lr]);
          }
          acc = mma_f16_k16(a, b, acc);
        }
        // For the 16x16x16 MFMA the accumulator layout (row 4lg+i, column lr)
        // is the B-operand layout, so W feeds the next product from registers.
        f16x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = static_cast<_Float16>(Tb[(16 * bi3 + lr) * L::M_LD + 16 * bi3 + 4 * lg + e]);
          b[e] = static_cast<_Float16>(acc[e]);
        }
        f32x4 t = mma_f16_k16(a, b, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) Tb[(16 * bi3 + 4 * lg + i) * L::M_LD + 16 * bj3 + lr] = -t[i];
      }
      __syncthreads();
    }

    // ================= P4: X = V - Kt S,  O = Qt S   (rows of block w)
    f32x4 accO[NCT];
    {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 accX = {0.f, 0.f, 0.f, 0.f};
        accO[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int c0 = 32 * kk + 8 * lg;
          const f16x8 bh = *reinterpret_cast<const f16x8*>(sT + (16 * ct + lr) * L::ST_LD + c0);
          const f16x8 bl = *reinterpret_cast<const f16x8*>(sT + (DV + 16 * ct + lr) * L::ST_LD + c0);
          accX = mma_f16(Kt[kk], bh, accX);
          accX = mma_f16(Kt[kk], bl, accX);
          accO[ct] = mma_f16(Qt[kk], bh, accO[ct]);
          accO[ct] = mma_f16(Qt[kk], bl, accO[ct]);
        }
        f16x4 hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 16 * w + 4 * lg + i;
          const float vv = (rr < Lc)
              ? load1(v, (int64_t)(t0 + rr) * HD + (int64_t)h * D + col0 + 16 * ct + lr, QKV_BF16)
              : 0.0f;
          _Float16 a, b;
          split_f16(s_beta[rr] * (vv - accX[i]), a, b);
          hi[i] = a;
          lo[i] = b;
        }
        const int j = 16 * ct + lr, s = 16 * w + 4 * lg;
        *reinterpret_cast<f16x4*>(bxT + j * L::TT_LD + s) = hi;
        *reinterpret_cast<f16x4*>(bxT + (DV + j) * L::TT_LD + s) = lo;
      }
    }
    __syncthreads();

    // ================= P5: Delta = T (beta X)   (rows of block w)
    {
      const int nk = (w >> 1) + 1;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < nk; ++kk) {
          const int s0 = 32 * kk + 8 * lg;
          const f32x4 t0v = *reinterpret_cast<const f32x4*>(Tb + (16 * w + lr) * L::M_LD + s0);
          const f32x4 t1v = *reinterpret_cast<const f32x4*>(Tb + (16 * w + lr) * L::M_LD + s0 + 4);
          f16x8 a;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = static_cast<_Float16>(t0v[e]);
            a[4 + e] = static_cast<_Float16>(t1v[e]);
          }
          const f16x8 bh = *reinterpret_cast<const f16x8*>(bxT + (16 * ct + lr) * L::TT_LD + s0);
          const f16x8 bl = *reinterpret_cast<const f16x8*>(bxT + (DV + 16 * ct + lr) * L::TT_LD + s0);
          acc = mma_f16(a, bh, acc);
          acc = mma_f16(a, bl, acc);
        }
        f16x4 hi, lo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          _Float16 a, b;
          split_f16(acc[i], a, b);
          hi[i] = a;
          lo[i] = b;
        }
        const int j = 16 * ct + lr, s = 16 * w + 4 * lg;
        *reinterpret_cast<f16x4*>(dlT + j * L::TT_LD + s) = hi;
        *reinterpret_cast<f16x4*>(dlT + (DV + j) * L::TT_LD + s) = lo;
      }
    }
    __syncthreads();

    // ================= P6a: O += P Delta, store o   (rows of block w)
    {
      const int nk = (w >> 1) + 1;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        for (int kk = 0; kk < nk; ++kk) {
          const int s0 = 32 * kk + 8 * lg;
          const f32x4 p0 = *reinterpret_cast<const f32x4*>(Pb + (16 * w + lr) * L::M_LD + s0);
          const f32x4 p1 = *reinterpret_cast<const f32x4*>(Pb + (16 * w + lr) * L::M_LD + s0 + 4);
          f16x8 ph, pl;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            _Float16 a, b;
            split_f16(e < 4 ? p0[e] : p1[e - 4], a, b);
            ph[e] = a;
            pl[e] = b;
          }
          const f16x8 dh = *reinterpret_cast<const f16x8*>(dlT + (16 * ct + lr) * L::TT_LD + s0);
          const f16x8 dl = *reinterpret_cast<const f16x8*>(dlT + (DV + 16 * ct + lr) * L::TT_LD + s0);
          accO[ct] = mma_f16(ph, dh, accO[ct]);
          accO[ct] = mma_f16(pl, dh, accO[ct]);
          accO[ct] = mma_f16(ph, dl, accO[ct]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 16 * w + 4 * lg + i;
          if (rr < Lc) {
            const int64_t oi = (int64_t)(t0 + rr) * HD + (int64_t)h * D + col0 + 16 * ct + lr;
            const float val = scale * accO[ct][i];
            if (O_BF16) static_cast<uint16_t*>(o)[oi] = f32_to_bf16_bits(val);
            else static_cast<float*>(o)[oi] = val;
          }
        }
      }
    }

    // ================= P6b: S <- e^gamma_C S + Khat^T Delta  (key rows 32w..)
    {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float dec = cst[17 * D + 32 * w + 16 * rt + 4 * lg + i];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) sacc[rt][ct][i] *= dec;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int s0 = 32 * kk + 8 * lg;
          const f16x8 a = *reinterpret_cast<const f16x8*>(KhT + (32 * w + 16 * rt + lr) * L::TT_LD + s0);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const f16x8 dh = *reinterpret_cast<const f16x8*>(dlT + (16 * ct + lr) * L::TT_LD + s0);
            const f16x8 dl = *reinterpret_cast<const f16x8*>(dlT + (DV + 16 * ct + lr) * L::TT_LD + s0);
            sacc[rt][ct] = mma_f16(a, dh, sacc[rt][ct]);
            sacc[rt][ct] = mma_f16(a, dl, sacc[rt][ct]);
          }
        }
      }
      write_sT();
    }
    __syncthreads();
  }

  if (Sf) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 32 * w + 16 * rt + 4 * lg + i;
          Sf[sbase + (int64_t)row * D + col0 + 16 * ct + lr] = sacc[rt][ct][i];
        }
  }
}

}  // namespace

hipError_t launch_chunk_prefill(const void* q, const void* k, const void* v, bool qkv_bf16,
                                const float* g, const float* beta, const int32_t* cu, int N,
                                const float* S0, float* S_final, void* o, bool o_bf16,
                                int64_t T_tot, int H, float scale, hipStream_t s) {
  constexpr int DV = 64;
  constexpr int NT = D / DV;
  const int64_t P = (int64_t)N * H;
  const int64_t blocks = 8 * NT * ((P + 7) / 8);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks));
  const int T = static_cast<int>(T_tot);
#define KDA_LAUNCH(QB, OB)                                                                       \
  chunk_kernel<DV, QB, OB><<<grid, NTHR, 0, s>>>(q, k, v, g, beta, cu, N, S0, S_final, o, T, H, \
                                                 scale)
  if (qkv_bf16 && o_bf16) KDA_LAUNCH(true, true);
  else if (qkv_bf16) KDA_LAUNCH(true, false);
  else if (o_bf16) KDA_LAUNCH(false, true);
  else KDA_LAUNCH(false, false);
#undef KDA_LAUNCH
  return hipGetLastError();
}

}  // namespace kda
