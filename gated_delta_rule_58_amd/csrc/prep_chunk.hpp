// The prep computation of the chunked prefill: everything about one (chunk,
// head) that does not depend on the state.  prep_chunk runs it on one unit of
// 4 waves (the prep kernel's workgroup, or one of the fused kernel's prep
// units) and writes that chunk's
// workspace image (layout in chunk_common.hpp): K e^gamma, Q e^gamma,
// (K e^(gamma_C - gamma))^T, the decay-weighted P, the lower triangular
// (I + A)^-1 diag(beta) that maps X to Delta, and e^gamma_C.
//
// Wave i owns chunk rows 16i..16i+15 (block i); lane (lr, lg) owns row
// 16i + lr and, in k-step kk, the 8 consecutive channels 32kk + 8lg + e.
// g, k and q are loaded straight into registers in that layout.
//  S1  gamma = cumsum(g) down the rows: a 16-lane DPP scan inside each block,
//      block sums exchanged through LDS.
//  S2  per-(block, channel) decay constants from the block sums.
//  P1  decay factors, K e^gamma and Q e^gamma (to the image), the decayed
//      K^T (transposed by an MFMA against a 0/1 selector, to the image), the
//      off-diagonal factors (LDS), the diagonal tiles A_ii and P_ii, and
//      T_ii = (I + A_ii)^-1 by repeated squaring.
//  P2  off-diagonal tiles (i, j < i) of A and P, two per wave at most.
//  P3  the blocks of (I + A)^-1 below the diagonal, by forward substitution
//      down each block column (one column per wave), from T_ii and -A_ij.
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
// pairs, which keep fp32 range.  fp32 range needs every 8-token span of one
// channel's decay below 126 (log2 units): the per-token decay is floored at
// -DECAY_FLOOR_LOG2 (15.5) before the scan, which keeps the spans at 124 or
// less for any g <= 0 (NaN passes through unchanged).
#pragma once

#include <type_traits>

#include "chunk_common.hpp"
#include "gate_math.hpp"

namespace kda {
namespace chunk {
namespace {

struct PrepLds {
  static constexpr int SC_LD = 17;  // fp32 [4][16][17] per-wave transpose scratch
  static constexpr int off_R = 0;                         // fp16 6 x [16][128], rl_off layout
  static constexpr int off_L3 = off_R + 96 * D * 2;       // fp16 [32][128], rl_off layout
  static constexpr int off_scr = off_L3 + 32 * D * 2;
  static constexpr int off_btot = off_scr + 4 * 16 * SC_LD * 4;  // fp32 [4][128] block sums
  static constexpr int off_bmid = off_btot + 4 * D * 4;   // fp32 [4][128] block sums to row 7
  static constexpr int off_gm = off_bmid + 4 * D * 4;     // fp32 [4][128] gamma at mid rows
  static constexpr int off_cst = off_gm + 4 * D * 4;      // fp32 [18][128]
  static constexpr int off_beta = off_cst + 18 * D * 4;
  static constexpr int off_flag = off_beta + C * 4;      // int [4]: block needs wide range
  static constexpr int total = off_flag + 16;
};
static_assert(PrepLds::total <= 160 * 1024 / 3, "three prep workgroups per CU");

// byte offset of (row r, channel c) in the fp16 [rows][128] factor buffers:
// 16-byte chunks swizzled by row so a 16-lane column of rows is conflict-free
__device__ __forceinline__ int rl_off(int r, int c) {
  return r * 256 + ((((c >> 3) ^ (r & 15))) << 4) + ((c & 7) << 1);
}

// Per-channel constant slots (after exp2, all <= 1).  m_i = 16i + 7 is the
// mid row of block i, b_i = 16i - 1 the row before it (gamma_{b_0} = 0):
//  0..3   em_i = 2^gamma_{m_i}
//  4..6   cL_i = 2^(gamma_{m_i} - gamma_{b_i}), i = 1..3
//  7..12  cR(i,j) = 2^(gamma_{b_i} - gamma_{m_j}), pairs (i, j > ... ) in rset order
//  13     eC = 2^gamma_C
//  14..17 eL_i = 2^(gamma_C - gamma_{m_i})
// An off-diagonal tile (i, j < i) is then the product of the left factor
// k_r 2^(gamma_r - gamma_{b_i}) = (k E)_r cL_i (one per row block) and the
// right factor k_s 2^(gamma_{b_i} - gamma_s) = (k F)_s cR(i,j), both <= 1.
// Right-factor set of tile (i, j): (1,0) (2,0) (3,0) (2,1) (3,1) (3,2).
__device__ __forceinline__ int rset(int i, int j) { return j == 0 ? i - 1 : (j == 1 ? i + 1 : 5); }

// v + (v of the lane K rows up, inside each 16-lane row; 0 above the row)
template <int K>
__device__ __forceinline__ float add_row_shr(float v) {
  const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x110 + K, 0xf, 0xf,
                                            true);
  return v + __builtin_bit_cast(float, s);
}

template <bool BF16>
struct Row8;  // 8 consecutive channels per k-step, 4 k-steps
template <>
struct Row8<true> {
  u16x8 v[4];
  __device__ __forceinline__ float at(int kk, int e) const { return bf16_bits_to_f32(v[kk][e]); }
};
template <>
struct Row8<false> {
  f32x4 v[4][2];
  __device__ __forceinline__ float at(int kk, int e) const { return v[kk][e >> 2][e & 3]; }
};

template <bool BF16>
__device__ __forceinline__ void load_row8(Row8<BF16>& R, __amdgpu_buffer_rsrc_t rs, int off0) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if constexpr (BF16) {
      R.v[kk] = __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off0 + 64 * kk, 0, 0));
    } else {
#pragma unroll
      for (int a = 0; a < 2; ++a)
        R.v[kk][a] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off0 + 128 * kk + 16 * a, 0, 0));
    }
  }
}

// The decay input: log-decay g (fp32), or the raw gate logits x (fp32 or
// bf16) from which g and beta are formed in registers (gate_math.hpp).
// kPC (or-ed into kX32 / kX16): A_log per (head, channel), [H, 128].
enum GateIn { kG = 0, kX32 = 1, kX16 = 2, kPC = 4 };
struct GateArgs {
  const void* b;         // beta logits [T, H] (gated input) or post-sigmoid beta (fp32)
  bool b_bf16;
  const float* A_log;    // [H], or [H, 128] with kPC
  const float* dt_bias;  // [H, 128]
};

}  // namespace

// One chunk of one head, computed by one unit of 4 waves: `tid` in [0, 256) is
// the thread's index in the unit and `lds` the unit's PrepLds::total bytes.
// Rows [t0, t0 + Lc) of head h (h < H).  Lc == 0 is a unit without a task: every
// load reads 0 and the image goes to `img`, a scratch slot, so that the unit
// still meets every workgroup barrier.
template <bool QKV_BF16, int GIN>
__device__ __forceinline__ void prep_chunk(const void* __restrict__ q, const void* __restrict__ k,
                                           const void* __restrict__ g, const GateArgs& ga, int H,
                                           int h, int t0, int Lc, char* __restrict__ img,
                                           char* lds, int tid) {
  char* Rb = lds + PrepLds::off_R;
  char* L3 = lds + PrepLds::off_L3;
  float* btot = reinterpret_cast<float*>(lds + PrepLds::off_btot);
  float* bmid = reinterpret_cast<float*>(lds + PrepLds::off_bmid);
  float* gmv = reinterpret_cast<float*>(lds + PrepLds::off_gm);
  float* cst = reinterpret_cast<float*>(lds + PrepLds::off_cst);
  float* s_beta = reinterpret_cast<float*>(lds + PrepLds::off_beta);
  int* s_flag = reinterpret_cast<int*>(lds + PrepLds::off_flag);

  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave of the unit (uniform)
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  float* scr = reinterpret_cast<float*>(lds + PrepLds::off_scr) + w * 16 * PrepLds::SC_LD;
  const int HD = H * D;
  constexpr int QS = QKV_BF16 ? 2 : 4;
  const int bi = w;
  const int r = 16 * w + lr;  // chunk row of this lane

  // chunk buffers: rows [t0, t0 + Lc) of head h; loads past Lc return 0 (all
  // of them when Lc == 0)
  auto buf_tok = [&](const void* base, int esz) {
    const char* b = static_cast<const char*>(base) + ((int64_t)t0 * HD + (int64_t)h * D) * esz;
    return make_buf(b, Lc > 0 ? (uint32_t)(Lc * HD * esz - h * D * esz) : 0u);
  };

  // ---- loads: row r, channels 32kk + 8lg .. +7 (dt_bias first: every gate
  // element needs it)
  f32x4 dtb[4][2], alc[4][2];
  if constexpr (GIN != kG) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        dtb[kk][a] = *reinterpret_cast<const f32x4*>(ga.dt_bias + h * D + 32 * kk + 8 * lg + 4 * a);
        if constexpr ((GIN & kPC) != 0)
          alc[kk][a] = *reinterpret_cast<const f32x4*>(ga.A_log + h * D + 32 * kk + 8 * lg + 4 * a);
      }
  }
  f32x4 graw[4][2];
  {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    if constexpr ((GIN & 3) == kX16) {
      const auto rg = buf_tok(g, 2);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u16x8 x8 = __builtin_bit_cast(
            u16x8, __builtin_amdgcn_raw_buffer_load_b128(rg, r * HD * 2 + (32 * kk + 8 * lg) * 2, 0, 0));
#pragma unroll
        for (int e = 0; e < 8; ++e) graw[kk][e >> 2][e & 3] = bf16_bits_to_f32(x8[e]);
      }
    } else {
      const auto rg = buf_tok(g, 4);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int a = 0; a < 2; ++a)
          graw[kk][a] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, r * HD * 4 + (32 * kk + 8 * lg + 4 * a) * 4, 0, 0));
    }
  }
  Row8<QKV_BF16> kv8, qv8;
  load_row8<QKV_BF16>(kv8, buf_tok(k, QS), (r * HD + 8 * lg) * QS);
  load_row8<QKV_BF16>(qv8, buf_tok(q, QS), (r * HD + 8 * lg) * QS);
  float bval;
  {
    const int bs = (GIN != kG && ga.b_bf16) ? 2 : 4;
    const char* bb = static_cast<const char*>(ga.b) + ((int64_t)t0 * H + h) * bs;
    const auto rb = make_buf(bb, Lc > 0 ? (uint32_t)(Lc * H * bs - h * bs) : 0u);
    if (bs == 2) bval = bf16_bits_to_f32((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rb, r * H * 2, 0, 0));
    else bval = buf_f32(rb, r * H * 4);
  }
  if constexpr (GIN != kG) {
    // g log2(e) = -exp(A_log[h]) softplus(x + dt_bias[h, c]) log2(e) straight in
    // the scan's log2 units, beta = sigmoid(b).  Computed on every row and
    // masked (rows past the chunk end read x = b = 0, finite): a select here
    // becomes per-element branches that serialize the dt_bias loads.
    const float neg_a = (GIN & kPC) != 0 ? 0.0f : -expf(ga.A_log[h]);
    const float keep = r < Lc ? 1.0f : 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float na = (GIN & kPC) != 0 ? -expf(alc[kk][a][j]) : neg_a;
          graw[kk][a][j] = keep * gate_log2_decay_fast(na, gate_input(graw[kk][a][j], dtb[kk][a][j]));
        }
    bval = keep * gate_beta(bval);
  }

  // ================= S1: gamma (log2 units), in-block scan down the 16 rows
  float gam[4][8];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = GIN == kG ? graw[kk][e >> 2][e & 3] * LOG2E : graw[kk][e >> 2][e & 3];
      x = x < -DECAY_FLOOR_LOG2 ? -DECAY_FLOOR_LOG2 : x;
      x = add_row_shr<1>(x);
      x = add_row_shr<2>(x);
      x = add_row_shr<4>(x);
      x = add_row_shr<8>(x);
      gam[kk][e] = x;
    }
  if (lr == 15 || lr == 7) {
    float* dst = (lr == 15 ? btot : bmid) + w * D;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int a = 0; a < 2; ++a)
        *reinterpret_cast<f32x4*>(dst + 32 * kk + 8 * lg + 4 * a) =
            f32x4{gam[kk][4 * a], gam[kk][4 * a + 1], gam[kk][4 * a + 2], gam[kk][4 * a + 3]};
  }
  if (lg == 0) s_beta[r] = bval;
  if (tid < 4) s_flag[tid] = 0;
  __syncthreads();

  // ================= S2: gamma at the block ends and mid rows, decay constants;
  // every lane adds the sums of the blocks above its own.
  {
    const int c = tid & 127, half = tid >> 7;
    const float t0v = btot[c], t1v = btot[D + c], t2v = btot[2 * D + c], t3v = btot[3 * D + c];
    const float gb1 = t0v, gb2 = gb1 + t1v, gb3 = gb2 + t2v, gl = gb3 + t3v;
    const float gm0 = bmid[c], gm1 = gb1 + bmid[D + c], gm2 = gb2 + bmid[2 * D + c],
                gm3 = gb3 + bmid[3 * D + c];
    if (half == 0) {
      gmv[c] = gm0;
      gmv[D + c] = gm1;
      cst[0 * D + c] = ex2(gm0);
      cst[1 * D + c] = ex2(gm1);
      cst[2 * D + c] = ex2(gm2);
      cst[3 * D + c] = ex2(gm3);
      cst[4 * D + c] = ex2(gm1 - gb1);
      cst[5 * D + c] = ex2(gm2 - gb2);
      cst[6 * D + c] = ex2(gm3 - gb3);
      cst[14 * D + c] = ex2(gl - gm0);
      cst[15 * D + c] = ex2(gl - gm1);
      // gamma of block i spans [gamma_{b_{i+1}}, gamma_{b_i}] (non-increasing)
      if (fmaxf(-gm0, gm0 - gb1) > 7.0f) s_flag[0] = 1;
      if (fmaxf(gb1 - gm1, gm1 - gb2) > 7.0f) s_flag[1] = 1;
    } else {
      gmv[2 * D + c] = gm2;
      gmv[3 * D + c] = gm3;
      cst[7 * D + c] = ex2(gb1 - gm0);
      cst[8 * D + c] = ex2(gb2 - gm0);
      cst[9 * D + c] = ex2(gb3 - gm0);
      cst[10 * D + c] = ex2(gb2 - gm1);
      cst[11 * D + c] = ex2(gb3 - gm1);
      cst[12 * D + c] = ex2(gb3 - gm2);
      cst[13 * D + c] = ex2(gl);
      cst[16 * D + c] = ex2(gl - gm2);
      cst[17 * D + c] = ex2(gl - gm3);
      if (fmaxf(gb2 - gm2, gm2 - gb3) > 7.0f) s_flag[2] = 1;
      if (fmaxf(gb3 - gm3, gm3 - gl) > 7.0f) s_flag[3] = 1;
    }
  }
  // prefix of the blocks above (same summation order as gb_i above)
  if (w > 0) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int c0 = 32 * kk + 8 * lg + 4 * a;
        f32x4 pre = *reinterpret_cast<const f32x4*>(btot + c0);
        for (int j = 1; j < w; ++j) pre += *reinterpret_cast<const f32x4*>(btot + j * D + c0);
#pragma unroll
        for (int i = 0; i < 4; ++i) gam[kk][4 * a + i] += pre[i];
      }
  }
  __syncthreads();

  // 16x16 tile helpers (one wave): accumulator layout (rows 4lg+i, column lr)
  // -> operand layout (row lr, columns 4lg+e) through the wave's LDS scratch,
  // and the 16x16x16 product of an operand-layout left factor (one fp16) with
  // an accumulator-layout right factor (hi+lo fp16), added to acc.
  auto to_a = [&](const f32x4& xb) -> f32x4 {
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 4; ++i) scr[(4 * lg + i) * PrepLds::SC_LD + lr] = xb[i];
    wave_lds_sync();
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = scr[lr * PrepLds::SC_LD + 4 * lg + e];
    return x;
  };
  auto mac16 = [&](const f16x4& a, const f32x4& yb, f32x4 acc) -> f32x4 {
    f16x4 bh, bl;
    bfrag16_split(yb, bh, bl);
    acc = mma_f16_k16(a, bh, acc);
    return mma_f16_k16(a, bl, acc);
  };
  auto mul = [&](const f32x4& xa, const f32x4& yb) -> f32x4 {
    return mac16(cvt_f16(xa), yb, f32x4{0.f, 0.f, 0.f, 0.f});
  };
  // P3 operands: fp32 T_ii tiles (row-major, over the block sums, dead since
  // S2) and fp16 N_ij = -A_ij tiles (row-major, over constant slots 0..5, dead
  // after P1)
  float* Tt = btot;
  _Float16* Nt = reinterpret_cast<_Float16*>(cst);
  auto n_tile = [](int i, int j) { return ((i * (i - 1)) >> 1) + j; };

  // ================= P1: per 32-channel step kk: decay factors, the image's
  // K e^gamma, Q e^gamma and transposed decayed K, the right factors of the
  // tiles below this block (LDS), this block's left factors (registers; LDS
  // for tile (3,0)), and the diagonal tiles A_ii, P_ii.  Only the left factors
  // outlive a step.
  // Diagonal tiles A_ii = (k E)(k F)^T (accumulator layout: rows 4lg+i) and
  // P_ii = (q E)(k F)^T computed as (k F)(q E)^T, so a lane holds row lr,
  // columns 4lg .. +3 (the image's row-major tile).  E and F span at most
  // the block's decay: plain fp16 when that is <= 2^7, otherwise hi+lo bf16.
  const bool wide = s_flag[bi] != 0;
  f16x8 lk[4], lq[4];
  f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
  {
    // Kd x Sel_h with Sel_h[k][n] = (k == 16h + n) puts Kd[16bi + 4lg + i][32kk + 16h + lr]
    // in lane (lr, lg): four tokens of one channel (512 contiguous bytes per store)
    f16x8 sel[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sel[hh][e] = static_cast<_Float16>((8 * lg + e == 16 * hh + lr) ? 1.0f : 0.0f);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      // the factors a row block uses: block 0 none of the left factors, blocks
      // 0..2 the right factors of the tiles below them (block 0 three, block 1
      // two, block 2 one); each half of 4 channels is converted to fp16 as soon
      // as it is formed (two values per conversion)
      f32x4 keh[2], qeh[2], kfh[2];
      f16x4 kth[2], qth[2], kdh[2], lkh[2], lqh[2], r0h[2], r1h[2], r2h[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int c = 32 * kk + 8 * lg + 4 * a;
        const f32x4 gm = *reinterpret_cast<const f32x4*>(gmv + bi * D + c);
        const f32x4 em = *reinterpret_cast<const f32x4*>(cst + bi * D + c);
        const f32x4 eL = *reinterpret_cast<const f32x4*>(cst + (14 + bi) * D + c);
        f32x4 kv4, qv4, E, F;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kv4[j] = kv8.at(kk, 4 * a + j);
          qv4[j] = qv8.at(kk, 4 * a + j);
          const float dg = gam[kk][4 * a + j] - gm[j];
          E[j] = ex2(dg);
          F[j] = ex2(-dg);
        }
        const f32x4 ke = kv4 * E, qe = qv4 * E, kf = kv4 * F;
        keh[a] = ke;
        qeh[a] = qe;
        kfh[a] = kf;
        kth[a] = cvt_f16(ke * em);
        qth[a] = cvt_f16(qe * em);
        kdh[a] = cvt_f16(kf * eL);
        // computed on every wave (the stores below pick what each block needs):
        // per-wave branches here cost more in registers than they save
        const f32x4 cl = *reinterpret_cast<const f32x4*>(cst + (bi > 0 ? 3 + bi : 4) * D + c);
        lkh[a] = cvt_f16(ke * cl);
        lqh[a] = cvt_f16(qe * cl);
        // right-factor scales of the tiles (i, bi), i > bi
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(
            cst + (7 + rset(bi < 3 ? bi + 1 : 3, bi < 3 ? bi : 2)) * D + c);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(
            cst + (7 + rset(bi < 2 ? bi + 2 : 3, bi < 2 ? bi : 1)) * D + c);
        const f32x4 s2 = *reinterpret_cast<const f32x4*>(cst + 9 * D + c);
        r0h[a] = cvt_f16(kf * s0);
        r1h[a] = cvt_f16(kf * s1);
        r2h[a] = cvt_f16(kf * s2);
      }
      auto cat = [](const f16x4& x, const f16x4& y) -> f16x8 {
        return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      const f16x8 kd = cat(kdh[0], kdh[1]);
      lk[kk] = cat(lkh[0], lkh[1]);
      lq[kk] = cat(lqh[0], lqh[1]);
      // K e^gamma, Q e^gamma: two 8-byte halves per lane
      *reinterpret_cast<f16x4*>(img + Ws::KE + keqe_at(bi, kk, 8 * lg, lr)) = kth[0];
      *reinterpret_cast<f16x4*>(img + Ws::KE + keqe_at(bi, kk, 8 * lg + 4, lr)) = kth[1];
      *reinterpret_cast<f16x4*>(img + Ws::QE + keqe_at(bi, kk, 8 * lg, lr)) = qth[0];
      *reinterpret_cast<f16x4*>(img + Ws::QE + keqe_at(bi, kk, 8 * lg + 4, lr)) = qth[1];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4 dt = mma_f16(kd, sel[hh], f32x4{0.f, 0.f, 0.f, 0.f});
        *reinterpret_cast<f16x4*>(img + Ws::KDT + kdt_at(bi, 2 * kk + hh, lr, lg)) = cvt_f16(dt);
      }
      // right factors of the tiles below: block 0 -> (1,0) (2,0) (3,0);
      // block 1 -> (2,1) (3,1); block 2 -> (3,2)
      const int co = 32 * kk + 8 * lg;
      if (bi < 3) *reinterpret_cast<f16x8*>(Rb + rl_off(16 * rset(bi + 1, bi) + lr, co)) = cat(r0h[0], r0h[1]);
      if (bi < 2) *reinterpret_cast<f16x8*>(Rb + rl_off(16 * rset(bi + 2, bi) + lr, co)) = cat(r1h[0], r1h[1]);
      if (bi == 0) *reinterpret_cast<f16x8*>(Rb + rl_off(16 * rset(3, 0) + lr, co)) = cat(r2h[0], r2h[1]);
      if (bi == 3) {  // left factors of tile (3,0), which wave 0 multiplies
        *reinterpret_cast<f16x8*>(L3 + rl_off(lr, co)) = lk[kk];
        *reinterpret_cast<f16x8*>(L3 + rl_off(16 + lr, co)) = lq[kk];
      }
      // diagonal tiles, this step's 32 channels
      if (!wide) {
        const f16x8 ek = cat(cvt_f16(keh[0]), cvt_f16(keh[1])),
                    eq = cat(cvt_f16(qeh[0]), cvt_f16(qeh[1])),
                    fk = cat(cvt_f16(kfh[0]), cvt_f16(kfh[1]));
        accA = mma_f16(ek, fk, accA);
        accP = mma_f16(fk, eq, accP);
      } else {
        bf16x8 ekh, ekl, eqh, eql, fkh, fkl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 x0, x1;
          split_bf16(keh[e >> 2][e & 3], x0, x1); ekh[e] = x0; ekl[e] = x1;
          split_bf16(qeh[e >> 2][e & 3], x0, x1); eqh[e] = x0; eql[e] = x1;
          split_bf16(kfh[e >> 2][e & 3], x0, x1); fkh[e] = x0; fkl[e] = x1;
        }
        accA = mma_bf16(ekh, fkh, accA);
        accA = mma_bf16(ekh, fkl, accA);
        accA = mma_bf16(ekl, fkh, accA);
        accP = mma_bf16(fkh, eqh, accP);
        accP = mma_bf16(fkl, eqh, accP);
        accP = mma_bf16(fkh, eql, accP);
      }
    }
  }
  {
    // -- diagonal tile (bi, bi)
    f32x4 nB;  // N = A_ii (strictly lower, beta-scaled rows) in accumulator layout
    f32x4 pd;  // P_ii row lr, columns 4lg + i (lower triangle kept)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 4 * lg + i, row = 16 * bi + rr;
      nB[i] = (lr < rr) ? accA[i] * s_beta[row] : 0.0f;
      pd[i] = (rr <= lr) ? accP[i] : 0.0f;
    }
    *reinterpret_cast<f16x4*>(img + Ws::PM + tri_at(bi, bi, lr, lg)) = cvt_f16(pd);
    // -- T_ii = (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8), exact since
    // N^16 = 0.  Products are 16x16x16 MFMAs: the left factor is read in operand
    // layout through a wave-private LDS transpose, the right factor is an
    // accumulator (hi+lo fp16).
    f32x4 eye;
#pragma unroll
    for (int i = 0; i < 4; ++i) eye[i] = (4 * lg + i == lr) ? 1.0f : 0.0f;  // same in both layouts
    const f32x4 nA = to_a(nB);
    const f32x4 n2B = mul(nA, nB);
    const f32x4 n4B = mul(to_a(n2B), n2B);
    const f32x4 n8B = mul(to_a(n4B), n4B);
    const f32x4 m2B = mul(eye - nA, eye + n2B);
    const f32x4 m3B = mul(to_a(m2B), eye + n4B);
    const f32x4 tA = to_a(mul(to_a(m3B), eye + n8B));  // row lr, columns 4lg + e
    // fp32 T_ii for the blocks below the diagonal; the image gets T_ii diag(beta)
    *reinterpret_cast<f32x4*>(Tt + bi * 256 + lr * 16 + 4 * lg) = tA;
    const f32x4 bc = *reinterpret_cast<const f32x4*>(s_beta + 16 * bi + 4 * lg);
    *reinterpret_cast<f16x4*>(img + Ws::AT + tri_at(bi, bi, lr, lg)) = cvt_f16(tA * bc);
  }
  __syncthreads();

  // ================= P2: off-diagonal tiles (i, j<i): two per wave at most.
  // Wave w multiplies its own left factors (rows of block w) except wave 0,
  // which takes tile (3,0) with the left factors wave 3 left in LDS.
  {
    auto offdiag = [&](int ti, int tj) {
      f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int co = 32 * kk + 8 * lg;
        f16x8 lkk, lqk;
        if (ti == bi) {
          lkk = lk[kk];
          lqk = lq[kk];
        } else {
          lkk = *reinterpret_cast<const f16x8*>(L3 + rl_off(lr, co));
          lqk = *reinterpret_cast<const f16x8*>(L3 + rl_off(16 + lr, co));
        }
        const f16x8 rb = *reinterpret_cast<const f16x8*>(Rb + rl_off(16 * rset(ti, tj) + lr, co));
        // transposed products: lane (lr, lg) gets row lr, columns 4lg .. +3
        aA = mma_f16(rb, lkk, aA);
        aP = mma_f16(rb, lqk, aP);
      }
      const float nb = -s_beta[16 * ti + lr];
      *reinterpret_cast<f16x4*>(Nt + n_tile(ti, tj) * 256 + lr * 16 + 4 * lg) = cvt_f16(aA * nb);
      *reinterpret_cast<f16x4*>(img + Ws::PM + tri_at(ti, tj, lr, lg)) = cvt_f16(aP);
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

  // ================= P3: the blocks of T = (I + A)^-1 below the diagonal.  Column
  // block j is a forward substitution down the column: T_ij = T_ii sum_{k=j}^{i-1}
  // N_ik T_kj for i > j.  Wave j < 3 takes column j; the image gets T_ij
  // diag(beta_j), so that the state kernel's Delta = (T diag(beta)) X needs no
  // substitution of its own.
  auto column = [&](auto J) {
    constexpr int j = decltype(J)::value;
    f32x4 X[4];  // X[k] = T_kj, accumulator layout
#pragma unroll
    for (int i = 0; i < 4; ++i) X[j][i] = Tt[j * 256 + (4 * lg + i) * 16 + lr];
    const float bcol = s_beta[16 * j + lr];
#pragma unroll
    for (int i = j + 1; i < 4; ++i) {
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = j; kb < i; ++kb)
        y = mac16(*reinterpret_cast<const f16x4*>(Nt + n_tile(i, kb) * 256 + lr * 16 + 4 * lg), X[kb], y);
      X[i] = mul(*reinterpret_cast<const f32x4*>(Tt + i * 256 + lr * 16 + 4 * lg), y);
      const f32x4 xa = to_a(X[i] * bcol);  // row lr, columns 4lg + e
      *reinterpret_cast<f16x4*>(img + Ws::AT + tri_at(i, j, lr, lg)) = cvt_f16(xa);
    }
  };
  if (w == 0) column(std::integral_constant<int, 0>{});
  else if (w == 1) column(std::integral_constant<int, 1>{});
  else if (w == 2) column(std::integral_constant<int, 2>{});

  // ---- EC
  {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    if (w == 3 && lane < 32)
      *reinterpret_cast<u32x4*>(img + Ws::EC + 16 * lane) =
          *reinterpret_cast<const u32x4*>(cst + 13 * D + 4 * lane);
  }
}

}  // namespace chunk
}  // namespace kda
