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
// float index of element (row, c) of the swizzled gamma buffer
__device__ __forceinline__ int gidx(int row, int c) {
  return row * 128 + ((((c >> 2) ^ (row & 15))) << 2) + (c & 3);
}

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
  static constexpr int GAM_LD = 128;   // fp32 [64][128]   g of the next chunk, then gamma (log2 units);
                                       // 16-byte chunk j of row r stored at chunk j ^ (r & 15)
  static constexpr int OP_LD = 136;    // fp16 [64][136]   Kt, Qt (channel-permuted); R [48][136]; L3 [32][136]
  static constexpr int TT_LD = 72;     // fp16 [..][72]    Khat^T, P hi/lo (token-permuted)
  static constexpr int AT_LD = 72;     // fp16 [64][72]    -A_ij below the diagonal blocks, T_ii on them
  static constexpr int SC_LD = 20;     // fp32 [4][16][20] per-wave transpose scratch

  static constexpr int off_gam = 0;
  static constexpr int off_R = off_gam + C * GAM_LD * 4;
  static constexpr int off_L3 = off_R + 48 * OP_LD * 2;
  static constexpr int off_Kt = off_L3 + 32 * OP_LD * 2;
  static constexpr int off_Qt = off_Kt + C * OP_LD * 2;
  static constexpr int off_KhT = off_Qt + C * OP_LD * 2;
  static constexpr int off_Ph = off_KhT + D * TT_LD * 2;
  static constexpr int off_Pl = off_Ph + C * TT_LD * 2;
  static constexpr int off_AT = off_Pl + C * TT_LD * 2;
  static constexpr int off_scr = off_AT + C * AT_LD * 2;
  static constexpr int off_cst = off_scr + 4 * 16 * SC_LD * 4;
  static constexpr int off_beta = off_cst + 18 * D * 4;
  static constexpr int off_seq = off_beta + C * 4;
  static constexpr int total = off_seq + 16;
};
static_assert(Lds::total <= 160 * 1024, "LDS budget");

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

// Raw buffer resource over [base, base + nbytes): loads past the end return 0
// and stores past the end are dropped, which is how partial chunks are masked.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_buf(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                           0x00020000);
}
__device__ __forceinline__ float buf_f32(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// 16 bytes per lane from a buffer straight into LDS (lane l writes dst + 16 l).
// Kept out of templates: the size check of this builtin misfires in the host
// pass of a template instantiation and silently drops the kernel's host stub.
__device__ __forceinline__ void buf_to_lds16_inl(__amdgpu_buffer_rsrc_t r, lds_ptr_t dst,
                                                 int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
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
__device__ __forceinline__ void load_qk(QKRaw<BF16>& R, __amdgpu_buffer_rsrc_t rs, int off0) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int c = 32 * kk + 16 * a;   // plus 4lg, folded into off0
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

template <bool QKV_BF16, bool O_BF16>
__global__ void __launch_bounds__(NTHR, 1) chunk_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int N, const float* __restrict__ S0,
    float* __restrict__ Sf, void* __restrict__ o, int T_tot, int H, float scale) {
  __shared__ __attribute__((aligned(16))) char lds[Lds::total];
  float* gam = reinterpret_cast<float*>(lds + Lds::off_gam);
  _Float16* Rb = reinterpret_cast<_Float16*>(lds + Lds::off_R);
  _Float16* L3 = reinterpret_cast<_Float16*>(lds + Lds::off_L3);
  _Float16* Kt = reinterpret_cast<_Float16*>(lds + Lds::off_Kt);
  _Float16* Qt = reinterpret_cast<_Float16*>(lds + Lds::off_Qt);
  _Float16* KhT = reinterpret_cast<_Float16*>(lds + Lds::off_KhT);
  _Float16* Ph = reinterpret_cast<_Float16*>(lds + Lds::off_Ph);
  _Float16* Pl = reinterpret_cast<_Float16*>(lds + Lds::off_Pl);
  _Float16* AT = reinterpret_cast<_Float16*>(lds + Lds::off_AT);
  float* cst = reinterpret_cast<float*>(lds + Lds::off_cst);
  float* s_beta = reinterpret_cast<float*>(lds + Lds::off_beta);
  int* s_seq = reinterpret_cast<int*>(lds + Lds::off_seq);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave (uniform)
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
  const int HD = H * D;                  // elements per token row (fits int32: H <= 2^24/128)
  const int col0 = tile * DV;
  const int jcol = col0 + 16 * w + lr;   // value column owned by this lane (state products)
  constexpr int QS = QKV_BF16 ? 2 : 4;   // q/k/v element size
  constexpr int OS = O_BF16 ? 2 : 4;     // o element size

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

  // ---- per-lane byte offsets inside one chunk (rows of the packed token axis)
  const int gc = tid >> 1, ghf = tid & 1;    // gamma pass: channel, half (lane pairs)
  const int rA = 16 * w + lr;                // chunk row of this lane in the operand phase
  const int off_g = (32 * ghf * HD + gc) * 4;
  const int off_qk = rA * HD * QS + 4 * lg * QS;
  const int off_v = (4 * lg * HD + jcol) * QS;  // + 16 rt HD + i HD
  const int off_o = (4 * lg * HD + jcol) * OS;

  // chunk buffers: [t0, min(eos, t0 + C)) tokens of head h
  auto rows_of = [&](int t0c) { return (eos - t0c) < C ? (eos - t0c) : C; };
  auto buf_tok = [&](const void* base, int esz, int t0c) {
    const char* b = static_cast<const char*>(base) + ((int64_t)t0c * HD + (int64_t)h * D) * esz;
    return make_buf(b, (uint32_t)(rows_of(t0c) * HD * esz - h * D * esz));
  };

  // ---- next-chunk prefetch (loads past the chunk end return 0).  g goes
  // straight to LDS (the gamma region, where P0 turns it into gamma in place);
  // k, q, beta and v go to registers.
  QKRaw<QKV_BF16> kpf, qpf;
  uint32_t vraw[16];
  float bpf = 0.0f;
  auto stage_g = [&](int t0n) {
    const auto rg = buf_tok(g, 4, t0n);
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // rows 16w + 2j + (lane >> 5): lane writes physical chunk lane & 31
      const int row0 = 16 * w + 2 * j;
      const int hi = lane >> 5;
      const int lchunk = (lane & 31) ^ ((2 * j + hi) & 15);
      buf_to_lds16_inl(rg, (lds_ptr_t)(gam + row0 * Lds::GAM_LD), hi * HD * 4 + lchunk * 16,
                       row0 * HD * 4);
    }
  };
  auto prefetch_kq = [&](int t0n) {
    load_qk<QKV_BF16>(kpf, buf_tok(k, QS, t0n), off_qk);
    load_qk<QKV_BF16>(qpf, buf_tok(q, QS, t0n), off_qk);
    const char* bb = reinterpret_cast<const char*>(beta) + ((int64_t)t0n * H + h) * 4;
    const auto rb = make_buf(bb, (uint32_t)(rows_of(t0n) * H * 4 - h * 4));
    bpf = buf_f32(rb, lane * H * 4);
  };
  auto prefetch_v = [&](int t0n) {
    const auto rv = buf_tok(v, QS, t0n);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int soff = (16 * rt + i) * HD * QS;
        if constexpr (QKV_BF16) vraw[4 * rt + i] = __builtin_amdgcn_raw_buffer_load_b16(rv, off_v, soff, 0);
        else vraw[4 * rt + i] = __builtin_amdgcn_raw_buffer_load_b32(rv, off_v, soff, 0);
      }
  };
  auto vval = [&](int idx) -> float {
    if constexpr (QKV_BF16) return __uint_as_float(vraw[idx] << 16);
    else return __uint_as_float(vraw[idx]);
  };
  // all of this wave's loads (to LDS or registers) have landed
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(0x0f70); };
  if (bos < eos) {
    stage_g(bos);
    prefetch_kq(bos);
    prefetch_v(bos);
    wait_loads();
  }
  __syncthreads();

  for (int t0 = bos; t0 < eos; t0 += C) {
    const int Lc = rows_of(t0);

    // ================= P0: gamma (cumsum of g, log2 units) and decay constants.
    // Lanes 2c and 2c+1 own channel c, rows 0..31 and 32..63; they exchange
    // their totals and the key-row values with a cross-lane shuffle.
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
      if (tid < C) s_beta[tid] = bpf;
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
      const int kpos = ppos64(r);  // token-permuted column of this row in Khat^T
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
          const f32x4 eL = *reinterpret_cast<const f32x4*>(cst + (4 + bi) * D + c);
          const f32x4 eR = *reinterpret_cast<const f32x4*>(cst + (14 + (bi < 3 ? bi : 0)) * D + c);
          const f32x4 c30 = *reinterpret_cast<const f32x4*>(cst + 13 * D + c);
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
            KhT[(c + j) * Lds::TT_LD + kpos] = static_cast<_Float16>(kf * eL[j]);
            if (bi < 3) rr8[e] = static_cast<_Float16>(kf * eR[j]);
            if (bi == 3) {
              l3k[e] = static_cast<_Float16>(ke * c30[j]);
              l3q[e] = static_cast<_Float16>(qe * c30[j]);
            }
          }
        }
        *reinterpret_cast<f16x8*>(Kt + r * Lds::OP_LD + 32 * kk + 8 * lg) = kt;
        *reinterpret_cast<f16x8*>(Qt + r * Lds::OP_LD + 32 * kk + 8 * lg) = qt;
        if (bi < 3) *reinterpret_cast<f16x8*>(Rb + r * Lds::OP_LD + 32 * kk + 8 * lg) = rr8;
        if (bi == 3) {  // left factors of tile (3,0), which wave 0 multiplies
          *reinterpret_cast<f16x8*>(L3 + lr * Lds::OP_LD + 32 * kk + 8 * lg) = l3k;
          *reinterpret_cast<f16x8*>(L3 + (16 + lr) * Lds::OP_LD + 32 * kk + 8 * lg) = l3q;
        }
      }
      // Diagonal tiles A_ii = (k E)(k F)^T and P_ii = (q E)(k F)^T.  When every
      // |gamma_r - gamma_mid| of the block is <= 7 (log2), E and F lie in
      // [2^-7, 2^7] and the factors are plain fp16 operands; otherwise they
      // are split into hi+lo bf16 pairs, which keep fp32 range.
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
      // -- P1w: diagonal tile (bi, bi): lane holds rows 16bi + 4lg + i, column s = 16bi + lr
      const int sp = ppos64(16 * bi + lr);
      f32x4 nB;  // N = A_ii (strictly lower, beta-scaled rows) in accumulator layout
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 4 * lg + i, row = 16 * bi + rr;
        nB[i] = (lr < rr) ? accA[i] * s_beta[row] : 0.0f;
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
      // -- P1t: T_ii = (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8), exact since
      // N^16 = 0.  Products are 16x16x16 MFMAs: the left factor is read in operand
      // layout through a wave-private LDS transpose, the right factor is an
      // accumulator (hi+lo fp16).
      auto to_a = [&](const f32x4& xb) -> f32x4 {  // accumulator layout -> A-operand layout
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i) scr[(4 * lg + i) * Lds::SC_LD + lr] = xb[i];
        wave_lds_sync();
        return *reinterpret_cast<const f32x4*>(scr + lr * Lds::SC_LD + 4 * lg);
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
        AT[(16 * bi + 4 * lg + i) * Lds::AT_LD + 16 * bi + lr] = static_cast<_Float16>(tB[i]);
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
            lk = *reinterpret_cast<const f16x8*>(L3 + lr * Lds::OP_LD + 32 * kk + 8 * lg);
            lq = *reinterpret_cast<const f16x8*>(L3 + (16 + lr) * Lds::OP_LD + 32 * kk + 8 * lg);
          }
          const f16x8 rb = *reinterpret_cast<const f16x8*>(Rb + (16 * tj + lr) * Lds::OP_LD + 32 * kk + 8 * lg);
          accA = mma_f16(lk, rb, accA);
          accP = mma_f16(lq, rb, accP);
        }
        const int sp = ppos64(16 * tj + lr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * ti + 4 * lg + i;
          AT[row * Lds::AT_LD + 16 * tj + lr] = static_cast<_Float16>(-accA[i] * s_beta[row]);
          _Float16 x0, x1;
          split_f16(accP[i], x0, x1);
          Ph[row * Lds::TT_LD + sp] = x0;
          Pl[row * Lds::TT_LD + sp] = x1;
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

    // ================= P3: state products for value column jcol (no barriers)
    {
      const bool more = t0 + C < eos;
      if (more) {  // operands of this chunk are consumed: fetch the next chunk's
        stage_g(t0 + C);
        prefetch_kq(t0 + C);
      }
      // S as B fragments (hi/lo), contraction over key channels
      f16x8 sbh[4], sbl[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) bfrag_split(Sacc[2 * kk], Sacc[2 * kk + 1], sbh[kk], sbl[kk]);
      // X = V - Kt S ;  O = Qt S   (8 independent accumulator chains)
      f32x4 Xacc[4], Oacc[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) Xacc[rt] = Oacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const f16x8 ak = *reinterpret_cast<const f16x8*>(Kt + (16 * rt + lr) * Lds::OP_LD + 32 * kk + 8 * lg);
          const f16x8 aq = *reinterpret_cast<const f16x8*>(Qt + (16 * rt + lr) * Lds::OP_LD + 32 * kk + 8 * lg);
          Xacc[rt] = mma_f16(ak, sbh[kk], Xacc[rt]);
          Oacc[rt] = mma_f16(aq, sbh[kk], Oacc[rt]);
          Xacc[rt] = mma_f16(ak, sbl[kk], Xacc[rt]);
          Oacc[rt] = mma_f16(aq, sbl[kk], Oacc[rt]);
        }
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) Xacc[rt][i] = vval(4 * rt + i) - Xacc[rt][i];
      if (more) prefetch_v(t0 + C);  // v of this chunk is consumed
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
      // -- P3c: O += P Delta ; store o (rows past the chunk end are dropped)
      const char* ob = static_cast<const char*>(o) + ((int64_t)t0 * HD + (int64_t)h * D) * OS;
      const auto ro = make_buf(ob, (uint32_t)(Lc * HD * OS - h * D * OS));
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
          const int soff = (16 * rt + i) * HD * OS;
          const float val = scale * ao[i];
          if constexpr (O_BF16)
            __builtin_amdgcn_raw_buffer_store_b16(
                __builtin_bit_cast(uint16_t, static_cast<__bf16>(val)), ro, off_o, soff, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), ro, off_o, soff, 0);
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
    wait_loads();
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
