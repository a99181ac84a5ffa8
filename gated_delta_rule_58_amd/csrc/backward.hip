// kda_chunk_prefill_backward: gradients of the chunked KDA prefill.
//
// For one (sequence, head) the forward is the recurrence S_t = (I - b_t k_t
// k_t^T) Diag(exp(g_t)) S_{t-1} + b_t k_t v_t^T, o_t = scale S_t^T q_t, so its
// gradient is the reverse-mode of the same chunk identities the forward uses.
// Per chunk of L <= 64 tokens with entry state S (d_k x d_v), gamma the
// within-chunk cumulative sum of g, E = exp(gamma), K_E = K.E, Q_E = Q.E,
// K_D = K.exp(gamma_C - gamma) (gamma_C the chunk's last row),
//   At[r,s] = sum_c k_rc k_sc exp(gamma_rc - gamma_sc)  (s < r),  A = diag(b) At
//   P[r,s]  = sum_c q_rc k_sc exp(gamma_rc - gamma_sc)  (s <= r)
//   M = (I + A)^-1,  X = V - K_E S,  Y = diag(b) X,  Delta = M Y
//   O = scale (Q_E S + P Delta),  S_next = Diag(exp(gamma_C)) S + K_D^T Delta.
// With W = M diag(b) K_E, U = M diag(b) V and Qt = scale (Q_E - P W):
//   S_next = Diag(e^gamma_C) S - K_D^T (W S) + K_D^T U                 (forward)
//   dS     = Diag(e^gamma_C) dS_next - W^T (K_D dS_next) + Qt^T dO     (backward)
// Both walks have one shape: Z = A1 R; R <- e^gamma_C R - A2^T Z + A3^T B.
//
// Three kernels, all to fp32 accuracy: the products on fp32 MFMA, except the
// walk's (its state update, and Z = A1 R with bf16 d_o), which run on bf16
// MFMA as three-term splits that carry fp32's 24 bits (walk_dir):
//   bwd_prep  one workgroup per (chunk, head): gamma, At, P, M, W, U, Qt, K_D
//             and e^gamma_C into a per-(chunk, head) record;
//   bwd_walk  one workgroup per (sequence, head, 64-column tile) and
//             direction, both directions in one launch: forward, the entry
//             state of every chunk; backward, the state gradient at every
//             chunk's end and the initial state's gradient;
//   bwd_grad  one workgroup per (chunk, head), each with a scratch slot of
//             its own, in launches of at most grad_slots workgroups: with S
//             and dS_next known, the chunk's gradients dq, dk, dv, dg, dbeta
//             by the chain rule through the identities above (the pairwise
//             decay terms of At and P per 16-channel slab, dg as the
//             reverse cumulative sum of dgamma within the same slab).
#include <type_traits>

#include "chunk_common.hpp"
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace bwd {
namespace {

constexpr int C = 64;
constexpr int D = 128;
constexpr int NT = 256;

// The per-token decay floor of the forward prefill, in natural-log units: g
// enters as max(g, -15.5 / log2 e) (the test taken in log2 units, as the
// forward takes it; NaN passes through), so the backward differentiates the
// function the forward computes and its decay factors keep their range
// bounds.  The gradient of a floored g is 0.
__device__ __forceinline__ bool decay_floored(float g) {
  return g * chunk::LOG2E < -chunk::DECAY_FLOOR_LOG2;
}
__device__ __forceinline__ float floor_decay(float g) {
  return decay_floored(g) ? -chunk::DECAY_FLOOR_LOG2 / chunk::LOG2E : g;
}

// Per-(chunk, head) record written by bwd_prep (offsets in floats).
struct Rec {
  static constexpr int W = 0;             // [C][D]  M diag(b) K_E
  static constexpr int U = W + C * D;     // [C][D]  M diag(b) V
  static constexpr int QT = U + C * D;    // [C][D]  scale (Q_E - P W)
  static constexpr int KD = QT + C * D;   // [C][D]  K exp(gamma_C - gamma)
  static constexpr int G = KD + C * D;    // [C][D]  gamma (rows past the chunk end repeat the last)
  static constexpr int M = G + C * D;     // [C][C]  (I + A)^-1
  static constexpr int P = M + C * C;     // [C][C]  P (s <= r)
  static constexpr int AT = P + C * C;    // [C][C]  At (s < r)
  static constexpr int EC = AT + C * C;   // [D]     exp(gamma_C)
  static constexpr int floats = EC + D;
};
// Per-(chunk, head) scratch of bwd_grad (offsets in floats, each [C][D]).
struct Scr {
  static constexpr int DL = 0, DD = C * D, DX = 2 * C * D, DKE = 3 * C * D, DQE = 4 * C * D,
                       DKD = 5 * C * D, floats = 6 * C * D;
};

constexpr int KT = 16;
// Slab rows of the staged products: the contraction index contiguous, rows
// 4 x odd floats apart, so the 16-byte fills and reads of 16 lanes land on
// distinct banks.
constexpr int SKP = KT + 4;
constexpr int STAGE_FLOATS = (64 + 128) * SKP;  // the largest product's slabs
// acc += a b for a (16 TM / 4 x 4 waves) x (16 TN) output over the 256
// threads, on fp32 MFMA, with the operands staged through LDS in slabs of
// KT = 16 along the contraction (each element read once from memory instead
// of once per thread that uses it).  acc[i][j][v] is element
// (orow<TM>(4 i + v), ocol(j)): wave w owns whole 16-row output tiles and
// keeps them in MFMA accumulator registers for the whole product.  A_KC:
// a(m, kk) is contiguous along kk in memory (else along m); B_NC: b(kk, n)
// is contiguous along n (else along kk); the slab fill follows the
// contiguous index.  Slab rows are 17 floats past a multiple of 32 apart, so
// the MFMA reads (16 consecutive elements of 4 consecutive rows) and the
// kk-fastest fills both spread over the banks.  Two slabs are in flight:
// slab k0 + 2 KT is read into registers while slab k0 is used, and the
// barriers order LDS only, so those loads stay in flight across them (a
// __syncthreads fence would wait for them at every slab).  K, always 64 or
// 128, is a multiple of 2 KT; a caller orders any global data it wrote
// before the call itself.  Contains barriers: every thread of the block
// calls it.
// NP products of one shape in a row through one slab pipeline: a(p, m, k)
// and b(p, k, n) give product p's operands, and after product p < NP - 1
// epi(p, ct) takes its result and ct starts again from zero (the last one is
// left in ct).  The two slabs in flight run on across product boundaries, so
// a product's first slabs are read while the previous one finishes.
template <int NP, int TM, int TN, bool A_KC, bool B_NC, typename FA, typename FB, typename FE>
__device__ __forceinline__ void gemm_staged2_seq(f32x4 (&ct)[TM / 4][TN], int K, float* stage,
                                                 FA a, FB b, FE epi) {
  constexpr int M = 16 * TM, N = 16 * TN;
  float* sa = stage;           // [M][SKP]
  float* sb = stage + M * SKP;  // [N][SKP]
  constexpr int QA = M * KT / 4 / NT, QB = N * KT / 4 / NT;  // quads a thread fills
  static_assert(TM % 4 == 0 && QA >= 1 && QB >= 1 && (M * KT) % (4 * NT) == 0 &&
                    (N * KT) % (4 * NT) == 0,
                "whole 16-row tiles per wave, whole quads per thread");
  const int t = threadIdx.x;
  // quad u of thread t: row m (column n) and contraction indices 4 q .. 4 q + 3,
  // the lanes running along the index that is contiguous in memory
  auto a_pos = [&](int u, int& m, int& q) {
    const int e = t + NT * u;
    m = A_KC ? e / (KT / 4) : e % M;
    q = A_KC ? e % (KT / 4) : e / M;
  };
  auto b_pos = [&](int u, int& n, int& q) {
    const int e = t + NT * u;
    n = B_NC ? e % N : e / (KT / 4);
    q = B_NC ? e / N : e % (KT / 4);
  };
  // A lambda that returns an f32x4 gives a whole quad at once: a(p, m, k) the
  // contraction indices k .. k + 3 of row m (b(p, k, n) those of column n).
  constexpr bool AQ = std::is_same_v<decltype(a(0, 0, 0)), f32x4>;
  constexpr bool BQ = std::is_same_v<decltype(b(0, 0, 0)), f32x4>;
  f32x4 ra[2][QA], rb[2][QB];
  auto fetch = [&](int g0, int sl) {  // slab at g0 of the products' joint contraction
    const int p = g0 / K, k0 = g0 - p * K;
#pragma unroll
    for (int u = 0; u < QA; ++u) {
      int m, q;
      a_pos(u, m, q);
      if constexpr (AQ) {
        ra[sl][u] = a(p, m, k0 + 4 * q);
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) ra[sl][u][s2] = a(p, m, k0 + 4 * q + s2);
      }
    }
#pragma unroll
    for (int u = 0; u < QB; ++u) {
      int n, q;
      b_pos(u, n, q);
      if constexpr (BQ) {
        rb[sl][u] = b(p, k0 + 4 * q, n);
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) rb[sl][u][s2] = b(p, k0 + 4 * q + s2, n);
      }
    }
  };
  constexpr int TR = TM / 4;
  const int KA = NP * K;
  fetch(0, 0);
  fetch(KT, 1);
  for (int g0 = 0; g0 < KA; g0 += 2 * KT) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
      for (int u = 0; u < QA; ++u) {
        int m, q;
        a_pos(u, m, q);
        *reinterpret_cast<f32x4*>(sa + m * SKP + 4 * q) = ra[sl][u];
      }
#pragma unroll
      for (int u = 0; u < QB; ++u) {
        int n, q;
        b_pos(u, n, q);
        *reinterpret_cast<f32x4*>(sb + n * SKP + 4 * q) = rb[sl][u];
      }
      barrier_lds();
      if (g0 + (2 + sl) * KT < KA) fetch(g0 + (2 + sl) * KT, sl);
      // sub-step s of lane group lq takes contraction index 4 lq + s: a
      // lane's four are one 16-byte read of each operand
      const int lane = t & 63, w = t >> 6, lr = lane & 15, lq = lane >> 4;
      f32x4 av[TR], bv[TN];
#pragma unroll
      for (int i = 0; i < TR; ++i)
        av[i] = *reinterpret_cast<const f32x4*>(sa + (16 * (TR * w + i) + lr) * SKP + 4 * lq);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bv[j] = *reinterpret_cast<const f32x4*>(sb + (16 * j + lr) * SKP + 4 * lq);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
        for (int i = 0; i < TR; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            ct[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i][s2], bv[j][s2], ct[i][j], 0, 0, 0);
      barrier_lds();
    }
    if constexpr (NP > 1) {
      const int g1 = g0 + 2 * KT;
      if (g1 < KA && g1 % K == 0) {
        epi(g1 / K - 1, ct);
#pragma unroll
        for (int i = 0; i < TR; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) ct[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  }
}
template <int TM, int TN, bool A_KC, bool B_NC, typename FA, typename FB>
__device__ __forceinline__ void gemm_staged2(f32x4 (&ct)[TM / 4][TN], int K, float* stage, FA a,
                                             FB b) {
  gemm_staged2_seq<1, TM, TN, A_KC, B_NC>(
      ct, K, stage, [&](int, int m, int k) { return a(m, k); },
      [&](int, int k, int n) { return b(k, n); }, [](int, f32x4(&)[TM / 4][TN]) {});
}

// Two products of one shape over one contraction, c_p += a(p) b(p) for p < 2,
// through one slab pipeline (the gemm_staged2 scheme with both products'
// slabs filled and read each step): each slab step does twice the MFMA work
// per barrier.  a(p, m, k) returns the quad k .. k + 3 of row m (A_KC), b(p,
// k, n) one element (B_NC).  hook(k0, sb0, sb1) runs once per slab, while
// the B slabs of contraction indices k0 .. k0 + KT - 1 are in LDS: element
// (k0 + kk, n) of operand p at sb_p[n SKP + kk].  Stage: 2 (M + N) SKP floats.
template <int TM, int TN, typename FA, typename FB, typename FH>
__device__ __forceinline__ void gemm_staged2_pair(f32x4 (&c0)[TM / 4][TN], f32x4 (&c1)[TM / 4][TN],
                                                  int K, float* stage, FA a, FB b, FH hook) {
  constexpr int M = 16 * TM, N = 16 * TN;
  float* sa0 = stage;
  float* sa1 = sa0 + M * SKP;
  float* sb0 = sa1 + M * SKP;
  float* sb1 = sb0 + N * SKP;
  constexpr int QA = M * KT / 4 / NT, QB = N * KT / 4 / NT;
  static_assert(TM % 4 == 0 && QA >= 1 && QB >= 1 && (M * KT) % (4 * NT) == 0 &&
                    (N * KT) % (4 * NT) == 0,
                "whole 16-row tiles per wave, whole quads per thread");
  const int t = threadIdx.x;
  // one slab in flight: a slab step is both products' MFMA work, as long as
  // two steps of a single product
  f32x4 ra[2][QA], rb[2][QB];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int u = 0; u < QA; ++u) {
        const int e = t + NT * u;
        ra[p][u] = a(p, e / (KT / 4), k0 + 4 * (e % (KT / 4)));
      }
#pragma unroll
      for (int u = 0; u < QB; ++u) {
        const int e = t + NT * u, n = e % N, q = e / N;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) rb[p][u][s2] = b(p, k0 + 4 * q + s2, n);
      }
    }
  };
  constexpr int TR = TM / 4;
  fetch(0);
  for (int k0 = 0; k0 < K; k0 += KT) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int u = 0; u < QA; ++u) {
        const int e = t + NT * u;
        *reinterpret_cast<f32x4*>((p ? sa1 : sa0) + (e / (KT / 4)) * SKP + 4 * (e % (KT / 4))) =
            ra[p][u];
      }
#pragma unroll
      for (int u = 0; u < QB; ++u) {
        const int e = t + NT * u;
        *reinterpret_cast<f32x4*>((p ? sb1 : sb0) + (e % N) * SKP + 4 * (e / N)) = rb[p][u];
      }
    }
    barrier_lds();
    if (k0 + KT < K) fetch(k0 + KT);
    const int lane = t & 63, w = t >> 6, lr = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float* xa = p ? sa1 : sa0;
      const float* xb = p ? sb1 : sb0;
      f32x4 av[TR], bv[TN];
#pragma unroll
      for (int i = 0; i < TR; ++i)
        av[i] = *reinterpret_cast<const f32x4*>(xa + (16 * (TR * w + i) + lr) * SKP + 4 * lq);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bv[j] = *reinterpret_cast<const f32x4*>(xb + (16 * j + lr) * SKP + 4 * lq);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
        for (int i = 0; i < TR; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            f32x4& c = p ? c1[i][j] : c0[i][j];
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i][s2], bv[j][s2], c, 0, 0, 0);
          }
    }
    hook(k0, static_cast<const float*>(sb0), static_cast<const float*>(sb1));
    barrier_lds();
  }
}

// gemm_staged2 with operands read 4 at a time: a4(m, k) returns a(m, k .. k+3)
// when A_KC (contiguous along k), else a(m .. m+3, k); b4(k, n) returns
// b(k, n .. n+3) when B_NC, else b(k .. k+3, n).  Index arguments are
// multiples of 4 along the vector's direction.
template <int TM, int TN, bool A_KC, bool B_NC, typename FA4, typename FB4>
__device__ __forceinline__ void gemm_staged2v(f32x4 (&ct)[TM / 4][TN], int K, float* stage, FA4 a4,
                                              FB4 b4) {
  constexpr int M = 16 * TM, N = 16 * TN, MS = M + 17, NS = N + 17;
  float* sa = stage;
  float* sb = stage + KT * MS;
  constexpr int PA4 = M * KT / NT / 4, PB4 = N * KT / NT / 4;
  static_assert(TM % 4 == 0 && PA4 >= 1 && PB4 >= 1 && (M * KT) % (4 * NT) == 0 &&
                    (N * KT) % (4 * NT) == 0,
                "whole 16-row tiles per wave, whole 4-vectors per thread");
  const int t = threadIdx.x;
  f32x4 ra[2][PA4], rb[2][PB4];
  auto a_pos = [&](int u, int& m, int& kt) {
    const int e = t + NT * u;
    m = A_KC ? e / (KT / 4) : 4 * (e % (M / 4));
    kt = A_KC ? 4 * (e % (KT / 4)) : e / (M / 4);
  };
  auto b_pos = [&](int u, int& n, int& kt) {
    const int e = t + NT * u;
    n = B_NC ? 4 * (e % (N / 4)) : e / (KT / 4);
    kt = B_NC ? e / (N / 4) : 4 * (e % (KT / 4));
  };
  auto fetch = [&](int k0, int sl) {
#pragma unroll
    for (int u = 0; u < PA4; ++u) {
      int m, kt;
      a_pos(u, m, kt);
      ra[sl][u] = a4(m, k0 + kt);
    }
#pragma unroll
    for (int u = 0; u < PB4; ++u) {
      int n, kt;
      b_pos(u, n, kt);
      rb[sl][u] = b4(k0 + kt, n);
    }
  };
  constexpr int TR = TM / 4;
  fetch(0, 0);
  fetch(KT, 1);
  for (int k0 = 0; k0 < K; k0 += 2 * KT) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
      for (int u = 0; u < PA4; ++u) {
        int m, kt;
        a_pos(u, m, kt);
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[(A_KC ? (kt + i) * MS + m : kt * MS + m + i)] = ra[sl][u][i];
      }
#pragma unroll
      for (int u = 0; u < PB4; ++u) {
        int n, kt;
        b_pos(u, n, kt);
#pragma unroll
        for (int i = 0; i < 4; ++i) sb[(B_NC ? kt * NS + n + i : (kt + i) * NS + n)] = rb[sl][u][i];
      }
      barrier_lds();
      if (k0 + (2 + sl) * KT < K) fetch(k0 + (2 + sl) * KT, sl);
      const int lane = t & 63, w = t >> 6, lr = lane & 15, lq = lane >> 4;
#pragma unroll
      for (int kg = 0; kg < KT / 4; ++kg) {
        const int kk = 4 * kg + lq;
        float av[TR], bv[TN];
#pragma unroll
        for (int i = 0; i < TR; ++i) av[i] = sa[kk * MS + 16 * (TR * w + i) + lr];
#pragma unroll
        for (int j = 0; j < TN; ++j) bv[j] = sb[kk * NS + 16 * j + lr];
#pragma unroll
        for (int i = 0; i < TR; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            ct[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[j], ct[i][j], 0, 0, 0);
      }
      barrier_lds();
    }
  }
}

// Output element of acc[i][j][v] after gemm_staged2<TM, TN>: row
// orow<TM>(4 i + v), column ocol(j).
template <int TM>
__device__ __forceinline__ int orow(int i) {
  const int t = threadIdx.x;
  return 16 * ((TM / 4) * (t >> 6) + (i >> 2)) + 4 * ((t & 63) >> 4) + (i & 3);
}
__device__ __forceinline__ int ocol(int j) { return 16 * j + (threadIdx.x & 15); }

template <int TR, int TN>
__device__ __forceinline__ void zero(f32x4 (&acc)[TR][TN]) {
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// Chunk c of sequence n: its packed index (bos / 64 + n + c) is unique and
// below T_tot / 64 + N.
struct ChunkPos {
  int n, c, h, Lc;
  int64_t t0, pair;
};
__device__ __forceinline__ bool chunk_of_block(const int32_t* cu, int N, int T_tot, int H,
                                               int maxnch, ChunkPos& p, int64_t b) {
  p.h = static_cast<int>(b % H);
  const int64_t rest = b / H;
  p.c = static_cast<int>(rest % maxnch);
  p.n = static_cast<int>(rest / maxnch);
  if (p.n >= N) return false;
  int64_t bos = cu[p.n], eos = cu[p.n + 1];
  bos = bos < 0 ? 0 : (bos > T_tot ? T_tot : bos);
  eos = eos < bos ? bos : (eos > T_tot ? T_tot : eos);
  const int64_t L = eos - bos;
  if ((int64_t)p.c * C >= L) return false;
  p.Lc = static_cast<int>(L - (int64_t)p.c * C < C ? L - (int64_t)p.c * C : C);
  p.t0 = bos + (int64_t)p.c * C;
  p.pair = (bos / C + p.n + p.c) * H + p.h;
  return true;
}

// The chunk's rows of one head of a token-major [T, H, 128] tensor as a
// buffer resource: rows at or past the chunk's end (and every row when the
// tensor is absent) read as 0.  Loads through it carry no branch: with a
// branch per element (r < Lc ? load : 0) every load waited alone, and the
// staged products' operand fetches ran one memory round trip per element.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rows(const void* base, int esz,
                                                             const ChunkPos& p, int64_t HD) {
  const char* b = base ? static_cast<const char*>(base) +
                             ((int64_t)p.t0 * HD + (int64_t)p.h * D) * esz
                       : nullptr;
  const int64_t n = (base && p.Lc > 0) ? ((int64_t)(p.Lc - 1) * HD + D) * esz : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(b), (short)0, (int)n, 0x00020000);
}
// elements (row r < 64, channels cc .. cc + 3) through chunk_rows, cc a
// multiple of 4; HDi = H * 128
template <bool BF16>
__device__ __forceinline__ f32x4 row4_at(__amdgpu_buffer_rsrc_t rs, int HDi, int r, int cc) {
  if constexpr (BF16) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (r * HDi + cc) * 2, 0, 0));
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                 __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
  } else {
    return __builtin_bit_cast(f32x4,
                              __builtin_amdgcn_raw_buffer_load_b128(rs, (r * HDi + cc) * 4, 0, 0));
  }
}
// element (row r < 64, channel cc) through chunk_rows
template <bool BF16>
__device__ __forceinline__ float row_at(__amdgpu_buffer_rsrc_t rs, int HDi, int r, int cc) {
  if constexpr (BF16)
    return bf16_bits_to_f32(static_cast<uint16_t>(
        __builtin_amdgcn_raw_buffer_load_b16(rs, (r * HDi + cc) * 2, 0, 0)));
  else
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (r * HDi + cc) * 4, 0, 0));
}

// At[r, s] = sum_c k_rc k_sc e^(gamma_rc - gamma_sc) (s < r) and P[r, s] =
// sum_c q_rc k_sc e^(...) (s <= r) as fp32 16x16x4 MFMA products over 16-row
// tiles, with the decay split into two factors taken relative to an anchor
// row a: (k_r e^(gamma_r - gamma_a)) (k_s e^(gamma_a - gamma_s)).
//  * Tile (i, j < i): a = 16 i - 1, the row before block i; both factors <= 1.
//  * Diagonal tile (i, i), by quadrants of 8 rows: the top-left and the
//    bottom-right ones take a = 16 i + 3 and 16 i + 11 (one product, each row
//    and column with the anchor of its own half), the bottom-left one
//    a = 16 i + 7 (factors <= 1, a second product); the top-right one lies
//    above the diagonal.  A factor then spans at most 4 tokens of decay,
//    below e^43 with the per-token decay floored (DECAY_FLOOR_NAT).  The
//    first product's mixed-anchor quadrants may overflow; they are dropped.
// MFMA lanes: lane (ln, lq) supplies A[ln][lq] (row ln of the tile, channel
// ch) and B[lq][ln] (channel ch, column ln), and holds D[4 lq + v][ln].
struct AtpDiag {
  f32x4 a1, p1, a3, p3;  // first product (same-half quadrants), second (bottom-left)
};
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
constexpr int ATP_LD = 17;  // row stride of the K / Q / gamma slabs (16 channels + 1)
constexpr int ATP_GL = 2 * C + 2;  // row stride of gamma in LDS (all 128 channels)
__device__ __forceinline__ void atp_diag(AtpDiag& d, int i, const float* sK, const float* sQ,
                                         const float* sG, int ch, int ln) {
  const int r = 16 * i + ln;
  const float kr = sK[r * ATP_LD + ch], qr = sQ[r * ATP_LD + ch], gr = sG[r * ATP_GL + ch];
  const float ga = sG[(16 * i + (ln < 8 ? 3 : 11)) * ATP_GL + ch];
  const float e1 = __expf(gr - ga), b1 = kr * __expf(ga - gr);
  d.a1 = mfma4(kr * e1, b1, d.a1);
  d.p1 = mfma4(qr * e1, b1, d.p1);
  const float g7 = sG[(16 * i + 7) * ATP_GL + ch];
  const bool lower = ln >= 8;  // row of the bottom half (A) / column of the top half (B)
  const float e3 = __expf(lower ? gr - g7 : g7 - gr);
  const float ka = lower ? kr * e3 : 0.0f, qa = lower ? qr * e3 : 0.0f;
  const float kb = lower ? 0.0f : kr * e3;
  d.a3 = mfma4(ka, kb, d.a3);
  d.p3 = mfma4(qa, kb, d.p3);
}
// tiles (i, j) for j < n into slots SLOT0 + j (n <= 3 - SLOT0)
template <int SLOT0>
__device__ __forceinline__ void atp_off(f32x4 (&oa)[3], f32x4 (&op)[3], int i, int n,
                                        const float* sK, const float* sQ, const float* sG,
                                        int ch, int ln) {
  if (i == 0) return;
  const int r = 16 * i + ln;
  const float gb = sG[(16 * i - 1) * ATP_GL + ch];
  const float eo = __expf(sG[r * ATP_GL + ch] - gb);
  const float ka = sK[r * ATP_LD + ch] * eo, qa = sQ[r * ATP_LD + ch] * eo;
#pragma unroll
  for (int j = 0; j < 3 - SLOT0; ++j) {
    if (j < n) {
      const int s = 16 * j + ln;
      const float kb = sK[s * ATP_LD + ch] * __expf(gb - sG[s * ATP_GL + ch]);
      oa[SLOT0 + j] = mfma4(ka, kb, oa[SLOT0 + j]);
      op[SLOT0 + j] = mfma4(qa, kb, op[SLOT0 + j]);
    }
  }
}
// store (add = false) or add and finish (add = true) one wave's share of a tile
__device__ __forceinline__ void atp_put_diag(const AtpDiag& d, int i, float (*sA)[C + 1],
                                             float (*sP)[C + 1], int ln, int lq, bool add) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rr = 4 * lq + v, r = 16 * i + rr, s = 16 * i + ln;
    const bool bl = rr >= 8 && ln < 8;
    float a = bl ? d.a3[v] : d.a1[v], p = bl ? d.p3[v] : d.p1[v];
    if (add) {
      a = ln < rr ? a + sA[r][s] : 0.0f;
      p = ln <= rr ? p + sP[r][s] : 0.0f;
    }
    sA[r][s] = a;
    sP[r][s] = p;
  }
}
__device__ __forceinline__ void atp_put_off(f32x4 a, f32x4 p, int i, int j, float (*sA)[C + 1],
                                            float (*sP)[C + 1], int ln, int lq, bool add) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 16 * i + 4 * lq + v, s = 16 * j + ln;
    sA[r][s] = add ? a[v] + sA[r][s] : a[v];
    sP[r][s] = add ? p[v] + sP[r][s] : p[v];
  }
}

template <bool QB>
__global__ void __launch_bounds__(NT, 3) bwd_prep_kernel(const void* __restrict__ q,
                                                         const void* __restrict__ k,
                                                         const void* __restrict__ v,
                                                         const float* __restrict__ g,
                                                         const float* __restrict__ beta,
                                                         const int32_t* __restrict__ cu, int N,
                                                         int T_tot, int H, int maxnch,
                                                         float scale, float* __restrict__ img) {
  constexpr int CS = 16;  // channels per slab of the At / P sums
  // At, P and M (three workgroups per CU); the At / P phase keeps gamma (all
  // channels) where At and P go later and its slabs of K and Q where M goes
  // later, the products after M stage through At's place
  constexpr int SLAB = C * (CS + 1);
  __shared__ __attribute__((aligned(16))) float sPool[3 * C * (C + 1)];
  __shared__ float sB[C];
  static_assert(2 * SLAB <= C * (C + 1) && STAGE_FLOATS <= C * (C + 1), "slabs fit");
  static_assert(C * ATP_GL <= 2 * C * (C + 1), "gamma fits in At's and P's place");
  static_assert(2 * (C + D) * SKP <= 2 * C * (C + 1), "paired slabs fit in At's and P's place");
  float(*sA)[C + 1] = reinterpret_cast<float(*)[C + 1]>(sPool);
  float(*sP)[C + 1] = reinterpret_cast<float(*)[C + 1]>(sPool + C * (C + 1));
  float(*sM)[C + 1] = reinterpret_cast<float(*)[C + 1]>(sPool + 2 * C * (C + 1));
  float* sS = sPool + 2 * C * (C + 1);  // the At / P slabs (over M)
  float* sGam = sPool;                  // gamma [C][ATP_GL] until At and P are stored
  ChunkPos p;
  if (!chunk_of_block(cu, N, T_tot, H, maxnch, p, blockIdx.x)) return;
  const int t = threadIdx.x;
  const int64_t HD = (int64_t)H * D;
  float* im = img + p.pair * Rec::floats;
  const int HDi = static_cast<int>(HD);
  const auto rk = chunk_rows(k, QB ? 2 : 4, p, HD), rq = chunk_rows(q, QB ? 2 : 4, p, HD),
             rv = chunk_rows(v, QB ? 2 : 4, p, HD), rg = chunk_rows(g, 4, p, HD);
  if (t < C) sB[t] = t < p.Lc ? beta[(p.t0 + t) * H + p.h] : 0.0f;
  if (t < D) {  // gamma: running sum of the floored g down channel t (rows past the end repeat the last)
    float gv[C];
#pragma unroll
    for (int r = 0; r < C; ++r) gv[r] = row_at<false>(rg, HDi, r, t);
    float run = 0.0f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      run += floor_decay(gv[r]);
      im[Rec::G + r * D + t] = run;
      sGam[r * ATP_GL + t] = run;
    }
  }
  __syncthreads();
  auto Gf = [&](int r, int cc) { return im[Rec::G + r * D + cc]; };
  {  // At and P (see atp_diag / atp_off): wave w sums the channels of half
     // w >> 1 for the row blocks {0, 3} (w even) or {1, 2} (w odd), 14
     // products per 4 channels either way.  Slab sl holds the channels
     // 8 sl .. 8 sl + 7 (columns 0..7) and 64 + 8 sl .. 64 + 8 sl + 7 (8..15),
     // so slab column ch of half hf is channel ch + 56 hf + 8 sl of gamma.
    float* sK = sS;
    float* sQ = sS + SLAB;
    const int l = t & 63, w = t >> 6, ln = l & 15, lq = l >> 4, hf = w >> 1;
    const int bA = w & 1, bB = 3 - bA;
    AtpDiag dA{}, dB{};
    f32x4 oa[3] = {}, op[3] = {};
    // thread t reads row t / 4, slab columns 4 (t % 4) .. + 3 (4 contiguous channels)
    static_assert(C * CS == 4 * NT, "one 4-channel group a thread");
    const int fr = t >> 2, fc = 4 * (t & 3);
    f32x4 rk4, rq4;
    auto fetch_slab = [&](int sl) {
      const int cc = fc < 8 ? 8 * sl + fc : 64 + 8 * sl + fc - 8;
      rk4 = row4_at<QB>(rk, HDi, fr, cc);
      rq4 = row4_at<QB>(rq, HDi, fr, cc);
    };
    fetch_slab(0);
    for (int sl = 0; sl < D / CS; ++sl) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sK[fr * (CS + 1) + fc + i] = rk4[i];
        sQ[fr * (CS + 1) + fc + i] = rq4[i];
      }
      barrier_lds();
      if (sl + 1 < D / CS) fetch_slab(sl + 1);
      const float* sG = sGam + 56 * hf + 8 * sl;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ch = 8 * hf + 4 * kk + lq;
        atp_diag(dA, bA, sK, sQ, sG, ch, ln);
        atp_diag(dB, bB, sK, sQ, sG, ch, ln);
        // tiles (bB, j < bB) in slots j; tile (1, 0) of the pair {1, 2} in slot 2
        atp_off<0>(oa, op, bB, bB, sK, sQ, sG, ch, ln);
        if (bA == 1) atp_off<2>(oa, op, 1, 1, sK, sQ, sG, ch, ln);
      }
      barrier_lds();
    }
    // gamma is read for the last time above: the tiles above the diagonal
    // (never summed) take zeros, the others are stored below
    for (int e = t; e < C * (C + 1); e += NT) {
      const int r = e / (C + 1), s2 = e % (C + 1);
      if (s2 / 16 > r / 16) {
        (&sA[0][0])[e] = 0.0f;
        (&sP[0][0])[e] = 0.0f;
      }
    }
    // the second channel half stores its sums, the first adds its own and
    // masks the diagonal tiles
    for (int pass = 1; pass >= 0; --pass) {
      if (hf == pass) {
        atp_put_diag(dA, bA, sA, sP, ln, lq, pass == 0);
        atp_put_diag(dB, bB, sA, sP, ln, lq, pass == 0);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int ti = j < bB ? bB : 1, tj = j < bB ? j : 0;
          if (j < bB || bA == 1) atp_put_off(oa[j], op[j], ti, tj, sA, sP, ln, lq, pass == 0);
        }
      }
      barrier_lds();
    }
    for (int e = t; e < C * C / 4; e += NT) {  // 4 columns a thread
      const int r = e / (C / 4), s4 = 4 * (e % (C / 4));
      *reinterpret_cast<f32x4*>(im + Rec::AT + r * C + s4) =
          f32x4{sA[r][s4], sA[r][s4 + 1], sA[r][s4 + 2], sA[r][s4 + 3]};
      *reinterpret_cast<f32x4*>(im + Rec::P + r * C + s4) =
          f32x4{sP[r][s4], sP[r][s4 + 1], sP[r][s4 + 2], sP[r][s4 + 3]};
    }
  }
  __syncthreads();
  // M = (I + A)^-1, A = diag(b) At strictly lower, by 16-row blocks on fp32
  // MFMA: the diagonal blocks M_ii = (I - N)(I + N^2)(I + N^4)(I + N^8) with
  // N = A_ii (nilpotent, N^16 = 0), then block column j on wave j by forward
  // substitution, M_ij = -M_ii sum_{k=j}^{i-1} A_ik M_kj.  P's LDS copy is
  // free from here (the Qt product reads P from the record): it holds each
  // wave's 16 x 16 intermediates.
  {
    const int l = t & 63, w = t >> 6, lr = l & 15, lq = l >> 4;
    float* scr = &sP[0][0] + w * 1024;  // four 16 x 16 matrices per wave
    float* X2 = scr;
    float* X4 = scr + 256;
    float* X8 = scr + 512;
    float* Q = scr + 768;
    // acc += X Y over 16 x 16 x 16; X (m, k) at x[m xs + k] times xrow[m],
    // Y (k, n) at y[k ys + n] times yrow[k] (1 when the pointers are null)
    auto mm16 = [&](const float* x, int xs, const float* xrow, const float* y, int ys,
                    const float* yrow, f32x4 acc) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int k = 4 * kk + lq;
        const float a = x[lr * xs + k] * (xrow ? xrow[lr] : 1.0f);
        const float b = y[k * ys + lr] * (yrow ? yrow[k] : 1.0f);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
      }
      return acc;
    };
    auto put16 = [&](float* d, int ds, f32x4 v, float sgn) {
#pragma unroll
      for (int i = 0; i < 4; ++i) d[(4 * lq + i) * ds + lr] = sgn * v[i];
    };
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    {  // the diagonal block of row block w
      const int b0 = 16 * w;
      const float* N = &sA[b0][b0];
      const float* bw = sB + b0;
      put16(X2, 16, mm16(N, C + 1, bw, N, C + 1, bw, z4), 1.0f);
      put16(X4, 16, mm16(X2, 16, nullptr, X2, 16, nullptr, z4), 1.0f);
      put16(X8, 16, mm16(X4, 16, nullptr, X4, 16, nullptr, z4), 1.0f);
      f32x4 q;  // I - N in the accumulator layout: element (4 lq + i, lr)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * lq + i;
        q[i] = (r == lr ? 1.0f : 0.0f) - bw[r] * N[r * (C + 1) + lr];
      }
      put16(Q, 16, q, 1.0f);
      q = mm16(Q, 16, nullptr, X2, 16, nullptr, q);  // (I - N)(I + N^2)
      put16(Q, 16, q, 1.0f);
      q = mm16(Q, 16, nullptr, X4, 16, nullptr, q);  // ... (I + N^4)
      put16(Q, 16, q, 1.0f);
      q = mm16(Q, 16, nullptr, X8, 16, nullptr, q);  // ... (I + N^8)
      put16(&sM[b0][b0], C + 1, q, 1.0f);
      for (int j = w + 1; j < 4; ++j) put16(&sM[b0][16 * j], C + 1, z4, 1.0f);
    }
    __syncthreads();
    // block column j = w: rows i = j + 1 .. 3 in order
    for (int i = w + 1; i < 4; ++i) {
      f32x4 acc = z4;
      for (int k = w; k < i; ++k)
        acc = mm16(&sA[16 * i][16 * k], C + 1, sB + 16 * i, &sM[16 * k][16 * w], C + 1, nullptr,
                   acc);
      put16(Q, 16, acc, 1.0f);
      put16(&sM[16 * i][16 * w], C + 1,
            mm16(&sM[16 * i][16 * i], C + 1, nullptr, Q, 16, nullptr, z4), -1.0f);
    }
  }
  __syncthreads();
  for (int e = t; e < C * C / 4; e += NT) {
    const int r = e / (C / 4), s4 = 4 * (e % (C / 4));
    *reinterpret_cast<f32x4*>(im + Rec::M + r * C + s4) =
        f32x4{sM[r][s4], sM[r][s4 + 1], sM[r][s4 + 2], sM[r][s4 + 3]};
  }
  float* sa = sPool;  // the products' slabs, over At (read for the last time above)
  {  // W = M diag(b) K_E; the operand fetch, which reads each K and gamma
     // element once, also writes K_D = K e^(gamma_C - gamma) to the record
    f32x4 acc[1][8];
    zero(acc);
    gemm_staged2v<4, 8, true, true>(
        acc, C, sa,
        [&](int r, int s2) { return f32x4{sM[r][s2], sM[r][s2 + 1], sM[r][s2 + 2], sM[r][s2 + 3]}; },
        [&](int s2, int cc) {
          const f32x4 kv = row4_at<QB>(rk, HDi, s2, cc);
          const f32x4 gv = *reinterpret_cast<const f32x4*>(im + Rec::G + s2 * D + cc);
          const f32x4 gl = *reinterpret_cast<const f32x4*>(im + Rec::G + (C - 1) * D + cc);
          *reinterpret_cast<f32x4*>(im + Rec::KD + s2 * D + cc) =
              f32x4{kv[0] * __expf(gl[0] - gv[0]), kv[1] * __expf(gl[1] - gv[1]),
                    kv[2] * __expf(gl[2] - gv[2]), kv[3] * __expf(gl[3] - gv[3])};
          const float b = sB[s2];
          return f32x4{b * kv[0] * __expf(gv[0]), b * kv[1] * __expf(gv[1]),
                       b * kv[2] * __expf(gv[2]), b * kv[3] * __expf(gv[3])};
        });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) im[Rec::W + orow<4>(i) * D + ocol(j)] = acc[0][j][i];
  }
  __syncthreads();  // W complete
  {  // U = M diag(b) V and Qt = scale (Q_E - P W) in one pipeline; Qt's
     // accumulator starts at -Q_E (its reads overlap the product's)
    f32x4 acc[1][8], aq[1][8];
    zero(acc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = orow<4>(i), cc = ocol(j);
        aq[0][j][i] = -row_at<QB>(rq, HDi, r, cc) * __expf(Gf(r, cc));
      }
    gemm_staged2_pair<4, 8>(
        acc, aq, C, sa,
        [&](int p2, int r, int s2) {
          if (p2 == 0) return f32x4{sM[r][s2], sM[r][s2 + 1], sM[r][s2 + 2], sM[r][s2 + 3]};
          return *reinterpret_cast<const f32x4*>(im + Rec::P + r * C + s2);
        },
        [&](int p2, int s2, int j) {
          return p2 == 0 ? sB[s2] * row_at<QB>(rv, HDi, s2, j) : im[Rec::W + s2 * D + j];
        },
        [](int, const float*, const float*) {});
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        im[Rec::U + orow<4>(i) * D + ocol(j)] = acc[0][j][i];
        im[Rec::QT + orow<4>(i) * D + ocol(j)] = -scale * aq[0][j][i];
      }
  }
  if (t < D) im[Rec::EC + t] = __expf(Gf(C - 1, t));
}

// One chunk walk of a (sequence, head, 64-column tile).  Lane (lr, lq) of
// wave w holds R[32 w + 16 i + 4 lq + v][16 j + lr] of the tile in R[i][j][v]
// (i < 2, j < 4), the 16x16 MFMA accumulator layout.
// Forward (FWD): R = S from the initial state; rec[chunk] = R at the chunk's
// entry.  Backward: R = dS from dS_final; rec[chunk] = R at the chunk's end,
// R_end gets the gradient of the initial state.
// A chunk step is Z = A1 R (A1 = W forward, K_D backward; 16 rows of Z per
// wave), then R <- e^gamma_C R + K_D^T (U - Z) forward, or e^gamma_C R -
// W^T Z + Qt^T dO backward (dO the tile's columns of d_o).  The MFMA A
// operands come straight from the chunk record into registers, one product
// ahead of their use: rows of A1 16 or 32 bytes a lane (the contraction
// index of lane group lq and sub-step s is 16 u + 4 lq + s on the fp32 MFMA,
// 32 g + 8 lq + s on the bf16 one, and the B operand is read in that order),
// the transposed operands one float a lane (16 lanes on 64 contiguous
// bytes).  The B operands sit transposed in LDS, so the contraction indices
// a lane needs are one 16-byte read.  Two barriers per chunk step.
// The products run on the bf16 16x16x32 MFMA with three-term splits: x = hi
// + mid + lo in bf16 carries the 24 bits of an fp32 x, a product of two
// such sums is the six bf16 products whose terms reach 2^-16 of the leading
// one (the three left out are below 2^-24 of it), and bf16 products are
// exact in the fp32 accumulator, so the result is the fp32 product up to
// fp32 rounding at three eighths of the fp32 MFMA cycles.  The state update
// always does so; Z = A1 R does so with bf16 d_o (R as three bf16 planes in
// LDS), and with fp32 d_o, whose tile takes the LDS those planes would
// need, stays on the fp32 16x16x4 MFMA.  With bf16 d_o, Qt^T dO takes dO as
// is (three products); with fp32 d_o it stays on the fp32 MFMA.
constexpr int WTS = 2 * C + 4;  // row stride of the transposed fp32 tile: 4 WTS = 16 (mod 64 banks)
constexpr int DTS = C + 8;      // the bf16 tiles': 16-lane reads of 16 bytes land on distinct banks
constexpr int FTS = C + 4;      // the fp32 d_o tile's
// With bf16 d_o the walk also runs Z = A1 R on split-bf16 products, with R
// as three bf16 planes; its three bf16 tiles then fit two workgroups per CU
// (80 KB) only unpadded, with the 16-byte groups of a row XOR-swizzled so
// that the 16 lanes of a read (rows 16 j + l, one group each) still hit
// distinct banks.  Offsets in bf16 elements:
//   R planes [3][64][128]: group g of row r at g ^ (r % 16);
//   Z planes [3][64][64] and d_o [64][64]: group g of row r at g ^ (r / 2 % 8).
__device__ __forceinline__ int rp_off(int p, int r, int k) {
  return (p * 64 + r) * 128 + ((((k >> 3) ^ (r & 15))) << 3) + (k & 7);
}
__device__ __forceinline__ int zp_off(int p, int r, int k) {
  return (p * 64 + r) * 64 + ((((k >> 3) ^ ((r >> 1) & 7))) << 3) + (k & 7);
}
__device__ __forceinline__ void split3(const chunk::f32x8& x, bf16x8& hi, bf16x8& mi, bf16x8& lo) {
  hi = __builtin_convertvector(x, bf16x8);
  const chunk::f32x8 r = x - __builtin_convertvector(hi, chunk::f32x8);
  mi = __builtin_convertvector(r, bf16x8);
  lo = __builtin_convertvector(r - __builtin_convertvector(mi, chunk::f32x8), bf16x8);
}
__device__ __forceinline__ void split3(const f32x4& x, bf16x4& hi, bf16x4& mi, bf16x4& lo) {
  hi = __builtin_convertvector(x, bf16x4);
  const f32x4 r = x - __builtin_convertvector(hi, f32x4);
  mi = __builtin_convertvector(r, bf16x4);
  lo = __builtin_convertvector(r - __builtin_convertvector(mi, f32x4), bf16x4);
}
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
template <bool FWD, bool DOB>
__device__ __forceinline__ void walk_dir(const float* __restrict__ img, const void* d_o,
                                         int64_t bos, int64_t L, int n, int h, int tile, int H,
                                         const float* __restrict__ R_init,
                                         float* __restrict__ rec, float* __restrict__ R_end,
                                         void* sR, void* sZ, void* sDo) {
  // ZB: Z = A1 R on split-bf16 products (bf16 d_o), else on the fp32 MFMA
  constexpr bool ZB = DOB;
  float(*sRt)[WTS] = reinterpret_cast<float(*)[WTS]>(sR);  // fp32 R^T (not ZB)
  uint16_t* sRp = reinterpret_cast<uint16_t*>(sR);          // R planes (ZB)
  uint16_t* sZp = reinterpret_cast<uint16_t*>(sZ);
  // element (p, r, k) of the Z planes; d_o (bf16) is plane 0 of its own tile
  auto zo = [](int p, int r, int k) { return ZB ? zp_off(p, r, k) : (p * 64 + r) * DTS + k; };
  const int nch = static_cast<int>((L + C - 1) / C);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, lr = lane & 15, lq = lane >> 4;
  const int64_t HD = (int64_t)H * D;
  const int HDi = static_cast<int>(HD);
  const int64_t sbase = ((int64_t)n * H + h) * D * D + 64 * tile;
  auto rrow = [&](int i, int v) { return 32 * w + 16 * i + 4 * lq + v; };
  f32x4 R[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        R[i][j][v] = R_init ? R_init[sbase + (int64_t)rrow(i, v) * D + 16 * j + lr] : 0.0f;
  auto pair_of = [&](int it) {
    const int c = FWD ? it : nch - 1 - it;
    return (bos / C + n + c) * H + h;
  };
  // Record reads through a buffer resource: the lane's part of the offset in
  // one register, the rest a constant, so the many operand loads share it.
  auto rec_buf = [&](int64_t pair) {
    return chunk::make_buf(img + pair * Rec::floats, Rec::floats * 4);
  };
  auto ld1 = [](__amdgpu_buffer_rsrc_t rs, int vo, int so) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vo, so, 0));
  };
  constexpr int A1 = FWD ? Rec::W : Rec::KD;
  // A1 rows 16 w + lr; fp32 MFMA: zA[u] the contraction 16 u + 4 lq .. + 3;
  // ZB: zA[2 g + e] the contraction 32 g + 8 lq + 4 e .. + 3
  f32x4 zA[8];
  const int vo_zA = ((16 * w + lr) * D + (ZB ? 8 : 4) * lq) * 4;
  auto load_zA = [&](__amdgpu_buffer_rsrc_t rs) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      zA[u] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rs, vo_zA, (A1 + (ZB ? 32 * (u >> 1) + 4 * (u & 1) : 16 * u)) * 4, 0));
  };
  if (nch > 0) load_zA(rec_buf(pair_of(0)));
  // the transposed update operand: K_D forward, W backward, as bf16 A
  // fragments (row 32 w + 16 i + lr, contraction 32 g + 8 lq + e)
  constexpr int A2 = FWD ? Rec::KD : Rec::W;
  const int vo_a = (8 * lq * D + 32 * w + lr) * 4;
  for (int it = 0; it < nch; ++it) {
    const int c = FWD ? it : nch - 1 - it;
    const int64_t pair = pair_of(it);
    const auto rs = rec_buf(pair);
    float* rc = rec + pair * (int64_t)(D * D) + 64 * tile;
    // (1) R into the record and, transposed, into LDS
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int v = 0; v < 4; ++v) rc[rrow(i, v) * D + 16 * j + lr] = R[i][j][v];
        if constexpr (ZB) {
          bf16x4 ph, pm, pl;
          split3(R[i][j], ph, pm, pl);
          *reinterpret_cast<bf16x4*>(sRp + rp_off(0, 16 * j + lr, rrow(i, 0))) = ph;
          *reinterpret_cast<bf16x4*>(sRp + rp_off(1, 16 * j + lr, rrow(i, 0))) = pm;
          *reinterpret_cast<bf16x4*>(sRp + rp_off(2, 16 * j + lr, rrow(i, 0))) = pl;
        } else {
          *reinterpret_cast<f32x4*>(&sRt[16 * j + lr][rrow(i, 0)]) = R[i][j];
        }
      }
    // the state update's operands, in flight during Z = A1 R
    float a2[2][2][8];  // [g][i][e]
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) a2[g][i][e] = ld1(rs, vo_a, (A2 + (32 * g + e) * D + 16 * i) * 4);
    // Qt^T dO: bf16 A fragments (like a2) with bf16 d_o, fp32 16x16x4 ones
    // (contraction 16 u + 4 lq + s) with fp32 d_o
    float qa[2][2][8];
    float qf[4][4][2];
    if constexpr (!FWD) {
      if constexpr (DOB) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              qa[g][i][e] = ld1(rs, vo_a, (Rec::QT + (32 * g + e) * D + 16 * i) * 4);
      } else {
        const int vo_q = (4 * lq * D + 32 * w + lr) * 4;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 2; ++i)
              qf[u][s][i] = ld1(rs, vo_q, (Rec::QT + (16 * u + s) * D + 16 * i) * 4);
      }
    }
    float ec[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        ec[i][v] = ld1(rs, (32 * w + 4 * lq) * 4, (Rec::EC + 16 * i + v) * 4);
    u32x4 draw[2];  // bf16 d_o row `lane`, columns 16 w .. + 15, as stored
    f32x4 ext[4];   // forward: U at Z's elements; fp32 d_o: that row segment
    if constexpr (FWD) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          ext[j][v] = ld1(rs, ((16 * w + 4 * lq) * D + 64 * tile + lr) * 4,
                          (Rec::U + v * D + 16 * j) * 4);
    } else {
      ChunkPos cp;
      cp.t0 = bos + (int64_t)c * C;
      cp.h = h;
      cp.Lc = static_cast<int>(L - (int64_t)c * C < C ? L - (int64_t)c * C : C);
      const auto rdo = chunk_rows(d_o, DOB ? 2 : 4, cp, HD);
      const int off = lane * HDi + 64 * tile + 16 * w;
      if constexpr (DOB) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          draw[hh] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(rdo, (off + 8 * hh) * 2, 0, 0));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ext[e] = __builtin_bit_cast(
              f32x4, __builtin_amdgcn_raw_buffer_load_b128(rdo, (off + 4 * e) * 4, 0, 0));
      }
    }
    barrier_lds();
    // (2) Z = A1 R, rows 16 w .. + 15 of the chunk
    f32x4 z[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (ZB) {  // six split products per contraction step of 32
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x8 ah, am, al;
        split3(__builtin_shufflevector(zA[2 * g], zA[2 * g + 1], 0, 1, 2, 3, 4, 5, 6, 7), ah, am,
               al);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * j + lr, k = 32 * g + 8 * lq;
          const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(sRp + rp_off(0, r, k));
          const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(sRp + rp_off(1, r, k));
          const bf16x8 b2 = *reinterpret_cast<const bf16x8*>(sRp + rp_off(2, r, k));
          z[j] = mfma_bf16(am, b1, z[j]);
          z[j] = mfma_bf16(al, b0, z[j]);
          z[j] = mfma_bf16(ah, b2, z[j]);
          z[j] = mfma_bf16(am, b0, z[j]);
          z[j] = mfma_bf16(ah, b1, z[j]);
          z[j] = mfma_bf16(ah, b0, z[j]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 b = *reinterpret_cast<const f32x4*>(&sRt[16 * j + lr][16 * u + 4 * lq]);
#pragma unroll
          for (int s = 0; s < 4; ++s)
            z[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(zA[u][s], b[s], z[j], 0, 0, 0);
        }
    }
    if (it + 1 < nch) load_zA(rec_buf(pair_of(it + 1)));
    // (3) U - Z (forward) or -Z (backward) as three bf16 planes, transposed,
    // and d_o, into LDS
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 ph, pm, pl;
      split3(FWD ? ext[j] - z[j] : -z[j], ph, pm, pl);
      *reinterpret_cast<bf16x4*>(sZp + zo(0, 16 * j + lr, 16 * w + 4 * lq)) = ph;
      *reinterpret_cast<bf16x4*>(sZp + zo(1, 16 * j + lr, 16 * w + 4 * lq)) = pm;
      *reinterpret_cast<bf16x4*>(sZp + zo(2, 16 * j + lr, 16 * w + 4 * lq)) = pl;
    }
    if constexpr (!FWD) {
      if constexpr (DOB) {
        uint16_t* sDt = reinterpret_cast<uint16_t*>(sDo);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          sDt[zo(0, 16 * w + e, lane)] =
              static_cast<uint16_t>(draw[e >> 3][(e & 7) >> 1] >> (16 * (e & 1)));
      } else {
        float(*sDf)[FTS] = reinterpret_cast<float(*)[FTS]>(sDo);
#pragma unroll
        for (int e = 0; e < 16; ++e) sDf[16 * w + e][lane] = ext[e >> 2][e & 3];
      }
    }
    barrier_lds();
    // (4) the state update
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) R[i][j][v] *= ec[i][v];
#pragma unroll
    for (int g = 0; g < 2; ++g) {  // + A2^T (U - Z) or A2^T (-Z), contraction 32 g + 8 lq + e
      bf16x8 bz[3][4];
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bz[p][j] = *reinterpret_cast<const bf16x8*>(sZp + zo(p, 16 * j + lr, 32 * g + 8 * lq));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        bf16x8 ah, am, al;
        split3(chunk::f32x8_of(a2[g][i]), ah, am, al);
#pragma unroll
        for (int j = 0; j < 4; ++j) R[i][j] = mfma_bf16(am, bz[1][j], R[i][j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) R[i][j] = mfma_bf16(al, bz[0][j], R[i][j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) R[i][j] = mfma_bf16(ah, bz[2][j], R[i][j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) R[i][j] = mfma_bf16(am, bz[0][j], R[i][j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) R[i][j] = mfma_bf16(ah, bz[1][j], R[i][j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) R[i][j] = mfma_bf16(ah, bz[0][j], R[i][j]);
      }
    }
    if constexpr (!FWD && DOB) {  // + Qt^T dO, dO exact in bf16
      const uint16_t* sDt = reinterpret_cast<const uint16_t*>(sDo);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        bf16x8 bo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bo[j] = *reinterpret_cast<const bf16x8*>(sDt + zo(0, 16 * j + lr, 32 * g + 8 * lq));
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          bf16x8 qh, qm, ql;
          split3(chunk::f32x8_of(qa[g][i]), qh, qm, ql);
#pragma unroll
          for (int j = 0; j < 4; ++j) R[i][j] = mfma_bf16(ql, bo[j], R[i][j]);
#pragma unroll
          for (int j = 0; j < 4; ++j) R[i][j] = mfma_bf16(qm, bo[j], R[i][j]);
#pragma unroll
          for (int j = 0; j < 4; ++j) R[i][j] = mfma_bf16(qh, bo[j], R[i][j]);
        }
      }
    } else if constexpr (!FWD) {  // + Qt^T dO on the fp32 MFMA
      float(*sDf)[FTS] = reinterpret_cast<float(*)[FTS]>(sDo);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 b = *reinterpret_cast<const f32x4*>(&sDf[16 * j + lr][16 * u + 4 * lq]);
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 2; ++i)
              R[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(qf[u][s][i], b[s], R[i][j], 0, 0, 0);
        }
    }
  }
  if (R_end) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          R_end[sbase + (int64_t)rrow(i, v) * D + 16 * j + lr] = R[i][j][v];
  }
}

// Both chunk walks in one launch: block b < nb walks forward (when both run),
// the others backward; one (sequence, head, 64-column tile) each.  Forward:
// rec_f[chunk] = S at the chunk's entry; backward: rec_b[chunk] = dS at the
// chunk's end, dS0 = the initial state's gradient.
template <bool DOB>
__global__ void __launch_bounds__(NT, 2) bwd_walk_kernel(
    const float* __restrict__ img, const void* __restrict__ d_o,
    const int32_t* __restrict__ cu, int N, int T_tot, int H, int both,
    const float* __restrict__ S0, float* __restrict__ rec_f, const float* __restrict__ dSf,
    float* __restrict__ dS0, float* __restrict__ rec_b) {
  // R transposed: three bf16 planes (bf16 d_o) or fp32 [64][WTS]; the
  // update's B operand as three bf16 planes; d_o of the chunk's tile,
  // transposed, bf16 or fp32 [64][FTS] (walk_dir gives the layouts)
  constexpr int R_BYTES = DOB ? 3 * 64 * 128 * 2 : 64 * WTS * 4;
  constexpr int Z_BYTES = DOB ? 3 * 64 * 64 * 2 : 3 * 64 * DTS * 2;
  constexpr int DO_BYTES = DOB ? 64 * 64 * 2 : 64 * FTS * 4;
  static_assert(R_BYTES + Z_BYTES + DO_BYTES <= 80 * 1024, "two workgroups per CU");
  __shared__ __attribute__((aligned(16))) unsigned char sR[R_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char sZ[Z_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char sDo[DO_BYTES];
  const int64_t nb = (int64_t)N * H * 2;
  int64_t b = blockIdx.x;
  const bool fwd = both && b < nb;
  if (both && !fwd) b -= nb;
  const int tile = static_cast<int>(b & 1);
  const int h = static_cast<int>((b >> 1) % H);
  const int n = static_cast<int>((b >> 1) / H);
  if (n >= N) return;
  int64_t bos = cu[n], eos = cu[n + 1];
  bos = bos < 0 ? 0 : (bos > T_tot ? T_tot : bos);
  eos = eos < bos ? bos : (eos > T_tot ? T_tot : eos);
  const int64_t L = eos - bos;
  if (fwd)
    walk_dir<true, DOB>(img, d_o, bos, L, n, h, tile, H, S0, rec_f, nullptr, sR, sZ, sDo);
  else
    walk_dir<false, DOB>(img, d_o, bos, L, n, h, tile, H, dSf, rec_b, dS0, sR, sZ, sDo);
}

// Three workgroups per CU (50 KB of LDS, at most 168 VGPRs): the kernel is
// bound by latency, and a third workgroup hides it better than the few
// registers the compiler spills to fit (one workgroup per CU measured 35 %
// slower than two, three 7 % faster).
template <bool QB, bool DOB>
__global__ void __launch_bounds__(NT, 3) bwd_grad_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ d_o, const float* __restrict__ g, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int N, int T_tot, int H, int maxnch, float scale,
    const float* __restrict__ img, const float* __restrict__ Srec,
    const float* __restrict__ dSrec, float* __restrict__ scr, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dg,
    float* __restrict__ dbeta, int64_t item0) {
  // sT, sDP: [C][C + 1] each, written from dM on.  Before that the first
  // products' slabs (gemm_staged2_pair) sit there, then X transposed (sXT,
  // [D][C]: X[r][c] in row c, its 4-float groups XOR-swizzled by c % 16, so
  // that 16 lanes reading one group each of rows c .. c + 15 hit distinct
  // banks) until dM has read it.  sU: the other products' LDS slabs (and, during the first
  // pipeline, its per-wave row sums), then (pairwise phase) K, Q and gamma of
  // a 16-channel slab and the per-wave partial sums.
  constexpr int SC = 16, SS = SC + 1;
  constexpr int PAIR_FLOATS = 3 * C * SS + 8 * SC;
  constexpr int TP = C * (C + 1);
  constexpr int STAGE_PAIR = 2 * (C + D) * SKP;
  static_assert(STAGE_PAIR <= 2 * TP && C * D <= 2 * TP, "paired slabs, then X, in sT, sDP");
  static_assert(4 * D <= STAGE_FLOATS, "row sums in sU");
  __shared__ __attribute__((aligned(16))) float
      sPool[2 * TP + (PAIR_FLOATS > STAGE_FLOATS ? PAIR_FLOATS : STAGE_FLOATS)];
  __shared__ __attribute__((aligned(16))) float sB[C];
  __shared__ float sDB[C], sGC[D];
  float(*sT)[C + 1] = reinterpret_cast<float(*)[C + 1]>(sPool);
  float(*sDP)[C + 1] = reinterpret_cast<float(*)[C + 1]>(sPool + TP);
  float* sU = sPool + 2 * TP;
  float* sRed = sU;    // [4][D], during the first pipeline
  float* sXT = sPool;  // X^T, from the first pipeline's end until dM
  auto xto = [](int c, int r) { return c * C + ((((r >> 2) ^ (c & 15))) << 2) + (r & 3); };
  float* sa = sU;
  ChunkPos p;
  if (!chunk_of_block(cu, N, T_tot, H, maxnch, p, item0 + blockIdx.x)) return;
  const int t = threadIdx.x;
  const int tc = t & 15;
  const int64_t HD = (int64_t)H * D;
  const float* im = img + p.pair * Rec::floats;
  const float* S = Srec + p.pair * (int64_t)(D * D);
  const float* dS = dSrec + p.pair * (int64_t)(D * D);
  // one scratch slot per workgroup of a launch (a launch has at most grad_slots)
  float* sc = scr + (int64_t)blockIdx.x * Scr::floats;
  const int Lc = p.Lc;
  auto tok = [&](int r, int cc) { return (p.t0 + r) * HD + (int64_t)p.h * D + cc; };
  const int HDi = static_cast<int>(HD);
  const auto rk = chunk_rows(k, QB ? 2 : 4, p, HD), rq = chunk_rows(q, QB ? 2 : 4, p, HD),
             rv = chunk_rows(v, QB ? 2 : 4, p, HD), ro = chunk_rows(d_o, DOB ? 2 : 4, p, HD);
  auto Vf = [&](int r, int cc) { return row_at<QB>(rv, HDi, r, cc); };
  auto dOf = [&](int r, int cc) { return row_at<DOB>(ro, HDi, r, cc); };
  auto Gf = [&](int r, int cc) { return im[Rec::G + r * D + cc]; };
  // quads (4 consecutive contraction indices) for the staged products
  auto ld4 = [](const float* x) { return *reinterpret_cast<const f32x4*>(x); };
  auto dO4 = [&](int r, int cc) { return row4_at<DOB>(ro, HDi, r, cc); };
  // a staged product's 64 x 128 result in the lane's own order: tile j of
  // thread t at off + 4 (NT j + t), one 16-byte store (read back only by the
  // same thread, in the pairwise phase)
  auto put8own = [&](const f32x4 (&acc)[1][8], int off, float mul) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<f32x4*>(sc + off + 4 * (NT * j + t)) =
          f32x4{mul * acc[0][j][0], mul * acc[0][j][1], mul * acc[0][j][2], mul * acc[0][j][3]};
  };
  auto put8 = [&](f32x4 (&acc)[1][8], int off, float mul) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) sc[off + orow<4>(i) * D + ocol(j)] = mul * acc[0][j][i];
  };
  if (t < C) {
    sB[t] = t < Lc ? beta[(p.t0 + t) * H + p.h] : 0.0f;
    sDB[t] = 0.0f;
  }
  __syncthreads();
  f32x4 accD[1][8];  // dDelta
  {  // X = V - K_E S and K_D dS_next in one pipeline.  While a slab of rows
     // of S and dS_next is in LDS, thread t sums row t % 16 of S . dS_next over
     // the columns 4 lq + w + 16 i (i < 8; the 16-lane groups of a wave read
     // distinct banks); summed over the wave's lane groups, then over the waves
     // below, this is d e^gamma_C[c] = sum_j dS_next[c, j] S[c, j].
    f32x4 acc[1][8];
    zero(acc);
    zero(accD);
    const int w = t >> 6, lq = (t & 63) >> 4, kk = t & 15;
    gemm_staged2_pair<4, 8>(
        acc, accD, D, sPool,
        [&](int p2, int r, int cc) {
          if (p2 == 1) return ld4(im + Rec::KD + r * D + cc);
          const f32x4 kv = row4_at<QB>(rk, HDi, r, cc);
          const f32x4 gv = ld4(im + Rec::G + r * D + cc);
          return f32x4{kv[0] * __expf(gv[0]), kv[1] * __expf(gv[1]), kv[2] * __expf(gv[2]),
                       kv[3] * __expf(gv[3])};
        },
        [&](int p2, int cc, int j) { return (p2 == 0 ? S : dS)[cc * D + j]; },
        [&](int k0, const float* b0, const float* b1) {
          float part = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int o = (4 * lq + w + 16 * i) * SKP + kk;
            part = fmaf(b0[o], b1[o], part);
          }
          part += __shfl_xor(part, 16);
          part += __shfl_xor(part, 32);
          if (lq == 0) sRed[w * D + k0 + kk] = part;
        });
    // lane (l % 16, l / 16) of wave w holds X rows 16 w + 4 (l / 16) + i
    // (i < 4) of column 16 j + l % 16: one 16-byte group of X^T
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = ocol(j), r0 = orow<4>(0);
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = Vf(r0 + i, col) - acc[0][j][i];
      *reinterpret_cast<f32x4*>(sXT + xto(col, r0)) = x;
    }
  }
  if (t < D)  // the gradient of gamma_C through e^gamma_C (the pairwise phase adds the rest)
    sGC[t] = (sRed[t] + sRed[D + t] + sRed[2 * D + t] + sRed[3 * D + t]) * __expf(Gf(C - 1, t));
  barrier_lds();  // X complete, the row sums read (sU takes the next slabs)
  // dDelta += scale P^T dO
  gemm_staged2<4, 8, false, true>(accD, C, sa,
                                 [&](int r, int s) { return scale * im[Rec::P + s * C + r]; },
                                 [&](int s, int j) { return dOf(s, j); });
  put8(accD, Scr::DD, 1.0f);
  __syncthreads();
  {  // Delta = M diag(b) X, without staging: wave w forms rows 16 w .. + 15
     // from its rows of M diag(b) in registers (lane (lr, lq): row 16 w + lr,
     // contraction 16 u + 4 lq + s) and X^T read from LDS in the same order
    const int lr = t & 15, lq = (t & 63) >> 4, w = t >> 6;
    f32x4 am[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) am[u] = ld4(im + Rec::M + (16 * w + lr) * C + 16 * u + 4 * lq);
    f32x4 acc[1][8];
    zero(acc);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4 bq = ld4(sB + 16 * u + 4 * lq);
      const f32x4 a = am[u] * bq;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 b = ld4(sXT + xto(16 * j + lr, 16 * u + 4 * lq));
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
          acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s2], b[s2], acc[0][j], 0, 0, 0);
      }
    }
    put8(acc, Scr::DL, 1.0f);
  }
  {  // dY = M^T dDelta, dX = diag(b) dY (= dv), dbeta += rowsum(dY . X)
    // (X through an opaque zero offset: its addresses are recomputed here
    // rather than kept in registers, which spills, since X's epilogue)
    int oz = 0;
    asm volatile("" : "+v"(oz));
    const float* qX = sXT + oz;
    f32x4 acc[1][8];
    zero(acc);
    gemm_staged2<4, 8, false, true>(acc, C, sa,
                                   [&](int r, int s) { return im[Rec::M + s * C + r]; },
                                   [&](int s, int j) { return sc[Scr::DD + s * D + j]; });
    f32x4 xv[8];  // X at the lane's elements: one 16-byte group of X^T per tile
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = ld4(qX + xto(ocol(j), orow<4>(0)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = orow<4>(i);
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = ocol(j);
        const float dX = sB[r] * acc[0][j][i];
        sc[Scr::DX + r * D + col] = dX;
        if (r < Lc) dv[tok(r, col)] = dX;
        part = fmaf(acc[0][j][i], xv[j][i], part);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) part += __shfl_xor(part, off);
      if (tc == 0) sDB[r] += part;  // the 16 lanes holding row r
    }
  }
  __syncthreads();
  {  // dM = dDelta Y^T (Y = diag(b) X, X from LDS), then dP = scale dO Delta^T
     // on s <= r, in one pipeline; dM goes over X once the pipeline has read
     // it (X is read by the first product only)
    f32x4 a4[1][4];
    zero(a4);
    gemm_staged2_seq<2, 4, 4, true, false>(
        a4, D, sa,
        [&](int p2, int r, int j) { return p2 == 0 ? ld4(sc + Scr::DD + r * D + j) : dO4(r, j); },
        [&](int p2, int j, int s) {
          return p2 == 0 ? sB[s] * f32x4{sXT[xto(j, s)], sXT[xto(j + 1, s)], sXT[xto(j + 2, s)],
                                         sXT[xto(j + 3, s)]}
                         : ld4(sc + Scr::DL + s * D + j);
        },
        [&](int, f32x4(&c)[1][4]) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) sT[orow<4>(i)][ocol(j)] = c[0][j][i];
        });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = orow<4>(i), s = ocol(j);
        sDP[r][s] = (s <= r && r < Lc) ? scale * a4[0][j][i] : 0.0f;
      }
  }
  __syncthreads();
  // dM M^T and dA = -M^T (dM M^T) without staging: wave w forms rows
  // 16 w .. + 15 of each product from its rows of M (or M^T) in registers and
  // the other operand read from sT (lane (lr, lq), sub-step s: contraction
  // index 16 u + 4 lq + s)
  {
    const int lr = t & 15, lq = (t & 63) >> 4, w = t >> 6;
    {  // dM M^T as its transpose M dM^T (M's rows in registers); lane (lr, lq)
       // then holds (dM M^T)[16 j + lr][16 w + 4 lq + v], written over dM once
       // every wave has read it
      f32x4 am[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) am[u] = ld4(im + Rec::M + (16 * w + lr) * C + 16 * u + 4 * lq);
      f32x4 acc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(am[u][s2], sT[16 * j + lr][16 * u + 4 * lq + s2],
                                                          acc[j], 0, 0, 0);
      barrier_lds();  // dM read by every wave
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) sT[16 * j + lr][16 * w + 4 * lq + v] = acc[j][v];
    }
    barrier_lds();
    {  // dA = -M^T (dM M^T) on s < r; its epilogue adds sum_s dA[r, s] At[r, s]
       // to dbeta (At read before the product, at the lane's elements) and
       // stores dA scaled by beta_r, the factor the pairwise terms take it
       // with, over dM M^T in sT once every wave has read that
      float at[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) at[i][j] = im[Rec::AT + orow<4>(i) * C + ocol(j)];
      float mt[4][4];  // M^T row 16 w + lr: M[16 u + 4 lq + s][16 w + lr]
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) mt[u][s2] = im[Rec::M + (16 * u + 4 * lq + s2) * C + 16 * w + lr];
      f32x4 a4[1][4];
      zero(a4);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            a4[0][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(mt[u][s2], sT[16 * u + 4 * lq + s2][16 * j + lr],
                                                            a4[0][j], 0, 0, 0);
      barrier_lds();  // dM M^T read by every wave
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = orow<4>(i);
        const float br = sB[r];
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int s = ocol(j);
          const float da = (s < r && r < Lc) ? -a4[0][j][i] : 0.0f;
          part = fmaf(da, at[i][j], part);
          sT[r][s] = da * br;
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) part += __shfl_xor(part, off);
        if (tc == 0) sDB[r] += part;  // the 16 lanes holding row r
      }
    }
  }
  {  // dK_E = -dX S^T, dQ_E = scale dO S^T, dK_D = Delta dS_next^T in one pipeline
    f32x4 acc[1][8];
    zero(acc);
    gemm_staged2_seq<3, 4, 8, true, false>(
        acc, D, sa,
        [&](int p2, int r, int j) {
          return p2 == 1 ? dO4(r, j) : ld4(sc + (p2 == 0 ? Scr::DX : Scr::DL) + r * D + j);
        },
        [&](int p2, int j, int cc) { return ld4((p2 == 2 ? dS : S) + cc * D + j); },
        [&](int p2, f32x4(&c)[1][8]) {
          if (p2 == 0)
            put8own(c, Scr::DKE, -1.0f);
          else
            put8own(c, Scr::DQE, scale);
        });
    put8own(acc, Scr::DKD, 1.0f);
  }
  __syncthreads();  // dK_E, dQ_E, dK_D (scratch) and the scaled dA complete
  // The terms of the decay factors and the pairwise terms of At and P, 16
  // channels at a time.  For a row x and channel c (w(a, b) = e^(gamma_a -
  // gamma_b) <= 1 for a >= b):
  //   L1[x] = sum_{s < x} dA~[x, s] k_s w(x, s)     (dA~: dA with beta_x folded in)
  //   L2[x] = sum_{s <= x} dP[x, s] k_s w(x, s)
  //   R[x]  = sum_{r >= x} (dA~[r, x] k_r + dP[r, x] q_r) w(r, x)
  //   dk += L1 + R,  dq += L2,  dgamma += k L1 + q L2 - k R.
  // For x in 16-row block i and s in an earlier block, w(x, s) = w(x, b)
  // w(b, s) with b the row before block i, both <= 1: L1 and L2 of block i are
  // products of the dA~ / dP rows with the right factors k_s w(b, s) over all
  // earlier rows, scaled by w(x, b) (fp32 MFMA).  Likewise R of block j uses
  // e, the block's last row: (dA~ / dP columns)^T times k_r w(r, e) and
  // q_r w(r, e) over all later rows, scaled by w(e, x).  Pairs inside one
  // block take w directly (a pair's factors could both be huge there).
  float* sK = sU;                  // [C][SS] k of the slab's channels
  float* sQ = sK + C * SS;         // q
  float* sG = sQ + C * SS;         // gamma
  float* sPart = sG + C * SS;      // [4][SC] partial sums of the gamma_C term
  float* sBlk = sPart + 4 * SC;    // [4][SC] dgamma summed over each wave's rows
  const int lane = t & 63, w = t >> 6, ln = lane & 15, lq = lane >> 4;
  // Thread t reads row t / 4, channels 4 (t % 4) .. + 3 of the slab's k, q
  // and gamma into LDS (4-wide loads, one slab ahead so that the reads stay
  // in flight across the slab's barriers, which order LDS only).  Lane
  // (ln, lq) of wave w then owns rows 16 w + 4 lq + v (v < 4) of channel
  // c0 + ln: it reads those elements' decay-factor gradients (which it wrote
  // itself, put8own) and g (for the floor), one slab ahead as well, adds the
  // pairwise terms and writes dq and dk; the slab's dgamma, summed down its
  // 64 rows, gives dg.
  // (16 channels per slab: the MFMA tiles below use the 16 lanes of a row
  // as the slab's channels)
  static_assert(SC == 16, "one slab channel per lane of a 16-lane row");
  const int xr = t >> 2, n4 = 4 * (t & 3);
  const auto rgf = chunk_rows(g, 4, p, HD);
  const auto rsc = chunk::make_buf(sc, Scr::floats * 4);
  f32x4 pk, pq, pg;          // the LDS fill
  f32x4 eke, eqe, ekd, egv;  // the lane's own elements, rows 16 w + 4 lq + v
  auto fetch_slab = [&](int c0) {
    const int cc = c0 + n4;
    pk = row4_at<QB>(rk, HDi, xr, cc);
    pq = row4_at<QB>(rq, HDi, xr, cc);
    pg = *reinterpret_cast<const f32x4*>(im + Rec::G + xr * D + cc);
    const int x0 = 16 * w + 4 * lq, vo = 4 * (NT * (c0 / SC) + t) * 4;
    // the lane's own elements of dK_E, dQ_E, dK_D (put8own: tile c0 / 16)
    eke = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsc, vo, Scr::DKE * 4, 0));
    eqe = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsc, vo, Scr::DQE * 4, 0));
    ekd = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsc, vo, Scr::DKD * 4, 0));
#pragma unroll
    for (int v = 0; v < 4; ++v)
      egv[v] = row_at<false>(rgf, HDi, x0 + v, c0 + ln);  // rows past the chunk end read 0
  };
  fetch_slab(0);
  for (int c0 = 0; c0 < D; c0 += SC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sK[xr * SS + n4 + i] = pk[i];
      sQ[xr * SS + n4 + i] = pq[i];
      sG[xr * SS + n4 + i] = pg[i];
    }
    const f32x4 dke = eke, dqe = eqe, dkd = ekd, gv = egv;  // this slab's
    float dgs[4];  // dgamma of the lane's rows (0 past the chunk end)
    barrier_lds();
    if (c0 + SC < D) fetch_slab(c0 + SC);
    {  // pairs across blocks on fp32 MFMA: wave w owns the rows of block w.
       // Lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and holds
       // D[4 (l / 16) + v][l % 16]; n = l % 16 is the channel of B and D.
      f32x4 L1 = {0.f, 0.f, 0.f, 0.f}, L2 = L1, R = L1;
      if (w >= 1) {  // s < 16 w, reference b = 16 w - 1
        const int b = 16 * w - 1;
        const float gb = sG[b * SS + ln];
        for (int ks = 0; ks < 4 * w; ++ks) {
          const int s2 = 4 * ks + lq;
          const float bv = sK[s2 * SS + ln] * __expf(gb - sG[s2 * SS + ln]);
          L1 = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[16 * w + ln][s2], bv, L1, 0, 0, 0);
          L2 = __builtin_amdgcn_mfma_f32_16x16x4f32(sDP[16 * w + ln][s2], bv, L2, 0, 0, 0);
        }
      }
      if (w <= 2) {  // r >= 16 (w + 1), reference e = 16 w + 15
        const int e = 16 * w + 15;
        const float ge = sG[e * SS + ln];
        for (int ks = 4 * (w + 1); ks < C / 4; ++ks) {
          const int r = 4 * ks + lq;
          const float wr = __expf(sG[r * SS + ln] - ge);
          R = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[r][16 * w + ln], sK[r * SS + ln] * wr, R,
                                                   0, 0, 0);
          R = __builtin_amdgcn_mfma_f32_16x16x4f32(sDP[r][16 * w + ln], sQ[r * SS + ln] * wr, R,
                                                   0, 0, 0);
        }
      }
      // Pairs inside block w, by 8-row halves as in the prep's diagonal At / P
      // tiles: same-half pairs relative to the half's anchor a (rows 3 and 11
      // of the block: at most 4 tokens from any row of the half), pairs across
      // the halves relative to row 7 (factors <= 1).  Each product's operand
      // A is masked to its pairs; with L the later row:
      //   Ls / Lx: rows x, columns s <= x, B = k_s e^(gamma_a(s) - gamma_s) /
      //            k_s e^(gamma_7 - gamma_s), scaled by e^(gamma_x - gamma_a(x)) /
      //            e^(gamma_x - gamma_7);
      //   Rs / Rx: rows x, columns r >= x (A transposed), B = (k_r, q_r)
      //            e^(gamma_r - gamma_a(r)) / e^(gamma_r - gamma_7), scaled by
      //            e^(gamma_a(x) - gamma_x) / e^(gamma_7 - gamma_x).
      f32x4 L1s = {0.f, 0.f, 0.f, 0.f}, L2s = L1s, L1x = L1s, L2x = L1s, Rs = L1s, Rx = L1s;
      {
        const int x = 16 * w + ln;
        const float g7 = sG[(16 * w + 7) * SS + ln];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int sl = 4 * ks + lq, s2 = 16 * w + sl;  // k index of A, row of B
          const bool same = (ln < 8) == (sl < 8);
          const bool cl = ln >= 8 && sl < 8, cr = ln < 8 && sl >= 8;
          const float gs = sG[s2 * SS + ln], ks2 = sK[s2 * SS + ln], qs2 = sQ[s2 * SS + ln];
          const float ga = sG[(16 * w + (sl < 8 ? 3 : 11)) * SS + ln];
          const float fa = __expf(ga - gs), ea = __expf(gs - ga);
          const float e7 = __expf(sl < 8 ? g7 - gs : gs - g7);
          const float ta = sT[x][s2], tp = sDP[x][s2];      // A of L: (x, s)
          const float ua = sT[s2][x], up = sDP[s2][x];      // A of R: (r, x)
          const float b1 = ks2 * fa, b3 = sl < 8 ? ks2 * e7 : 0.0f;
          L1s = __builtin_amdgcn_mfma_f32_16x16x4f32(same ? ta : 0.0f, b1, L1s, 0, 0, 0);
          L2s = __builtin_amdgcn_mfma_f32_16x16x4f32(same ? tp : 0.0f, b1, L2s, 0, 0, 0);
          L1x = __builtin_amdgcn_mfma_f32_16x16x4f32(cl ? ta : 0.0f, b3, L1x, 0, 0, 0);
          L2x = __builtin_amdgcn_mfma_f32_16x16x4f32(cl ? tp : 0.0f, b3, L2x, 0, 0, 0);
          Rs = __builtin_amdgcn_mfma_f32_16x16x4f32(same ? ua : 0.0f, ks2 * ea, Rs, 0, 0, 0);
          Rs = __builtin_amdgcn_mfma_f32_16x16x4f32(same ? up : 0.0f, qs2 * ea, Rs, 0, 0, 0);
          const float rk = sl >= 8 ? ks2 * e7 : 0.0f, rq = sl >= 8 ? qs2 * e7 : 0.0f;
          Rx = __builtin_amdgcn_mfma_f32_16x16x4f32(cr ? ua : 0.0f, rk, Rx, 0, 0, 0);
          Rx = __builtin_amdgcn_mfma_f32_16x16x4f32(cr ? up : 0.0f, rq, Rx, 0, 0, 0);
        }
      }
      const float gb = w >= 1 ? sG[(16 * w - 1) * SS + ln] : 0.0f;
      const float ge = sG[(16 * w + 15) * SS + ln];
      const float g7 = sG[(16 * w + 7) * SS + ln];
      const float gc = sG[(C - 1) * SS + ln];  // gamma_C of channel c0 + ln
      float dcs = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int xl = 4 * lq + v, x = 16 * w + xl;
        dgs[v] = 0.0f;
        const float gx = sG[x * SS + ln];
        const float gax = sG[(16 * w + (xl < 8 ? 3 : 11)) * SS + ln];
        const float ex = __expf(gx - gax), fx = __expf(gax - gx);
        const float e7 = __expf(xl < 8 ? g7 - gx : gx - g7);  // <= 1 either way
        float l1 = L1s[v] * ex, l2 = L2s[v] * ex, rr = Rs[v] * fx;
        if (xl >= 8) {
          l1 += L1x[v] * e7;
          l2 += L2x[v] * e7;
        } else {
          rr += Rx[v] * e7;
        }
        if (w >= 1) {
          const float eb = __expf(gx - gb);
          l1 += L1[v] * eb;
          l2 += L2[v] * eb;
        }
        if (w <= 2) rr += R[v] * __expf(ge - gx);
        // plus the terms of the decay factors of K_E = K e^gamma, Q_E = Q
        // e^gamma and K_D = K e^(gamma_C - gamma)
        const float kx = sK[x * SS + ln], qx = sQ[x * SS + ln];
        if (x < Lc) {
          const float E = __expf(gx), F = __expf(gc - gx);
          const int cc = c0 + ln;
          dk[tok(x, cc)] = dke[v] * E + dkd[v] * F + l1 + rr;
          dq[tok(x, cc)] = dqe[v] * E + l2;
          dgs[v] = (dke[v] * kx + dqe[v] * qx) * E - dkd[v] * kx * F + kx * l1 + qx * l2 - kx * rr;
          dcs += dkd[v] * kx * F;
        }
      }
      // the gamma_C terms of channel c0 + ln summed over the wave's 16 rows
      dcs += __shfl_xor(dcs, 16);
      dcs += __shfl_xor(dcs, 32);
      if (lq == 0) sPart[w * SC + ln] = dcs;
    }
    // dg = the reverse cumulative sum of dgamma down the rows plus the gamma_C
    // terms.  The lane's rows 16 w + 4 lq + v, summed from the last: within
    // the lane, then the later lane groups of the wave, then (after the
    // barrier) the later waves and the gamma_C terms of the channel.
#pragma unroll
    for (int v = 2; v >= 0; --v) dgs[v] += dgs[v + 1];
    const float o1 = __shfl(dgs[0], (lane + 16) & 63), o2 = __shfl(dgs[0], (lane + 32) & 63),
                o3 = __shfl(dgs[0], (lane + 48) & 63);
    const float later = (lq < 3 ? o1 : 0.0f) + (lq < 2 ? o2 : 0.0f) + (lq < 1 ? o3 : 0.0f);
    if (lq == 0) sBlk[w * SC + ln] = dgs[0] + o1 + o2 + o3;
    barrier_lds();  // sPart, sBlk complete; the slab's arrays are refilled next
    {
      float run = sGC[c0 + ln] + sPart[ln] + sPart[SC + ln] + sPart[2 * SC + ln] +
                  sPart[3 * SC + ln] + later;
      for (int w2 = w + 1; w2 < 4; ++w2) run += sBlk[w2 * SC + ln];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int x = 16 * w + 4 * lq + v;
        if (x < Lc) dg[tok(x, c0 + ln)] = decay_floored(gv[v]) ? 0.0f : run + dgs[v];
      }
    }
  }
  if (t < Lc) dbeta[(p.t0 + t) * H + p.h] = sDB[t];
}

}  // namespace

// The gradient kernel runs in launches of at most grad_slots workgroups, each
// with a scratch slot of its own: one slot per (chunk, head) up to
// GRAD_SLOTS_MAX (1.6 GB of scratch), so that up to that size one launch
// covers every chunk and the GPU's dispatcher refills each CU as its
// workgroups finish (a launch per 512 workgroups cost 4 % at T = 4096,
// H = 96 in drained launch tails).
constexpr int64_t GRAD_SLOTS_MAX = 8192;
int64_t grad_slots(size_t pairs) {
  return pairs == 0 ? 1 : (pairs < (size_t)GRAD_SLOTS_MAX ? (int64_t)pairs : GRAD_SLOTS_MAX);
}

size_t workspace_bytes(int64_t T_tot, int N, int H) {
  const size_t pairs = (size_t)(T_tot / C + N) * (size_t)H;
  return (pairs * (size_t)(Rec::floats + 2 * D * D) + (size_t)grad_slots(pairs) * Scr::floats) *
         sizeof(float);
}

hipError_t launch(const void* q, const void* k, const void* v, bool qkv_bf16, const float* g,
                  const float* beta, const int32_t* cu, const int32_t* cu_host, int N,
                  const float* S0, const void* d_o, bool do_bf16, const float* dS_final,
                  float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dS0,
                  int64_t T_tot, int H, float scale, void* ws, hipStream_t s) {
  int64_t maxnch = (T_tot + C - 1) / C;
  if (cu_host) {
    maxnch = 0;
    for (int n = 0; n < N; ++n) {
      const int64_t nc = ((int64_t)cu_host[n + 1] - cu_host[n] + C - 1) / C;
      if (nc > maxnch) maxnch = nc;
    }
  }
  const size_t pairs = (size_t)(T_tot / C + N) * (size_t)H;
  float* img = static_cast<float*>(ws);
  float* Srec = img + pairs * Rec::floats;
  float* dSrec = Srec + pairs * (size_t)(D * D);
  float* scr = dSrec + pairs * (size_t)(D * D);
  const int T = static_cast<int>(T_tot);
  const int64_t chunk_blocks = (int64_t)N * maxnch * H;
  const int64_t walk_blocks = (int64_t)N * H * 2;
  if (chunk_blocks > 0x7fffffff || 2 * walk_blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (chunk_blocks > 0) {
    if (qkv_bf16)
      bwd_prep_kernel<true><<<dim3((unsigned)chunk_blocks), NT, 0, s>>>(
          q, k, v, g, beta, cu, N, T, H, (int)maxnch, scale, img);
    else
      bwd_prep_kernel<false><<<dim3((unsigned)chunk_blocks), NT, 0, s>>>(
          q, k, v, g, beta, cu, N, T, H, (int)maxnch, scale, img);
  }
  {  // the forward and backward walks together (backward only when no chunk exists)
    const int both = chunk_blocks > 0 ? 1 : 0;
    const dim3 grid((unsigned)(walk_blocks * (both ? 2 : 1)));
    if (do_bf16)
      bwd_walk_kernel<true><<<grid, NT, 0, s>>>(img, d_o, cu, N, T, H, both, S0, Srec, dS_final,
                                                dS0, dSrec);
    else
      bwd_walk_kernel<false><<<grid, NT, 0, s>>>(img, d_o, cu, N, T, H, both, S0, Srec,
                                                 dS_final, dS0, dSrec);
  }
  const int64_t slots = grad_slots(pairs);
  for (int64_t item0 = 0; item0 < chunk_blocks; item0 += slots) {
    const int64_t nb = chunk_blocks - item0 < slots ? chunk_blocks - item0 : slots;
#define KDA_BG(QB, OB)                                                                        \
  bwd_grad_kernel<QB, OB><<<dim3((unsigned)nb), NT, 0, s>>>(                                  \
      q, k, v, d_o, g, beta, cu, N, T, H, (int)maxnch, scale, img, Srec, dSrec, scr, dq, dk, dv, \
      dg, dbeta, item0)
    if (qkv_bf16 && do_bf16) KDA_BG(true, true);
    else if (qkv_bf16) KDA_BG(true, false);
    else if (do_bf16) KDA_BG(false, true);
    else KDA_BG(false, false);
#undef KDA_BG
  }
  return hipGetLastError();
}

}  // namespace bwd
}  // namespace kda
