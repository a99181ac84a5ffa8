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
// Three kernels, all in fp32 (the products on fp32 MFMA):
//   bwd_prep  one workgroup per (chunk, head): gamma, At, P, M, W, U, Qt, K_D
//             and e^gamma_C into a per-(chunk, head) record;
//   bwd_walk  one workgroup per (sequence, head, 64-column tile) and
//             direction, both directions in one launch: forward, the entry
//             state of every chunk; backward, the state gradient at every
//             chunk's end and the initial state's gradient;
//   bwd_grad  in launches of at most GRAD_SLOTS workgroups, one per (chunk,
//             head), each with a scratch slot of its own: with S and dS_next known, the
//             chunk's gradients dq, dk, dv, dg, dbeta by the chain rule
//             through the identities above (the pairwise decay terms of At
//             and P per key channel, then a reverse cumulative sum for dg).
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace bwd {
namespace {

constexpr int C = 64;
constexpr int D = 128;
constexpr int NT = 256;

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
  static constexpr int X = 0, DL = C * D, DD = 2 * C * D, DX = 3 * C * D, DKE = 4 * C * D,
                       DQE = 5 * C * D, DKD = 6 * C * D, floats = 7 * C * D;
};

// acc += a b for a (16 TM) x (16 TN) output over the 256 threads, on fp32
// MFMA, with the operands staged through LDS in slabs of KT = 16 along the
// contraction (each element read once from memory instead of once per thread
// that uses it).  acc[i][j] is element (orow<TM>(i), ocol(j)).  A_KC: a(m, kk) is contiguous along kk in memory
// (else along m); B_NC: b(kk, n) is contiguous along n (else along kk); the
// slab fill follows the contiguous index.  sa: 16 x (16 TM + 1) floats, sb:
// 16 x (16 TN + 1) floats.  Contains barriers: every thread of the block calls it.
constexpr int KT = 16;
template <int TM, int TN, bool A_KC, bool B_NC, typename FA, typename FB>
__device__ __forceinline__ void gemm_staged(float (&acc)[TM][TN], int K, float* stage, FA a,
                                            FB b) {
  // slab rows 17 floats past a multiple of 32 apart: the MFMA reads (16
  // consecutive elements of 4 consecutive rows) and the kk-fastest fills
  // both spread over the banks
  constexpr int M = 16 * TM, N = 16 * TN, MS = M + 17, NS = N + 17;
  float* sa = stage;
  float* sb = stage + KT * MS;
  constexpr int PA = M * KT / NT, PB = N * KT / NT;  // slab elements per thread
  static_assert(TM % 4 == 0, "whole 16-row tiles per wave");
  const int t = threadIdx.x;
  // the next slab is read into registers while the current one is in use
  float ra[PA], rb[PB];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < PA; ++u) {
      const int e = t + NT * u;
      const int m = A_KC ? e / KT : e % M, kt = A_KC ? e % KT : e / M;
      ra[u] = a(m, k0 + kt);
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int e = t + NT * u;
      const int n = B_NC ? e % N : e / KT, kt = B_NC ? e / N : e % KT;
      rb[u] = b(k0 + kt, n);
    }
  };
  // the accumulators as MFMA tiles for the whole product (4 consecutive
  // registers each), converted from and to acc once
  constexpr int TR = TM / 4;
  f32x4 ct[TR][TN];
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      ct[i][j] = f32x4{acc[4 * i][j], acc[4 * i + 1][j], acc[4 * i + 2][j], acc[4 * i + 3][j]};
  fetch(0);
  for (int k0 = 0; k0 < K; k0 += KT) {
#pragma unroll
    for (int u = 0; u < PA; ++u) {
      const int e = t + NT * u;
      const int m = A_KC ? e / KT : e % M, kt = A_KC ? e % KT : e / M;
      sa[kt * MS + m] = ra[u];
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int e = t + NT * u;
      const int n = B_NC ? e % N : e / KT, kt = B_NC ? e / N : e % KT;
      sb[kt * NS + n] = rb[u];
    }
    __syncthreads();
    if (k0 + KT < K) fetch(k0 + KT);
    // fp32 16x16x4 MFMA: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]
    // and holds D[4 (l / 16) + v][l % 16]; wave w owns the output tile rows
    // TR w .. TR w + TR - 1 and every tile column.
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
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[4 * i + v][j] = ct[i][j][v];
}
constexpr int STAGE_FLOATS = KT * (64 + 17) + KT * (128 + 17);  // the largest product's slabs
// gemm_staged with two slabs in flight, for kernels with the registers to
// spare: slab k0 + 2 KT is read into registers while slab k0 is used, and
// the barriers order LDS only, so those loads stay in flight across them (a
// __syncthreads fence would wait for them at every slab).  With one slab in
// flight each slab costs about one memory latency, the products being short.
// K, always 64 or 128, is a multiple of 2 KT; a caller orders any global
// data it wrote before the call itself.
template <int TM, int TN, bool A_KC, bool B_NC, typename FA, typename FB>
__device__ __forceinline__ void gemm_staged2(float (&acc)[TM][TN], int K, float* stage, FA a,
                                             FB b) {
  constexpr int M = 16 * TM, N = 16 * TN, MS = M + 17, NS = N + 17;
  float* sa = stage;
  float* sb = stage + KT * MS;
  constexpr int PA = M * KT / NT, PB = N * KT / NT;
  static_assert(TM % 4 == 0, "whole 16-row tiles per wave");
  const int t = threadIdx.x;
  float ra[2][PA], rb[2][PB];
  auto fetch = [&](int k0, int sl) {
#pragma unroll
    for (int u = 0; u < PA; ++u) {
      const int e = t + NT * u;
      const int m = A_KC ? e / KT : e % M, kt = A_KC ? e % KT : e / M;
      ra[sl][u] = a(m, k0 + kt);
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int e = t + NT * u;
      const int n = B_NC ? e % N : e / KT, kt = B_NC ? e / N : e % KT;
      rb[sl][u] = b(k0 + kt, n);
    }
  };
  constexpr int TR = TM / 4;
  f32x4 ct[TR][TN];
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      ct[i][j] = f32x4{acc[4 * i][j], acc[4 * i + 1][j], acc[4 * i + 2][j], acc[4 * i + 3][j]};
  fetch(0, 0);
  fetch(KT, 1);
  for (int k0 = 0; k0 < K; k0 += 2 * KT) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
      for (int u = 0; u < PA; ++u) {
        const int e = t + NT * u;
        const int m = A_KC ? e / KT : e % M, kt = A_KC ? e % KT : e / M;
        sa[kt * MS + m] = ra[sl][u];
      }
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        const int e = t + NT * u;
        const int n = B_NC ? e % N : e / KT, kt = B_NC ? e / N : e % KT;
        sb[kt * NS + n] = rb[sl][u];
      }
      barrier_lds();
      if (k0 + (2 + sl) * KT < K) fetch(k0 + (2 + sl) * KT, sl);
      // the fp32 16x16x4 MFMA fragments of gemm_staged
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
#pragma unroll
  for (int i = 0; i < TR; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[4 * i + v][j] = ct[i][j][v];
}

// Output element of acc[i][j] after gemm_staged<TM, TN>: row orow<TM>(i),
// column ocol(j).
template <int TM>
__device__ __forceinline__ int orow(int i) {
  const int t = threadIdx.x;
  return 16 * ((TM / 4) * (t >> 6) + (i >> 2)) + 4 * ((t & 63) >> 4) + (i & 3);
}
__device__ __forceinline__ int ocol(int j) { return 16 * j + (threadIdx.x & 15); }

template <int TM, int TN>
__device__ __forceinline__ void zero(float (&acc)[TM][TN]) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;
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
// element (row r < 64, channel cc) through chunk_rows; HDi = H * 128
template <bool BF16>
__device__ __forceinline__ float row_at(__amdgpu_buffer_rsrc_t rs, int HDi, int r, int cc) {
  if constexpr (BF16)
    return bf16_bits_to_f32(static_cast<uint16_t>(
        __builtin_amdgcn_raw_buffer_load_b16(rs, (r * HDi + cc) * 2, 0, 0)));
  else
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (r * HDi + cc) * 4, 0, 0));
}

template <bool QB>
__global__ void __launch_bounds__(NT, 2) bwd_prep_kernel(const void* __restrict__ q,
                                                         const void* __restrict__ k,
                                                         const void* __restrict__ v,
                                                         const float* __restrict__ g,
                                                         const float* __restrict__ beta,
                                                         const int32_t* __restrict__ cu, int N,
                                                         int T_tot, int H, int maxnch,
                                                         float scale, float* __restrict__ img) {
  constexpr int CS = 16;  // channels per slab of the At / P sums
  __shared__ float sA[C][C + 1], sP[C][C + 1], sM[C][C + 1], sB[C];
  // slabs of K, Q, gamma (CS channels), later the products' LDS slabs
  constexpr int SLAB = C * (CS + 1);
  __shared__ float sS[(3 * SLAB > STAGE_FLOATS ? 3 * SLAB : STAGE_FLOATS)];
  ChunkPos p;
  if (!chunk_of_block(cu, N, T_tot, H, maxnch, p, blockIdx.x)) return;
  const int t = threadIdx.x;
  const int64_t HD = (int64_t)H * D;
  float* im = img + p.pair * Rec::floats;
  const int HDi = static_cast<int>(HD);
  const auto rk = chunk_rows(k, QB ? 2 : 4, p, HD), rq = chunk_rows(q, QB ? 2 : 4, p, HD),
             rv = chunk_rows(v, QB ? 2 : 4, p, HD), rg = chunk_rows(g, 4, p, HD);
  auto Kf = [&](int r, int cc) { return row_at<QB>(rk, HDi, r, cc); };
  auto Qf = [&](int r, int cc) { return row_at<QB>(rq, HDi, r, cc); };
  if (t < C) sB[t] = t < p.Lc ? beta[(p.t0 + t) * H + p.h] : 0.0f;
  if (t < D) {  // gamma: running sum of g down channel t (rows past the end repeat the last)
    float gv[C];
#pragma unroll
    for (int r = 0; r < C; ++r) gv[r] = row_at<false>(rg, HDi, r, t);
    float run = 0.0f;
#pragma unroll
    for (int r = 0; r < C; ++r) {
      run += gv[r];
      im[Rec::G + r * D + t] = run;
    }
  }
  __syncthreads();
  auto Gf = [&](int r, int cc) { return im[Rec::G + r * D + cc]; };
  {  // At and P over the strictly lower pairs, folded so that no lane idles:
     // wave w, step u takes the rows lo = w + 4u and hi = 63 - lo (lo + hi = 63
     // pairs s < r between them); lane l < lo takes (lo, l), lanes lo .. 62
     // take (hi, l - lo), and lane 63 the two diagonal entries of P (q_r . k_r,
     // the decay over zero tokens being 1; At is 0 on the diagonal).
    float* sK = sS;
    float* sQ = sS + C * (CS + 1);
    float* sG = sS + 2 * C * (CS + 1);
    constexpr int NU = C / 2 / (NT / 64);  // row pairs per wave
    const int l = t & 63, w = t >> 6;
    float a[NU], pp[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) a[u] = pp[u] = 0.0f;
    // slab c0 is read into registers while the previous one is in use
    constexpr int PS = C * CS / NT;
    float rk[PS], rq[PS], rg[PS];
    auto fetch_slab = [&](int c0) {
#pragma unroll
      for (int u = 0; u < PS; ++u) {
        const int e = t + NT * u, r = e / CS, ch = e % CS;
        rk[u] = Kf(r, c0 + ch);
        rq[u] = Qf(r, c0 + ch);
        rg[u] = Gf(r, c0 + ch);
      }
    };
    fetch_slab(0);
    for (int c0 = 0; c0 < D; c0 += CS) {
#pragma unroll
      for (int u = 0; u < PS; ++u) {
        const int e = t + NT * u, r = e / CS, ch = e % CS;
        sK[r * (CS + 1) + ch] = rk[u];
        sQ[r * (CS + 1) + ch] = rq[u];
        sG[r * (CS + 1) + ch] = rg[u];
      }
      __syncthreads();
      if (c0 + CS < D) fetch_slab(c0 + CS);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int lo = w + 4 * u, hi = C - 1 - lo;
        if (l < C - 1) {
          const int r = l < lo ? lo : hi, s2 = l < lo ? l : l - lo;
#pragma unroll
          for (int ch = 0; ch < CS; ++ch) {
            const float ks = sK[s2 * (CS + 1) + ch] *
                             __expf(sG[r * (CS + 1) + ch] - sG[s2 * (CS + 1) + ch]);
            a[u] = fmaf(sK[r * (CS + 1) + ch], ks, a[u]);
            pp[u] = fmaf(sQ[r * (CS + 1) + ch], ks, pp[u]);
          }
        } else {
#pragma unroll
          for (int ch = 0; ch < CS; ++ch) {
            a[u] = fmaf(sQ[lo * (CS + 1) + ch], sK[lo * (CS + 1) + ch], a[u]);
            pp[u] = fmaf(sQ[hi * (CS + 1) + ch], sK[hi * (CS + 1) + ch], pp[u]);
          }
        }
      }
      __syncthreads();
    }
    // each lower pair (r, s) also writes the zero of its mirror (s, r)
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int lo = w + 4 * u, hi = C - 1 - lo;
      if (l < C - 1) {
        const int r = l < lo ? lo : hi, s2 = l < lo ? l : l - lo;
        sA[r][s2] = a[u];
        sP[r][s2] = pp[u];
        sA[s2][r] = 0.0f;
        sP[s2][r] = 0.0f;
        im[Rec::AT + r * C + s2] = a[u];
        im[Rec::P + r * C + s2] = pp[u];
        im[Rec::AT + s2 * C + r] = 0.0f;
        im[Rec::P + s2 * C + r] = 0.0f;
      } else {
        sA[lo][lo] = sA[hi][hi] = 0.0f;
        sP[lo][lo] = a[u];
        sP[hi][hi] = pp[u];
        im[Rec::AT + lo * C + lo] = im[Rec::AT + hi * C + hi] = 0.0f;
        im[Rec::P + lo * C + lo] = a[u];
        im[Rec::P + hi * C + hi] = pp[u];
      }
    }
  }
  __syncthreads();
  // M = (I + diag(b) At)^-1, unit lower triangular, by forward substitution
  // down each column: M[r][s] = -b_r sum_{s <= u < r} At[r][u] M[u][s].
  // Column s belongs to lanes 4s .. 4s + 3 of one wave (a quarter of the
  // sum each, combined by shuffles); rows go in order.
  {
    const int s2 = t >> 2, qd = t & 3;
    for (int r = 0; r < C; ++r) {
      float acc = 0.0f;
      for (int u = s2 + qd; u < r; u += 4) acc = fmaf(sA[r][u], sM[u][s2], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      if (qd == 0) sM[r][s2] = r < s2 ? 0.0f : (r == s2 ? 1.0f : -sB[r] * acc);
    }
  }
  __syncthreads();
  for (int e = t; e < C * C; e += NT) im[Rec::M + e] = sM[e / C][e % C];
  float* sa = sS;
  {  // W = M diag(b) K_E
    float acc[4][8];
    zero(acc);
    gemm_staged<4, 8, true, true>(acc, C, sa, [&](int r, int s2) { return sM[r][s2]; },
                                  [&](int s2, int cc) {
                                    return sB[s2] * Kf(s2, cc) * __expf(Gf(s2, cc));
                                  });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) im[Rec::W + orow<4>(i) * D + ocol(j)] = acc[i][j];
  }
  {  // U = M diag(b) V
    float acc[4][8];
    zero(acc);
    gemm_staged<4, 8, true, true>(acc, C, sa, [&](int r, int s2) { return sM[r][s2]; },
                                  [&](int s2, int j) {
                                    return sB[s2] * row_at<QB>(rv, HDi, s2, j);
                                  });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) im[Rec::U + orow<4>(i) * D + ocol(j)] = acc[i][j];
  }
  __syncthreads();  // W complete
  {  // Qt = scale (Q_E - P W)
    float acc[4][8];
    zero(acc);
    gemm_staged<4, 8, true, true>(acc, C, sa, [&](int r, int s2) { return sP[r][s2]; },
                                  [&](int s2, int cc) { return im[Rec::W + s2 * D + cc]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = orow<4>(i), cc = ocol(j);
        im[Rec::QT + r * D + cc] = scale * (Qf(r, cc) * __expf(Gf(r, cc)) - acc[i][j]);
      }
  }
  for (int e = t; e < C * D; e += NT) {
    const int r = e / D, cc = e % D;
    im[Rec::KD + e] = Kf(r, cc) * __expf(Gf(C - 1, cc) - Gf(r, cc));
  }
  if (t < D) im[Rec::EC + t] = __expf(Gf(C - 1, t));
}

// Both chunk walks in one launch: block b < nb walks forward (when both run),
// the others backward; one (sequence, head, 64-column tile) each.  Thread t
// holds R[16 i + t / 16][16 j + t % 16] of the tile, i < 8, j < 4.
// Forward: R = S from the initial state; rec_f[chunk] = R at the chunk's entry.
// Backward: R = dS from dS_final; rec_b[chunk] = R at the chunk's end; dS0
// gets the gradient of the initial state.
template <bool DOB>
__global__ void __launch_bounds__(NT, 2) bwd_walk_kernel(
    const float* __restrict__ img, const void* __restrict__ d_o,
    const int32_t* __restrict__ cu, int N, int T_tot, int H, int both,
    const float* __restrict__ S0, float* __restrict__ rec_f, const float* __restrict__ dSf,
    float* __restrict__ dS0, float* __restrict__ rec_b) {
  __shared__ float sR[D][64 + 1], sZ[C][64 + 1];
  __shared__ float sS[STAGE_FLOATS];
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
  const int nch = static_cast<int>((L + C - 1) / C);
  const int t = threadIdx.x;
  const int64_t HD = (int64_t)H * D;
  const int HDi = static_cast<int>(HD);
  const int64_t sbase = ((int64_t)n * H + h) * D * D + 64 * tile;
  const float* R_init = fwd ? S0 : dSf;
  float* rec = fwd ? rec_f : rec_b;
  float R[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      R[i][j] = R_init ? R_init[sbase + (int64_t)orow<8>(i) * D + ocol(j)] : 0.0f;
  for (int it = 0; it < nch; ++it) {
    const int c = fwd ? it : nch - 1 - it;
    const int64_t pair = (bos / C + n + c) * H + h;
    const float* im = img + pair * Rec::floats;
    const int Lc = static_cast<int>(L - (int64_t)c * C < C ? L - (int64_t)c * C : C);
    const int64_t t0 = bos + (int64_t)c * C;
    ChunkPos cp;
    cp.t0 = t0;
    cp.h = h;
    cp.Lc = Lc;
    const auto rdo = chunk_rows(d_o, DOB ? 2 : 4, cp, HD);
    float* rc = rec + pair * (int64_t)(D * D) + 64 * tile;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rc[orow<8>(i) * D + ocol(j)] = R[i][j];
        sR[orow<8>(i)][ocol(j)] = R[i][j];
      }
    __syncthreads();
    {  // Z = A1 R, A1 = W (forward) or K_D (backward)
      const float* A1 = im + (fwd ? Rec::W : Rec::KD);
      float z[4][4];
      zero(z);
      gemm_staged2<4, 4, true, true>(z, D, sS,
                                    [&](int r, int cc) { return A1[r * D + cc]; },
                                    [&](int cc, int j) { return sR[cc][j]; });
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) sZ[orow<4>(i)][ocol(j)] = z[i][j];
    }
    __syncthreads();
    // R <- e^gamma_C R + [A2; A3]^T [-Z; B]: A2 = K_D / W, A3 = K_D / Qt,
    // B = U (forward) or the d_o tile (backward)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float ec = im[Rec::EC + orow<8>(i)];
#pragma unroll
      for (int j = 0; j < 4; ++j) R[i][j] *= ec;
    }
    // as three products whose operand reads have no branch of their own (a
    // branch per element made every operand load wait alone)
    const float* A2 = im + (fwd ? Rec::KD : Rec::W);
    const float* A3 = im + (fwd ? Rec::KD : Rec::QT);
    gemm_staged2<8, 4, false, true>(
        R, C, sS, [&](int cr, int kk) { return A2[kk * D + cr]; },
        [&](int kk, int j) { return -sZ[kk][j]; });
    if (fwd) {
      gemm_staged2<8, 4, false, true>(
          R, C, sS, [&](int cr, int kk) { return A3[kk * D + cr]; },
          [&](int kk, int j) { return im[Rec::U + kk * D + 64 * tile + j]; });
    } else {
      gemm_staged2<8, 4, false, true>(
          R, C, sS, [&](int cr, int kk) { return A3[kk * D + cr]; },
          [&](int kk, int j) { return row_at<DOB>(rdo, HDi, kk, 64 * tile + j); });
    }
  }
  float* R_end = fwd ? nullptr : dS0;
  if (R_end) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) R_end[sbase + (int64_t)orow<8>(i) * D + ocol(j)] = R[i][j];
  }
}

template <bool QB, bool DOB>
__global__ void __launch_bounds__(NT, 2) bwd_grad_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ d_o, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int N, int T_tot, int H, int maxnch, float scale,
    const float* __restrict__ img, const float* __restrict__ Srec,
    const float* __restrict__ dSrec, float* __restrict__ scr, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dg,
    float* __restrict__ dbeta, int64_t item0) {
  __shared__ float sT[C][C + 1], sDP[C][C + 1];
  __shared__ float sB[C], sDB[C], sGC[D];
  // the products' LDS slabs, then (pairwise phase) K, Q and gamma of a
  // quarter of the channels and the per-row-group partial sums
  constexpr int QC = D / 4;
  __shared__ float sU[3 * C * QC + 8 * QC];
  float* sa = sU;
  static_assert(STAGE_FLOATS <= 3 * C * (D / 4) + 8 * (D / 4), "stage fits the union");
  ChunkPos p;
  if (!chunk_of_block(cu, N, T_tot, H, maxnch, p, item0 + blockIdx.x)) return;
  const int t = threadIdx.x;
  const int tc = t & 15;
  const int64_t HD = (int64_t)H * D;
  const float* im = img + p.pair * Rec::floats;
  const float* S = Srec + p.pair * (int64_t)(D * D);
  const float* dS = dSrec + p.pair * (int64_t)(D * D);
  // one scratch slot per workgroup of a launch (a launch has at most GRAD_SLOTS)
  float* sc = scr + (int64_t)blockIdx.x * Scr::floats;
  const int Lc = p.Lc;
  auto tok = [&](int r, int cc) { return (p.t0 + r) * HD + (int64_t)p.h * D + cc; };
  const int HDi = static_cast<int>(HD);
  const auto rk = chunk_rows(k, QB ? 2 : 4, p, HD), rq = chunk_rows(q, QB ? 2 : 4, p, HD),
             rv = chunk_rows(v, QB ? 2 : 4, p, HD), ro = chunk_rows(d_o, DOB ? 2 : 4, p, HD);
  auto Kf = [&](int r, int cc) { return row_at<QB>(rk, HDi, r, cc); };
  auto Qf = [&](int r, int cc) { return row_at<QB>(rq, HDi, r, cc); };
  auto Vf = [&](int r, int cc) { return row_at<QB>(rv, HDi, r, cc); };
  auto dOf = [&](int r, int cc) { return row_at<DOB>(ro, HDi, r, cc); };
  auto Gf = [&](int r, int cc) { return im[Rec::G + r * D + cc]; };
  auto put8 = [&](float (&acc)[4][8], int off, float mul) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) sc[off + orow<4>(i) * D + ocol(j)] = mul * acc[i][j];
  };
  if (t < C) {
    sB[t] = t < Lc ? beta[(p.t0 + t) * H + p.h] : 0.0f;
    sDB[t] = 0.0f;
  }
  __syncthreads();
  {  // X = V - K_E S
    float acc[4][8];
    zero(acc);
    gemm_staged<4, 8, true, true>(acc, D, sa,
                                  [&](int r, int cc) { return Kf(r, cc) * __expf(Gf(r, cc)); },
                                  [&](int cc, int j) { return S[cc * D + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = orow<4>(i), col = ocol(j);
        sc[Scr::X + r * D + col] = Vf(r, col) - acc[i][j];
      }
  }
  __syncthreads();
  {  // Delta = M diag(b) X
    float acc[4][8];
    zero(acc);
    gemm_staged<4, 8, true, true>(acc, C, sa, [&](int r, int s) { return im[Rec::M + r * C + s]; },
                                  [&](int s, int j) { return sB[s] * sc[Scr::X + s * D + j]; });
    put8(acc, Scr::DL, 1.0f);
  }
  {  // dDelta = K_D dS_next + scale P^T dO
    float acc[4][8];
    zero(acc);
    gemm_staged<4, 8, true, true>(acc, D, sa,
                                  [&](int r, int cc) { return im[Rec::KD + r * D + cc]; },
                                  [&](int cc, int j) { return dS[cc * D + j]; });
    gemm_staged<4, 8, false, true>(acc, C, sa,
                                   [&](int r, int s) { return scale * im[Rec::P + s * C + r]; },
                                   [&](int s, int j) { return dOf(s, j); });
    put8(acc, Scr::DD, 1.0f);
  }
  __syncthreads();
  {  // dY = M^T dDelta, dX = diag(b) dY (= dv), dbeta += rowsum(dY . X)
    float acc[4][8];
    zero(acc);
    gemm_staged<4, 8, false, true>(acc, C, sa,
                                   [&](int r, int s) { return im[Rec::M + s * C + r]; },
                                   [&](int s, int j) { return sc[Scr::DD + s * D + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = orow<4>(i);
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = ocol(j);
        const float dX = sB[r] * acc[i][j];
        sc[Scr::DX + r * D + col] = dX;
        if (r < Lc) dv[tok(r, col)] = dX;
        part = fmaf(acc[i][j], sc[Scr::X + r * D + col], part);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) part += __shfl_xor(part, off);
      if (tc == 0) sDB[r] += part;  // the 16 lanes holding row r
    }
  }
  __syncthreads();
  {  // dM = dDelta Y^T
    float a4[4][4];
    zero(a4);
    gemm_staged<4, 4, true, false>(a4, D, sa,
                                   [&](int r, int j) { return sc[Scr::DD + r * D + j]; },
                                   [&](int j, int s) { return sB[s] * sc[Scr::X + s * D + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sT[orow<4>(i)][ocol(j)] = a4[i][j];
  }
  {  // dP = scale dO Delta^T on s <= r
    float a4[4][4];
    zero(a4);
    gemm_staged<4, 4, true, false>(a4, D, sa, [&](int r, int j) { return dOf(r, j); },
                                   [&](int j, int s) { return sc[Scr::DL + s * D + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = orow<4>(i), s = ocol(j);
        sDP[r][s] = (s <= r && r < Lc) ? scale * a4[i][j] : 0.0f;
      }
  }
  __syncthreads();
  float* dMMt = sc + Scr::DKE;  // [C][C], until dK_E is written
  {  // dM M^T
    float a4[4][4];
    zero(a4);
    gemm_staged<4, 4, true, false>(a4, C, sa, [&](int r, int u) { return sT[r][u]; },
                                   [&](int u, int s) { return im[Rec::M + s * C + u]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) dMMt[orow<4>(i) * C + ocol(j)] = a4[i][j];
  }
  __syncthreads();
  {  // dA = -M^T (dM M^T) on s < r
    float a4[4][4];
    zero(a4);
    gemm_staged<4, 4, false, true>(a4, C, sa,
                                   [&](int r, int u) { return im[Rec::M + u * C + r]; },
                                   [&](int u, int s) { return dMMt[u * C + s]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = orow<4>(i), s = ocol(j);
        sT[r][s] = (s < r && r < Lc) ? -a4[i][j] : 0.0f;
      }
  }
  {  // dK_E = -dX S^T
    float acc[4][8];
    zero(acc);
    gemm_staged<4, 8, true, false>(acc, D, sa,
                                   [&](int r, int j) { return sc[Scr::DX + r * D + j]; },
                                   [&](int j, int cc) { return S[cc * D + j]; });
    put8(acc, Scr::DKE, -1.0f);
  }
  {  // dQ_E = scale dO S^T
    float acc[4][8];
    zero(acc);
    gemm_staged<4, 8, true, false>(acc, D, sa, [&](int r, int j) { return dOf(r, j); },
                                   [&](int j, int cc) { return S[cc * D + j]; });
    put8(acc, Scr::DQE, scale);
  }
  {  // dK_D = Delta dS_next^T
    float acc[4][8];
    zero(acc);
    gemm_staged<4, 8, true, false>(acc, D, sa,
                                   [&](int r, int j) { return sc[Scr::DL + r * D + j]; },
                                   [&](int j, int cc) { return dS[cc * D + j]; });
    put8(acc, Scr::DKD, 1.0f);
  }
  {  // dbeta += sum_s dA[r, s] At[r, s]: row r on lanes 4r .. 4r + 3; each lane
     // then scales the dA entries it read by beta_r, the factor the pairwise
     // terms below take them with (the barriers of the next block order it)
    const int r = t >> 2, qd = t & 3;
    const float br = sB[r];
    float a = 0.0f;
#pragma unroll
    for (int u = 0; u < C / 4; ++u) {
      const int s2 = 4 * u + qd;
      const float da = sT[r][s2];
      a = fmaf(da, im[Rec::AT + r * C + s2], a);  // dA is 0 for s >= r
      sT[r][s2] = da * br;
    }
    a += __shfl_xor(a, 1);
    a += __shfl_xor(a, 2);
    if (qd == 0) sDB[r] += a;
  }
  {  // d e^gamma_C[c] = sum_j dS_next[c, j] S[c, j]: channel c on threads c, c + 128
    const int cc = t & (D - 1), half = t >> 7;
    float d = 0.0f;
#pragma unroll 16
    for (int j = 64 * half; j < 64 * half + 64; ++j) d = fmaf(dS[cc * D + j], S[cc * D + j], d);
    if (half == 1) sU[cc] = d;
    __syncthreads();
    if (half == 0) sGC[cc] = (d + sU[cc]) * __expf(Gf(C - 1, cc));
    __syncthreads();
  }
  // The pairwise terms, a quarter of the channels at a time: thread (channel
  // cc of the quarter, row group grp) finishes the rows x = grp, grp + 8, ...:
  // the decay-factor terms of K_E, Q_E, K_D, then the pairwise terms of At
  // and P with x as the later token (s <= x) and as the earlier one (r >= x).
  float* sK = sU;
  float* sQ = sU + C * QC;
  float* sG = sU + 2 * C * QC;
  float* sPart = sU + 3 * C * QC;  // [8][QC]
  const int cl = t & (QC - 1), grp = t >> 5;
  for (int quarter = 0; quarter < 4; ++quarter) {
    const int c0 = quarter * QC;
    for (int e = t; e < C * QC; e += NT) {
      const int r = e / QC, ch = c0 + e % QC;
      sK[e] = Kf(r, ch);
      sQ[e] = Qf(r, ch);
      sG[e] = Gf(r, ch);
    }
    __syncthreads();
    const int cc = c0 + cl;
    const float gC = sG[(C - 1) * QC + cl];
    float dgC = 0.0f;
    float nke = 0.0f, nqe = 0.0f, nkd = 0.0f;  // the next row's terms, read ahead
    if (grp < Lc) {
      nke = sc[Scr::DKE + grp * D + cc];
      nqe = sc[Scr::DQE + grp * D + cc];
      nkd = sc[Scr::DKD + grp * D + cc];
    }
    for (int x = grp; x < Lc; x += 8) {
      const float kx = sK[x * QC + cl], qx = sQ[x * QC + cl], gx = sG[x * QC + cl];
      const float E = __expf(gx), F = __expf(gC - gx);
      const float dke = nke, dqe = nqe, dkd = nkd;
      if (x + 8 < Lc) {
        nke = sc[Scr::DKE + (x + 8) * D + cc];
        nqe = sc[Scr::DQE + (x + 8) * D + cc];
        nkd = sc[Scr::DKD + (x + 8) * D + cc];
      }
      float dkx = dke * E + dkd * F;
      float dgx = (dke * kx + dqe * qx) * E - dkd * kx * F;
      float dqx = dqe * E;
      dgC = fmaf(dkd * kx, F, dgC);
      // sT rows carry beta of the row and are 0 on and above the diagonal;
      // the row's factors (kx, qx) multiply the two sums once at the end
      float sum_at = 0.0f, sum_p = 0.0f;
#pragma unroll 4
      for (int s2 = 0; s2 <= x; ++s2) {  // x later: pairs (x, s)
        const float u = __expf(gx - sG[s2 * QC + cl]) * sK[s2 * QC + cl];
        sum_at = fmaf(sT[x][s2], u, sum_at);
        sum_p = fmaf(sDP[x][s2], u, sum_p);
      }
      dkx += sum_at;
      dqx += sum_p;
      dgx += sum_at * kx + sum_p * qx;
      float sum_e = 0.0f;
#pragma unroll 4
      for (int r = x; r < Lc; ++r) {  // x earlier: pairs (r, x)
        const float w = __expf(sG[r * QC + cl] - gx);
        const float phi = sT[r][x] * sK[r * QC + cl] + sDP[r][x] * sQ[r * QC + cl];
        sum_e = fmaf(phi, w, sum_e);
      }
      dkx += sum_e;
      dgx -= sum_e * kx;
      dq[tok(x, cc)] = dqx;
      dk[tok(x, cc)] = dkx;
      sc[Scr::DX + x * D + cc] = dgx;  // dgamma, summed below
    }
    sPart[grp * QC + cl] = dgC;
    __syncthreads();
    if (t < QC) {
      float a = 0.0f;
#pragma unroll
      for (int g2 = 0; g2 < 8; ++g2) a += sPart[g2 * QC + t];
      sGC[c0 + t] += a;
    }
    __syncthreads();  // sK / sQ / sG / sPart are refilled for the next quarter
  }
  if (t < D) {  // dg: reverse cumulative sum of dgamma, plus the gamma_C terms
    const int cc = t;
    float dgam[C];
#pragma unroll
    for (int x = 0; x < C; ++x) dgam[x] = x < Lc ? sc[Scr::DX + x * D + cc] : 0.0f;
    float run = sGC[cc];
#pragma unroll
    for (int x = C - 1; x >= 0; --x) {
      run += dgam[x];
      if (x < Lc) dg[tok(x, cc)] = run;
    }
  }
  if (t < Lc) dbeta[(p.t0 + t) * H + p.h] = sDB[t];
}

}  // namespace

// The gradient kernel runs in launches of at most GRAD_SLOTS workgroups (two
// per CU), each with a scratch slot of its own, so the scratch does not grow
// with the sequence length.
constexpr int64_t GRAD_SLOTS = 512;

size_t workspace_bytes(int64_t T_tot, int N, int H) {
  const size_t pairs = (size_t)(T_tot / C + N) * (size_t)H;
  return (pairs * (size_t)(Rec::floats + 2 * D * D) + (size_t)GRAD_SLOTS * Scr::floats) *
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
  for (int64_t item0 = 0; item0 < chunk_blocks; item0 += GRAD_SLOTS) {
    const int64_t nb = chunk_blocks - item0 < GRAD_SLOTS ? chunk_blocks - item0 : GRAD_SLOTS;
#define KDA_BG(QB, OB)                                                                        \
  bwd_grad_kernel<QB, OB><<<dim3((unsigned)nb), NT, 0, s>>>(                                  \
      q, k, v, d_o, beta, cu, N, T, H, (int)maxnch, scale, img, Srec, dSrec, scr, dq, dk, dv, \
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
