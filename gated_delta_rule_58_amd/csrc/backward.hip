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
// Four launches, all fp32 (a first, plain version: correctness over speed):
//   bwd_prep  one workgroup per (chunk, head): gamma, At, P, M, W, U, Qt, K_D
//             and e^gamma_C into a per-(chunk, head) record;
//   bwd_walk  one workgroup per (sequence, head, 64-column tile), forward:
//             the entry state of every chunk; backward: the state gradient at
//             every chunk's end, and the initial state's gradient;
//   bwd_grad  one workgroup per (chunk, head): with S and dS_next known, the
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

// acc[i][j] += sum_{kk < K} a(16 i + tr, kk) b(kk, 16 j + tc) with tr = tid / 16,
// tc = tid % 16: a (16 TM) x (16 TN) output over the 256 threads.
template <int TM, int TN, typename FA, typename FB>
__device__ __forceinline__ void gemm_acc(float (&acc)[TM][TN], int K, FA a, FB b) {
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
  for (int kk = 0; kk < K; ++kk) {
    float av[TM], bv[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) av[i] = a(16 * i + tr, kk);
#pragma unroll
    for (int j = 0; j < TN; ++j) bv[j] = b(kk, 16 * j + tc);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
  }
}

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
                                               int maxnch, ChunkPos& p) {
  const int64_t b = blockIdx.x;
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

template <bool QB>
__global__ void __launch_bounds__(NT) bwd_prep_kernel(const void* __restrict__ q,
                                                      const void* __restrict__ k,
                                                      const void* __restrict__ v,
                                                      const float* __restrict__ g,
                                                      const float* __restrict__ beta,
                                                      const int32_t* __restrict__ cu, int N,
                                                      int T_tot, int H, int maxnch, float scale,
                                                      float* img) {
  __shared__ float sK[C][D + 1], sQ[C][D + 1], sG[C][D + 1];
  __shared__ float sA[C][C + 1], sP[C][C + 1], sM[C][C + 1], sB[C];
  ChunkPos p;
  if (!chunk_of_block(cu, N, T_tot, H, maxnch, p)) return;
  const int t = threadIdx.x;
  const int64_t HD = (int64_t)H * D;
  float* im = img + p.pair * Rec::floats;
  for (int e = t; e < C * D; e += NT) {
    const int r = e / D, cc = e % D;
    const bool in = r < p.Lc;
    const int64_t off = (p.t0 + r) * HD + (int64_t)p.h * D + cc;
    sK[r][cc] = in ? load1(k, off, QB) : 0.0f;
    sQ[r][cc] = in ? load1(q, off, QB) : 0.0f;
  }
  if (t < C) sB[t] = t < p.Lc ? beta[(p.t0 + t) * H + p.h] : 0.0f;
  if (t < D) {
    float run = 0.0f;
    for (int r = 0; r < C; ++r) {
      if (r < p.Lc) run += g[(p.t0 + r) * HD + (int64_t)p.h * D + t];
      sG[r][t] = run;
    }
  }
  __syncthreads();
  for (int e = t; e < C * D; e += NT) im[Rec::G + e] = sG[e / D][e % D];
  // At and P, one (r, s) pair per thread at a time
  for (int e = t; e < C * C; e += NT) {
    const int r = e / C, s = e % C;
    float a = 0.0f, pp = 0.0f;
    if (s <= r) {
      for (int cc = 0; cc < D; ++cc) {
        const float ks = sK[s][cc] * __expf(sG[r][cc] - sG[s][cc]);
        a = fmaf(sK[r][cc], ks, a);
        pp = fmaf(sQ[r][cc], ks, pp);
      }
    }
    a = s < r ? a : 0.0f;
    sA[r][s] = a;
    sP[r][s] = pp;
    im[Rec::AT + e] = a;
    im[Rec::P + e] = pp;
  }
  __syncthreads();
  // M = (I + diag(b) At)^-1, unit lower triangular: column s per thread
  if (t < C) {
    const int s = t;
    for (int r = 0; r < C; ++r) {
      float m;
      if (r < s) {
        m = 0.0f;
      } else if (r == s) {
        m = 1.0f;
      } else {
        float acc = 0.0f;
        for (int u = s; u < r; ++u) acc = fmaf(sA[r][u], sM[u][s], acc);
        m = -sB[r] * acc;
      }
      sM[r][s] = m;
    }
  }
  __syncthreads();
  for (int e = t; e < C * C; e += NT) im[Rec::M + e] = sM[e / C][e % C];
  const int tr = t >> 4, tc = t & 15;
  {  // W = M diag(b) K_E
    float acc[4][8];
    zero(acc);
    gemm_acc(acc, C, [&](int r, int s) { return sM[r][s]; },
             [&](int s, int cc) { return sB[s] * sK[s][cc] * __expf(sG[s][cc]); });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) im[Rec::W + (16 * i + tr) * D + 16 * j + tc] = acc[i][j];
  }
  {  // U = M diag(b) V
    float acc[4][8];
    zero(acc);
    gemm_acc(acc, C, [&](int r, int s) { return sM[r][s]; },
             [&](int s, int j) {
               return s < p.Lc
                          ? sB[s] * load1(v, (p.t0 + s) * HD + (int64_t)p.h * D + j, QB)
                          : 0.0f;
             });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) im[Rec::U + (16 * i + tr) * D + 16 * j + tc] = acc[i][j];
  }
  __syncthreads();  // W complete
  {  // Qt = scale (Q_E - P W)
    float acc[4][8];
    zero(acc);
    gemm_acc(acc, C, [&](int r, int s) { return sP[r][s]; },
             [&](int s, int cc) { return im[Rec::W + s * D + cc]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 16 * i + tr, cc = 16 * j + tc;
        im[Rec::QT + r * D + cc] = scale * (sQ[r][cc] * __expf(sG[r][cc]) - acc[i][j]);
      }
  }
  for (int e = t; e < C * D; e += NT) {
    const int r = e / D, cc = e % D;
    im[Rec::KD + e] = sK[r][cc] * __expf(sG[C - 1][cc] - sG[r][cc]);
  }
  if (t < D) im[Rec::EC + t] = __expf(sG[C - 1][t]);
}

// One (sequence, head, 64-column tile): thread t holds rows 8 (t / 16) .. +7
// and tile columns 4 (t % 16) .. +3 of the 128 x 64 carried matrix R.
// FWD: R = S from the initial state; rec[chunk] = R at the chunk's entry.
// Backward: R = dS from dS_final; rec[chunk] = R at the chunk's end; R_end
// gets the gradient of the initial state.
template <bool FWD, bool DOB>
__global__ void __launch_bounds__(NT) bwd_walk_kernel(const float* __restrict__ img,
                                                      const void* __restrict__ d_o,
                                                      const int32_t* __restrict__ cu, int N,
                                                      int T_tot, int H,
                                                      const float* __restrict__ R_init,
                                                      float* __restrict__ R_end,
                                                      float* __restrict__ rec) {
  __shared__ float sR[D][64 + 1], sZ[C][64 + 1];
  const int64_t b = blockIdx.x;
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
  const int rg = t >> 4, cg = t & 15;
  const int row0 = 8 * rg, col0 = 4 * cg;  // col0 within the tile
  const int jg0 = 64 * tile + col0;        // global value column
  const int64_t HD = (int64_t)H * D;
  const int64_t sbase = ((int64_t)n * H + h) * D * D;
  float R[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      R[a][e] = R_init ? R_init[sbase + (int64_t)(row0 + a) * D + jg0 + e] : 0.0f;
  const int tr = t >> 4, tc = t & 15;
  for (int it = 0; it < nch; ++it) {
    const int c = FWD ? it : nch - 1 - it;
    const int64_t pair = (bos / C + n + c) * H + h;
    const float* im = img + pair * Rec::floats;
    const int Lc = static_cast<int>(L - (int64_t)c * C < C ? L - (int64_t)c * C : C);
    const int64_t t0 = bos + (int64_t)c * C;
    float* rc = rec + pair * (int64_t)(D * D);
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rc[(row0 + a) * D + jg0 + e] = R[a][e];
        sR[row0 + a][col0 + e] = R[a][e];
      }
    __syncthreads();
    {  // Z = A1 R, A1 = W (forward) or K_D (backward)
      float z[4][4];
      zero(z);
      const float* A1 = im + (FWD ? Rec::W : Rec::KD);
      gemm_acc(z, D, [&](int r, int cc) { return A1[r * D + cc]; },
               [&](int cc, int j) { return sR[cc][j]; });
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) sZ[16 * i + tr][16 * j + tc] = z[i][j];
    }
    __syncthreads();
    // R <- e^gamma_C R - A2^T Z + A3^T B
    const float* A2 = im + (FWD ? Rec::KD : Rec::W);
    const float* A3 = im + (FWD ? Rec::KD : Rec::QT);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const float ec = im[Rec::EC + row0 + a];
#pragma unroll
      for (int e = 0; e < 4; ++e) R[a][e] *= ec;
    }
    for (int r = 0; r < C; ++r) {
      float bb[4];
      if (FWD) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bb[e] = im[Rec::U + r * D + jg0 + e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bb[e] = (d_o && r < Lc) ? load1(d_o, (t0 + r) * HD + (int64_t)h * D + jg0 + e, DOB)
                                  : 0.0f;
      }
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const float a2 = A2[r * D + row0 + a], a3 = A3[r * D + row0 + a];
#pragma unroll
        for (int e = 0; e < 4; ++e) R[a][e] = fmaf(a3, bb[e], fmaf(-a2, sZ[r][col0 + e], R[a][e]));
      }
    }
    __syncthreads();  // sR / sZ are rewritten by the next chunk
  }
  if (R_end) {
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) R_end[sbase + (int64_t)(row0 + a) * D + jg0 + e] = R[a][e];
  }
}

template <bool QB, bool DOB>
__global__ void __launch_bounds__(NT) bwd_grad_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ d_o, const float* __restrict__ beta,
    const int32_t* __restrict__ cu, int N, int T_tot, int H, int maxnch, float scale,
    const float* __restrict__ img, const float* __restrict__ Srec,
    const float* __restrict__ dSrec, float* scr, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dg,
    float* __restrict__ dbeta) {
  __shared__ float sT[C][C + 1], sDA[C][C + 1], sDP[C][C + 1];
  __shared__ float sAk[C][D], sAg[C][D], sB[C], sDB[C];
  ChunkPos p;
  if (!chunk_of_block(cu, N, T_tot, H, maxnch, p)) return;
  const int t = threadIdx.x;
  const int tr = t >> 4, tc = t & 15;
  const int64_t HD = (int64_t)H * D;
  const float* im = img + p.pair * Rec::floats;
  const float* S = Srec + p.pair * (int64_t)(D * D);
  const float* dS = dSrec + p.pair * (int64_t)(D * D);
  float* sc = scr + p.pair * Scr::floats;
  const int Lc = p.Lc;
  auto tok = [&](int r, int cc) { return (p.t0 + r) * HD + (int64_t)p.h * D + cc; };
  auto Kf = [&](int r, int cc) { return r < Lc ? load1(k, tok(r, cc), QB) : 0.0f; };
  auto Qf = [&](int r, int cc) { return r < Lc ? load1(q, tok(r, cc), QB) : 0.0f; };
  auto Vf = [&](int r, int cc) { return r < Lc ? load1(v, tok(r, cc), QB) : 0.0f; };
  auto dOf = [&](int r, int cc) {
    return (d_o && r < Lc) ? load1(d_o, tok(r, cc), DOB) : 0.0f;
  };
  auto Gf = [&](int r, int cc) { return im[Rec::G + r * D + cc]; };
  if (t < C) {
    sB[t] = t < Lc ? beta[(p.t0 + t) * H + p.h] : 0.0f;
    sDB[t] = 0.0f;
  }
  __syncthreads();
  {  // X = V - K_E S
    float acc[4][8];
    zero(acc);
    gemm_acc(acc, D, [&](int r, int cc) { return Kf(r, cc) * __expf(Gf(r, cc)); },
             [&](int cc, int j) { return S[cc * D + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 16 * i + tr, col = 16 * j + tc;
        sc[Scr::X + r * D + col] = Vf(r, col) - acc[i][j];
      }
  }
  __syncthreads();
  {  // Delta = M diag(b) X
    float acc[4][8];
    zero(acc);
    gemm_acc(acc, C, [&](int r, int s) { return im[Rec::M + r * C + s]; },
             [&](int s, int j) { return sB[s] * sc[Scr::X + s * D + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) sc[Scr::DL + (16 * i + tr) * D + 16 * j + tc] = acc[i][j];
  }
  {  // dDelta = K_D dS_next + scale P^T dO
    float acc[4][8];
    zero(acc);
    gemm_acc(acc, D, [&](int r, int cc) { return im[Rec::KD + r * D + cc]; },
             [&](int cc, int j) { return dS[cc * D + j]; });
    gemm_acc(acc, C, [&](int r, int s) { return scale * im[Rec::P + s * C + r]; },
             [&](int s, int j) { return dOf(s, j); });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) sc[Scr::DD + (16 * i + tr) * D + 16 * j + tc] = acc[i][j];
  }
  __syncthreads();
  {  // dY = M^T dDelta, dX = diag(b) dY (= dv), dbeta += rowsum(dY . X)
    float acc[4][8];
    zero(acc);
    gemm_acc(acc, C, [&](int r, int s) { return im[Rec::M + s * C + r]; },
             [&](int s, int j) { return sc[Scr::DD + s * D + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * i + tr;
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = 16 * j + tc;
        const float dX = sB[r] * acc[i][j];
        sc[Scr::DX + r * D + col] = dX;
        if (r < Lc) dv[tok(r, col)] = dX;
        part = fmaf(acc[i][j], sc[Scr::X + r * D + col], part);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) part += __shfl_xor(part, off);
      if (tc == 0) sDB[r] += part;
    }
  }
  __syncthreads();
  {  // dM = dDelta Y^T
    float a4[4][4];
    zero(a4);
    gemm_acc(a4, D, [&](int r, int j) { return sc[Scr::DD + r * D + j]; },
             [&](int j, int s) { return sB[s] * sc[Scr::X + s * D + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sT[16 * i + tr][16 * j + tc] = a4[i][j];
  }
  {  // dP = scale dO Delta^T on s <= r
    float a4[4][4];
    zero(a4);
    gemm_acc(a4, D, [&](int r, int j) { return dOf(r, j); },
             [&](int j, int s) { return sc[Scr::DL + s * D + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * i + tr, s = 16 * j + tc;
        sDP[r][s] = (s <= r && r < Lc) ? scale * a4[i][j] : 0.0f;
      }
  }
  __syncthreads();
  {  // dM M^T
    float a4[4][4];
    zero(a4);
    gemm_acc(a4, C, [&](int r, int u) { return sT[r][u]; },
             [&](int u, int s) { return im[Rec::M + s * C + u]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sDA[16 * i + tr][16 * j + tc] = a4[i][j];
  }
  __syncthreads();
  {  // dA = -M^T (dM M^T) on s < r
    float a4[4][4];
    zero(a4);
    gemm_acc(a4, C, [&](int r, int u) { return im[Rec::M + u * C + r]; },
             [&](int u, int s) { return sDA[u][s]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * i + tr, s = 16 * j + tc;
        sT[r][s] = (s < r && r < Lc) ? -a4[i][j] : 0.0f;
      }
  }
  __syncthreads();
  if (t < C) {  // dbeta += sum_s dA[r, s] At[r, s]
    float a = 0.0f;
    for (int s = 0; s < t; ++s) a = fmaf(sT[t][s], im[Rec::AT + t * C + s], a);
    sDB[t] += a;
  }
  {  // dK_E = -dX S^T
    float acc[4][8];
    zero(acc);
    gemm_acc(acc, D, [&](int r, int j) { return sc[Scr::DX + r * D + j]; },
             [&](int j, int cc) { return S[cc * D + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) sc[Scr::DKE + (16 * i + tr) * D + 16 * j + tc] = -acc[i][j];
  }
  {  // dQ_E = scale dO S^T
    float acc[4][8];
    zero(acc);
    gemm_acc(acc, D, [&](int r, int j) { return dOf(r, j); },
             [&](int j, int cc) { return S[cc * D + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        sc[Scr::DQE + (16 * i + tr) * D + 16 * j + tc] = scale * acc[i][j];
  }
  {  // dK_D = Delta dS_next^T
    float acc[4][8];
    zero(acc);
    gemm_acc(acc, D, [&](int r, int j) { return sc[Scr::DL + r * D + j]; },
             [&](int j, int cc) { return dS[cc * D + j]; });
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) sc[Scr::DKD + (16 * i + tr) * D + 16 * j + tc] = acc[i][j];
  }
  __syncthreads();
  if (t < D) {  // key channel cc: the decay factors and the pairwise terms of At and P
    const int cc = t;
    const float gC = Gf(C - 1, cc);
    float dgC = 0.0f;
    for (int j = 0; j < D; ++j) dgC = fmaf(dS[cc * D + j], S[cc * D + j], dgC);
    dgC *= __expf(gC);
    for (int r = 0; r < C; ++r) {
      const float kr = Kf(r, cc), qr = Qf(r, cc), gr = Gf(r, cc);
      const float E = __expf(gr), F = __expf(gC - gr);
      const float dke = sc[Scr::DKE + r * D + cc], dqe = sc[Scr::DQE + r * D + cc];
      const float dkd = sc[Scr::DKD + r * D + cc];
      sAk[r][cc] = dke * E + dkd * F;
      sAg[r][cc] = (dke * kr + dqe * qr) * E - dkd * kr * F;
      dgC = fmaf(dkd * kr, F, dgC);
    }
    for (int r = 0; r < Lc; ++r) {
      const float kr = Kf(r, cc), qr = Qf(r, cc), gr = Gf(r, cc), br = sB[r];
      float dkr = 0.0f, dqr = 0.0f, dgr = 0.0f;
      for (int s = 0; s <= r; ++s) {
        const float w = __expf(gr - Gf(s, cc));
        const float u = w * Kf(s, cc);
        const float al = s < r ? sT[r][s] * br : 0.0f;
        const float pi = sDP[r][s];
        const float phi = al * kr + pi * qr;
        dkr = fmaf(al, u, dkr);
        dqr = fmaf(pi, u, dqr);
        dgr = fmaf(phi, u, dgr);
        sAk[s][cc] = fmaf(phi, w, sAk[s][cc]);
        sAg[s][cc] = fmaf(-phi, u, sAg[s][cc]);
      }
      sAk[r][cc] += dkr;
      sAg[r][cc] += dgr;
      dq[tok(r, cc)] = sc[Scr::DQE + r * D + cc] * __expf(gr) + dqr;
    }
    float run = dgC;
    for (int r = Lc - 1; r >= 0; --r) {
      run += sAg[r][cc];
      dg[tok(r, cc)] = run;
      dk[tok(r, cc)] = sAk[r][cc];
    }
  }
  if (t < Lc) dbeta[(p.t0 + t) * H + p.h] = sDB[t];
}

}  // namespace

size_t workspace_bytes(int64_t T_tot, int N, int H) {
  const size_t pairs = (size_t)(T_tot / C + N) * (size_t)H;
  return pairs * (size_t)(Rec::floats + 2 * D * D + Scr::floats) * sizeof(float);
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
  if (chunk_blocks > 0x7fffffff || walk_blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (chunk_blocks > 0) {
    if (qkv_bf16)
      bwd_prep_kernel<true><<<dim3((unsigned)chunk_blocks), NT, 0, s>>>(
          q, k, v, g, beta, cu, N, T, H, (int)maxnch, scale, img);
    else
      bwd_prep_kernel<false><<<dim3((unsigned)chunk_blocks), NT, 0, s>>>(
          q, k, v, g, beta, cu, N, T, H, (int)maxnch, scale, img);
    bwd_walk_kernel<true, false><<<dim3((unsigned)walk_blocks), NT, 0, s>>>(
        img, nullptr, cu, N, T, H, S0, nullptr, Srec);
  }
  if (do_bf16)
    bwd_walk_kernel<false, true><<<dim3((unsigned)walk_blocks), NT, 0, s>>>(
        img, d_o, cu, N, T, H, dS_final, dS0, dSrec);
  else
    bwd_walk_kernel<false, false><<<dim3((unsigned)walk_blocks), NT, 0, s>>>(
        img, d_o, cu, N, T, H, dS_final, dS0, dSrec);
  if (chunk_blocks > 0) {
#define KDA_BG(QB, OB)                                                                        \
  bwd_grad_kernel<QB, OB><<<dim3((unsigned)chunk_blocks), NT, 0, s>>>(                        \
      q, k, v, d_o, beta, cu, N, T, H, (int)maxnch, scale, img, Srec, dSrec, scr, dq, dk, dv, \
      dg, dbeta)
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
