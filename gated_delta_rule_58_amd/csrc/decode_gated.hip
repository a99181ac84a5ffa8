// kda_recurrent_decode_gated: the one-token recurrent step of decode.hip for
// serving, with the gate fused in and the states kept in a slot pool.
//
// Per (sequence n, head h) with state S = pool[slot(n), h] (128 x 128, S[c][j]):
//   g     = -exp(A_log) softplus(x + dt_bias[h])   beta = sigmoid(b)
//           (A_log per head, or per (head, channel) when given as [H, 128])
//           (the arithmetic of kda_gate, per key channel; g never goes to memory)
//   S'    = Diag(exp(g)) S
//   delta = beta (v - S'^T k),   o = scale (S'^T q + (q.k) delta),   S = S' + k delta^T
// which is S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T with
// o = S_t^T q (the code audit's fused recurrent one-token decode regime); the
// gate's inputs are those of FlashKDA's interface (Kimi K3 artifact audit,
// §7.1).  The pool holds fp32 or bf16 states (bf16 halves the state traffic;
// each step rounds the new state to bf16, round to nearest even, which is
// part of what that mode computes).  slot(n) = state_indices[n], or n when no
// indices are given; a slot outside [0, num_slots) skips the sequence: its o
// is written as zeros and no state is touched.
//
// HBM-bound like decode.hip: one 512-thread workgroup handles two consecutive
// (sequence, head) pairs, the second pair's state loads are issued before the
// first pair's stores, and every wave-wide state access is 1 KiB contiguous.
// fp32 states: thread t holds 4 columns (4*(t%32)..) of the 8 key rows
// t/32 + 16 i; bf16 states: 8 columns (8*(t%16)..) of the 4 rows t/16 + 32 i.
// The column sums kS = S'^T k and qS = S'^T q run over a thread's rows, the
// lanes of a wave that share its columns (shuffles), then the 8 waves: one
// thread per column and sum adds the wave partials in LDS and every thread
// reads back only its own columns' totals.
#include <type_traits>

#include "gate_math.hpp"
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

constexpr int D = 128;
constexpr int NTHR = 512;
constexpr int PAIRS_PER_BLOCK = 2;
enum DecodeGate { kDX32 = 1, kDX16 = 2 };  // fp32 or bf16 gate logits

template <bool QKV_BF16, bool O_BF16, int GIN, bool S_BF16>
__global__ void __launch_bounds__(NTHR, 4) decode_gated_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ gx, const void* __restrict__ bb, bool b_bf16,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias, void* __restrict__ pool,
    const int32_t* __restrict__ slots, int64_t num_slots, void* __restrict__ o, float scale,
    int64_t pairs, int H, int alog_pc) {
  constexpr int CPT = S_BF16 ? 8 : 4;  // columns per thread
  constexpr int NCG = D / CPT;         // column groups
  constexpr int NRS = NTHR / NCG;      // row slots
  constexpr int RPT = D / NRS;         // rows per thread
  constexpr int NV = CPT / 4;          // float4 per row slice
  const int t = threadIdx.x;
  const int cg = t % NCG;
  const int rs = t / NCG;
  const int w = t >> 6;

  __shared__ float s_k[2][D], s_q[2][D], s_a[2][D];
  __shared__ f32x4 s_red[NTHR / 64][NCG][2 * NV];  // per-wave partial column sums
  __shared__ f32x4 s_sum[2][D / 4];                  // kS, qS per column
  __shared__ float s_qk[2][2];

  // state element offset of pair p, or -1 when its slot is outside the pool
  auto state_of = [&](int64_t p) -> int64_t {
    const int64_t n = p / H, h = p - n * H;
    const int64_t s = slots ? static_cast<int64_t>(slots[n]) : n;
    return (s >= 0 && s < num_slots) ? (s * H + h) * (D * D) : -1;
  };
  // Small inputs of a pair in two halves: fetch issues the loads (before the
  // previous pair's stores), commit uses them (after those stores): q, k,
  // decay and q.k into LDS buffer buf, this thread's v and beta.
  struct Small {
    float kk, qq, xv, db, alog, braw;
    f32x4 vv[NV];
  };
  auto fetch_small = [&](int64_t p, Small& sm) {
    const int h = static_cast<int>(p % H);
    if (t < D) {
      sm.kk = load1(k, p * D + t, QKV_BF16);
      sm.qq = load1(q, p * D + t, QKV_BF16);
      sm.xv = load1(gx, p * D + t, GIN == kDX16);
      sm.db = dt_bias[h * D + t];
      sm.alog = A_log[alog_pc ? h * D + t : h];
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) sm.vv[u] = load4(v, p * D + CPT * cg + 4 * u, QKV_BF16);
    sm.braw = load1(bb, p, b_bf16);
  };
  auto commit_small = [&](int buf, const Small& sm, f32x4* vv, float& b) {
    if (t < D) {
      s_k[buf][t] = sm.kk;
      s_q[buf][t] = sm.qq;
      s_a[buf][t] = expf(gate_log_decay(-expf(sm.alog), gate_input(sm.xv, sm.db)));
      float pr = sm.kk * sm.qq;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) pr += __shfl_xor(pr, off);
      if ((t & 63) == 0) s_qk[buf][t >> 6] = pr;
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) vv[u] = sm.vv[u];
    b = gate_beta(sm.braw);
  };
  // state rows as loaded (fp32 float4 or 8 bf16), widened to fp32 only when
  // used, so the next pair's loads stay in flight across this pair's stores
  typedef typename std::conditional<S_BF16, u16x8, f32x4>::type Raw;
  auto load_state = [&](int64_t so, Raw* raw) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int64_t e = so + (int64_t)(rs + NRS * i) * D + CPT * cg;
      if constexpr (S_BF16)
        raw[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(pool) + e));
      else
        raw[i] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(static_cast<const float*>(pool) + e));
    }
  };
  auto widen = [&](const Raw* raw, f32x4 (*st)[NV]) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      if constexpr (S_BF16) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
          st[i][u] = f32x4{bf16_bits_to_f32(raw[i][4 * u]), bf16_bits_to_f32(raw[i][4 * u + 1]),
                           bf16_bits_to_f32(raw[i][4 * u + 2]), bf16_bits_to_f32(raw[i][4 * u + 3])};
      } else {
        st[i][0] = raw[i];
      }
    }
  };
  auto store_state = [&](int64_t so, f32x4 (*st)[NV]) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int64_t e = so + (int64_t)(rs + NRS * i) * D + CPT * cg;
      if constexpr (S_BF16) {
        u16x8 r;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) r[4 * u + c] = f32_to_bf16_bits(st[i][u][c]);
        __builtin_nontemporal_store(r, reinterpret_cast<u16x8*>(static_cast<uint16_t*>(pool) + e));
      } else {
        __builtin_nontemporal_store(st[i][0],
                                    reinterpret_cast<f32x4*>(static_cast<float*>(pool) + e));
      }
    }
  };

  int64_t pair = (int64_t)blockIdx.x * PAIRS_PER_BLOCK;
  f32x4 st[RPT][NV];
  Raw raw[RPT];
  Small sm;
  f32x4 vv[NV];
  float b;
  int64_t so = state_of(pair);
  fetch_small(pair, sm);
  if (so >= 0) load_state(so, raw);
  commit_small(0, sm, vv, b);
  if (so >= 0) widen(raw, st);
#pragma unroll
  for (int j = 0; j < PAIRS_PER_BLOCK; ++j, ++pair) {
    const int buf = j & 1;
    const bool live = so >= 0;
    const bool more = j + 1 < PAIRS_PER_BLOCK && pair + 1 < pairs;
    const int64_t son = more ? state_of(pair + 1) : -1;  // its slot load overlaps the sums
    __syncthreads();
    f32x4 pk[NV], pq[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) pk[u] = pq[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (live) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = rs + NRS * i;
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          st[i][u] *= s_a[buf][r];
          pk[u] += s_k[buf][r] * st[i][u];
          pq[u] += s_q[buf][r] * st[i][u];
        }
      }
    }
    // lanes of this wave holding the same columns: lane bits above log2(NCG)
#pragma unroll
    for (int off = NCG; off < 64; off <<= 1)
#pragma unroll
      for (int u = 0; u < NV; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pk[u][e] += __shfl_xor(pk[u][e], off);
          pq[u][e] += __shfl_xor(pq[u][e], off);
        }
    if ((t & 63) < NCG) {
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        s_red[w][cg][u] = pk[u];
        s_red[w][cg][NV + u] = pq[u];
      }
    }
    __syncthreads();
    // the 8 wave partials of each column summed once (threads 0..255: kS, qS)
    if (t < 2 * D) {
      const int typ = t / D, col = t % D;
      const float* fr = reinterpret_cast<const float*>(s_red);
      const int off = ((col / CPT) * 2 * NV + typ * NV + (col % CPT) / 4) * 4 + col % 4;
      float acc = fr[off];
#pragma unroll
      for (int jj = 1; jj < NTHR / 64; ++jj) acc += fr[jj * NCG * 2 * NV * 4 + off];
      reinterpret_cast<float*>(s_sum)[typ * D + col] = acc;
    }
    __syncthreads();
    f32x4 kS[NV], qS[NV], delta[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      kS[u] = s_sum[0][(CPT * cg) / 4 + u];
      qS[u] = s_sum[1][(CPT * cg) / 4 + u];
      delta[u] = b * (vv[u] - kS[u]);
    }
    const float qk = s_qk[buf][0] + s_qk[buf][1];
    // next pair's loads go out before this pair's stores
    if (more) {
      fetch_small(pair + 1, sm);
      if (son >= 0) load_state(son, raw);
    }
    if (live) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float kr = s_k[buf][rs + NRS * i];
#pragma unroll
        for (int u = 0; u < NV; ++u) st[i][u] += kr * delta[u];
      }
      store_state(so, st);
    }
    if (rs == 0) {
#pragma unroll
      for (int u = 0; u < NV; ++u)
        store4(o, pair * D + CPT * cg + 4 * u,
               live ? scale * (qS[u] + qk * delta[u]) : f32x4{0.f, 0.f, 0.f, 0.f}, O_BF16);
    }
    if (!more) break;
    commit_small(buf ^ 1, sm, vv, b);
    if (son >= 0) widen(raw, st);
    so = son;
  }
}

}  // namespace

hipError_t launch_decode_gated(const void* q, const void* k, const void* v, bool qkv_bf16,
                               const void* gx, bool x_bf16, const void* b, bool b_bf16,
                               const float* A_log, bool alog_pc, const float* dt_bias, void* pool,
                               bool state_bf16, int64_t num_slots, const int32_t* slots, void* o,
                               bool o_bf16, int N, int H, float scale, hipStream_t s) {
  const int64_t pairs = (int64_t)N * H;
  if (pairs == 0) return hipSuccess;
  const int64_t blocks = (pairs + PAIRS_PER_BLOCK - 1) / PAIRS_PER_BLOCK;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
#define KDA_DG(QB, OB, GM, SB)                                                              \
  decode_gated_kernel<QB, OB, GM, SB><<<grid, NTHR, 0, s>>>(q, k, v, gx, b, b_bf16, A_log, \
                                                            dt_bias, pool, slots, num_slots, \
                                                            o, scale, pairs, H, alog_pc ? 1 : 0)
#define KDA_DG_S(QB, OB, GM) \
  do {                       \
    if (state_bf16)          \
      KDA_DG(QB, OB, GM, true); \
    else                     \
      KDA_DG(QB, OB, GM, false); \
  } while (0)
#define KDA_DG_G(QB, OB)                \
  do {                                  \
    if (x_bf16) KDA_DG_S(QB, OB, kDX16); \
    else KDA_DG_S(QB, OB, kDX32);       \
  } while (0)
  if (qkv_bf16 && o_bf16) KDA_DG_G(true, true);
  else if (qkv_bf16) KDA_DG_G(true, false);
  else if (o_bf16) KDA_DG_G(false, true);
  else KDA_DG_G(false, false);
#undef KDA_DG_G
#undef KDA_DG_S
#undef KDA_DG
  return hipGetLastError();
}

}  // namespace kda
