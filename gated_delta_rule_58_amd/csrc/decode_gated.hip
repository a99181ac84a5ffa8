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
// HBM-bound like decode.hip: one 512-thread workgroup handles two
// consecutive (sequence, head) pairs with fp32 states (the second pair's
// loads are issued before the first pair's stores) and one pair with bf16
// states (two workgroups per CU then keep more pairs in flight than the
// in-workgroup pipeline did); every wave-wide state access is 1 KiB
// contiguous.
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
enum DecodeGate { kDX32 = 1, kDX16 = 2 };  // fp32 or bf16 gate logits

template <bool QKV_BF16, bool O_BF16, int GIN, bool S_BF16>
__global__ void __launch_bounds__(NTHR, 4) decode_gated_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const void* __restrict__ gx, const void* __restrict__ bb, bool b_bf16,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias, void* __restrict__ pool,
    const int32_t* __restrict__ slots, int64_t num_slots, void* __restrict__ o, float scale,
    int64_t pairs, int H, int alog_pc) {
  // pairs per workgroup (bf16: 2 -> 1 took the 256 x 96 step 0.287 -> 0.266 ms)
  constexpr int PAIRS = S_BF16 ? 1 : 2;
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
  __shared__ f32x4 s_v[2][D / 4];
  __shared__ f32x4 s_red[NTHR / 64][NCG][2 * NV];  // per-wave partial column sums
  __shared__ f32x4 s_sum[2][D / 4];                  // kS, qS per column
  __shared__ float s_qk[2][2];

  // Buffer resource over the state of pair p: its 128 x 128 tile, or an empty
  // range when its slot is outside the pool, so that loads read zeros and
  // stores are dropped.  Every state access then runs unconditionally, which
  // keeps the compiler's count of outstanding loads the same on every path
  // (a branch around them makes it wait for all of them at the next use of
  // any earlier load).
  constexpr int ES = S_BF16 ? 2 : 4;  // state element bytes
  struct Tile {
    __amdgpu_buffer_rsrc_t r;
    bool live;
  };
  auto state_of = [&](int64_t p) -> Tile {
    const int64_t n = p / H, h = p - n * H;
    const int64_t s = slots ? static_cast<int64_t>(slots[n]) : n;
    const bool live = s >= 0 && s < num_slots;
    const char* base = static_cast<const char*>(pool) + (live ? (s * H + h) * (D * D * ES) : 0);
    return Tile{buffer_over(base, live ? D * D * ES : 0), live};
  };
  // Small inputs of a pair in two halves: fetch issues the loads (before the
  // previous pair's stores) and keeps the raw bits, commit widens and uses
  // them (after those stores): q, k, v, decay and q.k into LDS buffer buf,
  // beta into a register.  Every thread loads (threads past the 128 channels
  // repeat the first ones), so no load sits inside a branch.
  struct Small {
    typename Raw<QKV_BF16>::T1 kk, qq, vs;
    typename Raw<GIN == kDX16>::T1 xv;
    float db, alog;
    uint32_t bbits;  // beta logit: fp32 bits, or bf16 bits in the low half
  };
  auto fetch_small = [&](int64_t p, Small& sm) {
    const int h = static_cast<int>(p % H);
    const int c = t & (D - 1);
    sm.kk = load1_raw<QKV_BF16>(k, p * D + c);
    sm.qq = load1_raw<QKV_BF16>(q, p * D + c);
    sm.vs = load1_raw<QKV_BF16>(v, p * D + c);
    sm.xv = load1_raw<GIN == kDX16>(gx, p * D + c);
    sm.db = dt_bias[h * D + c];
    sm.alog = A_log[alog_pc ? h * D + c : h];
    sm.bbits = b_bf16 ? static_cast<uint32_t>(static_cast<const uint16_t*>(bb)[p])
                      : static_cast<const uint32_t*>(bb)[p];
  };
  auto commit_small = [&](int buf, Small& sm, float& b) {
    hold(sm.kk);
    hold(sm.qq);
    hold(sm.vs);
    hold(sm.xv);
    hold(sm.db);
    hold(sm.alog);
    hold(sm.bbits);
    if (t < D) {
      const float kk = widen1<QKV_BF16>(sm.kk), qq = widen1<QKV_BF16>(sm.qq);
      s_k[buf][t] = kk;
      s_q[buf][t] = qq;
      reinterpret_cast<float*>(s_v[buf])[t] = widen1<QKV_BF16>(sm.vs);
      s_a[buf][t] =
          expf(gate_log_decay(-expf(sm.alog), gate_input(widen1<GIN == kDX16>(sm.xv), sm.db)));
      float pr = kk * qq;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) pr += __shfl_xor(pr, off);
      if ((t & 63) == 0) s_qk[buf][t >> 6] = pr;
    }
    b = gate_beta(__uint_as_float(b_bf16 ? sm.bbits << 16 : sm.bbits));
  };
  // state rows as loaded (fp32 float4 or 8 bf16), widened to fp32 only when
  // used, so the next pair's loads stay in flight across this pair's stores
  typedef typename std::conditional<S_BF16, u16x8, f32x4>::type StateRaw;
  auto load_state = [&](const Tile& tl, StateRaw* raw) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int off = ((rs + NRS * i) * D + CPT * cg) * ES;
      raw[i] = __builtin_bit_cast(StateRaw, __builtin_amdgcn_raw_buffer_load_b128(tl.r, off, 0, kBufNT));
    }
  };
  auto widen = [&](const StateRaw* raw, f32x4 (*st)[NV]) {
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
  auto store_state = [&](const Tile& tl, f32x4 (*st)[NV]) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int off = ((rs + NRS * i) * D + CPT * cg) * ES;
      if constexpr (S_BF16) {
        u16x8 r;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) r[4 * u + c] = f32_to_bf16_bits(st[i][u][c]);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, r), tl.r, off, 0, kBufNT);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, st[i][0]), tl.r, off, 0,
                                               kBufNT);
      }
    }
  };

  // The next pair's loads are issued before this pair's stores and used after
  // them; the barriers wait for LDS only, so those loads and the stores stay
  // in flight across them.
  int64_t pair = (int64_t)blockIdx.x * PAIRS;
  f32x4 st[RPT][NV];
  StateRaw raw[RPT];
  Small sm;
  float b;
  Tile cur = state_of(pair), nxt = cur;
  fetch_small(pair, sm);
  load_state(cur, raw);
  commit_small(0, sm, b);
  widen(raw, st);
#pragma unroll
  for (int j = 0; j < PAIRS; ++j, ++pair) {
    const int buf = j & 1;
    const bool more = j + 1 < PAIRS && pair + 1 < pairs;
    if (more) nxt = state_of(pair + 1);  // its slot load overlaps the sums
    barrier_lds();
    f32x4 pk[NV], pq[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) pk[u] = pq[u] = f32x4{0.f, 0.f, 0.f, 0.f};
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
    barrier_lds();
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
    barrier_lds();
    f32x4 kS[NV], qS[NV], delta[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      kS[u] = s_sum[0][(CPT * cg) / 4 + u];
      qS[u] = s_sum[1][(CPT * cg) / 4 + u];
      delta[u] = b * (s_v[buf][(CPT * cg) / 4 + u] - kS[u]);
    }
    const float qk = s_qk[buf][0] + s_qk[buf][1];
    // the next pair's loads go out before this pair's stores
    if (more) {
      fetch_small(pair + 1, sm);
      load_state(nxt, raw);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float kr = s_k[buf][rs + NRS * i];
#pragma unroll
      for (int u = 0; u < NV; ++u) st[i][u] += kr * delta[u];
    }
    store_state(cur, st);  // dropped for a slot outside the pool
    if (rs == 0) {
#pragma unroll
      for (int u = 0; u < NV; ++u)
        store4(o, pair * D + CPT * cg + 4 * u,
               cur.live ? scale * (qS[u] + qk * delta[u]) : f32x4{0.f, 0.f, 0.f, 0.f}, O_BF16);
    }
    if (!more) break;
    commit_small(buf ^ 1, sm, b);
    cur = nxt;
    widen(raw, st);
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
  const int64_t per_block = state_bf16 ? 1 : 2;  // the kernel's PAIRS
  const int64_t blocks = (pairs + per_block - 1) / per_block;
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
