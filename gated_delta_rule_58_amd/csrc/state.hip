// State kernel of kda_chunk_prefill: the inter-chunk recurrence.
//
// One workgroup per (sequence, head, 64-column value tile); it walks the
// chunks of its sequence in order.  Per chunk, with the chunk's workspace
// image (written by the prep kernel) in LDS:
//   X     = V - (K e^gamma) S                      (S the entry state)
//   Delta = (I + A)^-1 diag(b) X                   (the prep kernel inverts)
//   O     = scale ((Q e^gamma) S + P Delta)
//   S    <- Diag(e^gamma_C) S + (K e^(gamma_C - gamma))^T Delta
//
// Waves 0..3 compute.  Every product is independent across value columns, so
// compute wave w owns columns 16w..16w+15 of the tile and keeps its 128x16
// slice of S, and its 64x16 slices of X, Delta and O, in MFMA accumulators:
// no barriers inside a chunk.  An accumulator tile holds rows 4lg..4lg+3 of
// column lr in lane (lr, lg); a pair of them is the B fragment of a 16x16x32
// product (contraction index 16(e>>2) + 4lg + (e&3)) and, unchanged, the A
// fragment of the transposed product, so S and Delta never leave their
// registers.  The image operands are read in the matching order.
// The output is computed transposed, O^T = S^T (Q e^gamma)^T + Delta^T P^T:
// the same fragments with the operands swapped, so each lane ends up with four
// consecutive columns of one token row.
//
// Waves 4 and 5 move data.  While chunk c is computed they store chunk c-1's
// output tile from LDS to o and copy chunk c+1's image (59 KiB) and v tile
// into the other LDS buffers with 16-byte buffer-to-LDS loads, so the compute
// waves never wait on a memory instruction.  The copy is split over two waves
// so that neither has more memory instructions in flight than its counter
// holds (63): one wave issuing all 75 of them stalls on its own first loads.
// Two workgroup barriers per chunk (image front, image back), so the copy of
// the next chunk streams without a gap.  (fp32 v or o, used only off the
// benchmarked path, go through the compute waves' registers instead.)
//
// Precision: operands are fp16 MFMA fragments with fp32 accumulation; X and
// Delta enter the products as hi+lo fp16 pairs, the state as one fp16 value
// (its rounding is not carried: S itself stays fp32 in the accumulators).
#include "chunk_common.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace chunk {
namespace {

constexpr int DV = 64;  // value columns per workgroup
constexpr int NT = D / DV;
constexpr int NTHR_S = NTHR + 128;  // 4 compute waves + 2 data waves
constexpr int IMG_UNITS = Ws::bytes / 1024;
constexpr int TILE_BYTES = C * DV * 2;  // bf16 v or o tile of one chunk

struct StateLds {
  static constexpr int off_img = 0;                             // 2 images
  static constexpr int off_v = off_img + 2 * Ws::bytes;         // 2 bf16 v tiles
  static constexpr int off_o = off_v + 2 * TILE_BYTES;          // 2 bf16 o tiles
  static constexpr int total = off_o + 2 * TILE_BYTES;
};
// byte offset of (row r, column j < 64) in the bf16 o tile, written 4 columns
// of one row per lane with the 16 rows of a tile on distinct 16-byte slots.
__device__ __forceinline__ int otile_off(int r, int j) {
  return r * 128 + ((((j >> 3) ^ (r & 7))) << 4) + ((j & 7) << 1);
}
__device__ __forceinline__ int otile_swz(int r) { return r & 7; }
// Image halves: the front (K e^gamma, Q e^gamma) is what a chunk's first
// products read, the back (the rest) what its later products read.
constexpr int FRONT_UNITS = Ws::KDT / 1024;          // 32
constexpr int BACK_UNITS = IMG_UNITS - FRONT_UNITS;  // 27
static_assert(Ws::KE == 0 && Ws::QE + 16384 == Ws::KDT, "front = KE, QE");
// s_waitcnt immediate that waits until at most N vector-memory operations of
// this wave are outstanding (lgkm and export counts left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
static_assert(StateLds::total <= 160 * 1024, "LDS budget");

// byte offset of (row r, column j < 64) in the bf16 v tile: 128-byte rows,
// 16-byte chunk j>>3 swizzled so the four row groups 4lg+i of an accumulator
// tile (read one element per lane) hit disjoint banks.
__device__ __forceinline__ int vtile_off(int r, int j) {
  return r * 128 + ((((j >> 3) ^ (((r >> 2) & 3) << 1))) << 4) + ((j & 7) << 1);
}
__device__ __forceinline__ int vtile_swz(int r) { return ((r >> 2) & 3) << 1; }

template <bool QKV_BF16, bool O_BF16>
__global__ void __launch_bounds__(NTHR_S, 1) state_kernel(
    const void* __restrict__ v, const int32_t* __restrict__ cu, int N, int T_tot, int H, int Hp,
    StateIO sio, void* __restrict__ o, float scale, int c_lo, int S_len,
    const char* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) char lds[StateLds::total];
  __shared__ int s_seq[1];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const bool mover = w >= 4;

  // ---- block -> (sequence rank, head, value tile); head % 8 == block % 8 so
  // both tiles of a head, and the prep blocks of its chunks, share one XCD.
  const int hx = blockIdx.x & 7;
  int rest = blockIdx.x >> 3;
  const int tile = rest % NT;
  rest /= NT;
  const int hgroups = Hp >> 3;
  const int h = (rest % hgroups) * 8 + hx;
  const int rank = rest / hgroups;
  if (h >= H) return;
  const int n = lpt_sequence(cu, N, T_tot, rank, s_seq);
  int bos = cu[n], eos = cu[n + 1];
  bos = bos < 0 ? 0 : (bos > T_tot ? T_tot : bos);
  eos = eos < bos ? bos : (eos > T_tot ? T_tot : eos);
  const int nch = (eos - bos + C - 1) / C;
  const int c_end = (c_lo + S_len) < nch ? (c_lo + S_len) : nch;
  const int HD = H * D;
  const int col0 = tile * DV;
  const int jl = 16 * (w & 3) + lr;  // column of the tile owned by this lane (compute waves)
  const int jcol = col0 + jl;
  constexpr int QS = QKV_BF16 ? 2 : 4;
  constexpr int OS = O_BF16 ? 2 : 4;
  auto rows_of = [&](int c) { return (eos - bos - c * C) < C ? (eos - bos - c * C) : C; };
  auto img_of = [&](int c) { return lds + StateLds::off_img + ((c - c_lo) & 1) * Ws::bytes; };
  auto vt_of = [&](int c) { return lds + StateLds::off_v + ((c - c_lo) & 1) * TILE_BYTES; };
  auto ot_of = [&](int c) { return lds + StateLds::off_o + ((c - c_lo) & 1) * TILE_BYTES; };
  // buffer over rows [bos + cC, bos + cC + rows) of head h, columns col0.. of the tile
  auto tok_buf = [&](const void* base, int esz, int c) {
    const char* b = static_cast<const char*>(base) +
                    ((int64_t)(bos + c * C) * HD + (int64_t)h * D + col0) * esz;
    return make_buf(b, (uint32_t)(rows_of(c) * HD * esz - (h * D + col0) * esz));
  };

  // ---- data waves: the front or the back of chunk c's image into LDS.  Each
  // wave takes half of either part; wave 5 adds the v tile to the front.
  const int mw = w - 4;
  constexpr int F0 = FRONT_UNITS / 2, B0 = BACK_UNITS / 2;  // wave 4: 16 + 13 ops
  constexpr int F1 = FRONT_UNITS - F0 + (QKV_BF16 ? 8 : 0);  // wave 5: 16 (+8 v) + 14 ops
  constexpr int B1 = BACK_UNITS - B0;
  auto img_src = [&](int c) {
    return make_buf(ws + ((int64_t)(n * S_len + (c - c_lo)) * H + h) * Ws::bytes, Ws::bytes);
  };
  auto load_front = [&](int c) {
    const auto rs = img_src(c);
    char* dst = img_of(c);
    const int u0 = mw == 0 ? 0 : FRONT_UNITS / 2, u1 = mw == 0 ? FRONT_UNITS / 2 : FRONT_UNITS;
#pragma unroll 2
    for (int u = u0; u < u1; ++u)
      buf_to_lds16(rs, (lds_ptr_t)(dst + u * 1024), lane * 16, u * 1024);
    if (mw == 0) return;
    if constexpr (QKV_BF16) {  // 8 rows of 128 bytes per round; lane writes slot lane&7
      const auto rv = tok_buf(v, 2, c);
      char* vt = vt_of(c);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = 8 * u + (lane >> 3);
        const int j = (lane & 7) ^ vtile_swz(r);  // logical chunk for LDS slot lane&7
        buf_to_lds16(rv, (lds_ptr_t)(vt + u * 1024), (lane >> 3) * HD * 2 + j * 16,
                     8 * u * HD * 2);
      }
    }
  };
  auto store_o = [&](int c) {  // rows [32 mw, 32 mw + 32) of chunk c's bf16 o tile
    const auto ro = tok_buf(o, 2, c);
    const char* ot = ot_of(c);
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int u = 4 * mw; u < 4 * mw + 4; ++u) {
      const int r = 8 * u + (lane >> 3);
      const int j = (lane & 7) ^ otile_swz(r);  // logical chunk held by slot lane&7
      const u32x4 x = *reinterpret_cast<const u32x4*>(ot + r * 128 + (lane & 7) * 16);
      __builtin_amdgcn_raw_buffer_store_b128(x, ro, (lane >> 3) * HD * 2 + j * 16,
                                             8 * u * HD * 2, 0);
    }
  };
  auto load_back = [&](int c) {
    const auto rs = img_src(c);
    char* dst = img_of(c);
    const int u0 = FRONT_UNITS + (mw == 0 ? 0 : B0), u1 = mw == 0 ? FRONT_UNITS + B0 : IMG_UNITS;
#pragma unroll 2
    for (int u = u0; u < u1; ++u)
      buf_to_lds16(rs, (lds_ptr_t)(dst + u * 1024), lane * 16, u * 1024);
  };

  // ---- state slice (compute waves): tile t holds key rows 16t + 4lg + i, column jcol.
  f32x4 Sacc[8];
  if (!mover) {
    const int64_t si = sio.in_idx ? static_cast<int64_t>(sio.in_idx[n]) : n;
    if (sio.in && si >= 0 && si < sio.in_slots) {
      const int64_t sbase = (si * H + h) * D * D;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t e = sbase + (int64_t)(16 * t + 4 * lg + i) * D + jcol;
          Sacc[t][i] = sio.in_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(sio.in)[e])
                                   : static_cast<const float*>(sio.in)[e];
        }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) Sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // fp32 v: loaded by the compute waves one chunk ahead
  uint32_t vraw[16];
  auto load_v_regs = [&](int c) {
    const auto rv = tok_buf(v, 4, c);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vraw[4 * rt + i] = __builtin_amdgcn_raw_buffer_load_b32(
            rv, (4 * lg * HD + jl) * 4, (16 * rt + i) * HD * 4, 0);
  };

  // Two workgroup barriers per chunk c: A once its image front (and v tile)
  // is in LDS, B once its back is.  The data waves keep the stream going:
  // the front of c+1 is issued right after B(c-1) (the front of c-1 is read
  // by then) and the back of c+1 right after A(c) (the back of c-1 likewise),
  // and each wave waits with a counter bound that leaves the later part in
  // flight.  The compute waves write o tiles into LDS (bf16 o), which the data
  // waves store after the next A barrier, or straight to o (fp32 o).  The
  // barriers carry no memory fence (a fence would drain the data waves'
  // loads): the data waves wait for their own copies with counter bounds, and
  // every LDS read of a buffer feeds a product before the barrier after which
  // that buffer is refilled.
  // (Separate loops for the two roles: the compiler's counter analysis then
  // never sees a buffer-to-LDS copy pending on the compute waves' path, which
  // would make every chunk's first LDS read wait for all their o stores.)
  if (mover) {
    if (c_lo < c_end) {
      load_front(c_lo);
      load_back(c_lo);
    }
    for (int c = c_lo; c < c_end; ++c) {
      const bool more = c + 1 < c_end;
      if (more) load_front(c + 1);
      // front of c done: at most back(c) [+ front(c+1)] outstanding
      if (mw == 0) {
        if (more) wait_vm_le<B0 + F0>();
        else wait_vm_le<B0>();
      } else {
        if (more) wait_vm_le<B1 + F1>();
        else wait_vm_le<B1>();
      }
      barrier_nofence();  // A(c)
      if (more) load_back(c + 1);
      // chunk c-1's o tile is complete (its writers passed A(c)); the stores
      // only add to the counter, which keeps the waits below conservative
      if constexpr (O_BF16) {
        if (c > c_lo) store_o(c - 1);
      }
      // back of c done: at most front(c+1) + back(c+1) outstanding
      if (more) {
        if (mw == 0) wait_vm_le<F0 + B0>();
        else wait_vm_le<F1 + B1>();
      } else {
        wait_vmem();
      }
      barrier_nofence();  // B(c)
    }
    if constexpr (O_BF16) {
      if (c_lo < c_end) {
        barrier_nofence();  // A(c_end): the last o tile is complete
        store_o(c_end - 1);
      }
    }
    return;
  }

  if constexpr (!QKV_BF16) {
    if (c_lo < c_end) load_v_regs(c_lo);
  }
  for (int c = c_lo; c < c_end; ++c) {
    const bool more = c + 1 < c_end;
    if constexpr (!QKV_BF16) wait_vmem();  // this chunk's v registers
    barrier_nofence();  // A(c)
    {
      const char* im = img_of(c);
      float vcur[16];
      if constexpr (QKV_BF16) {
        const char* vt = vt_of(c);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            vcur[4 * rt + i] = bf16_bits_to_f32(
                *reinterpret_cast<const uint16_t*>(vt + vtile_off(16 * rt + 4 * lg + i, jl)));
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) vcur[i] = __uint_as_float(vraw[i]);
        if (more) load_v_regs(c + 1);
      }

      // X = V - Ke S (rows = tokens) and O^T = S^T Qe^T (rows = value columns),
      // 16x16x32 products over the four 32-channel steps kk.  The S tile pair
      // (2kk, 2kk+1) is the B fragment of the first and, unchanged, the A
      // fragment of the second; the Ke / Qe fragment holds the matching
      // channels 32kk + 4lg + e and 32kk + 16 + 4lg + e.
      f32x4 Xacc[4], Oacc[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) Xacc[rt] = Oacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const f32x4 s0 = Sacc[2 * kk], s1 = Sacc[2 * kk + 1];
        const f16x8 sf = cvt_f16(f32x8{s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]});
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int po = keqe_frag(rt, kk, lr, lg);
          const f16x8 ak = *reinterpret_cast<const f16x8*>(im + Ws::KE + po);
          const f16x8 aq = *reinterpret_cast<const f16x8*>(im + Ws::QE + po);
          Xacc[rt] = mma_f16(ak, sf, Xacc[rt]);
          Oacc[rt] = mma_f16(sf, aq, Oacc[rt]);
        }
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) Xacc[rt][i] = vcur[4 * rt + i] - Xacc[rt][i];
      barrier_nofence();  // B(c): the image back is in LDS
      // -- Delta = (T diag(b)) X, T = (I + A)^-1 lower triangular: row block
      // rt sums the X block pairs ks with 2ks <= rt (the tile (rt, 2ks+1) above
      // the diagonal is 0); four independent chains of at most four products.
      f16x8 xh[2], xl[2];  // X block pairs as hi+lo fragments
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bfrag_split(Xacc[2 * ks], Xacc[2 * ks + 1], xh[ks], xl[ks]);
      f32x4 Dacc[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (2 * ks > rt) continue;
          const f16x4 t0 = *reinterpret_cast<const f16x4*>(im + Ws::AT + tri_at(rt, 2 * ks, lr, lg));
          f16x4 t1 = {0, 0, 0, 0};
          if (2 * ks + 1 <= rt)
            t1 = *reinterpret_cast<const f16x4*>(im + Ws::AT + tri_at(rt, 2 * ks + 1, lr, lg));
          const f16x8 ta = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
          d = mma_f16(ta, xh[ks], d);
          d = mma_f16(ta, xl[ks], d);
        }
        Dacc[rt] = d;
      }
      f16x8 dbh[2], dbl[2];  // Delta block pairs as hi+lo fragments
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) bfrag_split(Dacc[2 * ks], Dacc[2 * ks + 1], dbh[ks], dbl[ks]);
      // -- O^T += Delta^T P^T: lane (lr, lg) of tile rt then holds token row
      // 16rt + lr, value columns 16w + 4lg .. +3, stored straight to o (8 or
      // 16 bytes per lane; rows past the chunk end are dropped)
      const auto ro = tok_buf(o, OS, c);
      char* ot = ot_of(c);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 ao = Oacc[rt];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (2 * ks > rt) continue;
          // P row 16rt + lr, tokens 32ks + 4lg + e and 32ks + 16 + 4lg + e
          // (tile (rt, 2ks+1) lies above the diagonal when 2ks + 1 > rt)
          const f16x4 p0 = *reinterpret_cast<const f16x4*>(im + Ws::PM + tri_at(rt, 2 * ks, lr, lg));
          f16x4 p1 = {0, 0, 0, 0};
          if (2 * ks + 1 <= rt)
            p1 = *reinterpret_cast<const f16x4*>(im + Ws::PM + tri_at(rt, 2 * ks + 1, lr, lg));
          const f16x8 pm = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
          ao = mma_f16(dbh[ks], pm, ao);
          ao = mma_f16(dbl[ks], pm, ao);
        }
        ao = ao * scale;
        const int row = 16 * rt + lr;
        const int j0 = 16 * w + 4 * lg;
        if constexpr (O_BF16) {
          bf16x4 ob;
#pragma unroll
          for (int i = 0; i < 4; ++i) ob[i] = static_cast<__bf16>(ao[i]);
          *reinterpret_cast<bf16x4*>(ot + otile_off(row, j0)) = ob;
        } else {
          typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ao), ro,
                                                 (row * HD + j0) * 4, 0, 0);
        }
      }
      // -- S <- e^gamma_C S + Khat^T Delta
      const float* ec = reinterpret_cast<const float*>(im + Ws::EC);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const f32x4 dec = *reinterpret_cast<const f32x4*>(ec + 16 * t + 4 * lg);
        f32x4 s = Sacc[t] * dec;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const f16x8 a = *reinterpret_cast<const f16x8*>(im + Ws::KDT + kdt_frag(ks, t, lr, lg));
          s = mma_f16(a, dbh[ks], s);
          s = mma_f16(a, dbl[ks], s);
        }
        Sacc[t] = s;
      }
    }
  }

  if constexpr (O_BF16) {
    if (c_lo < c_end) barrier_nofence();  // A(c_end): hands the last o tile to the data waves
  }
  const int64_t so = sio.out_idx ? static_cast<int64_t>(sio.out_idx[n]) : n;
  if (sio.out && so >= 0 && so < sio.out_slots) {
    const int64_t sbase = (so * H + h) * D * D;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t e = sbase + (int64_t)(16 * t + 4 * lg + i) * D + jcol;
        if (sio.out_bf16) static_cast<uint16_t*>(sio.out)[e] = f32_to_bf16_bits(Sacc[t][i]);
        else static_cast<float*>(sio.out)[e] = Sacc[t][i];
      }
  }
}

}  // namespace

hipError_t launch_state(const void* v, bool qkv_bf16, const int32_t* cu, int N, int T_tot,
                        int H, const StateIO& sio, void* o, bool o_bf16,
                        float scale, int c_lo, int S_len, const char* ws, hipStream_t s) {
  const int Hp = (H + 7) & ~7;
  const int64_t blocks = (int64_t)N * Hp * NT;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(blocks));
#define KDA_LAUNCH(QB, OB)                                                                      \
  state_kernel<QB, OB><<<grid, NTHR_S, 0, s>>>(v, cu, N, T_tot, H, Hp, sio, o, scale,       \
                                               c_lo, S_len, ws)
  if (qkv_bf16 && o_bf16) KDA_LAUNCH(true, true);
  else if (qkv_bf16) KDA_LAUNCH(true, false);
  else if (o_bf16) KDA_LAUNCH(false, true);
  else KDA_LAUNCH(false, false);
#undef KDA_LAUNCH
  return hipGetLastError();
}

}  // namespace chunk
}  // namespace kda
