// Shared pieces of the two chunked-prefill kernels (prep.hip, state.hip):
// MFMA wrappers, operand permutations, buffer helpers and the layout of the
// per-(chunk, head) workspace image that the prep kernel writes and the state
// kernel copies verbatim into LDS.
//
// Chunked form (one sequence, one head, chunk of C=64 tokens, entry state S,
// d=128), from the recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1}
// + b_t k_t v_t^T, o_t = S_t^T q_t (the code audit's chunked training/prefill
// regime), with gamma_r = sum_{s<=r} g_s per key channel:
//   A[r,s] = b_r sum_c k_rc k_sc e^(gamma_rc - gamma_sc)   (s < r)
//   P[r,s] =     sum_c q_rc k_sc e^(gamma_rc - gamma_sc)   (s <= r)
//   X      = V - (K * e^gamma) S
//   Delta  = (I + A)^-1 diag(b) X
//   O      = scale * ((Q * e^gamma) S + P Delta)
//   S     <- Diag(e^gamma_C) S + (K * e^(gamma_C - gamma))^T Delta
// Everything left of the state is fixed by the chunk's own inputs; the prep
// kernel computes it for all chunks in parallel, the state kernel walks the
// chunks of each sequence in order and does only the products with S.
#pragma once

#include "kda_device.hpp"

namespace kda {
namespace chunk {

constexpr int C = 64;     // chunk length
constexpr int D = 128;    // dk = dv
constexpr int NTHR = 256; // 4 waves per workgroup
constexpr float LOG2E = 1.4426950408889634f;
// Floor of the per-token log2 decay in the prefill's cumulative sum.  The
// decay factors are built from references at most 8 tokens away, and 8 x 15.5
// = 124 keeps every such factor inside fp32 range for any g <= 0.  A floored
// decay factor is 2^-15.5 (2.2e-5) where the exact one is smaller, so o and
// the state move by far less than their rounding error (the audit's printed
// A_log maximum, 2.47, reaches tens of log2 units per token).
constexpr float DECAY_FLOOR_LOG2 = 15.5f;

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

typedef float f32x8 __attribute__((ext_vector_type(8)));
// fp32 -> fp16 rounding to nearest even, two values per instruction
// (v_cvt_pk_f16_f32) where a per-element cast costs a conversion and a pack.
__device__ __forceinline__ f16x8 cvt_f16(f32x8 x) { return __builtin_convertvector(x, f16x8); }
__device__ __forceinline__ f16x4 cvt_f16(f32x4 x) { return __builtin_convertvector(x, f16x4); }
__device__ __forceinline__ f32x8 f32x8_of(const float (&x)[8]) {
  return f32x8{x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
}

// Orders this wave's LDS writes before its later LDS reads (no workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

// 16x16x32 B fragment (hi and lo fp16) from an accumulator tile pair
// (t0 = rows 4lg+i, t1 = rows 16+4lg+i): fragment element e of lane group lg
// is contraction index 16(e>>2) + 4lg + (e&3) of the 32-wide step.  Every
// A operand paired with it is read in that same order.
__device__ __forceinline__ void bfrag_split(const f32x4& t0, const f32x4& t1, f16x8& hi,
                                            f16x8& lo) {
  const f32x8 t = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
  hi = cvt_f16(t);
  lo = cvt_f16(t - __builtin_convertvector(hi, f32x8));
}
// 16x16x16 B fragment (hi and lo fp16) from one accumulator tile.
__device__ __forceinline__ void bfrag16_split(const f32x4& t, f16x4& hi, f16x4& lo) {
  hi = cvt_f16(t);
  lo = cvt_f16(t - __builtin_convertvector(hi, f32x4));
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
// Called from non-template code paths only through this wrapper: the builtin's
// size check misfires in the host pass of a template instantiation and
// silently drops the kernel's host stub.
__device__ __forceinline__ void buf_to_lds16(__amdgpu_buffer_rsrc_t r, lds_ptr_t dst, int voff,
                                             int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}
// All of this wave's outstanding vector-memory operations have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }
// Workgroup barrier without the memory fence of __syncthreads, whose release
// half makes every wave drain its outstanding vector-memory operations
// (vmcnt 0) first.  Only the compiler is kept from moving memory operations
// across it.  For code where each wave that writes data for others waits for
// its own writes (counter waits on buffer-to-LDS copies) and every LDS read of
// a buffer is consumed before the barrier after which that buffer is refilled.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- workspace image of one (chunk, head), all offsets in bytes.
// The prep kernel writes each part straight from its registers (128 bytes to
// 1 KiB contiguous per instruction); the state kernel copies the image 1 KiB
// at a time into LDS and reads 8-byte operand pieces, ordered so that each
// 16-lane group of a read covers 128 contiguous bytes (no bank conflicts).
// Every part is a sequence of 8-byte units; lane (lr, lg) of a 16x16 operand
// tile reads unit 16 lg + lr of that tile's 512 bytes.
//   KE, QE  fp16 K e^gamma, Q e^gamma: per 16-row block rt and 32-channel
//           step kk a 1 KiB block of 16-byte units; unit 16 lg + lr holds row
//           16 rt + lr, channels 32kk + 4lg .. +3 then 32kk + 16 + 4lg .. +3
//           (the channel order of a 16x16x32 fragment paired with an
//           accumulator tile pair).
//   KDT     fp16 (K e^(gamma_C - gamma))^T: per 32-token step ks and
//           16-channel tile t a 1 KiB block; unit 16 lg + lr holds channel
//           16t + lr, tokens 32ks + 4lg .. +3 then 32ks + 16 + 4lg .. +3.
//   PM      fp16 P, ten 16x16 tiles (i, j <= i) at index i(i+1)/2 + j; unit
//           16 lg + lr holds row lr, columns 4lg .. +3 of the tile.
//   AT      fp16 the same ten tiles of (I + A)^-1 diag(b), the lower
//           triangular matrix that maps X to Delta (columns past the chunk end
//           are 0).
//   EC      fp32 [128]: e^gamma_C per key channel.
struct Ws {
  static constexpr int KE = 0;
  static constexpr int QE = KE + C * D * 2;
  static constexpr int KDT = QE + C * D * 2;
  static constexpr int PM = KDT + D * C * 2;
  static constexpr int AT = PM + 10 * 512;
  static constexpr int EC = AT + 10 * 512;
  static constexpr int used = EC + D * 4;
  static constexpr int bytes = ((used + 1023) / 1024) * 1024;  // copied in 1 KiB rounds
};
static_assert(Ws::bytes == 59 * 1024, "workspace image size");

// KE / QE: the 16-byte fragment of lane (lr, lg) for row block rt, step kk
__device__ __forceinline__ int keqe_frag(int rt, int kk, int lr, int lg) {
  return ((rt * 4 + kk) << 10) + ((((lg << 4) + lr)) << 4);
}
// KE / QE: where row 16rt + lr, channels 32kk + x .. x+3 (x = 0, 4, .., 28) go
__device__ __forceinline__ int keqe_at(int rt, int kk, int x, int lr) {
  return keqe_frag(rt, kk, lr, (x >> 2) & 3) + ((x >> 4) << 3);
}
// KDT: the 16-byte fragment of lane (lr, lg) for token step ks, channel tile t
__device__ __forceinline__ int kdt_frag(int ks, int t, int lr, int lg) {
  return ((ks * 8 + t) << 10) + ((((lg << 4) + lr)) << 4);
}
// KDT: where channel 16t + lr, tokens 16b + 4lg .. +3 go
__device__ __forceinline__ int kdt_at(int b, int t, int lr, int lg) {
  return kdt_frag(b >> 1, t, lr, lg) + ((b & 1) << 3);
}
// PM / AT: tile (i, j <= i), row lr, columns 4lg .. +3
__device__ __forceinline__ int tri_at(int i, int j, int lr, int lg) {
  return ((((i * (i + 1)) >> 1) + j) << 9) + ((((lg << 4) + lr)) << 3);
}

// Longest-first rank -> sequence index for N <= 64 sequences (ties by index),
// so that the workgroups of long sequences start first.  Needs 64 threads and
// one int of LDS; every thread of the workgroup must call it.
__device__ __forceinline__ int lpt_sequence(const int32_t* cu, int N, int T_tot, int rank,
                                            int* s_seq) {
  if (N <= 1 || N > 64) return rank;
  const int tid = threadIdx.x;
  if (tid < N) {
    auto clampi = [&](int x) { return x < 0 ? 0 : (x > T_tot ? T_tot : x); };
    const int li = clampi(cu[tid + 1]) - clampi(cu[tid]);
    int rk = 0;
    for (int j = 0; j < N; ++j) {
      const int lj = clampi(cu[j + 1]) - clampi(cu[j]);
      rk += (lj > li) || (lj == li && j < tid);
    }
    if (rk == rank) s_seq[0] = tid;
  }
  __syncthreads();
  return s_seq[0];
}

}  // namespace chunk
}  // namespace kda
