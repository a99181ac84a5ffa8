// KDA_DEBUG=1 validation mode.
//
// With the environment variable KDA_DEBUG set to 1, every entry point scans
// its inputs before its kernels run and its outputs after them, and reports
// through its status and kda_last_error:
//   before: q, k, v and states finite; g <= 0 (NaN fails); beta in [0, 1];
//           gate logits not NaN (infinite logits are the gate's limits);
//           A_log and dt_bias finite.  A failure returns KDA_ERR_DOMAIN and
//           the call's own kernels are not launched (nothing is written).
//   after:  every output value finite (the gate's g may be -inf, the limit
//           of an infinite logit, and only NaN fails there).  A failure
//           returns KDA_ERR_NONFINITE; the outputs have been written.
// The scans count offending values per scanned tensor into a small array of
// counters in device memory that belongs to the library (no allocation), and
// read them back with a copy and a stream synchronisation: debug calls are
// synchronous, and one host mutex serialises them.
//
// The PR review of the Kimi-K3 adapter (Model-Optimizer PR #2749) names the
// failure this mode makes visible: a recurrence fed out-of-domain beta
// diverges, and downstream only a NaN shows.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace dbg {
namespace {

constexpr int kMaxScans = 16;
constexpr int kMaxDevices = 64;

// Offending-value counters of the scans of one phase of one call.
__device__ __align__(64) uint32_t debug_counters[kMaxScans];

__global__ void clear_kernel(uint32_t* w) {
  if (threadIdx.x < kMaxScans) w[threadIdx.x] = 0u;
}

__device__ __forceinline__ bool value_ok(float x, int rule) {
  switch (rule) {
    case kFinite: return __builtin_isfinite(x);
    case kNotNaN: return !__builtin_isnan(x);
    case kNonPositive: return x <= 0.0f;  // NaN fails
    default: return x >= 0.0f && x <= 1.0f;  // kUnit; NaN fails
  }
}

template <bool BF16>
__global__ void scan_kernel(const void* __restrict__ p, int64_t n, int rule, uint32_t* word) {
  uint32_t bad = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float x = BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i])
                         : static_cast<const float*>(p)[i];
    bad += value_ok(x, rule) ? 0u : 1u;
  }
  if (bad) atomicAdd(word, bad);
}

// One workgroup per (sequence, head): the 128 x 128 state of slot idx[n]
// (n without indices); slots outside [0, slots) are skipped.
template <bool BF16>
__global__ void scan_states_kernel(const void* __restrict__ p, const int32_t* __restrict__ idx,
                                   int64_t slots, int H, uint32_t* word) {
  const int n = blockIdx.x / H, h = blockIdx.x % H;
  const int64_t s = idx ? static_cast<int64_t>(idx[n]) : n;
  if (s < 0 || s >= slots) return;
  const int64_t base = (s * H + h) * 128 * 128;
  uint32_t bad = 0;
  for (int i = threadIdx.x; i < 128 * 128; i += blockDim.x) {
    const float x = BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(p)[base + i])
                         : static_cast<const float*>(p)[base + i];
    bad += __builtin_isfinite(x) ? 0u : 1u;
  }
  if (bad) atomicAdd(word, bad);
}

std::mutex g_mutex;
uint32_t* g_words[kMaxDevices];  // per device: address of debug_counters

const char* rule_text(int rule) {
  switch (rule) {
    case kFinite: return "not finite";
    case kNotNaN: return "NaN";
    case kNonPositive: return "not <= 0";
    default: return "outside [0, 1]";
  }
}

}  // namespace

bool enabled() {
  const char* e = getenv("KDA_DEBUG");
  return e && e[0] == '1' && e[1] == '\0';
}

std::mutex& mutex() { return g_mutex; }

Session::Session(hipStream_t s) : stream_(s) {}

hipError_t Session::begin() {
  count_ = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!g_words[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(debug_counters));
    if (e != hipSuccess) return e;
    g_words[dev] = static_cast<uint32_t*>(ptr);
  }
  words_ = g_words[dev];
  clear_kernel<<<1, 64, 0, stream_>>>(words_);
  return hipGetLastError();
}

void Session::add(const char* what, const void* p, int64_t n, bool bf16, int rule) {
  if (!p || n <= 0 || count_ >= kMaxScans) return;
  const int64_t blocks64 = (n + 255) / 256;
  const unsigned blocks = (unsigned)(blocks64 < 2048 ? blocks64 : 2048);
  if (bf16) scan_kernel<true><<<blocks, 256, 0, stream_>>>(p, n, rule, words_ + count_);
  else scan_kernel<false><<<blocks, 256, 0, stream_>>>(p, n, rule, words_ + count_);
  what_[count_] = what;
  rule_[count_] = rule;
  n_[count_] = n;
  ++count_;
}

void Session::add_states(const char* what, const void* p, bool bf16, const int32_t* idx,
                         int64_t slots, int N, int H) {
  if (!p || N <= 0 || H <= 0 || count_ >= kMaxScans) return;
  const unsigned blocks = (unsigned)((int64_t)N * H);
  if (bf16) scan_states_kernel<true><<<blocks, 256, 0, stream_>>>(p, idx, slots, H, words_ + count_);
  else scan_states_kernel<false><<<blocks, 256, 0, stream_>>>(p, idx, slots, H, words_ + count_);
  what_[count_] = what;
  rule_[count_] = kFinite;
  n_[count_] = (int64_t)N * H * 128 * 128;
  ++count_;
}

hipError_t Session::finish(std::string* report) {
  report->clear();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint32_t host[kMaxScans] = {0};
  if (count_ > 0) {
    e = hipMemcpyAsync(host, words_, sizeof(uint32_t) * count_, hipMemcpyDeviceToHost, stream_);
    if (e != hipSuccess) return e;
  }
  e = hipStreamSynchronize(stream_);
  if (e != hipSuccess) return e;
  for (int i = 0; i < count_; ++i) {
    if (!host[i]) continue;
    char line[160];
    snprintf(line, sizeof(line), "%s%s %s (%u of %lld values)", report->empty() ? "" : "; ",
             what_[i], rule_text(rule_[i]), host[i], (long long)n_[i]);
    *report += line;
  }
  return hipSuccess;
}

}  // namespace dbg
}  // namespace kda
