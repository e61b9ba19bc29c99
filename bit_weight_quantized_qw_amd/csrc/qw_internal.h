// Internal helpers shared by the libqw translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "qw.h"
#include "qw_tuning.h"

namespace qw {

// Fails the enclosing entry point with QW_ERR_HIP when a HIP call fails.
#define QW_HIP_TRY(expr)                                   \
  do {                                                     \
    hipError_t qw_e_ = (expr);                             \
    if (qw_e_ != hipSuccess) return QW_ERR_HIP;            \
  } while (0)

// Returns a failed qw_status from the enclosing function.
#define QW_TRY(expr)                                       \
  do {                                                     \
    qw_status qw_s_ = (expr);                              \
    if (qw_s_ != QW_OK) return qw_s_;                      \
  } while (0)

// ---------------------------------------------------------------------------
// Kernel launches and per-call timing (qw_time_next_call). Every entry point
// that enqueues kernels opens a CallScope before validating its arguments;
// launch() attaches the armed events of that scope to the kernels it
// dispatches (start on the first, stop on every one).
struct CallScope {
  CallScope();
  ~CallScope();
  CallScope(const CallScope &) = delete;
  CallScope &operator=(const CallScope &) = delete;
};

hipError_t launch_raw(const void *fn, dim3 grid, dim3 block, void **argv, size_t lds,
                      hipStream_t s);
// Cooperative launch (all workgroups co-resident, or it fails) with the
// call's events recorded on the stream around it.
hipError_t launch_cooperative_raw(const void *fn, dim3 grid, dim3 block, void **argv, size_t lds,
                                  hipStream_t s);

template <typename Tup, size_t... I>
inline void fill_argv(Tup &t, void **argv, std::index_sequence<I...>) {
  ((argv[I] = (void *)&std::get<I>(t)), ...);
}

template <typename... P, typename... A>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                         A &&...args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> t(std::forward<A>(args)...);
  void *argv[sizeof...(P) + 1];
  fill_argv(t, argv, std::index_sequence_for<P...>{});
  return launch_raw(reinterpret_cast<const void *>(kernel), grid, block, argv, lds, s);
}

inline bool aligned16(const void *p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Current value of a test hook of qw_tuning.h (QW_TUNE_AUTO when unset).
int tune(qw_tune_key key);

// Checks that the current device is a gfx950 and returns its CU count.
qw_status current_device(int *cu_count);

// NF4 levels as fp32 (computed once on the host).
const float *nf4_levels_host();

// Returns the padded anchor row stride for n_out anchors.
inline int pad8(int n) { return (n + 7) & ~7; }

// Validates a packed-weight view against its format (sizes, NULLs,
// alignment of every buffer it uses). K_expect > 0 also pins K.
qw_status check_weight_view(const qw_weight *w, int format, int K_expect);

// ---------------------------------------------------------------------------
// Exact fp64 -> fp16 round-to-nearest-even, subnormals kept, by integer
// manipulation (one rounding, never through fp32). Returns the bit pattern.
__host__ __device__ inline uint16_t f64_to_f16_rne(double v) {
  uint64_t b = __builtin_bit_cast(uint64_t, v);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  int ex = (int)((b >> 52) & 0x7FF);
  uint64_t mant = b & ((1ull << 52) - 1);
  if (ex == 0x7FF) return sign | (mant ? 0x7E00u : 0x7C00u);
  if (ex == 0) return sign;  // fp64 subnormal: far below fp16 range
  int e = ex - 1023;
  if (e > 15) return sign | 0x7C00u;
  if (e < -26) return sign;
  uint64_t m = mant | (1ull << 52);            // 53-bit significand
  int shift = (e >= -14) ? 42 : 42 + (-14 - e);  // bits dropped
  uint64_t keep = m >> shift;
  uint64_t rem = m & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (keep & 1))) keep++;
  if (e >= -14) {
    int he = e + 15;
    if (keep == (1ull << 11)) { keep >>= 1; he++; }
    if (he >= 31) return sign | 0x7C00u;
    return sign | (uint16_t)(he << 10) | (uint16_t)(keep & 0x3FF);
  }
  // subnormal result; keep == 0x400 is exactly the smallest normal's code
  return sign | (uint16_t)keep;
}

// Exact fp16 bits -> fp32.
__host__ __device__ inline float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

}  // namespace qw
