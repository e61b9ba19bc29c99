// Host-side entry points of libqw that launch nothing: version, status text,
// buffer sizes, format constants, and the device check used by the others.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include <hip/hip_ext.h>

#include "qw_internal.h"

#pragma STDC FP_CONTRACT OFF

namespace qw {

namespace {
struct DevInfo {
  int state = 0;  // 0 unknown, 1 ok, 2 not gfx950
  int cus = 0;
};
DevInfo g_dev[64];
std::mutex g_dev_mu;

float g_nf4[16];
std::once_flag g_nf4_once;

// Standard normal CDF from the complementary error function.
double norm_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

// Inverse standard normal CDF: bisection to bracket, then Newton steps on
// Phi(x) - p with derivative phi(x).
double norm_ppf(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200 && hi - lo > 1e-12; ++i) {
    double mid = 0.5 * (lo + hi);
    if (norm_cdf(mid) < p) lo = mid; else hi = mid;
  }
  double x = 0.5 * (lo + hi);
  const double inv_sqrt_2pi = 0.39894228040143267794;
  for (int i = 0; i < 4; ++i) {
    double pdf = inv_sqrt_2pi * exp(-0.5 * x * x);
    x = x - (norm_cdf(x) - p) / pdf;
  }
  return x;
}

void build_nf4() {
  // "Fontes" of the AirQuant README cites QLoRA for NF4; the levels are the
  // normalised normal quantiles described in qw.h.
  const double delta = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0);
  double v[16];
  int n = 0;
  {
    double step = (0.5 - delta) / 8.0;
    for (int i = 0; i < 8; ++i) v[n++] = norm_ppf((double)i * step + delta);
  }
  {
    double step = (0.5 - delta) / 7.0;
    for (int i = 0; i < 7; ++i) v[n++] = -norm_ppf((double)i * step + delta);
  }
  v[n++] = 0.0;
  // insertion sort, ascending
  for (int i = 1; i < 16; ++i) {
    double t = v[i];
    int j = i - 1;
    while (j >= 0 && v[j] > t) { v[j + 1] = v[j]; --j; }
    v[j + 1] = t;
  }
  double mx = v[15];
  for (int i = 0; i < 16; ++i) g_nf4[i] = (float)(v[i] / mx);
}
}  // namespace

// Test hooks (qw_tuning.h), indexed by key; -1 = automatic.
constexpr int kTuneKeys = 7;
std::atomic<int> g_tune[kTuneKeys] = {{-1}, {-1}, {-1}, {-1}, {-1}, {-1}, {-1}};

int tune(qw_tune_key key) {
  const int k = (int)key;
  return (k > 0 && k < kTuneKeys) ? g_tune[k].load(std::memory_order_relaxed) : QW_TUNE_AUTO;
}

const float *nf4_levels_host() {
  std::call_once(g_nf4_once, build_nf4);
  return g_nf4;
}

qw_status current_device(int *cu_count) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QW_ERR_NO_DEVICE;
  if (dev < 0 || dev >= 64) return QW_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo &d = g_dev[dev];
  if (d.state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QW_ERR_NO_DEVICE;
    d.state = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    d.cus = prop.multiProcessorCount;
  }
  if (d.state != 1) return QW_ERR_NO_DEVICE;
  if (cu_count) *cu_count = d.cus;
  return QW_OK;
}

qw_status check_weight_view(const qw_weight *w, int format, int K_expect) {
  if (!w || w->format != format) return QW_ERR_INVALID_ARG;
  qw_sizes z;
  qw_status st = qw_packed_sizes((qw_format)format, w->N, w->K, w->n_out, &z);
  if (st != QW_OK) return st;
  if (K_expect > 0 && w->K != K_expect) return QW_ERR_INVALID_ARG;
  if (!w->codes || !w->scales) return QW_ERR_INVALID_ARG;
  if (!aligned16(w->codes) || !aligned16(w->scales)) return QW_ERR_ALIGNMENT;
  if (w->n_out > 0 && format == QW_FMT_INT4_G32) {
    // the products read the anchors only; the permutation is qw_pack's input
    if (!w->out_w) return QW_ERR_INVALID_ARG;
    if (w->n_out_pad < z.n_out_pad || (w->n_out_pad & 7)) return QW_ERR_INVALID_ARG;
    if (!aligned16(w->out_w)) return QW_ERR_ALIGNMENT;
  } else if (w->n_out > 0) {
    if (!w->out_idx || !w->out_w || !w->out_mask) return QW_ERR_INVALID_ARG;
    if (w->n_out_pad < z.n_out_pad || (w->n_out_pad & 7)) return QW_ERR_INVALID_ARG;
    if (!aligned16(w->out_idx) || !aligned16(w->out_w) || !aligned16(w->out_mask))
      return QW_ERR_ALIGNMENT;
  }
  return QW_OK;
}

// Events armed by qw_time_next_call on this host thread, and the pair taken
// by the entry point currently running on it.
namespace {
thread_local hipEvent_t tl_armed_start = nullptr, tl_armed_stop = nullptr;
thread_local hipEvent_t tl_call_start = nullptr, tl_call_stop = nullptr;
}  // namespace

CallScope::CallScope() {
  tl_call_start = tl_armed_start;
  tl_call_stop = tl_armed_stop;
  tl_armed_start = tl_armed_stop = nullptr;
}

CallScope::~CallScope() { tl_call_start = tl_call_stop = nullptr; }

hipError_t launch_raw(const void *fn, dim3 grid, dim3 block, void **argv, size_t lds,
                      hipStream_t s) {
  if (!tl_call_start && !tl_call_stop) return hipLaunchKernel(fn, grid, block, argv, lds, s);
  hipEvent_t start = tl_call_start;
  tl_call_start = nullptr;  // only the call's first kernel records the start
  return hipExtLaunchKernel(fn, grid, block, argv, lds, s, start, tl_call_stop, 0);
}

hipError_t launch_cooperative_raw(const void *fn, dim3 grid, dim3 block, void **argv, size_t lds,
                                  hipStream_t s) {
  // a cooperative launch takes no attached events: the call's start (if
  // still unrecorded) and stop go on the stream around it
  if (tl_call_start) {
    const hipError_t e = hipEventRecord(tl_call_start, s);
    tl_call_start = nullptr;
    if (e != hipSuccess) return e;
  }
  const hipError_t e = hipLaunchCooperativeKernel(fn, grid, block, argv, (unsigned)lds, s);
  if (e != hipSuccess || !tl_call_stop) return e;
  return hipEventRecord(tl_call_stop, s);
}

}  // namespace qw

extern "C" {

qw_status qw_time_next_call(void *start_event, void *stop_event) {
  qw::tl_armed_start = reinterpret_cast<hipEvent_t>(start_event);
  qw::tl_armed_stop = reinterpret_cast<hipEvent_t>(stop_event);
  return QW_OK;
}

int qw_abi_version(void) { return QW_ABI_VERSION; }

qw_status qw_tune_set(qw_tune_key key, int value) {
  const int k = (int)key;
  if (k <= 0 || k >= qw::kTuneKeys || value < QW_TUNE_AUTO) return QW_ERR_INVALID_ARG;
  qw::g_tune[k].store(value, std::memory_order_relaxed);
  return QW_OK;
}

int qw_tune_get(qw_tune_key key) { return qw::tune(key); }

size_t qw_select_workspace_bytes(int K) {
  return K > 0 ? (size_t)K * (2 * sizeof(double) + sizeof(int32_t)) : 0;
}

const char *qw_status_str(qw_status s) {
  switch (s) {
    case QW_OK: return "ok";
    case QW_ERR_INVALID_ARG: return "invalid argument";
    case QW_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case QW_ERR_UNSUPPORTED: return "unsupported request";
    case QW_ERR_HIP: return "HIP runtime error";
    case QW_ERR_NO_DEVICE: return "no gfx950 device is current";
    case QW_ERR_SCRATCH_LIMIT: return "request needs more than the library's static scratch array";
  }
  return "unknown status";
}

qw_status qw_packed_sizes(qw_format fmt, int N, int K, int n_out, qw_sizes *out) {
  if (!out || N <= 0 || K <= 0 || n_out < 0 || n_out >= K) return QW_ERR_INVALID_ARG;
  qw_sizes z{};
  if (fmt == QW_FMT_2BIT_G32) {
    if (K % 32) return QW_ERR_INVALID_ARG;
    z.codes = (size_t)N * (size_t)(K / 4);
    z.scales = (size_t)N * (size_t)(K / 32) * 4;
    if (n_out > 0) {
      z.n_out_pad = qw::pad8(n_out);
      z.out_idx = (size_t)n_out * 4;
      z.out_w = (size_t)N * (size_t)z.n_out_pad * 2;
      z.out_mask = (size_t)(K / 32) * 4;
    }
  } else if (fmt == QW_FMT_NF4_B64) {
    if (K % 64 || n_out != 0) return QW_ERR_INVALID_ARG;
    z.codes = (size_t)N * (size_t)(K / 2);
    z.scales = (size_t)N * (size_t)(K / 64) * 4;
  } else if (fmt == QW_FMT_INT4_G32) {
    if (K % 32) return QW_ERR_INVALID_ARG;
    z.codes = (size_t)N * (size_t)(K / 2);
    z.scales = (size_t)N * (size_t)(K / 32) * 2;
    z.out_idx = (size_t)K * 4;  // the permutation
    if (n_out > 0) {
      z.n_out_pad = qw::pad8(n_out);
      z.out_w = (size_t)N * (size_t)z.n_out_pad * 2;
    }
  } else {
    return QW_ERR_INVALID_ARG;
  }
  *out = z;
  return QW_OK;
}

int qw_outlier_count(int K, double frac) {
  if (K < 0 || !(frac >= 0.0 && frac < 1.0)) return -1;
  return (int)floor(frac * (double)K);
}

qw_status qw_codebook_2bit(float *out) {
  if (!out) return QW_ERR_INVALID_ARG;
  out[0] = -1.52f; out[1] = -0.45f; out[2] = 0.45f; out[3] = 1.52f;
  return QW_OK;
}

qw_status qw_nf4_levels(float *out) {
  if (!out) return QW_ERR_INVALID_ARG;
  memcpy(out, qw::nf4_levels_host(), 16 * sizeof(float));
  return QW_OK;
}

}  // extern "C"
