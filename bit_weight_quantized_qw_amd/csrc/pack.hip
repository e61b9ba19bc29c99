// qw_pack and qw_select_outliers: pack-time kernels.
//
// 2-bit: "On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)", sections 2-4
// (codebook, per-group least squares scale/offset, fp16 outlier anchors) and
// "Key v4.0 Innovations" (four codes per byte).
// NF4: "AirQuant" README, "Fundamentacao Teorica e Arquitetura" item 2.
//
// One thread per group (2-bit: 32 weights) or block (NF4: 64 weights); all
// arithmetic in fp64 with fused multiply-add disabled and every sum taken
// left to right, so the packed result is bit-identical to a plain
// sequential fp64 evaluation of the same formulas.
#include <math.h>

#include "qw_internal.h"

namespace qw {
namespace {

struct Levels16 { float v[16]; };

__global__ __launch_bounds__(256) void pack2_kernel(
    const float *__restrict__ W, int N, int K, const int32_t *__restrict__ idx,
    int n_out, uint32_t *__restrict__ codes, uint32_t *__restrict__ sz) {
#pragma clang fp contract(off)
  const int G = K / 32;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)N * G) return;
  const int n = (int)(gid / G), g = (int)(gid % G);
  const float4 *wp = reinterpret_cast<const float4 *>(W + (size_t)n * K + (size_t)g * 32);

  // positions of this group that are anchor channels
  uint32_t omask = 0;
  if (n_out > 0) {
    const int k0 = g * 32;
    int lo = 0, hi = n_out;
    while (lo < hi) {
      int mid = (lo + hi) >> 1;
      if (idx[mid] < k0) lo = mid + 1; else hi = mid;
    }
    for (int o = lo; o < n_out && idx[o] < k0 + 32; ++o) omask |= 1u << (idx[o] - k0);
  }

  double w[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 v = wp[i];
    w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if ((omask >> i) & 1u) w[i] = 0.0;

  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) acc = acc + w[i];
  const double m = acc / 32.0;
  double d[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) d[i] = w[i] - m;
  acc = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) acc = acc + d[i] * d[i];
  const double var = acc / 32.0;

  const double C0 = (double)-1.52f, C1 = (double)-0.45f, C2 = (double)0.45f, C3 = (double)1.52f;
  const double t = 0.5 * (C2 + C3);
  const double thr = (t * t) * var;

  uint32_t q[32];
  double c[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const bool outer = (d[i] * d[i]) > thr;
    const bool upper = d[i] >= 0.0;
    q[i] = upper ? (outer ? 3u : 2u) : (outer ? 0u : 1u);
    c[i] = upper ? (outer ? C3 : C2) : (outer ? C0 : C1);
  }
  acc = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) acc = acc + c[i];
  const double cbar = acc / 32.0;
  double num = 0.0, den = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const double cc = c[i] - cbar;
    num = num + d[i] * cc;
    den = den + cc * cc;
  }
  den = den + 1e-8;
  const double S = num / den;
  const double Z = m - S * cbar;

  uint32_t lo32 = 0, hi32 = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    lo32 |= q[i] << (2 * i);
    hi32 |= q[16 + i] << (2 * i);
  }
  uint2 cw;
  cw.x = lo32;
  cw.y = hi32;
  reinterpret_cast<uint2 *>(codes)[(size_t)n * G + g] = cw;
  sz[(size_t)n * G + g] = (uint32_t)f64_to_f16_rne(S) | ((uint32_t)f64_to_f16_rne(Z) << 16);
}

__global__ __launch_bounds__(256) void anchors_kernel(
    const float *__restrict__ W, int N, int K, const int32_t *__restrict__ idx,
    int n_out, int n_out_pad, uint16_t *__restrict__ out_w) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)N * n_out_pad) return;
  const int n = (int)(gid / n_out_pad), o = (int)(gid % n_out_pad);
  uint16_t v = 0;
  if (o < n_out) {
    const int c = idx[o];
    if (c >= 0 && c < K) v = f64_to_f16_rne((double)W[(size_t)n * K + c]);
  }
  out_w[gid] = v;
}

// out_mask word i: bit b set iff channel 32*i + b is an anchor channel.
__global__ __launch_bounds__(256) void mask_kernel(const int32_t *__restrict__ idx, int n_out,
                                                   int K, uint32_t *__restrict__ mask) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= K / 32) return;
  const int k0 = 32 * i;
  int lo = 0, hi = n_out;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (idx[mid] < k0) lo = mid + 1; else hi = mid;
  }
  uint32_t m = 0;
  for (int o = lo; o < n_out && idx[o] < k0 + 32; ++o) {
    const int b = idx[o] - k0;
    if (b >= 0) m |= 1u << b;
  }
  mask[i] = m;
}

__global__ __launch_bounds__(256) void pack_nf4_kernel(
    const float *__restrict__ W, int N, int K, Levels16 L,
    uint32_t *__restrict__ codes, float *__restrict__ absmax) {
#pragma clang fp contract(off)
  const int G = K / 64;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)N * G) return;
  const int n = (int)(gid / G), g = (int)(gid % G);
  const float4 *wp = reinterpret_cast<const float4 *>(W + (size_t)n * K + (size_t)g * 64);
  float w[64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float4 v = wp[i];
    w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) a = fmaxf(a, fabsf(w[i]));
  double mids[15];
#pragma unroll
  for (int j = 0; j < 15; ++j) mids[j] = 0.5 * ((double)L.v[j] + (double)L.v[j + 1]);
  const double a64 = (double)a;
  uint32_t out[8];
#pragma unroll
  for (int dw = 0; dw < 8; ++dw) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double wi = (double)w[8 * dw + e];
      uint32_t q = 0;
#pragma unroll
      for (int j = 0; j < 15; ++j) q += (wi > mids[j] * a64) ? 1u : 0u;
      if (a == 0.0f) q = 7;
      word |= q << (4 * e);
    }
    out[dw] = word;
  }
  uint4 *cp = reinterpret_cast<uint4 *>(codes + ((size_t)n * G + g) * 8);
  cp[0] = make_uint4(out[0], out[1], out[2], out[3]);
  cp[1] = make_uint4(out[4], out[5], out[6], out[7]);
  absmax[(size_t)n * G + g] = a;
}

// --- outlier selection ------------------------------------------------------

__global__ __launch_bounds__(256) void score_kernel(
    const float *__restrict__ W, int N, int K, const float *__restrict__ X,
    int P, int kind, double *__restrict__ score) {
#pragma clang fp contract(off)
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= K) return;
  double acc = 0.0;
  if (kind == QW_SCORE_MEANABS) {
    for (int n = 0; n < N; ++n) acc = acc + fabs((double)W[(size_t)n * K + c]);
    acc = acc / (double)N;
  } else {
    for (int n = 0; n < N; ++n) {
      const double v = (double)W[(size_t)n * K + c];
      acc = acc + v * v;
    }
    acc = sqrt(acc);
  }
  double pm = 0.0;
  for (int p = 0; p < P; ++p) pm = pm + fabs((double)X[(size_t)p * K + c]);
  pm = pm / (double)P;
  score[c] = acc * pm;
}

// flag[c] = 1 when fewer than n channels beat c (higher score, or equal
// score and lower index).
__global__ __launch_bounds__(256) void rank_kernel(const double *__restrict__ score,
                                                   int K, int n, int32_t *__restrict__ flag) {
  __shared__ double tile[256];
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const double s = (c < K) ? score[c] : 0.0;
  int beat = 0;
  for (int base = 0; base < K; base += 256) {
    const int j = base + threadIdx.x;
    tile[threadIdx.x] = (j < K) ? score[j] : 0.0;
    __syncthreads();
    const int lim = min(256, K - base);
    for (int t = 0; t < lim; ++t) {
      const double o = tile[t];
      const int cj = base + t;
      beat += (o > s || (o == s && cj < c)) ? 1 : 0;
    }
    __syncthreads();
  }
  if (c < K) flag[c] = (beat < n) ? 1 : 0;
}

// One workgroup: ascending compaction of flagged channels.
__global__ __launch_bounds__(1024) void compact_kernel(const int32_t *__restrict__ flag,
                                                       int K, int n, int32_t *__restrict__ out) {
  __shared__ int part[1024];
  const int T = blockDim.x, t = threadIdx.x;
  const int per = (K + T - 1) / T;
  const int b = t * per, e = min(K, b + per);
  int cnt = 0;
  for (int i = b; i < e; ++i) cnt += flag[i];
  part[t] = cnt;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int i = 0; i < T; ++i) { int v = part[i]; part[i] = run; run += v; }
  }
  __syncthreads();
  int pos = part[t];
  // never more than n writes, even if non-finite scores upset the ranks
  for (int i = b; i < e; ++i)
    if (flag[i] && pos < n) out[pos++] = i;
}

unsigned grid_for(long work, int block) { return (unsigned)((work + block - 1) / block); }

}  // namespace
}  // namespace qw

extern "C" {

qw_status qw_pack(const float *W, const qw_weight *dst, void *stream) {
  using namespace qw;
  CallScope scope;
  if (!W || !dst) return QW_ERR_INVALID_ARG;
  qw_status st = check_weight_view(dst, dst->format, 0);
  if (st != QW_OK) return st;
  if (!aligned16(W)) return QW_ERR_ALIGNMENT;
  const int N = dst->N, K = dst->K, n_out = dst->n_out;
  st = current_device(nullptr);
  if (st != QW_OK) return st;
  hipStream_t s = as_stream(stream);
  if (dst->format == QW_FMT_2BIT_G32) {
    const long groups = (long)N * (K / 32);
    QW_HIP_TRY(launch(pack2_kernel, grid_for(groups, 256), 256, 0, s, W, N, K,
                      (const int32_t *)dst->out_idx, n_out,
                      reinterpret_cast<uint32_t *>(dst->codes),
                      reinterpret_cast<uint32_t *>(dst->scales)));
    if (n_out > 0) {
      const long cnt = (long)N * dst->n_out_pad;
      QW_HIP_TRY(launch(anchors_kernel, grid_for(cnt, 256), 256, 0, s, W, N, K,
                        (const int32_t *)dst->out_idx, n_out, (int)dst->n_out_pad,
                        dst->out_w));
      QW_HIP_TRY(launch(mask_kernel, grid_for(K / 32, 256), 256, 0, s,
                        (const int32_t *)dst->out_idx, n_out, K, dst->out_mask));
    }
  } else {
    Levels16 L;
    const float *h = nf4_levels_host();
    for (int i = 0; i < 16; ++i) L.v[i] = h[i];
    const long blocks = (long)N * (K / 64);
    QW_HIP_TRY(launch(pack_nf4_kernel, grid_for(blocks, 256), 256, 0, s, W, N, K, L,
                      reinterpret_cast<uint32_t *>(dst->codes),
                      reinterpret_cast<float *>(dst->scales)));
  }
  return QW_OK;
}

qw_status qw_select_outliers(const float *W, int N, int K, const float *X_prof, int P,
                             double frac, qw_score score, int32_t *out_idx, void *stream) {
  using namespace qw;
  CallScope scope;
  if (!W || !X_prof || N <= 0 || K <= 0 || P <= 0) return QW_ERR_INVALID_ARG;
  if (score != QW_SCORE_MEANABS && score != QW_SCORE_L2) return QW_ERR_INVALID_ARG;
  const int n = qw_outlier_count(K, frac);
  if (n < 0) return QW_ERR_INVALID_ARG;
  if (n > 0 && !out_idx) return QW_ERR_INVALID_ARG;
  if (!aligned16(W) || !aligned16(X_prof) || (n > 0 && !aligned16(out_idx))) return QW_ERR_ALIGNMENT;
  qw_status st = current_device(nullptr);
  if (st != QW_OK) return st;
  if (n == 0) return QW_OK;
  hipStream_t s = as_stream(stream);
  void *scratch = nullptr;
  const size_t bytes = (size_t)K * (sizeof(double) + sizeof(int32_t));
  QW_HIP_TRY(hipMallocAsync(&scratch, bytes, s));
  double *sc = reinterpret_cast<double *>(scratch);
  int32_t *flag = reinterpret_cast<int32_t *>(sc + K);
  hipError_t e = launch(score_kernel, grid_for(K, 256), 256, 0, s, W, N, K, X_prof, P,
                        (int)score, sc);
  if (e == hipSuccess)
    e = launch(rank_kernel, grid_for(K, 256), 256, 0, s, (const double *)sc, K, n, flag);
  if (e == hipSuccess)
    e = launch(compact_kernel, 1, 1024, 0, s, (const int32_t *)flag, K, n, out_idx);
  hipError_t fe = hipFreeAsync(scratch, s);
  if (e != hipSuccess || fe != hipSuccess) return QW_ERR_HIP;
  return QW_OK;
}

}  // extern "C"
