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
// sequential fp64 evaluation of the same formulas. Weights may be fp32,
// fp16 or bf16; each widens exactly to fp32 before anything else.
//
// Optional refinement of the 2-bit code (0 rounds by default): section 3
// fits S, Z to given codes and section 2 assigns each weight its nearest
// centroid; a round applies that rule to the fitted levels S*C[j] + Z (a
// weight keeps its code when that level is among the nearest, else takes the
// lowest nearest j) and refits, as in Lloyd's method. Each round can only
// lower the group's squared error (up to the epsilon of the fit).
#include <math.h>

#include <type_traits>

#include "qw_internal.h"

namespace qw {
namespace {

struct Levels16 { float v[16]; };

// Exact widening of one stored weight to fp32.
struct Bf16 { uint16_t bits; };
__device__ inline float widen(float v) { return v; }
__device__ inline float widen(_Float16 v) { return (float)v; }
__device__ inline float widen(Bf16 v) { return __builtin_bit_cast(float, (uint32_t)v.bits << 16); }

template <typename WT>
__device__ inline void load_row_run(const WT *__restrict__ p, float *out, int count) {
#pragma unroll
  for (int i = 0; i < count; ++i) out[i] = widen(p[i]);
}

template <typename WT>
__global__ __launch_bounds__(256) void pack2_kernel(
    const WT *__restrict__ W, int N, int K, const int32_t *__restrict__ idx,
    int n_out, int rounds, uint32_t *__restrict__ codes, uint32_t *__restrict__ sz) {
#pragma clang fp contract(off)
  const int G = K / 32;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)N * G) return;
  const int n = (int)(gid / G), g = (int)(gid % G);
  float wf[32];
  load_row_run(W + (size_t)n * K + (size_t)g * 32, wf, 32);

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
  for (int i = 0; i < 32; ++i) w[i] = ((omask >> i) & 1u) ? 0.0 : (double)wf[i];

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
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const bool outer = (d[i] * d[i]) > thr;
    const bool upper = d[i] >= 0.0;
    q[i] = upper ? (outer ? 3u : 2u) : (outer ? 0u : 1u);
  }
  const double Cv[4] = {C0, C1, C2, C3};
  // section-3 fit of the current codes
  double S, Z;
  auto fit = [&]() __attribute__((always_inline)) {
    double c[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) c[i] = q[i] == 0 ? C0 : (q[i] == 1 ? C1 : (q[i] == 2 ? C2 : C3));
    double a = 0.0;
#pragma unroll
    for (int i = 0; i < 32; ++i) a = a + c[i];
    const double cbar = a / 32.0;
    double num = 0.0, den = 0.0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const double cc = c[i] - cbar;
      num = num + d[i] * cc;
      den = den + cc * cc;
    }
    den = den + 1e-8;
    S = num / den;
    Z = m - S * cbar;
  };
  fit();
  for (int r = 0; r < rounds; ++r) {
    double lev[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) lev[j] = S * Cv[j] + Z;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      double dist[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) dist[j] = fabs(w[i] - lev[j]);
      const double best = fmin(fmin(dist[0], dist[1]), fmin(dist[2], dist[3]));
      const double cur = q[i] == 0 ? dist[0] : (q[i] == 1 ? dist[1] : (q[i] == 2 ? dist[2] : dist[3]));
      if (!(cur == best)) q[i] = dist[0] == best ? 0u : (dist[1] == best ? 1u : (dist[2] == best ? 2u : 3u));
    }
    fit();
  }

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

template <typename WT>
__global__ __launch_bounds__(256) void anchors_kernel(
    const WT *__restrict__ W, int N, int K, const int32_t *__restrict__ idx,
    int n_out, int n_out_pad, uint16_t *__restrict__ out_w) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)N * n_out_pad) return;
  const int n = (int)(gid / n_out_pad), o = (int)(gid % n_out_pad);
  uint16_t v = 0;
  if (o < n_out) {
    const int c = idx[o];
    if (c >= 0 && c < K) v = f64_to_f16_rne((double)widen(W[(size_t)n * K + c]));
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

template <typename WT>
__global__ __launch_bounds__(256) void pack_nf4_kernel(
    const WT *__restrict__ W, int N, int K, Levels16 L,
    uint32_t *__restrict__ codes, float *__restrict__ absmax) {
#pragma clang fp contract(off)
  const int G = K / 64;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)N * G) return;
  const int n = (int)(gid / G), g = (int)(gid % G);
  float w[64];
  load_row_run(W + (size_t)n * K + (size_t)g * 64, w, 64);
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

// INT4 (the OTF-LLM page's v3.2 format, "Comparative Analysis"): one thread
// per group of 32 permuted positions. The weights are read in original
// channel order through perm; positions below n_out are the fp16 anchors
// and count as 0 here. In fp64: a = max |w|, s = fp16(a / 7) (one
// round-to-nearest-even), q = clamp(rint(w / s), -7, 7) with the stored s
// (rint rounds ties to even; s == 0 gives q = 0); nibble q + 8, the even
// position in the low nibble.
template <typename WT>
__global__ __launch_bounds__(256) void pack_int4_kernel(
    const WT *__restrict__ W, int N, int K, const int32_t *__restrict__ perm, int n_out,
    uint32_t *__restrict__ codes, uint16_t *__restrict__ scales) {
#pragma clang fp contract(off)
  const int G = K / 32;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)N * G) return;
  const int n = (int)(gid / G), g = (int)(gid % G);
  const WT *row = W + (size_t)n * K;
  double w[32];
  double a = 0.0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int j = 32 * g + i;
    const int c = perm[j];
    const double v = (j < n_out || c < 0 || c >= K) ? 0.0 : (double)widen(row[c]);
    w[i] = v;
    a = fmax(a, fabs(v));
  }
  const uint16_t s16 = f64_to_f16_rne(a / 7.0);
  const double s = (double)f16_bits_to_f32(s16);
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    double q = 0.0;
    if (s > 0.0) q = fmin(7.0, fmax(-7.0, __builtin_rint(w[i] / s)));
    out[i >> 3] |= (uint32_t)((int)q + 8) << (4 * (i & 7));
  }
  reinterpret_cast<uint4 *>(codes)[(size_t)n * G + g] = make_uint4(out[0], out[1], out[2], out[3]);
  scales[(size_t)n * G + g] = s16;
}

// --- outlier selection ------------------------------------------------------

// Column sums over rows, in row order, in fp64: out[c] = init[c] + f(A[0][c])
// + f(A[1][c]) + ... with f = |a| (kind 0) or a*a (kind 1). One workgroup per
// 64 columns: all four waves load chunks of 128 rows (coalesced across the
// columns, 32 loads in flight per thread, rows past R as zeros) into LDS
// while wave 0 adds the previous chunk row by row, one column per lane, so
// every column's sum is the plain sequential one. init, if given, must be
// non-negative (it is an earlier sum of this kind).
constexpr int kColChunk = 128;

// One element through a buffer load: offsets past the descriptor's size
// read as zero, so guarded loads need no branch and all stay in flight.
__device__ inline __amdgpu_buffer_rsrc_t elem_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ inline float load_elem(__amdgpu_buffer_rsrc_t r, uint32_t off, const float *) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ inline float load_elem(__amdgpu_buffer_rsrc_t r, uint32_t off, const _Float16 *) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
}
__device__ inline float load_elem(__amdgpu_buffer_rsrc_t r, uint32_t off, const Bf16 *) {
  return __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0) << 16);
}
constexpr uint32_t kElemOob = 0x7FFFFFF0u;

template <typename T, int KIND>
__global__ __launch_bounds__(256) void colsum_kernel(const T *__restrict__ A, int R, int C,
                                                     const double *__restrict__ init,
                                                     double *__restrict__ out) {
#pragma clang fp contract(off)
  __shared__ float tile[2][kColChunk][64];
  const int t = threadIdx.x, lane = t & 63, r_off = t >> 6;
  const int c = blockIdx.x * 64 + lane;
  const bool cok = c < C;
  // the host keeps R * C * sizeof(T) below 2^31
  const auto rs = elem_rsrc(A, (uint32_t)((size_t)R * C * sizeof(T)));
  float v[kColChunk / 4];
  auto load = [&](int r0) {
#pragma unroll
    for (int i = 0; i < kColChunk / 4; ++i) {
      const int r = r0 + r_off + 4 * i;
      const uint32_t off = (cok && r < R) ? (uint32_t)(((size_t)r * C + c) * sizeof(T)) : kElemOob;
      v[i] = load_elem(rs, off, A);
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int i = 0; i < kColChunk / 4; ++i) tile[b][r_off + 4 * i][lane] = v[i];
  };
  double acc = (init && cok) ? init[c] : 0.0;
  const int nch = (R + kColChunk - 1) / kColChunk;
  load(0);
  store(0);
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const int b = ch & 1;
    if (ch + 1 < nch) load((ch + 1) * kColChunk);
    if (t < 64) {
      // rows past R hold +0: adding +0 to a sum that is never -0 (it starts
      // at +0 or at an earlier sum of non-negative terms) changes no bit, so
      // the whole chunk is added without a row test and the reads batch up
#pragma unroll
      for (int r = 0; r < kColChunk; ++r) {
        const double x = (double)tile[b][r][lane];
        acc = acc + (KIND == 0 ? fabs(x) : x * x);
      }
    }
    if (ch + 1 < nch) store(b ^ 1);
    __syncthreads();
  }
  if (t < 64 && cok) out[c] = acc;
}

// score[c] = stat(W column c) * profile mean of channel c, with the column
// sum of W already in score[c]: MEANABS divides it by N, L2 takes its root.
__global__ __launch_bounds__(256) void score_finish_kernel(double *__restrict__ score, int K, int N,
                                                          int kind, const double *__restrict__ prof_sum,
                                                          double rows) {
#pragma clang fp contract(off)
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= K) return;
  const double col = kind == QW_SCORE_MEANABS ? score[c] / (double)N : sqrt(score[c]);
  score[c] = col * (prof_sum[c] / rows);
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

// perm[rank(c)] = c, rank(c) = number of channels that beat c (higher
// score, or equal score and lower index): channels by descending score.
__global__ __launch_bounds__(256) void perm_kernel(const double *__restrict__ score, int K,
                                                   int32_t *__restrict__ perm) {
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
  // ranks of finite scores are distinct; NaN scores would collide, so a
  // rank is written only in range
  if (c < K && beat < K) perm[beat] = c;
}

// X_p[m][j] = X[m][perm[j]] for elements of ES bytes (2 or 4).
template <int ES>
__global__ __launch_bounds__(256) void permute_cols_kernel(const uint8_t *__restrict__ X, int M, int K,
                                                           const int32_t *__restrict__ perm,
                                                           uint8_t *__restrict__ Xp) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)M * K) return;
  const int m = (int)(i / K), j = (int)(i % K);
  const int c = perm[j];
  typedef typename std::conditional<ES == 2, uint16_t, uint32_t>::type T;
  T v = 0;
  if (c >= 0 && c < K) v = reinterpret_cast<const T *>(X)[(size_t)m * K + c];
  reinterpret_cast<T *>(Xp)[i] = v;
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

template <typename WT>
qw_status pack_typed(const WT *W, int rounds, const qw_weight *dst, hipStream_t s) {
  const int N = dst->N, K = dst->K, n_out = dst->n_out;
  if (dst->format == QW_FMT_2BIT_G32) {
    const long groups = (long)N * (K / 32);
    QW_HIP_TRY(launch(pack2_kernel<WT>, grid_for(groups, 256), 256, 0, s, W, N, K,
                      (const int32_t *)dst->out_idx, n_out, rounds,
                      reinterpret_cast<uint32_t *>(dst->codes),
                      reinterpret_cast<uint32_t *>(dst->scales)));
    if (n_out > 0) {
      const long cnt = (long)N * dst->n_out_pad;
      QW_HIP_TRY(launch(anchors_kernel<WT>, grid_for(cnt, 256), 256, 0, s, W, N, K,
                        (const int32_t *)dst->out_idx, n_out, (int)dst->n_out_pad,
                        dst->out_w));
      QW_HIP_TRY(launch(mask_kernel, grid_for(K / 32, 256), 256, 0, s,
                        (const int32_t *)dst->out_idx, n_out, K, dst->out_mask));
    }
  } else if (dst->format == QW_FMT_INT4_G32) {
    const long groups = (long)N * (K / 32);
    QW_HIP_TRY(launch(pack_int4_kernel<WT>, grid_for(groups, 256), 256, 0, s, W, N, K,
                      (const int32_t *)dst->out_idx, n_out, reinterpret_cast<uint32_t *>(dst->codes),
                      reinterpret_cast<uint16_t *>(dst->scales)));
    if (n_out > 0) {
      // anchors: the weights of channels perm[0..n_out)
      const long cnt = (long)N * dst->n_out_pad;
      QW_HIP_TRY(launch(anchors_kernel<WT>, grid_for(cnt, 256), 256, 0, s, W, N, K,
                        (const int32_t *)dst->out_idx, n_out, (int)dst->n_out_pad, dst->out_w));
    }
  } else {
    Levels16 L;
    const float *h = nf4_levels_host();
    for (int i = 0; i < 16; ++i) L.v[i] = h[i];
    const long blocks = (long)N * (K / 64);
    QW_HIP_TRY(launch(pack_nf4_kernel<WT>, grid_for(blocks, 256), 256, 0, s, W, N, K, L,
                      reinterpret_cast<uint32_t *>(dst->codes),
                      reinterpret_cast<float *>(dst->scales)));
  }
  return QW_OK;
}

// Top-n channels of a score vector in device scratch -> out_idx (ascending).
qw_status rank_and_compact(const double *sc, int32_t *flag, int K, int n, int32_t *out_idx,
                           hipStream_t s) {
  QW_HIP_TRY(launch(rank_kernel, grid_for(K, 256), 256, 0, s, sc, K, n, flag));
  QW_HIP_TRY(launch(compact_kernel, 1, 1024, 0, s, (const int32_t *)flag, K, n, out_idx));
  return QW_OK;
}

}  // namespace
}  // namespace qw

extern "C" {

qw_status qw_pack(const float *W, const qw_weight *dst, void *stream) {
  return qw_pack_ex(W, QW_DT_F32, 0, dst, stream);
}

qw_status qw_pack_ex(const void *W, qw_dtype w_dtype, int refine_rounds, const qw_weight *dst,
                     void *stream) {
  using namespace qw;
  CallScope scope;
  if (!W || !dst) return QW_ERR_INVALID_ARG;
  if (w_dtype != QW_DT_F32 && w_dtype != QW_DT_F16 && w_dtype != QW_DT_BF16) return QW_ERR_INVALID_ARG;
  qw_status st = check_weight_view(dst, dst->format, 0);
  if (st != QW_OK) return st;
  if (dst->format == QW_FMT_INT4_G32) {  // the permutation is an input
    if (!dst->out_idx) return QW_ERR_INVALID_ARG;
    if (!aligned16(dst->out_idx)) return QW_ERR_ALIGNMENT;
  }
  if (refine_rounds < 0 || refine_rounds > QW_MAX_REFINE_ROUNDS) return QW_ERR_INVALID_ARG;
  if (dst->format != QW_FMT_2BIT_G32 && refine_rounds != 0) return QW_ERR_INVALID_ARG;
  if (!aligned16(W)) return QW_ERR_ALIGNMENT;
  st = current_device(nullptr);
  if (st != QW_OK) return st;
  hipStream_t s = as_stream(stream);
  switch (w_dtype) {
    case QW_DT_F16: return pack_typed(reinterpret_cast<const _Float16 *>(W), refine_rounds, dst, s);
    case QW_DT_BF16: return pack_typed(reinterpret_cast<const Bf16 *>(W), refine_rounds, dst, s);
    default: return pack_typed(reinterpret_cast<const float *>(W), refine_rounds, dst, s);
  }
}

qw_status qw_profile_accumulate(const void *X, qw_dtype x_dtype, int M, int K, double *abs_sum,
                                void *stream) {
  using namespace qw;
  CallScope scope;
  if (!X || !abs_sum || M <= 0 || K <= 0) return QW_ERR_INVALID_ARG;
  if (x_dtype != QW_DT_F32 && x_dtype != QW_DT_F16 && x_dtype != QW_DT_BF16) return QW_ERR_INVALID_ARG;
  if ((size_t)M * K * (x_dtype == QW_DT_F32 ? 4 : 2) >= (1ull << 31)) return QW_ERR_UNSUPPORTED;
  if (!aligned16(X) || !aligned16(abs_sum)) return QW_ERR_ALIGNMENT;
  qw_status st = current_device(nullptr);
  if (st != QW_OK) return st;
  hipStream_t s = as_stream(stream);
  const unsigned grid = grid_for(K, 64);
  switch (x_dtype) {
    case QW_DT_F16:
      QW_HIP_TRY(launch(colsum_kernel<_Float16, 0>, grid, 256, 0, s, reinterpret_cast<const _Float16 *>(X), M, K,
                        (const double *)abs_sum, abs_sum));
      break;
    case QW_DT_BF16:
      QW_HIP_TRY(launch(colsum_kernel<Bf16, 0>, grid, 256, 0, s, reinterpret_cast<const Bf16 *>(X), M, K,
                        (const double *)abs_sum, abs_sum));
      break;
    default:
      QW_HIP_TRY(launch(colsum_kernel<float, 0>, grid, 256, 0, s, reinterpret_cast<const float *>(X), M, K,
                        (const double *)abs_sum, abs_sum));
  }
  return QW_OK;
}

qw_status qw_select_outliers(const float *W, int N, int K, const float *X_prof, int P,
                             double frac, qw_score score, int32_t *out_idx, void *workspace,
                             size_t workspace_bytes, void *stream) {
  using namespace qw;
  CallScope scope;
  if (!W || !X_prof || N <= 0 || K <= 0 || P <= 0) return QW_ERR_INVALID_ARG;
  if ((size_t)N * K * 4 >= (1ull << 31) || (size_t)P * K * 4 >= (1ull << 31)) return QW_ERR_UNSUPPORTED;
  if (score != QW_SCORE_MEANABS && score != QW_SCORE_L2) return QW_ERR_INVALID_ARG;
  const int n = qw_outlier_count(K, frac);
  if (n < 0) return QW_ERR_INVALID_ARG;
  if (n > 0 && !out_idx) return QW_ERR_INVALID_ARG;
  if (n > 0 && (!workspace || workspace_bytes < qw_select_workspace_bytes(K))) return QW_ERR_INVALID_ARG;
  if (!aligned16(W) || !aligned16(X_prof) || (n > 0 && (!aligned16(out_idx) || !aligned16(workspace))))
    return QW_ERR_ALIGNMENT;
  qw_status st = current_device(nullptr);
  if (st != QW_OK) return st;
  if (n == 0) return QW_OK;
  hipStream_t s = as_stream(stream);
  // workspace: scores [K] double, profile means [K] double, flags [K] int32
  double *sc = reinterpret_cast<double *>(workspace);
  double *prof = sc + K;
  int32_t *flag = reinterpret_cast<int32_t *>(prof + K);
  const unsigned cgrid = grid_for(K, 64);
  hipError_t e = score == QW_SCORE_MEANABS
                     ? launch(colsum_kernel<float, 0>, cgrid, 256, 0, s, W, N, K, (const double *)nullptr, sc)
                     : launch(colsum_kernel<float, 1>, cgrid, 256, 0, s, W, N, K, (const double *)nullptr, sc);
  if (e == hipSuccess)
    e = launch(colsum_kernel<float, 0>, cgrid, 256, 0, s, X_prof, P, K, (const double *)nullptr, prof);
  if (e == hipSuccess)
    e = launch(score_finish_kernel, grid_for(K, 256), 256, 0, s, sc, K, N, (int)score,
               (const double *)prof, (double)P);
  return e == hipSuccess ? rank_and_compact(sc, flag, K, n, out_idx, s) : QW_ERR_HIP;
}

qw_status qw_select_perm(const float *W, int N, int K, const float *X_prof, int P, qw_score score,
                         int32_t *perm_out, void *workspace, size_t workspace_bytes, void *stream) {
  using namespace qw;
  CallScope scope;
  if (!W || !X_prof || !perm_out || N <= 0 || K <= 0 || P <= 0) return QW_ERR_INVALID_ARG;
  if ((size_t)N * K * 4 >= (1ull << 31) || (size_t)P * K * 4 >= (1ull << 31)) return QW_ERR_UNSUPPORTED;
  if (score != QW_SCORE_MEANABS && score != QW_SCORE_L2) return QW_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < qw_select_workspace_bytes(K)) return QW_ERR_INVALID_ARG;
  if (!aligned16(W) || !aligned16(X_prof) || !aligned16(perm_out) || !aligned16(workspace))
    return QW_ERR_ALIGNMENT;
  qw_status st = current_device(nullptr);
  if (st != QW_OK) return st;
  hipStream_t s = as_stream(stream);
  // workspace: scores [K] double, profile sums [K] double
  double *sc = reinterpret_cast<double *>(workspace);
  double *prof = sc + K;
  const unsigned cgrid = grid_for(K, 64);
  QW_HIP_TRY(score == QW_SCORE_MEANABS
                 ? launch(colsum_kernel<float, 0>, cgrid, 256, 0, s, W, N, K, (const double *)nullptr, sc)
                 : launch(colsum_kernel<float, 1>, cgrid, 256, 0, s, W, N, K, (const double *)nullptr, sc));
  QW_HIP_TRY(launch(colsum_kernel<float, 0>, cgrid, 256, 0, s, X_prof, P, K, (const double *)nullptr, prof));
  QW_HIP_TRY(launch(score_finish_kernel, grid_for(K, 256), 256, 0, s, sc, K, N, (int)score,
                    (const double *)prof, (double)P));
  QW_HIP_TRY(launch(perm_kernel, grid_for(K, 256), 256, 0, s, (const double *)sc, K, perm_out));
  return QW_OK;
}

qw_status qw_permute_cols(const void *X, qw_dtype dtype, int M, int K, const int32_t *perm, void *X_p,
                          void *stream) {
  using namespace qw;
  CallScope scope;
  if (!X || !perm || !X_p || M <= 0 || K <= 0 || X == X_p) return QW_ERR_INVALID_ARG;
  if (dtype != QW_DT_F16 && dtype != QW_DT_BF16 && dtype != QW_DT_F32) return QW_ERR_INVALID_ARG;
  const size_t es = dtype == QW_DT_F32 ? 4 : 2;
  if ((size_t)M * K * es >= (1ull << 31)) return QW_ERR_UNSUPPORTED;
  if (!aligned16(X) || !aligned16(perm) || !aligned16(X_p)) return QW_ERR_ALIGNMENT;
  qw_status st = current_device(nullptr);
  if (st != QW_OK) return st;
  hipStream_t s = as_stream(stream);
  const unsigned grid = grid_for((long)M * K, 256);
  const uint8_t *src = reinterpret_cast<const uint8_t *>(X);
  uint8_t *dst = reinterpret_cast<uint8_t *>(X_p);
  if (es == 2)
    QW_HIP_TRY(launch(permute_cols_kernel<2>, grid, 256, 0, s, src, M, K, perm, dst));
  else
    QW_HIP_TRY(launch(permute_cols_kernel<4>, grid, 256, 0, s, src, M, K, perm, dst));
  return QW_OK;
}

qw_status qw_select_outliers_ex(const void *W, qw_dtype w_dtype, int N, int K,
                                const double *prof_abs_sum, long long prof_rows, double frac,
                                qw_score score, int32_t *out_idx, void *workspace,
                                size_t workspace_bytes, void *stream) {
  using namespace qw;
  CallScope scope;
  if (!W || !prof_abs_sum || N <= 0 || K <= 0 || prof_rows <= 0) return QW_ERR_INVALID_ARG;
  if (w_dtype != QW_DT_F32 && w_dtype != QW_DT_F16 && w_dtype != QW_DT_BF16) return QW_ERR_INVALID_ARG;
  if ((size_t)N * K * (w_dtype == QW_DT_F32 ? 4 : 2) >= (1ull << 31)) return QW_ERR_UNSUPPORTED;
  if (score != QW_SCORE_MEANABS && score != QW_SCORE_L2) return QW_ERR_INVALID_ARG;
  const int n = qw_outlier_count(K, frac);
  if (n < 0) return QW_ERR_INVALID_ARG;
  if (n > 0 && !out_idx) return QW_ERR_INVALID_ARG;
  if (n > 0 && (!workspace || workspace_bytes < qw_select_workspace_bytes(K))) return QW_ERR_INVALID_ARG;
  if (!aligned16(W) || !aligned16(prof_abs_sum) || (n > 0 && (!aligned16(out_idx) || !aligned16(workspace))))
    return QW_ERR_ALIGNMENT;
  qw_status st = current_device(nullptr);
  if (st != QW_OK) return st;
  if (n == 0) return QW_OK;
  hipStream_t s = as_stream(stream);
  // workspace: scores [K] double, flags [K] int32
  double *sc = reinterpret_cast<double *>(workspace);
  int32_t *flag = reinterpret_cast<int32_t *>(sc + K);
  const unsigned cgrid = grid_for(K, 64);
  const bool l2 = score == QW_SCORE_L2;
  hipError_t e;
  switch (w_dtype) {
    case QW_DT_F16: {
      const _Float16 *w = reinterpret_cast<const _Float16 *>(W);
      e = l2 ? launch(colsum_kernel<_Float16, 1>, cgrid, 256, 0, s, w, N, K, (const double *)nullptr, sc)
             : launch(colsum_kernel<_Float16, 0>, cgrid, 256, 0, s, w, N, K, (const double *)nullptr, sc);
      break;
    }
    case QW_DT_BF16: {
      const Bf16 *w = reinterpret_cast<const Bf16 *>(W);
      e = l2 ? launch(colsum_kernel<Bf16, 1>, cgrid, 256, 0, s, w, N, K, (const double *)nullptr, sc)
             : launch(colsum_kernel<Bf16, 0>, cgrid, 256, 0, s, w, N, K, (const double *)nullptr, sc);
      break;
    }
    default: {
      const float *w = reinterpret_cast<const float *>(W);
      e = l2 ? launch(colsum_kernel<float, 1>, cgrid, 256, 0, s, w, N, K, (const double *)nullptr, sc)
             : launch(colsum_kernel<float, 0>, cgrid, 256, 0, s, w, N, K, (const double *)nullptr, sc);
    }
  }
  if (e == hipSuccess)
    e = launch(score_finish_kernel, grid_for(K, 256), 256, 0, s, sc, K, N, (int)score, prof_abs_sum,
               (double)prof_rows);
  return e == hipSuccess ? rank_and_compact(sc, flag, K, n, out_idx, s) : QW_ERR_HIP;
}

}  // extern "C"
