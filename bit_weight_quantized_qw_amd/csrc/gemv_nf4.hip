// Decode GEMV against NF4 block-wise codes ("AirQuant" README,
// "Fundamentacao Teorica e Arquitetura" item 2: NormalFloat4 with
// block-wise absmax).
//
//   y[b][n] = sum_blk absmax[n][blk] * sum_{k in blk} x[b][k] L[q_k]
//
// Same mapping as the 2-bit GEMV: a workgroup owns a row range, its waves
// split K, lane `l` of wave `w` owns code dwords u = (j*W + w)*64 + l (8
// codes each) and keeps those x pairs in registers across rows.
//
// Decode: each code byte (two elements) indexes a 256-entry LDS table whose
// entry holds the pair (L[lo], L[hi]) split into an fp16 high part and an
// fp16 remainder (L = hi + lo to within 2^-22 relative), so one ds_read_b64
// feeds two v_dot2_f32_f16 for two weights with exact products and fp32
// accumulation.
#include "qw_internal.h"

namespace qw {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

struct Nf4Split { uint16_t hi[16], lo[16]; };

struct ArgsNf4 {
  const uint32_t *codes;  // [N][K/8]
  const float *absmax;    // [N][K/64]
  const uint16_t *x;      // [B][K]
  void *y;                // [B][N]
  int N, K, rows_per_wg;
  Nf4Split L;
};

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int B, int UW, bool F32OUT>
__global__ __launch_bounds__(512) void gemv_nf4_kernel(ArgsNf4 a) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int T = blockDim.x;
  const int K = a.K;
  const int KD = K >> 3;   // code dwords per row
  const int KB = K >> 6;   // absmax per row
  const int r0 = (int)blockIdx.x * a.rows_per_wg;
  const int r1 = min(a.N, r0 + a.rows_per_wg);

  uint2 *table = reinterpret_cast<uint2 *>(lds);         // [256]
  float *parts = reinterpret_cast<float *>(lds + 512);    // [rows][W][B]
  for (int v = threadIdx.x; v < 256; v += T) {
    const int q0 = v & 15, q1 = v >> 4;
    uint2 e;
    e.x = (uint32_t)a.L.hi[q0] | ((uint32_t)a.L.hi[q1] << 16);
    e.y = (uint32_t)a.L.lo[q0] | ((uint32_t)a.L.lo[q1] << 16);
    table[v] = e;
  }

  uint32_t xr[UW][B][4];
#pragma unroll
  for (int j = 0; j < UW; ++j) {
    const int u = (j * W + w) * 64 + lane;
    const bool ok = u < KD;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ok) v = *reinterpret_cast<const uint4 *>(a.x + (size_t)b * K + (size_t)u * 8);
      xr[j][b][0] = v.x; xr[j][b][1] = v.y; xr[j][b][2] = v.z; xr[j][b][3] = v.w;
    }
  }
  __syncthreads();

  constexpr int RU = (UW <= 4) ? 4 : 2;
  for (int r = r0; r < r1; r += RU) {
    uint32_t cw[RU][UW];
    float am[RU][UW];
#pragma unroll
    for (int i = 0; i < RU; ++i) {
      const int rr = r + i;
#pragma unroll
      for (int j = 0; j < UW; ++j) {
        const int u = (j * W + w) * 64 + lane;
        const bool ok = rr < r1 && u < KD;
        cw[i][j] = ok ? __builtin_nontemporal_load(a.codes + (size_t)rr * KD + u) : 0u;
        am[i][j] = ok ? __builtin_nontemporal_load(a.absmax + (size_t)rr * KB + (u >> 3)) : 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < RU; ++i) {
      const int rr = r + i;
      if (rr >= r1) break;
      float acc[B];
#pragma unroll
      for (int b = 0; b < B; ++b) acc[b] = 0.0f;
#pragma unroll
      for (int j = 0; j < UW; ++j) {
        const uint32_t c = cw[i][j];
        uint2 e[4];
        e[0] = table[c & 0xFFu];
        e[1] = table[(c >> 8) & 0xFFu];
        e[2] = table[(c >> 16) & 0xFFu];
        e[3] = table[c >> 24];
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float t = 0.0f;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            t = dot2(xr[j][b][p], e[p].x, t);
            t = dot2(xr[j][b][p], e[p].y, t);
          }
          acc[b] = __builtin_fmaf(am[i][j], t, acc[b]);
        }
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float v = wave_sum(acc[b]);
        if (lane == 0) parts[((rr - r0) * W + w) * B + b] = v;
      }
    }
  }
  __syncthreads();
  const int nrows = r1 - r0;
  for (int t = threadIdx.x; t < nrows * B; t += T) {
    const int rl = t / B, b = t - rl * B;
    float v = 0.0f;
    for (int i = 0; i < W; ++i) v += parts[(rl * W + i) * B + b];
    const size_t o = (size_t)b * a.N + (r0 + rl);
    if (F32OUT)
      reinterpret_cast<float *>(a.y)[o] = v;
    else
      reinterpret_cast<_Float16 *>(a.y)[o] = (_Float16)v;
  }
}

template <int B, int UW>
qw_status launch_uw(const ArgsNf4 &a, bool f32, int W, int grid, size_t lds, hipStream_t s) {
  if (f32)
    gemv_nf4_kernel<B, UW, true><<<grid, W * 64, lds, s>>>(a);
  else
    gemv_nf4_kernel<B, UW, false><<<grid, W * 64, lds, s>>>(a);
  QW_LAUNCH_CHECK();
  return QW_OK;
}

template <int B>
qw_status launch_b(const ArgsNf4 &a, bool f32, int UW, int W, int grid, size_t lds, hipStream_t s) {
  if constexpr (B == 1) {
    switch (UW) {
      case 1: return launch_uw<1, 1>(a, f32, W, grid, lds, s);
      case 2: return launch_uw<1, 2>(a, f32, W, grid, lds, s);
      case 3: return launch_uw<1, 3>(a, f32, W, grid, lds, s);
      case 4: return launch_uw<1, 4>(a, f32, W, grid, lds, s);
      case 6: return launch_uw<1, 6>(a, f32, W, grid, lds, s);
      case 8: return launch_uw<1, 8>(a, f32, W, grid, lds, s);
      case 5: case 7: return launch_uw<1, 8>(a, f32, W, grid, lds, s);
      case 12: return launch_uw<1, 12>(a, f32, W, grid, lds, s);
      default: return launch_uw<1, 16>(a, f32, W, grid, lds, s);
    }
  } else {
    switch (UW) {
      case 1: return launch_uw<B, 1>(a, f32, W, grid, lds, s);
      case 2: return launch_uw<B, 2>(a, f32, W, grid, lds, s);
      case 3: case 4: return launch_uw<B, 4>(a, f32, W, grid, lds, s);
      default: return launch_uw<B, 8>(a, f32, W, grid, lds, s);
    }
  }
}

int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return v ? atoi(v) : dflt;
}

Nf4Split split_levels() {
  Nf4Split sp;
  const float *L = nf4_levels_host();
  for (int i = 0; i < 16; ++i) {
    const uint16_t hb = f64_to_f16_rne((double)L[i]);
    const double hv = (double)f16_bits_to_f32(hb);
    sp.hi[i] = hb;
    sp.lo[i] = f64_to_f16_rne((double)L[i] - hv);
  }
  return sp;
}

}  // namespace
}  // namespace qw

extern "C" qw_status qgemv_nf4(const qw_weight *w, const void *x, int B, void *y,
                               qw_dtype y_dtype, void *stream) {
  using namespace qw;
  if (!w || w->format != QW_FMT_NF4_B64 || !x || !y) return QW_ERR_INVALID_ARG;
  if (B < 1 || B > 8) return QW_ERR_INVALID_ARG;
  if (y_dtype != QW_DT_F16 && y_dtype != QW_DT_F32) return QW_ERR_INVALID_ARG;
  qw_status st = qw_packed_sizes(QW_FMT_NF4_B64, w->N, w->K, w->n_out, nullptr, nullptr,
                                 nullptr, nullptr);
  if (st != QW_OK) return st;
  if (!w->codes || !w->scales) return QW_ERR_INVALID_ARG;
  if (!aligned16(w->codes) || !aligned16(w->scales) || !aligned16(x) || !aligned16(y))
    return QW_ERR_ALIGNMENT;
  int cus = 0;
  st = current_device(&cus);
  if (st != QW_OK) return st;
  const bool f32 = y_dtype == QW_DT_F32;
  const size_t esz = f32 ? 4 : 2;
  const int K = w->K;
  const int KD = K / 8;
  const int U = (KD + 63) / 64;
  static const Nf4Split sp = split_levels();
  int b0 = 0;
  while (b0 < B) {
    const int rest = B - b0;
    const int Bk = rest >= 4 ? 4 : (rest >= 2 ? 2 : 1);
    const int maxuw = Bk == 1 ? 16 : (Bk == 2 ? 8 : 4);
    const int W = (U + maxuw - 1) / maxuw;
    if (W > 8) return QW_ERR_UNSUPPORTED;
    const int UW = (U + W - 1) / W;
    int rpw = env_int("QW_GEMV_ROWS_PER_WG", 0);
    if (rpw <= 0) {
      const long target_waves = (long)cus * 16;
      rpw = (int)(((long)w->N * W + target_waves - 1) / target_waves);
      rpw = max(2, min(rpw, 32));
    }
    ArgsNf4 a{};
    a.codes = reinterpret_cast<const uint32_t *>(w->codes);
    a.absmax = reinterpret_cast<const float *>(w->scales);
    a.x = reinterpret_cast<const uint16_t *>(x) + (size_t)b0 * K;
    a.y = reinterpret_cast<char *>(y) + (size_t)b0 * w->N * esz;
    a.N = w->N;
    a.K = K;
    a.rows_per_wg = rpw;
    a.L = sp;
    const int grid = (w->N + rpw - 1) / rpw;
    const size_t lds = 256 * 8 + 4 * (size_t)rpw * W * Bk;
    switch (Bk) {
      case 1: st = launch_b<1>(a, f32, UW, W, grid, lds, as_stream(stream)); break;
      case 2: st = launch_b<2>(a, f32, UW, W, grid, lds, as_stream(stream)); break;
      default: st = launch_b<4>(a, f32, UW, W, grid, lds, as_stream(stream)); break;
    }
    if (st != QW_OK) return st;
    b0 += Bk;
  }
  return QW_OK;
}
