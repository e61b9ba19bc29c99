// Decode GEMV against NF4 block-wise codes ("AirQuant" README,
// "Fundamentacao Teorica e Arquitetura" item 2: NormalFloat4 with
// block-wise absmax).
//
//   y[b][n] = sum_blk absmax[n][blk] * sum_{k in blk} x[b][k] L[q_k]
//
// Work split as in the 2-bit GEMV: a workgroup owns a block of rows; workers
// of W waves walk sub-ranges and split K; lane l of wave w owns code dwords
// u = (j*W + w)*64 + l (8 codes each) and keeps those x pairs in registers
// (copied once per workgroup through LDS). Weights come in through buffer
// loads; the first 2*RU rows are requested before anything else, then rows
// stream through two register buffers.
//
// Decode: each code byte (two elements) indexes a 256-entry LDS table whose
// entry holds the pair (L[lo], L[hi]) split into an fp16 high part and an
// fp16 remainder (L = hi + lo to within 2^-22 relative), so one ds_read_b64
// feeds two v_dot2_f32_f16 for two weights with exact products and fp32
// accumulation.
#include <stdlib.h>

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
  int N, K, rows_per_wg, W, f32out;
  Nf4Split L;
};

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

template <int CTRL, int ROW_MASK>
__device__ inline float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                CTRL, ROW_MASK, 0xF, false));
}

__device__ inline float wave_sum_to_lane63(float v) {
  v += dpp_f<0xB1, 0xF>(v);
  v += dpp_f<0x4E, 0xF>(v);
  v += dpp_f<0x124, 0xF>(v);
  v += dpp_f<0x128, 0xF>(v);
  v += dpp_f<0x142, 0xA>(v);
  v += dpp_f<0x143, 0xC>(v);
  return v;
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uint32_t bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

constexpr uint32_t kOob = 0x7FFFFFF0u;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Upper bound on the 16-byte x loads one thread issues while staging x
// (the host checks ceil(B*K/8 / threads) against it).
constexpr int kXLoads = 16;

// LDS: table uint2 [256] | x uint32 [B][K/2] | parts float [rows_per_wg][W][B]
template <int B, int UW>
__global__ __launch_bounds__(512) void gemv_nf4_kernel(ArgsNf4 a) {
  // Both row buffers (2 loads per row and code dword) stay within the 63
  // loads one wave can have outstanding, so the wait that precedes the x
  // staging covers only the x loads.
  constexpr int RU0 = 60 / (2 * 2 * UW);
  constexpr int RU = RU0 < 1 ? 1 : (RU0 > 8 ? 8 : RU0);
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  uint2 *table = reinterpret_cast<uint2 *>(lds);
  uint32_t *xl = lds + 512;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const int T = blockDim.x;
  const int W = a.W;
  const int V = (T >> 6) / W;
  const int w = wave % W;
  const int K = a.K;
  const int KD = K >> 3;   // code dwords per row (8 codes each)
  const int KB = K >> 6;   // absmax per row
  float *parts = reinterpret_cast<float *>(xl + B * (K >> 1));
  const int g0 = (int)blockIdx.x * a.rows_per_wg;
  const int g1 = min(a.N, g0 + a.rows_per_wg);
  const int rpw = (a.rows_per_wg + V - 1) / V;
  const int r0 = min(g1, g0 + (wave / W) * rpw);
  const int r1 = min(g1, r0 + rpw);

  const auto rc = make_rsrc(a.codes, (uint32_t)((size_t)a.N * KD * 4));
  const auto rm = make_rsrc(a.absmax, (uint32_t)((size_t)a.N * KB * 4));
  uint32_t vc[UW], vm[UW];
#pragma unroll
  for (int j = 0; j < UW; ++j) {
    const int u = (j * W + w) * 64 + lane;
    vc[j] = u < KD ? (uint32_t)u * 4 : kOob;
    vm[j] = u < KD ? (uint32_t)(u >> 3) * 4 : kOob;
  }
  uint32_t cA[RU][UW], cB[RU][UW], mA[RU][UW], mB[RU][UW];
  // Rows past the worker's range read through a zero-length descriptor, so
  // every load is unconditional (no branch for the wait counters to merge).
  const auto rz = make_rsrc(a.codes, 0u);
  auto load = [&](uint32_t (&c)[RU][UW], uint32_t (&m)[RU][UW], int rb) {
#pragma unroll
    for (int i = 0; i < RU; ++i) {
      const int rr = rb + i;
      const bool ok = rr < r1;
      const auto rcr = ok ? rc : rz, rmr = ok ? rm : rz;
      const uint32_t so_c = ok ? (uint32_t)rr * KD * 4 : 0u, so_m = ok ? (uint32_t)rr * KB * 4 : 0u;
#pragma unroll
      for (int j = 0; j < UW; ++j) {
        c[i][j] = bload(rcr, vc[j], so_c);
        m[i][j] = bload(rmr, vm[j], so_m);
      }
    }
  };

  // This group's copy of x: 16-byte buffer loads issued ahead of the weight
  // prefetch, so the LDS stores below wait only for them.
  const auto rx = make_rsrc(a.x, (uint32_t)((size_t)B * K * 2));
  const int nx = (B * KD + T - 1) / T;  // uniform trip count
  constexpr int XMAX = kXLoads;
  u32x4 xv[XMAX];
#pragma unroll
  for (int q = 0; q < XMAX; ++q) {
    if (q < nx) {
      const int i = q * T + (int)threadIdx.x;
      xv[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, i < B * KD ? i * 16 : (int)kOob, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  load(cA, mA, r0);
  load(cB, mB, r0 + RU);
  __builtin_amdgcn_sched_barrier(0);

  // level-pair table
  // (levels picked by a select chain over scalar kernel arguments: a
  // per-lane indexed read of the argument block would be a memory load
  // queued behind the weight prefetch)
  for (int v = threadIdx.x; v < 256; v += T) {
    const int q0 = v & 15, q1 = v >> 4;
    uint32_t h0 = a.L.hi[0], l0 = a.L.lo[0], h1 = a.L.hi[0], l1 = a.L.lo[0];
#pragma unroll
    for (int t = 1; t < 16; ++t) {
      h0 = q0 == t ? a.L.hi[t] : h0;
      l0 = q0 == t ? a.L.lo[t] : l0;
      h1 = q1 == t ? a.L.hi[t] : h1;
      l1 = q1 == t ? a.L.lo[t] : l1;
    }
    uint2 e;
    e.x = h0 | (h1 << 16);
    e.y = l0 | (l1 << 16);
    table[v] = e;
  }
#pragma unroll
  for (int q = 0; q < XMAX; ++q) {
    const int i = q * T + (int)threadIdx.x;
    if (q < nx && i < B * KD) reinterpret_cast<u32x4 *>(xl)[i] = xv[q];
  }
  // LDS-only barrier: a full __syncthreads would also drain the prefetch.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  uint32_t xr[UW][B][4];
#pragma unroll
  for (int j = 0; j < UW; ++j) {
    const int u = (j * W + w) * 64 + lane;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (u < KD) v = reinterpret_cast<const u32x4 *>(xl)[b * KD + u];
      xr[j][b][0] = v[0]; xr[j][b][1] = v[1]; xr[j][b][2] = v[2]; xr[j][b][3] = v[3];
    }
  }

  auto compute = [&](const uint32_t (&c)[RU][UW], const uint32_t (&m)[RU][UW], int rb) {
#pragma unroll
    for (int i = 0; i < RU; ++i) {
      const int rr = rb + i;
      if (rr >= r1) break;
      float acc[B];
#pragma unroll
      for (int b = 0; b < B; ++b) acc[b] = 0.0f;
#pragma unroll
      for (int j = 0; j < UW; ++j) {
        const uint32_t cw = c[i][j];
        uint2 e[4];
        e[0] = table[cw & 0xFFu];
        e[1] = table[(cw >> 8) & 0xFFu];
        e[2] = table[(cw >> 16) & 0xFFu];
        e[3] = table[cw >> 24];
        const float am = __builtin_bit_cast(float, m[i][j]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float t = 0.0f;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            t = dot2(xr[j][b][p], e[p].x, t);
            t = dot2(xr[j][b][p], e[p].y, t);
          }
          acc[b] = __builtin_fmaf(am, t, acc[b]);
        }
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float v = wave_sum_to_lane63(acc[b]);
        if (lane == 63) {
          if (W == 1) {
            const size_t off = (size_t)b * a.N + rr;
            if (a.f32out)
              reinterpret_cast<float *>(a.y)[off] = v;
            else
              reinterpret_cast<_Float16 *>(a.y)[off] = (_Float16)v;
          } else {
            parts[((rr - g0) * W + w) * B + b] = v;
          }
        }
      }
    }
  };

  for (int r = r0; r < r1; r += 2 * RU) {
    compute(cA, mA, r);
    load(cA, mA, r + 2 * RU);
    compute(cB, mB, r + RU);
    load(cB, mB, r + 3 * RU);
  }

  if (W > 1) {
    __syncthreads();
    const int nrows = g1 - g0;
    for (int t = threadIdx.x; t < nrows * B; t += T) {
      const int rl = t / B, b = t - rl * B;
      float v = 0.0f;
      for (int i = 0; i < W; ++i) v += parts[(rl * W + i) * B + b];
      const size_t off = (size_t)b * a.N + (g0 + rl);
      if (a.f32out)
        reinterpret_cast<float *>(a.y)[off] = v;
      else
        reinterpret_cast<_Float16 *>(a.y)[off] = (_Float16)v;
    }
  }
}

template <int B, int UW>
qw_status launch_uw(const ArgsNf4 &a, int grid, int threads, size_t lds, hipStream_t s) {
  if (lds > 64 * 1024) {
    QW_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(&gemv_nf4_kernel<B, UW>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  }
  QW_HIP_TRY(launch(gemv_nf4_kernel<B, UW>, grid, threads, lds, s, a));
  return QW_OK;
}

template <int B>
qw_status launch_b(const ArgsNf4 &a, int UW, int grid, int threads, size_t lds, hipStream_t s) {
  if constexpr (B == 1) {
    if (UW <= 1) return launch_uw<1, 1>(a, grid, threads, lds, s);
    if (UW <= 2) return launch_uw<1, 2>(a, grid, threads, lds, s);
    if (UW <= 4) return launch_uw<1, 4>(a, grid, threads, lds, s);
    if (UW <= 6) return launch_uw<1, 6>(a, grid, threads, lds, s);
    if (UW <= 8) return launch_uw<1, 8>(a, grid, threads, lds, s);
    if (UW <= 12) return launch_uw<1, 12>(a, grid, threads, lds, s);
    return launch_uw<1, 16>(a, grid, threads, lds, s);
  } else if constexpr (B == 2) {
    if (UW <= 1) return launch_uw<2, 1>(a, grid, threads, lds, s);
    if (UW <= 2) return launch_uw<2, 2>(a, grid, threads, lds, s);
    if (UW <= 4) return launch_uw<2, 4>(a, grid, threads, lds, s);
    if (UW <= 6) return launch_uw<2, 6>(a, grid, threads, lds, s);
    return launch_uw<2, 8>(a, grid, threads, lds, s);
  } else {
    if (UW <= 1) return launch_uw<4, 1>(a, grid, threads, lds, s);
    if (UW <= 2) return launch_uw<4, 2>(a, grid, threads, lds, s);
    return launch_uw<4, 4>(a, grid, threads, lds, s);
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
  CallScope scope;
  qw_status st = check_weight_view(w, QW_FMT_NF4_B64, 0);
  if (st != QW_OK) return st;
  if (!x || !y || B < 1 || B > 8) return QW_ERR_INVALID_ARG;
  if (y_dtype != QW_DT_F16 && y_dtype != QW_DT_F32) return QW_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y)) return QW_ERR_ALIGNMENT;
  int cus = 0;
  st = current_device(&cus);
  if (st != QW_OK) return st;
  const bool f32 = y_dtype == QW_DT_F32;
  const size_t esz = f32 ? 4 : 2;
  const int K = w->K;
  const int KD = K / 8;
  const int U = (KD + 63) / 64;
  static const Nf4Split sp = split_levels();
  if ((size_t)w->N * (K / 2) >= (1ull << 31)) return QW_ERR_UNSUPPORTED;
  int b0 = 0;
  while (b0 < B) {
    const int rest = B - b0;
    int Bk = rest >= 4 ? 4 : (rest >= 2 ? 2 : 1);
    auto maxuw = [](int b) { return b == 1 ? 12 : (b == 2 ? 8 : 4); };
    int W = 0, UW = 0, rpg = 0, grid = 0, threads = 0;
    size_t lds = 0;
    for (;;) {
      W = (U + maxuw(Bk) - 1) / maxuw(Bk);
      UW = (U + W - 1) / W;
      const int V = 8 / W;
      threads = 64 * W * V;
      const long target_wgs = max(1L, (long)cus * env_int("QW_GEMV_WG_PER_CU", 1));
      rpg = env_int("QW_GEMV_ROWS_PER_WG", 0);
      if (rpg <= 0) rpg = (int)max(1L, ((long)w->N + target_wgs - 1) / target_wgs);
      grid = (w->N + rpg - 1) / rpg;
      lds = 256 * 8 + (size_t)Bk * K * 2 + (W > 1 ? 4 * (size_t)rpg * W * Bk : 0);
      if (W <= 8 && lds <= 160 * 1024 && (Bk * KD + threads - 1) / threads <= kXLoads) break;
      if (Bk == 1) return QW_ERR_UNSUPPORTED;
      Bk >>= 1;
    }
    ArgsNf4 a{};
    a.codes = reinterpret_cast<const uint32_t *>(w->codes);
    a.absmax = reinterpret_cast<const float *>(w->scales);
    a.x = reinterpret_cast<const uint16_t *>(x) + (size_t)b0 * K;
    a.y = reinterpret_cast<char *>(y) + (size_t)b0 * w->N * esz;
    a.N = w->N;
    a.K = K;
    a.rows_per_wg = rpg;
    a.W = W;
    a.f32out = f32 ? 1 : 0;
    a.L = sp;
    switch (Bk) {
      case 1: st = launch_b<1>(a, UW, grid, threads, lds, as_stream(stream)); break;
      case 2: st = launch_b<2>(a, UW, grid, threads, lds, as_stream(stream)); break;
      default: st = launch_b<4>(a, UW, grid, threads, lds, as_stream(stream)); break;
    }
    if (st != QW_OK) return st;
    b0 += Bk;
  }
  return QW_OK;
}
