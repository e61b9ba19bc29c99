// Decode GEMV against NF4 block-wise codes ("AirQuant" README,
// "Fundamentacao Teorica e Arquitetura" item 2: NormalFloat4 with
// block-wise absmax).
//
//   y[b][n] = sum_blk absmax[n][blk] * sum_{k in blk} x[b][k] L[q_k]
//
// Work split: a workgroup owns a block of rows; workers of W waves walk
// sub-ranges and split K; lane l of wave w owns the half blocks
// h = (j*W + w)*64 + l (32 codes = 16 bytes each, so every code load of a
// wave reads 1 KB contiguous, plus the absmax of block h/2) and keeps those
// x pairs in registers (copied once per workgroup through LDS). Rows stream through a ring of P row slots per wave;
// every refill is unconditional (rows past the end read through a zero-size
// descriptor) except in the last round, which only drains the ring.
//
// Decode: each code byte (two elements) selects an LDS entry holding the
// level pair (L[lo], L[hi]) as fp32, so one ds_read_b64 feeds two fp32 FMAs
// against x (converted to fp32 once): exact x, levels to 2^-24, fp32
// products and accumulation. Random byte indices into one 256-entry table
// would collide in the 32 LDS banks (about 3.5 distinct entries per bank
// pair and access); instead every entry is stored 16 times, replica r in
// bank pair r, at byte offset 256*v + 8*r, and lane l reads replica l % 16.
// The lanes of a 16-lane group then always touch distinct banks, whatever
// the codes. One v_perm builds the address: the code byte goes to byte 1
// and the lane's replica offset to byte 0.
#include <stdlib.h>

#include "qw_internal.h"

namespace qw {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

struct ArgsNf4 {
  const uint32_t *codes;  // [N][K/8]
  const float *absmax;    // [N][K/64]
  const uint16_t *x;      // [B][K]
  void *y;                // [B][N]
  int N, K, rows_per_wg, W, f32out;
  float L[16];             // NF4 levels
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
constexpr int kThreads = 512;

// Replicated level-pair table: entry v (code byte) replica r at byte
// 256*v + 8*r, r < 16; bytes 128..255 of each entry are unused.
constexpr int kPairStride = 256;
constexpr int kReplicas = 16;

__device__ inline float2 pair_at(const char *tab, uint32_t byte_off) {
  return *reinterpret_cast<const float2 *>(tab + byte_off);
}

// LDS: pair table (static, 64 KB) | x uint32 [B][K/2] | parts float [rows_per_wg][W][B]
template <int B, int UW, int P>
__global__ __launch_bounds__(kThreads) void gemv_nf4_kernel(ArgsNf4 a) {
  __shared__ __attribute__((aligned(16))) char pair_tab[256 * kPairStride];
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  uint32_t *xl = lds;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const int W = a.W;
  const int V = (kThreads >> 6) / W;
  const int w = wave % W;
  const int K = a.K;
  const int NB = K >> 6;    // NF4 blocks per row
  const int NH = K >> 5;    // half blocks per row
  const int KP = K >> 1;    // x pairs per row
  float *parts = reinterpret_cast<float *>(xl + B * KP);
  const int g0 = (int)blockIdx.x * a.rows_per_wg;
  const int g1 = min(a.N, g0 + a.rows_per_wg);
  // the group's rows split over its V workers as evenly as possible, the
  // extra rows to the lowest workers: waves v and v + 4 share a SIMD, so no
  // SIMD gets more than one row above another
  const int nrow = max(0, g1 - g0), vw = wave / W;
  const int rbase = nrow / V, rextra = nrow % V;
  const int r0 = g0 + vw * rbase + min(vw, rextra);
  const int r1 = r0 + rbase + (vw < rextra ? 1 : 0);

  const uint32_t row_cb = (uint32_t)K / 2, row_ab = (uint32_t)NB * 4;  // bytes per row
  uint32_t vc[UW], va[UW];
#pragma unroll
  for (int j = 0; j < UW; ++j) {
    const int h = (j * W + w) * 64 + lane;
    vc[j] = h < NH ? (uint32_t)h * 16 : kOob;
    va[j] = h < NH ? (uint32_t)(h >> 1) * 4 : kOob;
  }
  struct Slot {
    u32x4 c[UW];
    uint32_t am[UW];
  };
  Slot ring[P];
  const uint32_t n_cb = (uint32_t)((size_t)a.N * row_cb), n_ab = (uint32_t)((size_t)a.N * row_ab);
  // rows past the worker's range read through zero-size descriptors
  auto issue = [&](Slot &d, int rr) __attribute__((always_inline)) {
    const bool ok = rr < r1;
    const auto rc = make_rsrc(a.codes, ok ? n_cb : 0u);
    const auto ra = make_rsrc(a.absmax, ok ? n_ab : 0u);
    const uint32_t sc = ok ? (uint32_t)rr * row_cb : 0u, sa = ok ? (uint32_t)rr * row_ab : 0u;
#pragma unroll
    for (int j = 0; j < UW; ++j) {
      d.c[j] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)vc[j], (int)sc, 0);
      d.am[j] = bload(ra, va[j], sa);
    }
  };

  // This group's copy of x: 16-byte buffer loads issued ahead of the weight
  // prefetch, so the LDS stores below wait only for them.
  const auto rx = make_rsrc(a.x, (uint32_t)((size_t)B * K * 2));
  const int nx = (B * (K >> 3) + kThreads - 1) / kThreads;  // uniform trip count
  u32x4 xv[kXLoads];
#pragma unroll
  for (int q = 0; q < kXLoads; ++q) {
    if (q < nx) {
      const int i = q * kThreads + (int)threadIdx.x;
      xv[q] = __builtin_amdgcn_raw_buffer_load_b128(rx, i < B * (K >> 3) ? i * 16 : (int)kOob, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < P; ++i) issue(ring[i], r0 + i);
  __builtin_amdgcn_sched_barrier(0);

  // level-pair table: 16-byte chunk c = 512*i + tid holds two replicas of
  // entry v = c / 8 (8 used chunks per entry), i.e. low nibble (tid / 8) % 16
  // and high nibble 4*i + tid / 128, the latter wave-uniform.
  // (levels picked by select chains over scalar kernel arguments: a
  // per-lane indexed read of the argument block would be a memory load
  // queued behind the weight prefetch)
  {
    const int qlo = (int)(threadIdx.x >> 3) & 15;
    float llo = a.L[0];
#pragma unroll
    for (int t = 1; t < 16; ++t) llo = qlo == t ? a.L[t] : llo;
    const int hq = wave >> 1;  // threadIdx.x / 128
    const int sub = (int)(threadIdx.x & 7);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qhi = 4 * i + hq;
      float lhi = a.L[0];
#pragma unroll
      for (int t = 1; t < 16; ++t) lhi = qhi == t ? a.L[t] : lhi;
      const int v = 64 * i + (int)(threadIdx.x >> 3);
      const float4 two = make_float4(llo, lhi, llo, lhi);
      *reinterpret_cast<float4 *>(pair_tab + v * kPairStride + sub * 16) = two;
    }
  }
  const uint32_t lane_rep = 8u * (uint32_t)(lane % kReplicas);
#pragma unroll
  for (int q = 0; q < kXLoads; ++q) {
    const int i = q * kThreads + (int)threadIdx.x;
    if (q < nx && i < B * (K >> 3)) reinterpret_cast<u32x4 *>(xl)[i] = xv[q];
  }
  // LDS-only barrier: a full __syncthreads would also drain the prefetch.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  // x of this lane's half blocks as fp32 (zeros past the row end)
  float xf[UW][B][32];
#pragma unroll
  for (int j = 0; j < UW; ++j) {
    const int h = (j * W + w) * 64 + lane;
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (h < NH) v = reinterpret_cast<const u32x4 *>(xl + b * KP + h * 16)[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // the element goes through a scalar first: a bit cast of a vector
          // element reads element 0 with this compiler
          const uint32_t w32 = v[e];
          const h2 pr = __builtin_bit_cast(h2, w32);
          xf[j][b][8 * q + 2 * e] = (float)pr.x;
          xf[j][b][8 * q + 2 * e + 1] = (float)pr.y;
        }
      }
  }

  // eight independent accumulator chains (code byte position, element
  // parity) so the FMAs of one row do not wait on each other
  auto compute = [&](const Slot &sl, int rr) __attribute__((always_inline)) {
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;
#pragma unroll
    for (int j = 0; j < UW; ++j) {
      float t[B][8];
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int c = 0; c < 8; ++c) t[b][c] = 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t cw = sl.c[j][d];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // v_perm selector: byte 0 <- lane_rep (source byte 4), byte 1 <-
          // code byte k, bytes 2..3 <- zero
          const float2 e = pair_at(pair_tab, __builtin_amdgcn_perm(lane_rep, cw, 0x0C0C0004u | ((uint32_t)k << 8)));
#pragma unroll
          for (int b = 0; b < B; ++b) {
            t[b][2 * k] = __builtin_fmaf(xf[j][b][8 * d + 2 * k], e.x, t[b][2 * k]);
            t[b][2 * k + 1] = __builtin_fmaf(xf[j][b][8 * d + 2 * k + 1], e.y, t[b][2 * k + 1]);
          }
        }
      }
      const float am = __builtin_bit_cast(float, sl.am[j]);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float s4 = ((t[b][0] + t[b][1]) + (t[b][2] + t[b][3])) + ((t[b][4] + t[b][5]) + (t[b][6] + t[b][7]));
        acc[b] = __builtin_fmaf(am, s4, acc[b]);
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
  };

  // rounds of P rows; all but the last refill each slot after using it
  const int n_rows = r1 - r0;
  const int n_rounds = (n_rows + P - 1) / P;
  int r = r0;
  for (int rd = 1; rd < n_rounds; ++rd) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      compute(ring[i], r + i);
      issue(ring[i], r + i + P);
    }
    r += P;
  }
#pragma unroll
  for (int i = 0; i < P; ++i)
    if (r + i < r1) compute(ring[i], r + i);

  if (W > 1) {
    __syncthreads();
    const int nrows = g1 - g0;
    for (int t = threadIdx.x; t < nrows * B; t += kThreads) {
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

template <int B, int UW, int P>
qw_status launch_k(const ArgsNf4 &a, int grid, size_t lds, hipStream_t s) {
  if (lds > 64 * 1024) {
    QW_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(&gemv_nf4_kernel<B, UW, P>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  }
  QW_HIP_TRY(launch(gemv_nf4_kernel<B, UW, P>, grid, kThreads, lds, s, a));
  return QW_OK;
}

template <int B, int UW>
qw_status launch_p(const ArgsNf4 &a, bool deep, int grid, size_t lds, hipStream_t s) {
  return deep ? launch_k<B, UW, 6>(a, grid, lds, s) : launch_k<B, UW, 3>(a, grid, lds, s);
}

qw_status launch_b(const ArgsNf4 &a, int B, int UW, bool deep, int grid, size_t lds, hipStream_t s) {
  if (B == 1) {
    if (UW == 1) return launch_p<1, 1>(a, deep, grid, lds, s);
    if (UW == 2) return launch_p<1, 2>(a, deep, grid, lds, s);
    if (UW == 3) return launch_p<1, 3>(a, deep, grid, lds, s);
    return launch_p<1, 4>(a, deep, grid, lds, s);
  }
  if (B == 2) return UW == 1 ? launch_p<2, 1>(a, deep, grid, lds, s) : launch_p<2, 2>(a, deep, grid, lds, s);
  return launch_p<4, 1>(a, deep, grid, lds, s);
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
  const int NH = K / 32;  // half blocks per row
  if ((size_t)w->N * (K / 2) >= (1ull << 31)) return QW_ERR_UNSUPPORTED;
  int b0 = 0;
  while (b0 < B) {
    const int rest = B - b0;
    int Bk = rest >= 4 ? 4 : (rest >= 2 ? 2 : 1);
    int W = 0, UW = 0, rpg = 0, grid = 0;
    size_t lds = 0;
    for (;;) {
      // half blocks per lane: 4 at batch 1, 2 at batch 2, else 1 (x pairs and
      // the ring stay in registers); W, a power of two, waves split each row
      const int maxuw = Bk == 1 ? 4 : (Bk == 2 ? 2 : 1);
      W = 1;
      while (W < 8 && W * 64 * maxuw < NH) W *= 2;
      UW = (NH + 64 * W - 1) / (64 * W);
      // one workgroup per CU
      const long target_wgs = max(1L, (long)cus);
      rpg = (int)max(1L, ((long)w->N + target_wgs - 1) / target_wgs);
      grid = (w->N + rpg - 1) / rpg;
      lds = (size_t)Bk * K * 2 + (W > 1 ? 4 * (size_t)rpg * W * Bk : 0);
      if (UW <= maxuw && lds + 256 * kPairStride <= 160 * 1024 && (Bk * (K / 8) + kThreads - 1) / kThreads <= kXLoads) break;
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
    const float *lv = nf4_levels_host();
    for (int i = 0; i < 16; ++i) a.L[i] = lv[i];
    // 3 row slots per wave: measured on MI355X, 6 slots (all rows of a wave
    // in flight at once) are slower with weights coming from HBM; the test
    // hook QW_TUNE_NF4_DEEP_RING = 1 selects them (tests check both give the
    // same bits)
    const bool deep = tune(QW_TUNE_NF4_DEEP_RING) == 1;
    st = launch_b(a, Bk, UW, deep, grid, lds, as_stream(stream));
    if (st != QW_OK) return st;
    b0 += Bk;
  }
  return QW_OK;
}
