// Decode GEMV against the v3.2 INT4 format of "On-The-Fly Weight Synthesizer
// (OTF-LLM Engine v4.0)" ("Comparative Analysis: INT4 (v3.2) vs INT2
// Non-Uniform (v4.0)" and the "Method Comparison Table": two 4-bit codes per
// byte on a uniform symmetric grid with zero-point 0, a static channel
// permutation, the top 1% channels in fp16):
//
//   y[b][n] = sum_g s[n][g] * sum_{j in g} x_p[b][j] (u[n][j] - 8)
//           + sum_{o < n_out} x_p[b][o] W_O[n][o]
//
// with x_p the activations in permuted channel order (the anchor positions
// hold u = 8, the zero level, so they add nothing to the first sum).
//
// qgemv_int4 runs the matrix-core GEMV's INT4 branch (kernel_int4) wherever
// K is a multiple of 512 and a batch slice fits it; the vector-ALU kernel of
// this file takes the other shapes (and the test hook QW_TUNE_INT4_PATH = 1).
//
// Work split (as the NF4 GEMV): a workgroup owns a block of rows; workers of
// W waves walk sub-ranges of them and split K. Lane l of wave w owns the
// groups h = (j*W + w)*64 + l (32 codes = 16 bytes, so every code load of a
// wave reads 1 KB contiguous, plus the group's fp16 scale) and the anchor
// pairs (t*W + w)*64 + l, and keeps their x in registers (copied once per
// workgroup through LDS). Rows stream through a ring of 3 row slots per
// wave; every refill is unconditional (rows past the worker's range read
// through zero-size descriptors) except in the last round, which drains.
//
// Decode without a table: two nibbles of a code word masked into the
// mantissas of the fp16 pair 0x6400|u (= 1024 + u), minus 1032 in both
// halves with one packed fp16 add, are the exact pair (u_i - 8, u_{i+4} - 8)
// (integers up to 2048 are exact in fp16); one v_dot2_f32_f16 multiplies it
// with the pair (x_i, x_{i+4}): exact products, fp32 accumulation. Per 8
// weights: 3 shifts, 4 and-or, 4 packed adds and 4 dot2 per batch row.
#include "qw_internal.h"

namespace qw {
namespace gemv2m {
qw_status launch_int4(const qw_weight &w, const uint16_t *x, int B, void *y, bool f32, int cus,
                      hipStream_t s);
}  // namespace gemv2m

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct ArgsInt4 {
  const uint32_t *codes;   // [N][K/8]
  const uint16_t *scales;  // [N][K/32] fp16
  const uint32_t *wo;      // [N][n_out_pad/2] fp16 pairs
  const uint16_t *x;       // [B][K] fp16, permuted channel order
  void *y;                 // [B][N]
  int N, K, n_out_pad, rows_per_wg, W, f32out;
};

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kAnchorSlots = 2;  // anchor pairs per lane and row: n_out_pad <= 256 W
constexpr int kXLoads = 16;      // 16-byte x loads per thread while staging x
constexpr int kRing = 3;
constexpr uint32_t kOob = 0x7FFFFFF0u;

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

// (1024 + u0, 1024 + u1) -> (u0 - 8, u1 - 8), exact
__device__ inline uint32_t minus1032(uint32_t t) {
  const h2 r = __builtin_bit_cast(h2, t) + h2{(_Float16)-1032.0f, (_Float16)-1032.0f};
  return __builtin_bit_cast(uint32_t, r);
}

template <int CTRL, int ROW_MASK>
__device__ inline float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                CTRL, ROW_MASK, 0xF, false));
}

__device__ inline float wave_sum_to_lane63(float v) {
  v += dpp_f<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x124, 0xF>(v);  // row_ror:4
  v += dpp_f<0x128, 0xF>(v);  // row_ror:8
  v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_f<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// LDS: x pairs uint32 [B][K/2] | parts float [rows_per_wg][W][B] (W > 1)
template <int B, int UW, bool ANCH>
__global__ __launch_bounds__(kThreads) void gemv_int4_kernel(ArgsInt4 a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  uint32_t *xl = lds;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = a.W;
  const int V = kWaves / W;
  const int w = wave % W;
  const int K = a.K;
  const int NG = K >> 5;  // groups per row
  const int KP = K >> 1;  // x pairs per row
  const int KA = a.n_out_pad >> 1;
  float *parts = reinterpret_cast<float *>(xl + B * KP);
  const int g0 = (int)blockIdx.x * a.rows_per_wg;
  const int g1 = min(a.N, g0 + a.rows_per_wg);
  // rows split over the V workers as evenly as possible (extra rows to the
  // lowest workers)
  const int nrow = max(0, g1 - g0), vw = wave / W;
  const int rbase = nrow / V, rextra = nrow % V;
  const int r0 = g0 + vw * rbase + min(vw, rextra);
  const int r1 = r0 + rbase + (vw < rextra ? 1 : 0);

  uint32_t vc[UW], vs[UW], va[kAnchorSlots];
#pragma unroll
  for (int j = 0; j < UW; ++j) {
    const int h = (j * W + w) * 64 + lane;
    vc[j] = h < NG ? (uint32_t)h * 16 : kOob;
    vs[j] = h < NG ? (uint32_t)h * 2 : kOob;
  }
#pragma unroll
  for (int t = 0; t < kAnchorSlots; ++t) {
    const int ad = (t * W + w) * 64 + lane;
    va[t] = ad < KA ? (uint32_t)ad * 4 : kOob;
  }
  struct Slot {
    u32x4 c[UW];
    uint32_t s[UW];
    uint32_t o[kAnchorSlots];
  };
  Slot ring[kRing];
  const uint32_t row_cb = (uint32_t)K / 2, row_sb = (uint32_t)NG * 2, row_ob = (uint32_t)a.n_out_pad * 2;
  const uint32_t n_cb = (uint32_t)((size_t)a.N * row_cb), n_sb = (uint32_t)((size_t)a.N * row_sb);
  const uint32_t n_ob = (uint32_t)((size_t)a.N * row_ob);
  auto issue = [&](Slot &d, int rr) __attribute__((always_inline)) {
    const bool ok = rr < r1;
    const auto rc = make_rsrc(a.codes, ok ? n_cb : 0u);
    const auto rs = make_rsrc(a.scales, ok ? n_sb : 0u);
    const uint32_t sc = ok ? (uint32_t)rr * row_cb : 0u, ss = ok ? (uint32_t)rr * row_sb : 0u;
#pragma unroll
    for (int j = 0; j < UW; ++j) {
      d.c[j] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)vc[j], (int)sc, 0);
      d.s[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)vs[j], (int)ss, 0);
    }
    if (ANCH) {
      const auto ro = make_rsrc(a.wo, ok ? n_ob : 0u);
      const uint32_t so = ok ? (uint32_t)rr * row_ob : 0u;
#pragma unroll
      for (int t = 0; t < kAnchorSlots; ++t) d.o[t] = __builtin_amdgcn_raw_buffer_load_b32(ro, (int)va[t], (int)so, 0);
    }
  };

  // this group's copy of x: 16-byte loads issued ahead of the weight
  // prefetch, so the LDS stores below wait only for them
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
  for (int i = 0; i < kRing; ++i) issue(ring[i], r0 + i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < kXLoads; ++q) {
    const int i = q * kThreads + (int)threadIdx.x;
    if (q < nx && i < B * (K >> 3)) reinterpret_cast<u32x4 *>(xl)[i] = xv[q];
  }
  // LDS-only barrier: a full __syncthreads would also drain the prefetch
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  // x of this lane's groups as the pairs (x_{8d+i}, x_{8d+i+4}) that match
  // the decoded code pairs, and of its anchor pairs as given
  uint32_t xr[UW][B][16];
#pragma unroll
  for (int j = 0; j < UW; ++j) {
    const int h = (j * W + w) * 64 + lane;
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        u32x4 p = {0u, 0u, 0u, 0u};
        if (h < NG) p = reinterpret_cast<const u32x4 *>(xl + b * KP + h * 16)[d];
        // scalars first (a bit cast of a vector element can read element 0)
        const uint32_t p0 = p[0], p1 = p[1], p2 = p[2], p3 = p[3];
        xr[j][b][4 * d + 0] = __builtin_amdgcn_perm(p2, p0, 0x05040100u);
        xr[j][b][4 * d + 1] = __builtin_amdgcn_perm(p2, p0, 0x07060302u);
        xr[j][b][4 * d + 2] = __builtin_amdgcn_perm(p3, p1, 0x05040100u);
        xr[j][b][4 * d + 3] = __builtin_amdgcn_perm(p3, p1, 0x07060302u);
      }
  }
  uint32_t xa[kAnchorSlots][B];
#pragma unroll
  for (int t = 0; t < kAnchorSlots; ++t) {
    const int ad = (t * W + w) * 64 + lane;
#pragma unroll
    for (int b = 0; b < B; ++b) xa[t][b] = (ANCH && ad < KA) ? xl[b * KP + ad] : 0u;
  }

  auto compute = [&](const Slot &sl, int rr) __attribute__((always_inline)) {
    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;
#pragma unroll
    for (int j = 0; j < UW; ++j) {
      float t[B][2];
#pragma unroll
      for (int b = 0; b < B; ++b) t[b][0] = t[b][1] = 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t cw = sl.c[j][d];
        uint32_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = minus1032(((cw >> (4 * i)) & 0x000F000Fu) | 0x64006400u);
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) t[b][i & 1] = dot2(xr[j][b][4 * d + i], q[i], t[b][i & 1]);
      }
      const float s = f16_bits_to_f32((uint16_t)sl.s[j]);
#pragma unroll
      for (int b = 0; b < B; ++b) acc[b] = __builtin_fmaf(s, t[b][0] + t[b][1], acc[b]);
    }
    if (ANCH) {
#pragma unroll
      for (int t = 0; t < kAnchorSlots; ++t)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = dot2(xa[t][b], sl.o[t], acc[b]);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float v = wave_sum_to_lane63(acc[b]);
      if (lane == 63 && rr < r1) {
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

  // rounds of kRing rows; all but the last refill each slot after using it
  const int n_rows = r1 - r0;
  const int n_rounds = (n_rows + kRing - 1) / kRing;
  int r = r0;
  for (int rd = 1; rd < n_rounds; ++rd) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      compute(ring[i], r + i);
      issue(ring[i], r + i + kRing);
    }
    r += kRing;
  }
#pragma unroll
  for (int i = 0; i < kRing; ++i)
    if (r + i < r1) compute(ring[i], r + i);

  if (W > 1) {
    __syncthreads();
    for (int t = threadIdx.x; t < nrow * B; t += kThreads) {
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

// groups per lane the x registers allow at batch B (no spills at 2 waves
// per SIMD)
constexpr int max_uw(int B) { return B == 1 ? 6 : (B == 2 ? 3 : (B <= 4 ? 2 : 1)); }

template <int B, int UW, bool ANCH>
qw_status launch_k(const ArgsInt4 &a, int grid, size_t lds, hipStream_t s) {
  auto fn = gemv_int4_kernel<B, UW, ANCH>;
  if (lds > 64 * 1024)
    QW_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)lds));
  QW_HIP_TRY(launch(fn, grid, kThreads, lds, s, a));
  return QW_OK;
}

// UW is clamped to what B allows (the host never asks for more)
template <int B, bool ANCH>
qw_status launch_uw(const ArgsInt4 &a, int UW, int grid, size_t lds, hipStream_t s) {
  constexpr int M = max_uw(B);
  switch (UW) {
    case 1: return launch_k<B, 1, ANCH>(a, grid, lds, s);
    case 2: return launch_k<B, (M < 2 ? M : 2), ANCH>(a, grid, lds, s);
    case 3: return launch_k<B, (M < 3 ? M : 3), ANCH>(a, grid, lds, s);
    case 4: return launch_k<B, (M < 4 ? M : 4), ANCH>(a, grid, lds, s);
    case 5: return launch_k<B, (M < 5 ? M : 5), ANCH>(a, grid, lds, s);
    default: return launch_k<B, M, ANCH>(a, grid, lds, s);
  }
}

template <bool ANCH>
qw_status launch_b(const ArgsInt4 &a, int B, int UW, int grid, size_t lds, hipStream_t s) {
  switch (B) {
    case 1: return launch_uw<1, ANCH>(a, UW, grid, lds, s);
    case 2: return launch_uw<2, ANCH>(a, UW, grid, lds, s);
    case 3: return launch_uw<3, ANCH>(a, UW, grid, lds, s);
    case 4: return launch_uw<4, ANCH>(a, UW, grid, lds, s);
    case 5: return launch_uw<5, ANCH>(a, UW, grid, lds, s);
    case 6: return launch_uw<6, ANCH>(a, UW, grid, lds, s);
    case 7: return launch_uw<7, ANCH>(a, UW, grid, lds, s);
    default: return launch_uw<8, ANCH>(a, UW, grid, lds, s);
  }
}

}  // namespace
}  // namespace qw

extern "C" qw_status qgemv_int4(const qw_weight *w, const void *x, int B, void *y, qw_dtype y_dtype,
                                void *stream) {
  using namespace qw;
  CallScope scope;
  qw_status st = check_weight_view(w, QW_FMT_INT4_G32, 0);
  if (st != QW_OK) return st;
  if (!x || !y || B < 1 || B > 8) return QW_ERR_INVALID_ARG;
  if (y_dtype != QW_DT_F16 && y_dtype != QW_DT_F32) return QW_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y)) return QW_ERR_ALIGNMENT;
  int cus = 0;
  st = current_device(&cus);
  if (st != QW_OK) return st;
  const int K = w->K, N = w->N;
  if ((size_t)N * (K / 2) >= (1ull << 31)) return QW_ERR_UNSUPPORTED;
  const bool f32 = y_dtype == QW_DT_F32;
  // the matrix-core kernel where it takes the shape, else this file's kernel
  if (tune(QW_TUNE_INT4_PATH) != 1) {
    st = gemv2m::launch_int4(*w, reinterpret_cast<const uint16_t *>(x), B, y, f32, cus, as_stream(stream));
    if (st != QW_ERR_UNSUPPORTED) return st;
  }
  const int NG = K / 32;
  const int n_pad = w->n_out > 0 ? w->n_out_pad : 0;
  const size_t esz = f32 ? 4 : 2;
  const int rpg = (int)max(1L, ((long)N + cus - 1) / cus);  // one workgroup per CU
  const int grid = (N + rpg - 1) / rpg;
  int b0 = 0;
  while (b0 < B) {
    // the widest batch slice whose x fits LDS and the registers
    int Bk = B - b0, W = 1, UW = 1;
    size_t lds = 0;
    for (;; --Bk) {
      if (Bk == 0) return QW_ERR_UNSUPPORTED;
      W = 1;
      while (W < kWaves && W * 64 * max_uw(Bk) < NG) W *= 2;
      UW = (NG + 64 * W - 1) / (64 * W);
      lds = (size_t)Bk * K * 2 + (W > 1 ? (size_t)4 * rpg * W * Bk : 0);
      const bool fits = UW <= max_uw(Bk) && lds <= 160 * 1024 &&
                        (Bk * (K / 8) + kThreads - 1) / kThreads <= kXLoads && n_pad <= 128 * kAnchorSlots * W;
      if (fits) break;
    }
    ArgsInt4 a{};
    a.codes = reinterpret_cast<const uint32_t *>(w->codes);
    a.scales = reinterpret_cast<const uint16_t *>(w->scales);
    a.wo = reinterpret_cast<const uint32_t *>(w->out_w);
    a.x = reinterpret_cast<const uint16_t *>(x) + (size_t)b0 * K;
    a.y = reinterpret_cast<char *>(y) + (size_t)b0 * N * esz;
    a.N = N;
    a.K = K;
    a.n_out_pad = n_pad;
    a.rows_per_wg = rpg;
    a.W = W;
    a.f32out = f32 ? 1 : 0;
    st = n_pad > 0 ? launch_b<true>(a, Bk, UW, grid, lds, as_stream(stream))
                   : launch_b<false>(a, Bk, UW, grid, lds, as_stream(stream));
    if (st != QW_OK) return st;
    b0 += Bk;
  }
  return QW_OK;
}
