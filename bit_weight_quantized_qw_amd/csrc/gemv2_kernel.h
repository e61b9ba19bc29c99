// Decode GEMV against the adaptive non-uniform 2-bit code
// ("On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)": codebook of
// section 2, per-group scale/offset of section 3, fp16 anchors of section 4,
// four codes per byte and in-register decode from "Key v4.0 Innovations").
//
//   y[b][n] = sum_g S_g * sum_{k in g} x_R[b][k] C[q_k] + Z_g * X_g[b]
//           + sum_o x[b][idx_o] W_O[n][o]
//
// Work split. A workgroup owns a contiguous block of rows. Its waves form
// workers of W waves; a worker walks a contiguous sub-range of rows and its
// W waves split K. Lane l of wave w owns the 16-code dwords
// u = (j*W + w)*64 + l of every row (j < UW) and the anchor dwords
// a = (t*W + w)*64 + l (t < UA), so every load of a wave is contiguous and
// the lane's slice of x stays in registers for all its rows.
//
// x is prepared once per workgroup: the whole group loads x, zeroes the
// anchor channels and writes, per 16-element unit, the pre-scaled pairs, the
// unit's sum and its scale coefficients to LDS; each lane then reads its
// slice from LDS. Weights are fetched with buffer loads (row offset in an SGPR, fixed
// lane offset, hardware range check returning 0 for tail lanes), and the
// first 2*RU rows are requested before the x preparation starts; rows then
// stream through the two register buffers of RU rows each.
//
// Decode without a lookup table: with q = l + 2h (low/high bit of the code),
// C[q] = C0 + d1*l + d2*h exactly (d1 = C1-C0, d2 = C2-C0; C3-C0 = d1+d2 for
// the symmetric codebook), so per 16 weights
//   sum x C[q] = C0*X + d1*sum x q + (d2 - 2 d1)*sum x h.
// A 2-bit field masked in place inside the 32-bit code word is a subnormal
// fp16 (value q * 2^(2f-24) for the f-th field of each half-word), so one
// v_and_b32 turns two fields -- element f and element f+8 of the dword --
// into an fp16 pair that v_dot2_f32_f16 multiplies exactly with a pair of x
// values. x is pre-scaled by 2^(s-2f) per field so every product lands on
// the common scale 2^(s-24); fields 5..7 of each half are first shifted down
// by 10 bits. s <= 8 is chosen per 16-element unit from its max |x| so
// nothing overflows fp16; for |x| < 256 every product is exact and only the
// fp32 accumulation rounds.
#pragma once

#include "qw_internal.h"

namespace qw {
namespace gemv2 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kMaxMats = 4;
constexpr int kMaxWaves = 8;

struct Mat {
  const uint32_t *codes;  // [N][K/16]
  const uint32_t *sz;     // [N][K/32] : fp16 S | fp16 Z << 16
  const uint32_t *mask;   // [K/32] anchor-channel bits, null if no anchors
  const int32_t *idx;     // [n_out]
  const uint32_t *wo;     // [N][n_out_pad/2] fp16 pairs
  void *y;                // [B][N]
  int N, n_out, n_out_pad;
  int wg_begin;           // first workgroup of this matrix
  int rows_per_wg;
};

struct Args {
  Mat m[kMaxMats];
  int count;
  const uint16_t *x;  // [B][K] (this batch slice)
  int K;
  int W;              // waves per worker
  int f32out;
};

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

template <int CTRL, int ROW_MASK>
__device__ inline uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

template <int CTRL, int ROW_MASK>
__device__ inline float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes; the total lands in lane 63.
__device__ inline float wave_sum_to_lane63(float v) {
  v += dpp_f<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x124, 0xF>(v);  // row_ror:4
  v += dpp_f<0x128, 0xF>(v);  // row_ror:8
  v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_f<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// Max over the 64 lanes (unsigned); lands in lane 63.
__device__ inline uint32_t wave_max_to_lane63(uint32_t v) {
  v = max(v, dpp_u<0xB1, 0xF>(v));
  v = max(v, dpp_u<0x4E, 0xF>(v));
  v = max(v, dpp_u<0x124, 0xF>(v));
  v = max(v, dpp_u<0x128, 0xF>(v));
  v = max(v, dpp_u<0x142, 0xA>(v));
  v = max(v, dpp_u<0x143, 0xC>(v));
  return v;
}

// fp16 bits of 2^k (-14 <= k <= 15) in both halves.
__device__ inline uint32_t pow2_pair(int k) {
  const uint32_t h = (uint32_t)(k + 15) << 10;
  return h | (h << 16);
}

__device__ inline uint32_t pk_mul(uint32_t a, uint32_t b) {
  const h2 r = __builtin_bit_cast(h2, a) * __builtin_bit_cast(h2, b);
  return __builtin_bit_cast(uint32_t, r);
}

// Raw buffer over [p, p + bytes); loads beyond `bytes` return 0.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uint32_t bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline u32x4 bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

constexpr uint32_t kOob = 0x7FFFFFF0u;  // lane offset that is always out of range

// Rows per register buffer. A wave can track at most 63 outstanding vector
// memory instructions; the two buffers (2 * RU rows of 2*UW + UA loads) plus
// the x loads are kept within that so the x preparation can wait for x alone.
template <int B, int UW, int UA>
constexpr int rows_per_buffer() {
  constexpr int per_row = 2 * UW + UA;
  constexpr int budget = 60 - (1 + 2 * B + 2 * UA);
  constexpr int r = budget / (2 * per_row);
  return r < 1 ? 1 : (r > 8 ? 8 : r);
}

// x units (16 elements) each thread prepares; K/16 <= this * threads.
template <int B>
__host__ __device__ constexpr int x_units_per_thread() { return B == 1 ? 4 : (B == 2 ? 2 : 1); }

// LDS layout (dwords):
//   xp    uint32 [B][KD][8]  pre-scaled pairs per code dword
//   xs    float4 [B][KD]     per unit: sum of its 16 x, C0 * sum, and the
//                            coefficients of sum x q and sum x h for its scale
//   xraw  fp16   [B][K]      x as given (the anchors read it)
//   parts float  [rows_per_wg][W][B] when W > 1
template <int B, int UW, int UA>
__global__ __launch_bounds__(512) void kernel(Args a) {
  constexpr int RU = rows_per_buffer<B, UW, UA>();
  constexpr int UAk = UA > 0 ? UA : 1;
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const int NW = blockDim.x >> 6;
  const int W = a.W;
  const int V = NW / W;
  const int w = wave % W;
  const int T = blockDim.x;

  Mat M = a.m[0];
#pragma unroll
  for (int i = 1; i < kMaxMats; ++i)
    if (i < a.count && (int)blockIdx.x >= a.m[i].wg_begin) M = a.m[i];
  const int K = a.K;
  const int KD = K >> 4;
  const int KS = K >> 5;
  const int KA = M.n_out_pad >> 1;
  const int g0 = ((int)blockIdx.x - M.wg_begin) * M.rows_per_wg;
  const int g1 = min(M.N, g0 + M.rows_per_wg);
  const int rpw = (M.rows_per_wg + V - 1) / V;  // rows per worker
  const int r0 = min(g1, g0 + (wave / W) * rpw);
  const int r1 = min(g1, r0 + rpw);

  // ---- issue the first rows' weight loads ----
  const auto rc = make_rsrc(M.codes, (uint32_t)((size_t)M.N * KD * 4));
  const auto rs = make_rsrc(M.sz, (uint32_t)((size_t)M.N * KS * 4));
  const auto ro = make_rsrc(M.wo, (uint32_t)((size_t)M.N * KA * 4));
  uint32_t vc[UW], vs[UW], va[UAk];
#pragma unroll
  for (int j = 0; j < UW; ++j) {
    const int u = (j * W + w) * 64 + lane;
    vc[j] = u < KD ? (uint32_t)u * 4 : kOob;
    vs[j] = u < KD ? (uint32_t)(u >> 1) * 4 : kOob;
  }
#pragma unroll
  for (int t = 0; t < UA; ++t) {
    const int ad = (t * W + w) * 64 + lane;
    va[t] = ad < KA ? (uint32_t)ad * 4 : kOob;
  }
  uint32_t cA[RU][UW], sA[RU][UW], oA[RU][UAk];
  uint32_t cB[RU][UW], sB[RU][UW], oB[RU][UAk];
  // Rows past the worker's range read through zero-length descriptors
  // (selected with scalar ops), so every load is unconditional and returns 0.
  const auto rz = make_rsrc(M.codes, 0u);
  auto load = [&](uint32_t (&c)[RU][UW], uint32_t (&s)[RU][UW], uint32_t (&o)[RU][UAk], int rb) {
#pragma unroll
    for (int i = 0; i < RU; ++i) {
      const int rr = rb + i;
      const bool ok = rr < r1;
      const auto rcr = ok ? rc : rz, rsr = ok ? rs : rz, ror = ok ? ro : rz;
      const uint32_t so_c = ok ? (uint32_t)rr * KD * 4 : 0u, so_s = ok ? (uint32_t)rr * KS * 4 : 0u;
      const uint32_t so_o = ok ? (uint32_t)rr * KA * 4 : 0u;
#pragma unroll
      for (int j = 0; j < UW; ++j) {
        c[i][j] = bload(rcr, vc[j], so_c);
        s[i][j] = bload(rsr, vs[j], so_s);
      }
#pragma unroll
      for (int t = 0; t < UA; ++t) o[i][t] = bload(ror, va[t], so_o);
    }
  };
  // ---- prepare x once per workgroup ----
  uint32_t *xp_l = lds;                                            // [B][KD][8]
  float4 *xs_l = reinterpret_cast<float4 *>(lds + B * KD * 8);    // [B][KD]
  uint16_t *xraw_l = reinterpret_cast<uint16_t *>(lds + B * KD * 12);  // [B][K]
  float *parts = reinterpret_cast<float *>(lds + B * KD * 12 + B * (K >> 1));
  constexpr int XU = x_units_per_thread<B>();
  // (1) x units of this thread and their anchor-channel bits, and the anchor
  //     channel numbers of this lane's anchor dwords: requested before the
  //     weights so that waiting for them never waits for the weights
  const auto rx = make_rsrc(a.x, (uint32_t)(B * K * 2));
  const auto rmk = make_rsrc(M.mask, M.mask ? (uint32_t)(KS * 4) : 0u);
  const auto rid = make_rsrc(M.idx, (uint32_t)(M.n_out * 4));
  u32x4 xv[XU][B][2];
  uint32_t omk[XU];
#pragma unroll
  for (int q = 0; q < XU; ++q) {
    const int u = threadIdx.x + q * T;
    const bool ok = u < KD;
    omk[q] = 0;
#pragma unroll
    for (int b = 0; b < B; ++b) xv[q][b][0] = xv[q][b][1] = u32x4{0, 0, 0, 0};
    if (q * T < KD) {  // uniform: skip units no thread of the group has
      omk[q] = bload(rmk, ok ? (uint32_t)(u >> 1) * 4 : kOob, 0);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const uint32_t off = ok ? (uint32_t)(b * K + u * 16) * 2 : kOob;
        xv[q][b][0] = bload4(rx, off, 0);
        xv[q][b][1] = bload4(rx, off + 16, 0);
      }
    }
  }
  int ci0[UAk], ci1[UAk];
#pragma unroll
  for (int t = 0; t < UA; ++t) {
    const int ad = (t * W + w) * 64 + lane;
    const int o0 = 2 * ad;
    const bool v0 = ad < KA && o0 < M.n_out, v1 = ad < KA && o0 + 1 < M.n_out;
    ci0[t] = (int)bload(rid, v0 ? (uint32_t)o0 * 4 : kOob, 0);
    ci1[t] = (int)bload(rid, v1 ? (uint32_t)(o0 + 1) * 4 : kOob, 0);
    if (!v0) ci0[t] = -1;
    if (!v1) ci1[t] = -1;
  }
  // (2) the first 2*RU rows of weights, issued after (not interleaved with)
  //     the loads above
  __builtin_amdgcn_sched_barrier(0);
  load(cA, sA, oA, r0);
  load(cB, sB, oB, r0 + RU);
  __builtin_amdgcn_sched_barrier(0);
  // (3) per 16-element unit: raw copy (for the anchors), anchor channels
  //     zeroed, scale s from the unit's own max |x|, pre-scaled pairs, sum
  //     and the two scale coefficients, all into LDS
  {
    const float C0 = -1.52f, d1 = -0.45f - C0, d2 = 0.45f - C0;
#pragma unroll
    for (int q = 0; q < XU; ++q) {
      const int u = threadIdx.x + q * T;
      if (u < KD) {
        const uint32_t om = (omk[q] >> ((u & 1) * 16)) & 0xFFFFu;
#pragma unroll
        for (int b = 0; b < B; ++b) {
          u32x4 *raw = reinterpret_cast<u32x4 *>(xraw_l + (size_t)b * K + (size_t)u * 16);
          raw[0] = xv[q][b][0];
          raw[1] = xv[q][b][1];
          uint32_t d[8] = {xv[q][b][0].x, xv[q][b][0].y, xv[q][b][0].z, xv[q][b][0].w,
                           xv[q][b][1].x, xv[q][b][1].y, xv[q][b][1].z, xv[q][b][1].w};
          float xsum = 0.0f;
          uint32_t mx = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t keep = (((om >> (2 * i)) & 1u) ? 0u : 0xFFFFu) |
                                  (((om >> (2 * i + 1)) & 1u) ? 0u : 0xFFFF0000u);
            d[i] &= keep;
            xsum = dot2(d[i], 0x3C003C00u, xsum);
            mx = max(mx, max(d[i] & 0x7FFFu, (d[i] >> 16) & 0x7FFFu));
          }
          const int e5 = (int)(mx >> 10);
          const int sc = (e5 == 0) ? 8 : min(8, 30 - e5);
          uint32_t pr[8];
#pragma unroll
          for (int f = 0; f < 8; ++f) {
            const uint32_t lo = d[f >> 1], hi = d[4 + (f >> 1)];
            const uint32_t pair = __builtin_amdgcn_perm(hi, lo, (f & 1) ? 0x07060302u : 0x05040100u);
            const int fp = (f < 5) ? f : f - 5;
            pr[f] = pk_mul(pair, pow2_pair(sc - 2 * fp));
          }
          uint4 *dst = reinterpret_cast<uint4 *>(xp_l + ((size_t)b * KD + u) * 8);
          dst[0] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
          dst[1] = make_uint4(pr[4], pr[5], pr[6], pr[7]);
          xs_l[b * KD + u] = make_float4(xsum, C0 * xsum, d1 * __builtin_ldexpf(1.0f, 24 - sc),
                                         (d2 - 2.0f * d1) * __builtin_ldexpf(1.0f, 23 - sc));
        }
      }
    }
  }
  // (4) LDS-only barrier: the weight loads stay in flight across it
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

  // ---- this lane's slice of the prepared x ----
  uint32_t xp[UW][B][8];
  float Xh[UW][B], CX[UW][B], e1[UW][B], e2[UW][B];
#pragma unroll
  for (int j = 0; j < UW; ++j) {
    const int u = (j * W + w) * 64 + lane;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (u < KD) {
        const uint4 *src = reinterpret_cast<const uint4 *>(xp_l + ((size_t)b * KD + u) * 8);
        const uint4 p0 = src[0], p1 = src[1];
        xp[j][b][0] = p0.x; xp[j][b][1] = p0.y; xp[j][b][2] = p0.z; xp[j][b][3] = p0.w;
        xp[j][b][4] = p1.x; xp[j][b][5] = p1.y; xp[j][b][6] = p1.z; xp[j][b][7] = p1.w;
        const float4 xs = xs_l[b * KD + u];
        Xh[j][b] = xs.x;
        CX[j][b] = xs.y;
        e1[j][b] = xs.z;
        e2[j][b] = xs.w;
      } else {
#pragma unroll
        for (int f = 0; f < 8; ++f) xp[j][b][f] = 0;
        Xh[j][b] = CX[j][b] = e1[j][b] = e2[j][b] = 0.0f;
      }
    }
  }
  uint32_t xo[UAk][B];
#pragma unroll
  for (int t = 0; t < UA; ++t) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const uint32_t v0 = (ci0[t] >= 0 && ci0[t] < K) ? xraw_l[(size_t)b * K + ci0[t]] : 0u;
      const uint32_t v1 = (ci1[t] >= 0 && ci1[t] < K) ? xraw_l[(size_t)b * K + ci1[t]] : 0u;
      xo[t][b] = v0 | (v1 << 16);
    }
  }

  auto compute = [&](const uint32_t (&c)[RU][UW], const uint32_t (&s)[RU][UW],
                     const uint32_t (&o)[RU][UAk], int rb) {
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
        const uint32_t c2 = cw >> 10;
        uint32_t mq[8], mh[8];
#pragma unroll
        for (int f = 0; f < 5; ++f) {
          mq[f] = cw & (0x00030003u << (2 * f));
          mh[f] = cw & (0x00020002u << (2 * f));
        }
#pragma unroll
        for (int f = 5; f < 8; ++f) {
          mq[f] = c2 & (0x00030003u << (2 * (f - 5)));
          mh[f] = c2 & (0x00020002u << (2 * (f - 5)));
        }
        const float S = f16_bits_to_f32((uint16_t)(s[i][j] & 0xFFFFu));
        const float Z = f16_bits_to_f32((uint16_t)(s[i][j] >> 16));
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float aq = 0.0f, ah = 0.0f;
#pragma unroll
          for (int f = 0; f < 8; ++f) {
            aq = dot2(xp[j][b][f], mq[f], aq);
            ah = dot2(xp[j][b][f], mh[f], ah);
          }
          float t = __builtin_fmaf(e1[j][b], aq, CX[j][b]);
          t = __builtin_fmaf(e2[j][b], ah, t);
          acc[b] = __builtin_fmaf(S, t, acc[b]);
          acc[b] = __builtin_fmaf(Z, Xh[j][b], acc[b]);
        }
      }
#pragma unroll
      for (int t = 0; t < UA; ++t)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = dot2(xo[t][b], o[i][t], acc[b]);
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const float v = wave_sum_to_lane63(acc[b]);
        if (lane == 63) {
          if (W == 1) {
            const size_t off = (size_t)b * M.N + rr;
            if (a.f32out)
              reinterpret_cast<float *>(M.y)[off] = v;
            else
              reinterpret_cast<_Float16 *>(M.y)[off] = (_Float16)v;
          } else {
            parts[((rr - g0) * W + w) * B + b] = v;
          }
        }
      }
    }
  };

  for (int r = r0; r < r1; r += 2 * RU) {
    compute(cA, sA, oA, r);
    load(cA, sA, oA, r + 2 * RU);
    compute(cB, sB, oB, r + RU);
    load(cB, sB, oB, r + 3 * RU);
  }

  if (W > 1) {
    // partials of every row of this workgroup, indexed by row - g0
    __syncthreads();
    const int nrows = g1 - g0;
    for (int t = threadIdx.x; t < nrows * B; t += blockDim.x) {
      const int rl = t / B, b = t - rl * B;
      float v = 0.0f;
      for (int i = 0; i < W; ++i) v += parts[(rl * W + i) * B + b];
      const size_t off = (size_t)b * M.N + (g0 + rl);
      if (a.f32out)
        reinterpret_cast<float *>(M.y)[off] = v;
      else
        reinterpret_cast<_Float16 *>(M.y)[off] = (_Float16)v;
    }
  }
}

// LDS bytes the kernel needs.
inline size_t lds_bytes(int B, int K, int rows_per_wg, int W) {
  const size_t KD = K / 16;
  size_t n = (size_t)B * KD * 12 + (size_t)B * (K / 2);
  if (W > 1) n += (size_t)rows_per_wg * W * B;
  return n * 4;
}

// Launchers, one translation unit per batch width.
qw_status launch_b1(const Args &a, int UW, int UA, int grid, int threads, size_t lds, hipStream_t s);
qw_status launch_b2(const Args &a, int UW, int UA, int grid, int threads, size_t lds, hipStream_t s);
qw_status launch_b4(const Args &a, int UW, int UA, int grid, int threads, size_t lds, hipStream_t s);

template <int B, int UW, int UA>
qw_status launch_one(const Args &a, int grid, int threads, size_t lds, hipStream_t s) {
  if (lds > 64 * 1024) {
    QW_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(&kernel<B, UW, UA>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  }
  QW_HIP_TRY(launch(kernel<B, UW, UA>, grid, threads, lds, s, a));
  return QW_OK;
}

template <int B, int UW>
qw_status launch_ua(const Args &a, int UA, int grid, int threads, size_t lds, hipStream_t s) {
  if (UA == 0) return launch_one<B, UW, 0>(a, grid, threads, lds, s);
  if (UA <= 2) return launch_one<B, UW, 2>(a, grid, threads, lds, s);
  return launch_one<B, UW, 4>(a, grid, threads, lds, s);
}

}  // namespace gemv2
}  // namespace qw
