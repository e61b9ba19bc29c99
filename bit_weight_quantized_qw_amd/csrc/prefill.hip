// Prefill GEMM against block-wise quantized weights:
//   Y[m][n] = sum_k X[m][k] * w_bf16[n][k]
// with w_bf16 = bf16(fp32 fma(S, C[q], Z)) for the 2-bit code
// ("On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)", sections 2-4) or
// bf16(fp32 absmax * L[q]) for NF4 ("AirQuant" README, "Fundamentacao
// Teorica e Arquitetura" item 2). 2-bit anchor columns take bf16(out_w).
//
// Tiling: a 256-thread workgroup computes a 256 (M) x 256 (N) tile of Y; its
// four waves (2 x 2) each own 128 x 128 as 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16 (fp32 accumulators, 256 per lane). K advances 64
// at a time through two LDS buffers: while the waves multiply out of one,
// the next tile -- X copied, the packed W dequantized in registers straight
// to bf16 -- is written to the other and the one after that is in flight
// from memory; one LDS-only barrier per step. LDS rows are padded by 16
// bytes so 16-byte fragment reads of consecutive rows hit distinct banks.
// Workgroups are ordered M-tile fastest, so consecutive workgroups (spread
// over the eight XCDs) share a W tile and each XCD keeps one X slab in L2.
//
// 2-bit dequant: per group of 32 the four possible bf16 values
// v_q = bf16(fma(S, C[q], Z)) are formed once and packed into two dwords;
// a v_perm_b32 whose byte selectors are built from two code fields then
// assembles a bf16 pair, so each weight costs a few integer ops.
#include <stdlib.h>

#include <type_traits>

#include "qw_internal.h"

namespace qw {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDA = BK + 8;  // bf16 elements per LDS row (144 bytes)
constexpr int NT = 256;

struct PrefillArgs {
  const uint16_t *X;       // [M][K] bf16
  const uint32_t *codes;   // 2-bit: [N][K/16]; NF4, INT4: [N][K/8]
  const void *scales;      // 2-bit: uint32 [N][K/32]; NF4: float [N][K/64]; INT4: fp16 [N][K/32]
  const int32_t *idx;      // anchors (2-bit), may be null
  const uint16_t *wo;      // [N][n_out_pad]
  void *Y;                 // [M][N]
  int M, N, K, n_out, n_out_pad;
  int mt_count;            // number of 256-row tiles along M
  int n_begin;             // first output column of this launch's tiles
  int xcd_group;           // row tiles per group of the XCD-aware tile order (0: plain order)
  float nf4[16];           // level of each 4-bit code (NF4 table; u - 8 for INT4)
};

__device__ inline uint32_t f32_to_bf16_bits(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// RNE of both values, one v_cvt_pk_bf16_f32 (converting each half on its own
// costs two conversions plus a shift and an or)
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// 32 codes of one group (two code dwords c0, c1 = elements 0..15, 16..31)
// -> 16 dwords of bf16 pairs in natural element order. The four possible
// values bf16(fma(S, C[q], Z)) are packed in T1:T0 (byte 2q, 2q+1 = value
// q); codes are unpacked to bytes (d_t byte j = code of element 4j + t of a
// 16-code half), one v_perm gathers the two codes of an output pair, a
// shift-add turns them into byte selectors and a second v_perm looks the
// pair up: three integer ops per two weights.
__device__ inline void dequant_group_2bit(uint32_t c0, uint32_t c1, uint32_t szw,
                                          uint32_t out[16]) {
  const float S = f16_bits_to_f32((uint16_t)(szw & 0xFFFFu));
  const float Z = f16_bits_to_f32((uint16_t)(szw >> 16));
  const uint32_t T0 = pack_bf16x2(__builtin_fmaf(S, -1.52f, Z), __builtin_fmaf(S, -0.45f, Z));
  const uint32_t T1 = pack_bf16x2(__builtin_fmaf(S, 0.45f, Z), __builtin_fmaf(S, 1.52f, Z));
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t c = h ? c1 : c0;
    uint32_t d[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) d[t] = (c >> (2 * t)) & 0x03030303u;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      // elements 2p, 2p+1 = 4j + t, 4j + t + 1 with j = p / 2, t = 2 (p % 2)
      const int j = p >> 1, t = 2 * (p & 1);
      const uint32_t gsel = (uint32_t)j * 0x0101u + (uint32_t)(4 + j) * 0x01010000u;
      const uint32_t r = __builtin_amdgcn_perm(d[t + 1], d[t], gsel);  // q0 q0 q1 q1
      out[h * 8 + p] = __builtin_amdgcn_perm(T1, T0, (r << 1) + 0x01000100u);
    }
  }
}

template <int FMT, bool F32OUT>
__global__ __launch_bounds__(NT) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  // two buffers of X [BM][LDA] and W [BN][LDA] tiles, then the NF4 table
  auto As = [&](int buf) { return smem + buf * BM * LDA; };
  auto Bs = [&](int buf) { return smem + 2 * BM * LDA + buf * BN * LDA; };
  float2 *ltab = reinterpret_cast<float2 *>(smem + 2 * (BM + BN) * LDA);  // NF4 [256]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const int b = blockIdx.x;
  const int m_tile = b % a.mt_count;
  const int n_tile = b / a.mt_count;
  const int m0 = m_tile * BM, n0 = n_tile * BN;
  const int K = a.K;
  const int KT = K / BK;

  if (FMT != QW_FMT_2BIT_G32) {  // NF4 levels, or u - 8 for INT4
    for (int v = tid; v < 256; v += NT) ltab[v] = make_float2(a.nf4[v & 15], a.nf4[v >> 4]);
  }

  // ---- global prefetch registers: 8 x 16 bytes of X, one W column ----
  uint4 ra[8];
  uint32_t rb[9];
  const int gn = n0 + tid;  // this thread's W column
  const bool bvalid = gn < a.N;

  auto load_x = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * NT + tid;
      const int row = c >> 3, c16 = c & 7;
      const int gm = m0 + row;
      ra[i] = (gm < a.M)
                  ? *reinterpret_cast<const uint4 *>(a.X + (size_t)gm * K + k0 + c16 * 8)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto load_w = [&](int kt) {
    const int k0 = kt * BK;
    if (FMT == QW_FMT_2BIT_G32) {
      if (bvalid) {
        const u32x4 v = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(a.codes + (size_t)gn * (K / 16) + k0 / 16));
        rb[0] = v.x; rb[1] = v.y; rb[2] = v.z; rb[3] = v.w;
        const uint32_t *sp = reinterpret_cast<const uint32_t *>(a.scales) + (size_t)gn * (K / 32) + k0 / 32;
        rb[4] = __builtin_nontemporal_load(sp);
        rb[5] = __builtin_nontemporal_load(sp + 1);
      } else {
        rb[0] = rb[1] = rb[2] = rb[3] = rb[4] = rb[5] = 0;
      }
    } else {
      if (bvalid) {
        const u32x4 *cp = reinterpret_cast<const u32x4 *>(a.codes + (size_t)gn * (K / 8) + k0 / 8);
        const u32x4 v0 = __builtin_nontemporal_load(cp), v1 = __builtin_nontemporal_load(cp + 1);
        rb[0] = v0.x; rb[1] = v0.y; rb[2] = v0.z; rb[3] = v0.w;
        rb[4] = v1.x; rb[5] = v1.y; rb[6] = v1.z; rb[7] = v1.w;
        rb[8] = __builtin_bit_cast(uint32_t, __builtin_nontemporal_load(
            reinterpret_cast<const float *>(a.scales) + (size_t)gn * (K / 64) + k0 / 64));
      } else {
        for (int i = 0; i < 9; ++i) rb[i] = 0;
      }
    }
  };

  // X pieces of this thread (already in registers) into buffer buf
  auto store_x = [&](int buf) {
    uint16_t *A = As(buf);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * NT + tid;
      const int row = c >> 3, c16 = c & 7;
      *reinterpret_cast<uint4 *>(A + row * LDA + c16 * 8) = ra[i];
    }
  };
  // one 32-element group (half h of the 64 k of tile kt) of this thread's W
  // column, dequantized to bf16, into buffer buf
  auto store_w = [&](int kt, int buf, int h) {
    uint4 *bp = reinterpret_cast<uint4 *>(Bs(buf) + tid * LDA);
    uint32_t out[16];
    if (FMT == QW_FMT_2BIT_G32) {
      dequant_group_2bit(rb[2 * h], rb[2 * h + 1], rb[4 + h], out);
      if (a.n_out > 0 && bvalid) {
        // anchor columns of this group: idx is ascending, find the first >= k_lo
        const int k_lo = kt * BK + 32 * h;
        int lo = 0, hi = a.n_out;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (a.idx[mid] < k_lo) lo = mid + 1; else hi = mid;
        }
        for (int o = lo; o < a.n_out && a.idx[o] < k_lo + 32; ++o) {
          const int e = a.idx[o] - k_lo;
          const float v = f16_bits_to_f32(a.wo[(size_t)gn * a.n_out_pad + o]);
          const uint32_t bb = f32_to_bf16_bits(v);
          // static indexing only, so out[] stays in registers
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            if (q == (e >> 1))
              out[q] = (e & 1) ? ((out[q] & 0xFFFFu) | (bb << 16)) : ((out[q] & 0xFFFF0000u) | bb);
          }
        }
      }
    } else {
      // NF4: one fp32 absmax per 64; INT4: the fp16 scale of group h
      const float am = FMT == QW_FMT_NF4_B64 ? __builtin_bit_cast(float, rb[8])
                                            : f16_bits_to_f32((uint16_t)(rb[8] >> (16 * h)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t c = rb[4 * h + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float2 l = ltab[(c >> (8 * j)) & 0xFFu];
          out[i * 4 + j] = pack_bf16x2(am * l.x, am * l.y);
        }
      }
      // INT4 anchors: permuted positions below n_out take bf16(out_w)
      const int k_lo = kt * BK + 32 * h;
      if (FMT == QW_FMT_INT4_G32 && bvalid && k_lo < a.n_out) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int e = k_lo + 2 * q;
          const uint16_t *wr = a.wo + (size_t)gn * a.n_out_pad;
          const uint32_t b0 = e < a.n_out ? f32_to_bf16_bits(f16_bits_to_f32(wr[e])) : (out[q] & 0xFFFFu);
          const uint32_t b1 = e + 1 < a.n_out ? f32_to_bf16_bits(f16_bits_to_f32(wr[e + 1])) : (out[q] >> 16);
          out[q] = b0 | (b1 << 16);
        }
      }
    }
    bp[4 * h + 0] = make_uint4(out[0], out[1], out[2], out[3]);
    bp[4 * h + 1] = make_uint4(out[4], out[5], out[6], out[7]);
    bp[4 * h + 2] = make_uint4(out[8], out[9], out[10], out[11]);
    bp[4 * h + 3] = make_uint4(out[12], out[13], out[14], out[15]);
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // The products of tile kt out of buffer buf, with tile kt+1 written to the
  // other buffer between the 16-wide k slices (X after slice 0, the two W
  // groups after slices 1 and 2) so the writes and the dequantization run
  // beside the matrix cores; X and W of tile kt+2 are requested as soon as
  // their registers are free.
  auto read_frags = [&](int buf, int kk, bf16x8 (&af)[4], bf16x8 (&bfr)[4]) {
    const uint16_t *A = As(buf), *Bt = Bs(buf);
    const int kof = kk * 16 + (lane >> 5) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + (lane & 31);
      af[i] = *reinterpret_cast<const bf16x8 *>(A + row * LDA + kof);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wn * 128 + j * 32 + (lane & 31);
      bfr[j] = *reinterpret_cast<const bf16x8 *>(Bt + col * LDA + kof);
    }
  };
  // One K step: the products of tile kt out of buffer buf, with tile kt+1
  // written to the other buffer between the 16-wide k slices (X after slice
  // 0, the two W groups after slices 1 and 2) and X, W of tile kt+2
  // requested as soon as their registers are free. The side work is
  // unconditional (on the last step it fills the idle buffer; loads past the
  // end re-read the last tile) so each slice is one basic block, and
  // scheduling groups interleave it with the matrix-core instructions: with
  // one wave per SIMD, in-order issue would otherwise leave the matrix cores
  // idle while it runs.
  auto compute = [&](int kt, int buf) {
    const int kn = min(kt + 2, KT - 1);
    bf16x8 fa[2][4], fb[2][4];  // fragments of the current and the next k slice
    read_frags(buf, 0, fa[0], fb[0]);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) read_frags(buf, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][i], fb[kk & 1][j],
                                                               acc[i][j], 0, 0, 0);
      if (kk == 0) {
        store_x(buf ^ 1);
        load_x(kn);
      } else if (kk == 1) {
        store_w(kt + 1, buf ^ 1, 0);
      } else if (kk == 2) {
        store_w(kt + 1, buf ^ 1, 1);
        load_w(kn);
      }
      // 16 x {1 product, fragment reads, a few vector ops, an LDS write,
      // a memory read}
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      }
    }
  };

  // the NF4 table and tile 0 must be in LDS before the first step
  load_x(0);
  load_w(0);
  __syncthreads();
  store_x(0);
  store_w(0, 0, 0);
  store_w(0, 0, 1);
  if (KT > 1) {
    load_x(1);
    load_w(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  for (int kt = 0; kt < KT; ++kt) {
    compute(kt, kt & 1);
    // LDS-only barrier: the loads of tile kt+2 stay in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }

  // ---- epilogue: lane holds D[8*g + 4*(lane>>5) + r][lane & 31] ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn_ = n0 + wn * 128 + j * 32 + (lane & 31);
      if (gn_ >= a.N) continue;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gm = m0 + wm * 128 + i * 32 + 8 * g + 4 * (lane >> 5) + r;
          if (gm >= a.M) continue;
          const float v = acc[i][j][4 * g + r];
          const size_t o = (size_t)gm * a.N + gn_;
          if (F32OUT)
            reinterpret_cast<float *>(a.Y)[o] = v;
          else
            reinterpret_cast<uint16_t *>(a.Y)[o] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Prefill GEMM without anchor columns: W never goes through LDS.
//
// The four waves of a 256-thread workgroup each own 64 columns (two 32-wide
// sub-tiles) and all 256 rows of the 256 x 256 output tile (4 x ... = 8 x 2
// blocks of v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators per lane). Each
// lane loads the packed codes and scales of its two columns for the next K
// step itself and dequantizes the B fragments (8 consecutive k of one
// column) in registers right before the products that use them, so every
// weight is dequantized once per workgroup and W costs no LDS traffic; only
// X is staged through two LDS buffers. The K loop is unrolled by two so the
// two register sets of W (current step, next step) have static indices.

// 8 consecutive bf16 weights (elements 8h..8h+7 of code dword c, element
// 16u + i in bits 2i..2i+1) from the packed value table T1:T0 of their group.
__device__ inline void dequant8_2bit(uint32_t c, int h, uint32_t T0, uint32_t T1, uint32_t out[4]) {
  const uint32_t cc = c >> (16 * h);
  uint32_t d[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) d[t] = (cc >> (2 * t)) & 0x00030303u;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int j = p >> 1, t = 2 * (p & 1);
    const uint32_t gsel = (uint32_t)j * 0x0101u + (uint32_t)(4 + j) * 0x01010000u;
    const uint32_t r = __builtin_amdgcn_perm(d[t + 1], d[t], gsel);  // q0 q0 q1 q1
    out[p] = __builtin_amdgcn_perm(T1, T0, (r << 1) + 0x01000100u);
  }
}

// Tile of workgroup b for an mt x nt grid of output tiles, XCD-aware.
// Workgroups are dealt to the 8 XCDs round-robin (b % 8), each XCD with its
// own L2. The q-th workgroup of XCD x takes tile t = (start of x's share) + q
// of an order that walks groups of up to 4 row tiles column by column, so
// the workgroups one XCD runs at a time cover a few row tiles times several
// column tiles: each W column tile is fetched once per XCD for the row tiles
// sharing it, instead of once per row tile (row tiles on different XCDs).
// A bijection for every grid size.
__device__ inline void xcd_tile(int b, int mt, int nt, int gmax, int &m_tile, int &n_tile) {
  if (gmax <= 0) {  // plain order: row tile fastest
    m_tile = b % mt;
    n_tile = b / mt;
    return;
  }
  constexpr int kXcds = 8;
  const int total = mt * nt;
  const int xcd = b % kXcds, q = b / kXcds;
  const int per = total / kXcds, rem = total % kXcds;
  const int t = xcd < rem ? xcd * (per + 1) + q : rem * (per + 1) + (xcd - rem) * per + q;
  const int gm = mt < gmax ? mt : gmax;   // row tiles per group
  const int g = t / (gm * nt);            // group of row tiles
  const int rows_g = min(gm, mt - g * gm);  // the last group may be narrower
  const int w = t - g * gm * nt;
  m_tile = g * gm + w % rows_g;
  n_tile = w / rows_g;
}

__device__ inline __amdgpu_buffer_rsrc_t pf_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kPfOob = 0x7FFFFFF0u;  // an offset always past a buffer's end

template <int FMT, bool F32OUT, int NJ, int WM>
__global__ __launch_bounds__(256 * WM) void prefill_w_kernel(PrefillArgs a) {
  constexpr int NTW = 256 * WM;  // threads: WM x 4 waves
  constexpr int IM = 8 / WM;     // 32-row blocks per wave
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];  // X [BM][LDA] x 2 buffers
  // NF4 level pairs (L[lo], L[hi]) of each code byte v, 16 replicas: replica r
  // of entry v at byte 256 v + 8 r, in bank pair r. Lane l reads replica
  // l % 16, so the table reads of 16 lanes never share a bank whatever the
  // codes (one 256-entry copy would collide about 3.5 ways per access).
  // (NF4 only: 2-bit and INT4 fragments are built from registers alone)
  constexpr bool kTab = FMT == QW_FMT_NF4_B64;
  __shared__ __attribute__((aligned(16))) char pair_tab[kTab ? 256 * 256 : 16];
  const uint32_t lane_rep = 8u * (uint32_t)(threadIdx.x & 15);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 2, wn = wv & 3;  // wave's row half (WM = 2) and column quarter
  int m_tile, n_tile;
  xcd_tile((int)blockIdx.x, a.mt_count, (int)gridDim.x / a.mt_count, a.xcd_group, m_tile, n_tile);
  const int m0 = m_tile * BM, n0 = a.n_begin + n_tile * (128 * NJ);
  const int K = a.K;
  const int KT = K / BK;
  const int hk = lane >> 5;  // which 8 of each 16-wide k slice this lane holds

  if (kTab) {
    // 16-byte chunk c holds two replicas of entry c / 8
    for (int c = tid; c < 256 * 8; c += NTW) {
      const int v = c >> 3;
      const float2 p = make_float2(a.nf4[v & 15], a.nf4[v >> 4]);
      *reinterpret_cast<float4 *>(pair_tab + v * 256 + (c & 7) * 16) = make_float4(p.x, p.y, p.x, p.y);
    }
  }

  // ---- X prefetch registers (IM x 16 bytes per thread per step) ----
  // thread t copies 16-byte piece (t & 7) of rows (t >> 3) + 32 WM i, i < IM
  // (buffer loads: rows past M read through an out-of-range offset as 0)
  u32x4 ra[IM];
  const int xr = tid >> 3, xc = (tid & 7) * 8;
  const auto rx = pf_rsrc(a.X, (uint32_t)((size_t)a.M * K * 2));
  uint32_t xo[IM];
#pragma unroll
  for (int i = 0; i < IM; ++i) {
    const int gm = m0 + xr + 32 * WM * i;
    xo[i] = gm < a.M ? (uint32_t)(((size_t)gm * K + xc) * 2) : kPfOob;
  }
  // tiles at or past KT read as zeros (see the K loop below)
  auto load_x = [&](int kt) {
    const bool live = kt < KT;
    const uint32_t k0b = live ? (uint32_t)kt * BK * 2 : 0u;
#pragma unroll
    for (int i = 0; i < IM; ++i)
      ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(live ? xo[i] : kPfOob), (int)k0b, 0);
  };
  uint16_t *const xs = smem + xr * LDA + xc;  // + buf * BM * LDA + 32 WM i * LDA
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < IM; ++i)
      *reinterpret_cast<u32x4 *>(xs + buf * BM * LDA + 32 * WM * i * LDA) = ra[i];
  };

  // ---- W registers of this lane's two columns, two sets (step parity) ----
  constexpr int WR = FMT == QW_FMT_2BIT_G32 ? 6 : 9;  // dwords per column per step
  uint32_t wr[2][NJ][WR];
  int gcol[NJ];
  bool cvalid[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    gcol[j] = n0 + wn * 32 * NJ + j * 32 + (lane & 31);
    cvalid[j] = gcol[j] < a.N;
  }
  const uint32_t cb = FMT == QW_FMT_2BIT_G32 ? (uint32_t)K / 4 : (uint32_t)K / 2;  // code bytes per column
  const uint32_t sb = FMT == QW_FMT_2BIT_G32 ? (uint32_t)K / 8 : (uint32_t)K / 16;  // scale bytes per column
  const auto rcode = pf_rsrc(a.codes, (uint32_t)((size_t)a.N * cb));
  const auto rscale = pf_rsrc(a.scales, (uint32_t)((size_t)a.N * sb));
  uint32_t co[NJ], so[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    co[j] = cvalid[j] ? (uint32_t)gcol[j] * cb : kPfOob;
    so[j] = cvalid[j] ? (uint32_t)gcol[j] * sb : kPfOob;
  }
  auto load_w = [&](int kt, uint32_t (&dst)[NJ][WR]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (FMT == QW_FMT_2BIT_G32) {
        // 64 codes = 16 bytes, two S/Z words
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rcode, (int)co[j], kt * 16, 0);
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 sz = __builtin_amdgcn_raw_buffer_load_b64(rscale, (int)so[j], kt * 8, 0);
        dst[j][0] = v[0]; dst[j][1] = v[1]; dst[j][2] = v[2]; dst[j][3] = v[3];
        dst[j][4] = sz[0]; dst[j][5] = sz[1];
      } else {
        // 64 codes = 32 bytes, one absmax
        const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(rcode, (int)co[j], kt * 32, 0);
        const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(rcode, (int)co[j], kt * 32 + 16, 0);
        dst[j][0] = v0[0]; dst[j][1] = v0[1]; dst[j][2] = v0[2]; dst[j][3] = v0[3];
        dst[j][4] = v1[0]; dst[j][5] = v1[1]; dst[j][6] = v1[2]; dst[j][7] = v1[3];
        dst[j][8] = __builtin_amdgcn_raw_buffer_load_b32(rscale, (int)so[j], kt * 4, 0);
      }
    }
  };

  floatx16 acc[IM][NJ];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const uint16_t *const ar = smem + (wm * (BM / WM) + (lane & 31)) * LDA + hk * 8;  // + buf, i, kk offsets
  auto read_a = [&](int buf, int kk, bf16x8 (&af)[IM]) {
#pragma unroll
    for (int i = 0; i < IM; ++i)
      af[i] = *reinterpret_cast<const bf16x8 *>(ar + buf * BM * LDA + 32 * i * LDA + kk * 16);
  };

  // B fragment of column j for k slice kk of the step held in w
  auto make_b = [&](const uint32_t (&w)[NJ][WR], int j, int kk, const uint32_t (&T)[NJ][2][2]) {
    uint32_t o[4];
    if (FMT == QW_FMT_2BIT_G32) {
      const int g = kk >> 1;
      dequant8_2bit(w[j][kk], hk, T[j][g][0], T[j][g][1], o);
    } else if (FMT == QW_FMT_INT4_G32) {
      // the fp16 scale s of group kk / 2; elements kk*16 + hk*8 .. +7 are
      // the nibbles of code word 2kk + hk, element 2q in the low nibble of
      // byte q. Each nibble u becomes a float exactly (byte to float), and
      // u s - 8 s = (u - 8) s exactly (both products fit fp32), so the fma
      // gives fl32(s q) before the one rounding to bf16.
      const float s = f16_bits_to_f32((uint16_t)(w[j][8] >> (16 * (kk >> 1))));
      const float ns8 = -8.0f * s;
      // the word picked with a byte permute (a select here becomes an
      // indexed read that moves the W registers to private memory)
      const uint32_t c = __builtin_amdgcn_perm(w[j][2 * kk + 1], w[j][2 * kk], hk ? 0x07060504u : 0x03020100u);
      const uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = pack_bf16x2(__builtin_fmaf((float)((lo >> (8 * q)) & 0xFFu), s, ns8),
                           __builtin_fmaf((float)((hi >> (8 * q)) & 0xFFu), s, ns8));
    } else {
      // NF4: one fp32 absmax per 64
      const float am = __builtin_bit_cast(float, w[j][8]);
      // elements kk*16 + hk*8 .. +7 = bytes 4*(2kk+hk) .. +3 of the 32 code bytes
      const uint32_t c = hk ? w[j][2 * kk + 1] : w[j][2 * kk];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // v_perm: byte 0 <- lane_rep (source byte 4), byte 1 <- code byte q
        const uint32_t ad = __builtin_amdgcn_perm(lane_rep, c, 0x0C0C0004u | ((uint32_t)q << 8));
        const float2 l = *reinterpret_cast<const float2 *>(pair_tab + ad);
        o[q] = pack_bf16x2(am * l.x, am * l.y);
      }
    }
    return __builtin_bit_cast(bf16x8, u32x4{o[0], o[1], o[2], o[3]});
  };

  // One K step with the W register set PAR: products of tile kt out of LDS
  // buffer kt & 1; X of tile kt+1 is written to the other buffer after the
  // first k slice (the second for 2-bit), X of tile kt+2 and W of tile kt+1
  // (into the other set) are requested then too. W loads past the end re-read the last tile;
  // X loads past the end give zeros.
  // value tables of the two groups of each column (2-bit) from a W set
  auto make_tables = [&](const uint32_t (&w)[NJ][WR], uint32_t (&T)[NJ][2][2]) {
    if (FMT == QW_FMT_2BIT_G32) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const uint32_t szw = w[j][4 + g];
          const float S = f16_bits_to_f32((uint16_t)(szw & 0xFFFFu));
          const float Z = f16_bits_to_f32((uint16_t)(szw >> 16));
          T[j][g][0] = pack_bf16x2(__builtin_fmaf(S, -1.52f, Z), __builtin_fmaf(S, -0.45f, Z));
          T[j][g][1] = pack_bf16x2(__builtin_fmaf(S, 0.45f, Z), __builtin_fmaf(S, 1.52f, Z));
        }
    }
  };
  // 2-bit and INT4: the first slice's B fragments of a step (and the 2-bit
  // tables) depend on the lane's own W registers only, so they are built
  // during the previous step's last slice: after the step barrier only the
  // A reads remain before the first products (measured 3.6% faster for
  // 2-bit; NF4, whose fragments read the LDS pair table, keeps building
  // them at the step start: 30% slower otherwise).
  uint32_t T[NJ][2][2];
  bf16x8 fb0[NJ];

  auto step = [&](int kt, auto par_tag) {
    constexpr int PAR = decltype(par_tag)::value;
    constexpr int buf = PAR;  // kt has the parity of the register set
    const int kn1 = min(kt + 1, KT - 1), kn2 = kt + 2;
    // software pipeline: the A fragments and B fragments of slice kk+1 are
    // read and dequantized while the 16 products of slice kk run
    bf16x8 fa[2][IM], fb[2][NJ];
    read_a(buf, 0, fa[0]);
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb[0][j] = !kTab ? fb0[j] : make_b(wr[PAR], j, 0, T);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) {
        read_a(buf, kk + 1, fa[(kk + 1) & 1]);
#pragma unroll
        for (int j = 0; j < NJ; ++j) fb[(kk + 1) & 1][j] = make_b(wr[PAR], j, kk + 1, T);
      } else if constexpr (!kTab) {  // the next step's (W of tile kt+1)
        make_tables(wr[PAR ^ 1], T);
#pragma unroll
        for (int j = 0; j < NJ; ++j) fb0[j] = make_b(wr[PAR ^ 1], j, 0, T);
      }
#pragma unroll
      for (int i = 0; i < IM; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][i], fb[kk & 1][j], acc[i][j], 0, 0, 0);
      // 2-bit: the next step's W is requested before X (so waiting for it
      // at the next step's start does not wait for X), and X is stored and
      // refilled one slice later (its wait overlaps a slice of products);
      // measured 2% faster for 2-bit, not for the 4-bit formats
      if constexpr (!kTab) {
        if (kk == 0) load_w(kn1, wr[PAR ^ 1]);
        if (kk == 1) {
          store_x(buf ^ 1);
          load_x(kn2);
        }
      } else if (kk == 0) {
        store_x(buf ^ 1);
        load_x(kn2);
        load_w(kn1, wr[PAR ^ 1]);
      }
      // IM NJ x {1 product, a few vector ops, a fragment read, an LDS write,
      // a memory read}: the vector work runs while the products execute
#pragma unroll
      for (int t = 0; t < IM * NJ; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // LDS-only barrier: the loads of the next steps stay in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  // prologue: X of tile 0 into buffer 0, X of tile 1 in registers, W of
  // tile 0 in set 0
  load_x(0);
  load_w(0, wr[0]);
  __syncthreads();  // the NF4 table too
  store_x(0);
  load_x(1);
  if constexpr (!kTab) {
    make_tables(wr[0], T);
#pragma unroll
    for (int j = 0; j < NJ; ++j) fb0[j] = make_b(wr[0], j, 0, T);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  // Two steps per trip and a single exit: with an odd KT the last trip's
  // second step multiplies a zero X tile (one wasted step) rather than being
  // skipped, because a second loop exit makes the compiler copy the
  // accumulators out of the matrix-core registers on each path and spill.
  for (int kt = 0; kt < KT; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
  }

  // ---- epilogue: lane holds D[8*g + 4*(lane>>5) + r][lane & 31] of each
  //      32 x 32 block. Each wave passes its 32 x 64 slice of one row block
  //      at a time through its own LDS slab (the X buffers are free now):
  //      accumulators go out with ds_write straight from the accumulator
  //      registers, come back as rows, and leave as 16-byte stores when the
  //      row length allows it (one element at a time otherwise). Buffer
  //      stores drop rows past M and columns past N. ----
  const uint32_t esz = F32OUT ? 4u : 2u;
  const auto ry = pf_rsrc(a.Y, (uint32_t)((size_t)a.M * a.N * esz));
  constexpr int SL = 32 * NJ + 4;  // floats per slab row
  float *const slab = reinterpret_cast<float *>(smem) + wv * 32 * SL;
  const bool vec = F32OUT ? (a.N % 4 == 0) : (a.N % 8 == 0);
  // read-back mapping: CW columns per lane, RP rows per pass
  constexpr int CW = F32OUT ? 4 : 8;
  constexpr int LPR = 32 * NJ / CW;  // lanes per slab row
  constexpr int RP = 64 / LPR;
  // all lane-dependent epilogue addresses come from a copy of the lane index
  // the compiler cannot see through, so none of them is hoisted above the K
  // loop (where they would hold registers the whole time)
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int rr0 = ln / LPR, cc = (ln % LPR) * CW;
  // LDS byte address of this lane's first write: row 4 * (lane >> 5), column lane & 31
  const uint32_t slab_w = (uint32_t)reinterpret_cast<uintptr_t>(slab) +
                          (uint32_t)((4 * (ln >> 5) * SL + (ln & 31)) * 4);
  const int gc = n0 + wn * 32 * NJ + cc;
  static_assert(4 * WM * 32 * SL * 4 <= 2 * BM * LDA * 2, "slabs fit in the X buffers");
#pragma unroll
  for (int i = 0; i < IM; ++i) {
    // ds_write with the accumulator register as data operand: a plain store
    // makes the compiler copy acc to vector registers first, and that copy
    // pushes the allocator into spilling inside the K loop
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          asm volatile("ds_write_b32 %0, %1 offset:%2"
                       :
                       : "v"(slab_w), "a"(acc[i][j][4 * g + r]), "i"(((8 * g + r) * SL + j * 32) * 4)
                       : "memory");
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
    for (int pass = 0; pass < 32 / RP; ++pass) {
      const int rr = pass * RP + rr0;
      const int gm = m0 + wm * (BM / WM) + i * 32 + rr;
      float v[CW];
#pragma unroll
      for (int q = 0; q < CW; q += 4) {
        const float4 t = *reinterpret_cast<const float4 *>(slab + rr * SL + cc + q);
        v[q] = t.x; v[q + 1] = t.y; v[q + 2] = t.z; v[q + 3] = t.w;
      }
      const uint32_t rowb = gm < a.M ? (uint32_t)gm * a.N * esz : kPfOob;
      if (vec) {
        const uint32_t off = (rowb != kPfOob && gc < a.N) ? rowb + (uint32_t)gc * esz : kPfOob;
        if (F32OUT) {
          const u32x4 o = {__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                           __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])};
          __builtin_amdgcn_raw_buffer_store_b128(o, ry, (int)off, 0, 0);
        } else {
          const u32x4 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                           pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
          __builtin_amdgcn_raw_buffer_store_b128(o, ry, (int)off, 0, 0);
        }
      } else {
#pragma unroll
        for (int q = 0; q < CW; ++q) {
          const uint32_t off =
              (rowb != kPfOob && gc + q < a.N) ? rowb + (uint32_t)(gc + q) * esz : kPfOob;
          if (F32OUT)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[q]), ry, (int)off, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_bits(v[q]), ry, (int)off, 0, 0);
        }
      }
    }
    // the slab is rewritten by the next row block
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }
}

template <int FMT, bool F32, int NJ>
qw_status launch_w(const PrefillArgs &a, int n_begin, int n_tiles, hipStream_t s) {
  if (n_tiles <= 0) return QW_OK;
  PrefillArgs b = a;
  b.n_begin = n_begin;
  const size_t lds = (size_t)2 * BM * LDA * 2;  // the NF4 pair table is static
  // one wave per SIMD owning all 256 rows (WM = 1): measured on MI355X, two
  // waves per SIMD with 128 rows each (WM = 2) are slower, since the two
  // waves sharing a column both dequantize it
  constexpr int WM = 1;
  QW_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(&prefill_w_kernel<FMT, F32, NJ, WM>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  QW_HIP_TRY(launch(prefill_w_kernel<FMT, F32, NJ, WM>, a.mt_count * n_tiles, 256 * WM, lds, s, b));
  return QW_OK;
}

// Column split between 256-wide tiles and 128-wide tiles for the last
// columns: a whole number of rounds of wide tiles over the CUs, then one
// short round of narrow ones instead of a half-empty round of wide ones.
// Cost model in units of one wide-tile round; a narrow tile costs 0.55 of a
// wide one (half the products, same fixed per-step work).
int wide_column_tiles(int mt, int N, int cus) {
  const int nt = (N + 255) / 256;
  double best = 1e30;
  int best_n = nt;
  for (int n = nt; n >= 0; --n) {
    const long wide = (long)mt * n;
    const int rest = N - 256 * n;
    const long narrow = rest > 0 ? (long)mt * ((rest + 127) / 128) : 0;
    const double cost = (double)((wide + cus - 1) / cus) + 0.55 * (double)((narrow + cus - 1) / cus);
    if (cost < best - 1e-9) {
      best = cost;
      best_n = n;
    }
  }
  return best_n;
}

template <int FMT>
qw_status launch_fmt(const PrefillArgs &a, bool f32, int cus, hipStream_t s) {
  const size_t esz = f32 ? 4 : 2;
  const bool fits32 = (size_t)a.M * a.K * 2 < (1ull << 31) && (size_t)a.M * a.N * esz < (1ull << 31) &&
                      (size_t)a.N * (a.K / 2) < (1ull << 31);
  if (a.n_out == 0 && fits32) {  // W straight to registers
    // the test hook QW_TUNE_PREFILL_WIDE_TILES overrides the number of
    // 256-wide column tiles (tests run the 128-wide kernel on small shapes)
    const int nt = (a.N + 255) / 256;
    const int forced = tune(QW_TUNE_PREFILL_WIDE_TILES);
    const int nw = forced >= 0 ? min(forced, nt) : wide_column_tiles(a.mt_count, a.N, cus);
    const int rest = a.N - 256 * nw;
    const int nn = rest > 0 ? (rest + 127) / 128 : 0;
    if (f32) {
      QW_TRY((launch_w<FMT, true, 2>(a, 0, nw, s)));
      QW_TRY((launch_w<FMT, true, 1>(a, 256 * nw, nn, s)));
    } else {
      QW_TRY((launch_w<FMT, false, 2>(a, 0, nw, s)));
      QW_TRY((launch_w<FMT, false, 1>(a, 256 * nw, nn, s)));
    }
    return QW_OK;
  }
  const int nt = (a.N + BN - 1) / BN;
  const int grid = a.mt_count * nt;
  const size_t lds = (size_t)2 * (BM + BN) * LDA * 2 + (FMT != QW_FMT_2BIT_G32 ? 256 * 8 : 0);
  const void *fn = f32 ? reinterpret_cast<const void *>(&prefill_kernel<FMT, true>)
                       : reinterpret_cast<const void *>(&prefill_kernel<FMT, false>);
  QW_HIP_TRY(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  if (f32)
    QW_HIP_TRY(launch(prefill_kernel<FMT, true>, grid, NT, lds, s, a));
  else
    QW_HIP_TRY(launch(prefill_kernel<FMT, false>, grid, NT, lds, s, a));
  return QW_OK;
}

}  // namespace
}  // namespace qw

extern "C" qw_status qgemm_prefill(const qw_weight *w, const void *X, int M, void *Y,
                                   qw_dtype y_dtype, void *stream) {
  using namespace qw;
  CallScope scope;
  if (!w || !X || !Y || M < 1) return QW_ERR_INVALID_ARG;
  if (y_dtype != QW_DT_BF16 && y_dtype != QW_DT_F32) return QW_ERR_INVALID_ARG;
  if (!w || (w->format != QW_FMT_2BIT_G32 && w->format != QW_FMT_NF4_B64 && w->format != QW_FMT_INT4_G32))
    return QW_ERR_INVALID_ARG;
  qw_status st = check_weight_view(w, w->format, 0);
  if (st != QW_OK) return st;
  if (w->K % 64) return QW_ERR_UNSUPPORTED;
  if (!aligned16(X) || !aligned16(Y)) return QW_ERR_ALIGNMENT;
  int cus = 0;
  st = current_device(&cus);
  if (st != QW_OK) return st;
  PrefillArgs a{};
  a.X = reinterpret_cast<const uint16_t *>(X);
  a.codes = reinterpret_cast<const uint32_t *>(w->codes);
  a.scales = w->scales;
  a.idx = w->out_idx;
  a.wo = w->out_w;
  a.Y = Y;
  a.M = M;
  a.N = w->N;
  a.K = w->K;
  a.n_out = w->format == QW_FMT_NF4_B64 ? 0 : w->n_out;
  a.n_out_pad = w->n_out_pad;
  a.mt_count = (M + BM - 1) / BM;
  a.xcd_group = 4;  // row tiles an XCD walks per column sweep
  // level of each 4-bit code: the NF4 table, or u - 8 for INT4
  const float *L = nf4_levels_host();
  for (int i = 0; i < 16; ++i) a.nf4[i] = w->format == QW_FMT_INT4_G32 ? (float)(i - 8) : L[i];
  const bool f32 = y_dtype == QW_DT_F32;
  if (w->format == QW_FMT_2BIT_G32) return launch_fmt<QW_FMT_2BIT_G32>(a, f32, cus, as_stream(stream));
  if (w->format == QW_FMT_INT4_G32) return launch_fmt<QW_FMT_INT4_G32>(a, f32, cus, as_stream(stream));
  return launch_fmt<QW_FMT_NF4_B64>(a, f32, cus, as_stream(stream));
}
