// Prefill GEMM against block-wise quantized weights:
//   Y[m][n] = sum_k X[m][k] * w_bf16[n][k]
// with w_bf16 = bf16(fp32 fma(S, C[q], Z)) for the 2-bit code
// ("On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)", sections 2-4) or
// bf16(fp32 absmax * L[q]) for NF4 ("AirQuant" README, "Fundamentacao
// Teorica e Arquitetura" item 2). 2-bit anchor columns take bf16(out_w).
//
// Tiling: a 256-thread workgroup computes a 256 (M) x 128 (N) tile of Y; its
// four waves each own 128 x 64 as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16
// (fp32 accumulators). K advances 64 at a time: the X tile is copied to LDS,
// the packed W tile is dequantized in registers straight to bf16 and stored
// to LDS, and the next tile's global loads are in flight during the MFMAs.
// LDS rows are padded by 16 bytes so 16-byte fragment reads of 8 rows hit
// distinct banks.
//
// 2-bit dequant: per group of 32 the four possible bf16 values
// v_q = bf16(fma(S, C[q], Z)) are formed once and packed into two dwords;
// a v_perm_b32 whose byte selectors are built from two code fields then
// assembles a bf16 pair, so each weight costs a few integer ops.
#include "qw_internal.h"

namespace qw {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int LDA = BK + 8;  // bf16 elements per LDS row (144 bytes)
constexpr int NT = 256;

struct PrefillArgs {
  const uint16_t *X;       // [M][K] bf16
  const uint32_t *codes;   // 2-bit: [N][K/16]; NF4: [N][K/8]
  const void *scales;      // 2-bit: uint32 [N][K/32]; NF4: float [N][K/64]
  const int32_t *idx;      // anchors (2-bit), may be null
  const uint16_t *wo;      // [N][n_out_pad]
  void *Y;                 // [M][N]
  int M, N, K, n_out, n_out_pad;
  int mt_count;            // number of 256-row tiles along M
  float nf4[16];
};

__device__ inline uint32_t f32_to_bf16_bits(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// 32 codes of one group (two code dwords c0, c1 = elements 0..15, 16..31)
// -> 16 dwords of bf16 pairs in natural element order.
__device__ inline void dequant_group_2bit(uint32_t c0, uint32_t c1, uint32_t szw,
                                          uint32_t out[16]) {
  const float S = f16_bits_to_f32((uint16_t)(szw & 0xFFFFu));
  const float Z = f16_bits_to_f32((uint16_t)(szw >> 16));
  const uint32_t T0 = pack_bf16x2(__builtin_fmaf(S, -1.52f, Z), __builtin_fmaf(S, -0.45f, Z));
  const uint32_t T1 = pack_bf16x2(__builtin_fmaf(S, 0.45f, Z), __builtin_fmaf(S, 1.52f, Z));
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t c = h ? c1 : c0;
    uint32_t p[8];  // p[f] = (elem f, elem f + 8) of this 16-code dword
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const uint32_t t = (c >> (2 * f)) & 0x00030003u;
      const uint32_t sel = t * 0x0202u + 0x01000100u;
      p[f] = __builtin_amdgcn_perm(T1, T0, sel);
    }
    // natural order: (e0,e1) (e2,e3) ... (e14,e15)
#pragma unroll
    for (int f = 0; f < 8; f += 2) {
      out[h * 8 + f / 2] = __builtin_amdgcn_perm(p[f + 1], p[f], 0x05040100u);
      out[h * 8 + 4 + f / 2] = __builtin_amdgcn_perm(p[f + 1], p[f], 0x07060302u);
    }
  }
}

template <int FMT, bool F32OUT>
__global__ __launch_bounds__(NT) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t *As = smem;                    // [BM][LDA]
  uint16_t *Bs = smem + BM * LDA;         // [BN][LDA]
  float2 *ltab = reinterpret_cast<float2 *>(Bs + BN * LDA);  // NF4 [256]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int b = blockIdx.x;
  const int m_tile = b % a.mt_count;
  const int n_tile = b / a.mt_count;
  const int m0 = m_tile * BM, n0 = n_tile * BN;
  const int K = a.K;
  const int KT = K / BK;

  if (FMT == QW_FMT_NF4_B64) {
    for (int v = tid; v < 256; v += NT) ltab[v] = make_float2(a.nf4[v & 15], a.nf4[v >> 4]);
  }

  // ---- global prefetch registers ----
  uint4 ra[8];
  uint32_t rb[5];
  const int brow = tid >> 1, bhalf = tid & 1;
  const int gn = n0 + brow;
  const bool bvalid = gn < a.N;

  auto load_tile = [&](int kt) {
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
    if (FMT == QW_FMT_2BIT_G32) {
      if (bvalid) {
        const uint32_t *cp = a.codes + (size_t)gn * (K / 16) + k0 / 16 + 2 * bhalf;
        rb[0] = __builtin_nontemporal_load(cp);
        rb[1] = __builtin_nontemporal_load(cp + 1);
        rb[2] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(a.scales) +
                                           (size_t)gn * (K / 32) + k0 / 32 + bhalf);
      } else {
        rb[0] = rb[1] = rb[2] = 0;
      }
    } else {
      if (bvalid) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
            a.codes + (size_t)gn * (K / 8) + k0 / 8 + 4 * bhalf));
        rb[0] = v.x; rb[1] = v.y; rb[2] = v.z; rb[3] = v.w;
        rb[4] = __builtin_bit_cast(uint32_t, __builtin_nontemporal_load(
            reinterpret_cast<const float *>(a.scales) + (size_t)gn * (K / 64) + k0 / 64));
      } else {
        rb[0] = rb[1] = rb[2] = rb[3] = rb[4] = 0;
      }
    }
  };

  auto store_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = i * NT + tid;
      const int row = c >> 3, c16 = c & 7;
      *reinterpret_cast<uint4 *>(As + row * LDA + c16 * 8) = ra[i];
    }
    uint32_t out[16];
    if (FMT == QW_FMT_2BIT_G32) {
      dequant_group_2bit(rb[0], rb[1], rb[2], out);
      if (a.n_out > 0 && bvalid) {
        // anchor columns of this group: idx is ascending, find the first >= k_lo
        const int k_lo = kt * BK + 32 * bhalf;
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
      const float am = __builtin_bit_cast(float, rb[4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t c = rb[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float2 l = ltab[(c >> (8 * j)) & 0xFFu];
          out[i * 4 + j] = pack_bf16x2(am * l.x, am * l.y);
        }
      }
    }
    uint4 *bp = reinterpret_cast<uint4 *>(Bs + brow * LDA + bhalf * 32);
    bp[0] = make_uint4(out[0], out[1], out[2], out[3]);
    bp[1] = make_uint4(out[4], out[5], out[6], out[7]);
    bp[2] = make_uint4(out[8], out[9], out[10], out[11]);
    bp[3] = make_uint4(out[12], out[13], out[14], out[15]);
  };

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  load_tile(0);
  for (int kt = 0; kt < KT; ++kt) {
    __syncthreads();
    store_tile(kt);
    __syncthreads();
    if (kt + 1 < KT) load_tile(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int kof = kk * 16 + (lane >> 5) * 8;
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8 *>(As + row * LDA + kof);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8 *>(Bs + col * LDA + kof);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: lane holds D[8*g + 4*(lane>>5) + r][lane & 31] ----
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int gn_ = n0 + wn * 64 + j * 32 + (lane & 31);
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

template <int FMT>
qw_status launch_fmt(const PrefillArgs &a, bool f32, hipStream_t s) {
  const int nt = (a.N + BN - 1) / BN;
  const int grid = a.mt_count * nt;
  const size_t lds = (size_t)(BM + BN) * LDA * 2 + (FMT == QW_FMT_NF4_B64 ? 256 * 8 : 0);
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
  if (!w || (w->format != QW_FMT_2BIT_G32 && w->format != QW_FMT_NF4_B64)) return QW_ERR_INVALID_ARG;
  qw_status st = check_weight_view(w, w->format, 0);
  if (st != QW_OK) return st;
  if (w->K % 64) return QW_ERR_UNSUPPORTED;
  if (!aligned16(X) || !aligned16(Y)) return QW_ERR_ALIGNMENT;
  st = current_device(nullptr);
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
  a.n_out = w->format == QW_FMT_2BIT_G32 ? w->n_out : 0;
  a.n_out_pad = w->n_out_pad;
  a.mt_count = (M + BM - 1) / BM;
  const float *L = nf4_levels_host();
  for (int i = 0; i < 16; ++i) a.nf4[i] = L[i];
  const bool f32 = y_dtype == QW_DT_F32;
  if (w->format == QW_FMT_2BIT_G32) return launch_fmt<QW_FMT_2BIT_G32>(a, f32, as_stream(stream));
  return launch_fmt<QW_FMT_NF4_B64>(a, f32, as_stream(stream));
}
