// Decode GEMV against the adaptive non-uniform 2-bit code on the matrix
// cores ("On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)": codebook of
// section 2, per-group scale/offset of section 3, fp16 anchors of section 4).
//
//   y[b][n] = sum_g S_g * (C0 X_g + d1 sum_{k in g} x_R q + d3 sum_{k in g} x_R h)
//           + Z_g X_g + sum_o x[b][idx_o] W_O[n][o]
//
// with q = l + 2h the code, d1 = C1 - C0, d3 = (C2 - C0) - 2 d1 (exact for
// the symmetric codebook: C3 - C0 = d1 + (C2 - C0)) and X_g the group sum of
// x_R (x with the anchor channels zeroed).
//
// The two code sums run on v_mfma_scale_f32_16x16x128_f8f6f4 with the codes
// as the fp4 (e2m1) operand and x as the fp8 (e4m3) operand:
//  * a 2-bit code masked into the low two bits of a nibble is the e2m1 value
//    q/2 exactly, its high bit alone (bit 1) is the e2m1 value h; one AND
//    (plus one shift per 16 codes) turns 8 packed codes into 8 operands;
//  * x is split exactly into three e4m3 limbs after scaling each group of 32
//    by a power of two 2^s (max |x| 2^s in [128, 256)); a limb only loses
//    what underflows e4m3 (below 2^-10 absolute, 2^-17 of the group max);
//  * the matrix core sums each run of 8 products aligned to the largest of
//    them, dropping bits below 2^-13 of it; every D row holds one limb, so a
//    run never mixes limbs and only elements below about 2^-8 of their run's
//    largest lose bits.
// Operand placement (one 16x16x128 instruction = 16 output rows x 4 groups):
//  * B (codes, fp4): lane l holds output row l%16 and the 32 codes of one
//    group ("slot" l/16), as nibbles in the order even codes 0..14, odd
//    1..15, even 16..30, odd 17..31;
//  * A (x limbs, fp8): row i = 4*slot + limb (limb 3 zero); the 16 bytes of a
//    lane hold limb values of half a group in the same permuted order, in
//    bytes 0..15 for slots 0, 1 and bytes 16..31 for slots 2, 3;
//  * D: lane l holds rows 4*(l/16)..+3 of column l%16, i.e. the three limb
//    partials of (output row l%16, slot l/16) -- the same (row, group) whose
//    codes and S, Z that lane loaded, so the group's scale is applied in the
//    lane that owns it.
// Work: a wave computes 16 output rows; its K range is cut in super-chunks of
// 512 (16 groups, 4 instructions per stream), streamed through a ring of P
// register slots (two 16-byte code loads and one 16-byte S/Z load per lane),
// followed by anchor chunks of 96 anchors per row on the same ring.
// A workgroup of 8 waves owns a contiguous range of 16-row tiles; each tile's
// K range may be split over several waves, whose partial row sums meet in LDS
// and are added in a fixed order.
// The same body serves the merged gate/up product (pairs of gate and up tiles
// per workgroup, silu(gate) * up in the epilogue), the K parts of wide
// batches, the v3.2 INT4 format (kernel_int4), and the persistent decode
// stack at the end of this file.
#include <stdlib.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "qw_internal.h"

namespace qw {
namespace gemv2m {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMats = 4;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kXItems = 12;  // 16-byte x loads per thread in the prologue
constexpr int kIdxItems = 4; // anchor indices per thread in the prologue
constexpr int kAnchorChunk = 96;
// ring slots requested before the x preparation (the rest after it): more
// start the weight stream earlier but delay the preparation behind them
constexpr int kEarly = 2;
constexpr uint32_t kOob = 0x7FFFFFF0u;

struct Mat {
  const uint32_t *codes;  // [N][K/16]
  const uint32_t *sz;     // [N][K/32]: fp16 S | fp16 Z << 16
  const uint32_t *mask;   // [K/32] anchor-channel bits, null without anchors
  const int32_t *idx;     // [n_out]
  const uint16_t *wo;     // [N][ld_a] fp16
  void *y;                // [B][N]
  int N, n_out, n_out_pad; // anchors of this launch's share (padded to 8)
  int wg_begin, wg_count;  // this matrix's workgroups
  int tiles;               // ceil(N / 16)
  int W;                   // waves per tile (K splits); divides K/512
  int kbase;               // first channel of this K part (0 unless split);
                           // codes, sz and mask already point at it
  int ld_a;                // anchors per weight row (row stride of wo)
  int abase;               // first anchor of this part; idx and wo point at it
};

struct Args {
  Mat m[kMats];
  int count;
  const uint16_t *x;  // [B][ldk] fp16
  int K;              // channels per matrix of this launch (a K part when split)
  int ldk;            // channels per weight row and per x row
  int f32out;
  int xo_len;         // anchor index slots in LDS (multiple of 96)
  int units_max;      // max tiles per workgroup * W (partials in LDS)
  int xraw;           // 1: raw x copied to LDS for the anchor gather; 0:
                      // anchors gathered from global x (frees B*(K+8)*2
                      // bytes of LDS so wider batches fit one pass)
  int swiglu;         // 1: one merged gate/up matrix (m[0], 2I rows: gate
                      // rows 0..I-1, up rows I..2I-1, I % 16 == 0); y gets
                      // silu(gate) * up, I values per batch row
};

// SiLU of the gate projection's output, g * sigmoid(g), in fp32.
__device__ inline float silu(float g) { return g / (1.0f + expf(-g)); }

// LDS layout, bytes:
//   limbs  [B][G][3][32]   e4m3 limbs per group (two 16-byte halves)
//   zero   [32]
//   coef   [B][G] float4   {2 d1 2^-s, d3 2^-s, C0 X_g, X_g}
//   aidx   [xo_len] int32  anchor channels (entries past n_out unused)
//   xo     [B][xo_len] fp16 x at the anchor channels, zero past n_out
//   xraw   [B][K + 8] fp16 x as given, 8 zeros after each row (read at K);
//          absent when the anchors are gathered from global x
//   parts  [units_max][16][B] float  partial row sums of the units
struct Lds {
  size_t limbs, zero, coef, aidx, xo, xraw, parts, total;
};

__host__ __device__ inline Lds lds_layout(int B, int K, int xo_len, int units_max, int xraw = 1) {
  const size_t G = (size_t)K / 32;
  Lds l;
  l.limbs = 0;
  l.zero = (size_t)B * G * 96;
  l.coef = l.zero + 32;
  l.aidx = l.coef + (size_t)B * G * 16;
  l.xo = l.aidx + (((size_t)xo_len * 4 + 15) & ~(size_t)15);
  l.xraw = l.xo + (((size_t)B * xo_len * 2 + 15) & ~(size_t)15);
  l.parts = l.xraw + (xraw ? (size_t)B * (K + 8) * 2 : 0);
  l.total = l.parts + (size_t)units_max * 16 * B * 4;
  return l;
}

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ inline uint32_t ld1(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)v, (int)s, 0);
}
__device__ inline u32x2 ld2(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)v, (int)s, 0);
}
__device__ inline u32x4 ld4(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)v, (int)s, 0);
}
// Cache policy sc0 | sc1 (system coherence): the access goes to memory past
// the per-CU and per-XCD caches, so data written by workgroups on other XCDs
// is seen without invalidating any cache, and stores are visible to them as
// soon as they complete.
constexpr int kCoherent = 1 | 16;
__device__ inline u32x4 ld4_coherent(__amdgpu_buffer_rsrc_t r, uint32_t v, uint32_t s) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)v, (int)s, kCoherent);
}

// B scaled by 2^(scale_b - 127) (e8m0), added to c
__device__ inline v4f mfma_x_codes(v8i a_fp8, v8i b_fp4, v4f c = v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                   int scale_b = 0x7f) {
  // A format 0 = e4m3, B format 4 = e2m1; A scale 0x7f = 2^0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a_fp8, b_fp4, c, 0, 4, 0, 0x7f, 0, scale_b);
}

__device__ inline float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

template <int CTRL, int ROW_MASK>
__device__ inline float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                CTRL, ROW_MASK, 0xF, false));
}

// e4m3 bytes of four floats: a0, a1 in bytes 0, 1 and b0, b1 in bytes 2, 3
__device__ inline uint32_t to_fp8x4(float a0, float a1, float b0, float b1) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(b0, b1, lo, true);
}
__device__ inline float fp8_at(uint32_t w, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}

// Position of one wave in its stream of steps: unit (tile, split) and the
// step inside it (code super-chunks first, then anchor chunks). Units of a
// wave are u = wave, wave + 8, ...; unit u is (tile u / W, split u % W) and
// split s owns anchor chunks s, s + W, ... below NA. Kept incrementally so
// that advancing needs no division except once per unit.
struct Cursor {
  int unit;   // local unit index; >= n_units means past the end
  int tile;   // local tile index (unit / W)
  int split;  // unit % W
  int step;   // step inside the unit
  int len;    // steps of this unit
};

struct Stream {
  int n_units, W, L, NA, nw;  // nw: waves of the workgroup
  __device__ int unit_len(int split) const {
    return L + (split < NA ? (NA - 1 - split) / W + 1 : 0);
  }
  __device__ Cursor start(int u) const {
    Cursor c;
    c.unit = u;
    c.tile = u / W;
    c.split = u - c.tile * W;
    c.step = 0;
    c.len = unit_len(c.split);
    return c;
  }
  __device__ void advance(Cursor &c) const {
    if (++c.step >= c.len) {
      c.unit += nw;
      c.split += nw;
      while (c.split >= W) {
        c.split -= W;
        ++c.tile;
      }
      c.step = 0;
      c.len = unit_len(c.split);
    }
  }
};

// One ring slot: three 16-byte loads per lane (code step: codes of 32
// groups' halves and their S/Z words; anchor step: three pieces of 8 anchor
// weights).
struct Slot {
  u32x4 c0, c1, c2;
};
// INT4 (v3.2 format): code step: the 32 codes of four groups (four 16-byte
// loads) and their four fp16 scales (one 8-byte load); anchor step: three
// pieces of 8 anchor weights in c0..c2 (c3 and sz then read zeros).
struct Slot4 {
  u32x4 c0, c1, c2, c3;
  u32x2 sz;
};

// Select among four values that are all read (so the reads are not
// conditional: no chain of dependent scalar loads behind branches).
template <typename T>
__device__ inline T sel4(int i, T v0, T v1, T v2, T v3) {
  T r = v0;
  r = i == 1 ? v1 : r;
  r = i == 2 ? v2 : r;
  r = i == 3 ? v3 : r;
  return r;
}

// One workgroup's share (workgroup index bid of the launch the Args were
// planned for) of a grouped GEMV, with the group's LDS at lds.
// XR: raw x kept in LDS for the anchor gather (a.xraw == 1); false only for
// batches that fit one pass without it. NT: threads of the workgroup.
// SW: the merged gate/up product with the gated activation in the epilogue
// (a.swiglu == 1, a single matrix): the workgroup's items are tile pairs, the
// gate tile p and the up tile H + p (H = I / 16), so both factors of each of
// its outputs meet in its own LDS.
// I4: the v3.2 INT4 format ("On-The-Fly Weight Synthesizer (OTF-LLM Engine
// v4.0)", "Comparative Analysis: INT4 (v3.2) vs INT2 Non-Uniform (v4.0)"):
// codes u = q + 8 two per byte in element order, an fp16 scale s per group
// of 32, no anchor mask (anchor columns hold the zero level), anchors at
// the first n_out positions of x (x given in permuted order). A nibble
// u3 u2 u1 u0 masked to its low two bits is the e2m1 value (2 u1 + u0) / 2,
// its high two bits shifted down the value (2 u3 + u2) / 2, so
// u / 2 = P_lo + 4 P_hi: two fp4 products accumulated in one register, the
// second with the operand scale 2^2 of the scaled matrix-core instruction;
// per group sum x q = 2 (P_lo + 4 P_hi) - 8 X_g. x limbs are in element
// order.
template <int B, int P, bool MULTI, bool XC = false, bool XR = true, int NT = kThreads, bool SW = false,
          bool I4 = false>
__device__ __forceinline__ void body(const Args &a, const int bid, uint8_t *lds) {
  static_assert(!I4 || (!MULTI && !SW && !XC), "INT4 runs single-matrix launches");
  using SlotT = typename std::conditional<I4, Slot4, Slot>::type;
  constexpr int NW = NT / 64;
  // prologue items per thread: the same totals as at kThreads threads
  constexpr int XI = kXItems * kThreads / NT, IX = kIdxItems * kThreads / NT;
  // the thread index through an empty asm: values derived from it are
  // computed per call, so a persistent kernel that runs many bodies does not
  // keep them live (and spilled) across its whole loop
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int mi = 0;
  if (MULTI) {
#pragma unroll
    for (int i = 1; i < kMats; ++i)
      if (i < a.count && bid >= a.m[i].wg_begin) mi = i;
  }
  // each field picked with constant indices (scalar selects, no copy of the
  // argument block into private memory)
#define QW_SEL(f) (MULTI ? sel4(mi, a.m[0].f, a.m[1].f, a.m[2].f, a.m[3].f) : a.m[0].f)
  struct {
    const uint32_t *codes, *sz, *mask;
    const int32_t *idx;
    const uint16_t *wo;
    void *y;
    int N, n_out, n_out_pad, wg_begin, wg_count, tiles, W, kbase, ld_a, abase;
  } M = {QW_SEL(codes), QW_SEL(sz),    QW_SEL(mask),      QW_SEL(idx),      QW_SEL(wo),
         QW_SEL(y),     QW_SEL(N),     QW_SEL(n_out),     QW_SEL(n_out_pad), QW_SEL(wg_begin),
         QW_SEL(wg_count), QW_SEL(tiles), QW_SEL(W),      QW_SEL(kbase),     QW_SEL(ld_a),
         QW_SEL(abase)};
#undef QW_SEL
  const int K = a.K;
  // The raw-x variant serves unsplit launches only (the host never pairs it
  // with K parts), so there the part fields are constants: rows of K
  // channels and n_out_pad anchors, no part offsets.
  const int ldk = XR ? K : a.ldk;
  const int kbase = XR ? 0 : M.kbase;
  const int abase = XR ? 0 : M.abase;
  const int ld_a = XR ? M.n_out_pad : M.ld_a;
  const int G = K >> 5;
  const int SC = K >> 9;
  const int wi = bid - M.wg_begin;
  // (wi + 1) * tiles < 2^31: tiles <= 2^27 and workgroups per matrix <= 16
  // per CU of a 256-CU part are checked on the host
  // work items: tiles, or tile pairs (SW); this workgroup's are [t0, t1)
  const int H = SW ? M.tiles >> 1 : M.tiles;
  int t0, t1;
  if (SW && !XC && M.wg_count >= 2 && (M.wg_count & 1) == 0) {
    // the merged gate/up launch runs two workgroups per CU, w and w + G/2
    // sharing one: each pair of workgroups takes one CU's share of the
    // items, split between the two, so no CU holds more than its share
    // rounded up (a contiguous split puts the rounding of both workgroups
    // on the same CUs: 8 of 6.75 pairs per CU on the 32B block's 1728;
    // measured 26.9 -> 25.8 us)
    const int half = M.wg_count >> 1;
    const int c = wi < half ? wi : wi - half;
    const int u0 = (int)((uint32_t)(c * H) / (uint32_t)half);
    const int u1 = (int)((uint32_t)((c + 1) * H) / (uint32_t)half);
    const int mid = u0 + ((u1 - u0 + 1) >> 1);
    t0 = wi < half ? u0 : mid;
    t1 = wi < half ? mid : u1;
  } else {
    t0 = (int)((uint32_t)(wi * H) / (uint32_t)M.wg_count);
    t1 = (int)((uint32_t)((wi + 1) * H) / (uint32_t)M.wg_count);
  }
  const int np = t1 - t0;
  const int W = M.W;
  const int L = SC / W;
  const int NA = (M.n_out_pad + kAnchorChunk - 1) / kAnchorChunk;
  // local tiles: [0, np) the items' tiles, and with SW [np, 2 np) their up
  // tiles
  const int n_units = (SW ? 2 * np : np) * W;
  const Lds lay = lds_layout(B, K, a.xo_len, a.units_max, XR ? 1 : 0);
  uint8_t *limbs = lds + lay.limbs;
  uint8_t *zero = lds + lay.zero;
  float4 *coef = reinterpret_cast<float4 *>(lds + lay.coef);
  int32_t *aidx_l = reinterpret_cast<int32_t *>(lds + lay.aidx);
  uint16_t *xo = reinterpret_cast<uint16_t *>(lds + lay.xo);
  uint16_t *xraw = reinterpret_cast<uint16_t *>(lds + lay.xraw);
  float *parts = reinterpret_cast<float *>(lds + lay.parts);
  const int KX = K + 8;  // xraw row stride

  const int j = lane & 15;  // output row in the tile; A row
  const int g = lane >> 4;  // slot (group) of this lane's codes and D
  // ---- stream bookkeeping (wave-uniform) ----
  Stream st{n_units, W, L, NA, NW};

  // ---- per-lane load offsets ----
  const uint32_t rb_c = (uint32_t)ldk / (I4 ? 2 : 4);   // code bytes per row
  const uint32_t rb_s = (uint32_t)ldk / (I4 ? 16 : 8);  // scale (S/Z) bytes per row
  const uint32_t rb_a = (uint32_t)ld_a * 2;        // anchor bytes per row
  const uint32_t lim_a = (uint32_t)M.n_out_pad * 2; // this part's anchor bytes per row
  // sizes from the part's first channel (anchor) to the end of the matrix
  const uint32_t n_codes = (uint32_t)((size_t)M.N * rb_c - (uint32_t)kbase / (I4 ? 2 : 4));
  const uint32_t n_sz = (uint32_t)((size_t)M.N * rb_s - (uint32_t)kbase / (I4 ? 16 : 8));
  const uint32_t n_wo = (uint32_t)((size_t)M.N * rb_a - (uint32_t)abase * 2);

  // ring slot: code step: lane (row j, slot g) takes groups 16 sc + 4g ..
  // +3 of its row: codes bytes [32g, 32g+32) of the super-chunk's 128 and
  // their four S/Z words (INT4: bytes [64g, 64g+64) of 256 and four fp16
  // scales). Anchor step: three pieces of 8 anchor weights. One
  // branch-free issue path: descriptor and offsets are picked per step kind.
  auto issue = [&](SlotT &dst, const Cursor &c) __attribute__((always_inline)) {
    const bool live = c.unit < n_units;
    const int lt = live ? c.tile : 0;
    const int tile = SW ? (lt < np ? t0 + lt : H + t0 + (lt - np)) : t0 + lt;
    const int split = live ? c.split : 0;
    const bool row_ok = live && tile * 16 + j < M.N;
    const bool code = c.step < L;
    const int sc = split * L + c.step;
    const int an = split + W * (c.step - L);
    // descriptors built from a selected base and size (size 0 past the end)
    const auto r01 = rsrc(code ? (const void *)M.codes : (const void *)M.wo,
                          !live ? 0u : (code ? n_codes : n_wo));
    const auto r2 = rsrc(code ? (const void *)M.sz : (const void *)M.wo,
                         !live ? 0u : (code ? n_sz : n_wo));
    const uint32_t s01 = !live ? 0u : (code ? (uint32_t)tile * 16 * rb_c + (uint32_t)sc * (I4 ? 256 : 128)
                                            : (uint32_t)tile * 16 * rb_a);
    const uint32_t s2 = !live ? 0u : (code ? (uint32_t)tile * 16 * rb_s + (uint32_t)sc * (I4 ? 32 : 64)
                                           : (uint32_t)tile * 16 * rb_a);
    const uint32_t pa = (uint32_t)an * (kAnchorChunk * 2) + 16u * g;  // anchor piece 0
    if constexpr (I4) {
      // code step: four 16-byte code loads and one 8-byte scale load; anchor
      // step: the three anchor pieces (all from r01), the rest read zeros
      uint32_t v[4], vs;
      if (code) {  // uniform
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = row_ok ? (uint32_t)j * rb_c + 64u * g + 16u * t : kOob;
        vs = row_ok ? (uint32_t)j * rb_s + 8u * g : kOob;
      } else {
#pragma unroll
        for (int t = 0; t < 3; ++t)
          v[t] = row_ok && pa + 64u * t < lim_a ? (uint32_t)j * rb_a + pa + 64u * t : kOob;
        v[3] = kOob;
        vs = kOob;
      }
      dst.c0 = ld4(r01, v[0], s01);
      dst.c1 = ld4(r01, v[1], s01);
      dst.c2 = ld4(r01, v[2], s01);
      dst.c3 = ld4(r01, v[3], s01);
      dst.sz = ld2(r2, vs, s2);
      return;
    }
    uint32_t v0, v1, v2;
    if (code) {  // uniform
      v0 = row_ok ? (uint32_t)j * rb_c + 32u * g : kOob;
      v1 = row_ok ? v0 + 16 : kOob;
      v2 = row_ok ? (uint32_t)j * rb_s + 16u * g : kOob;
    } else {
      v0 = row_ok && pa < lim_a ? (uint32_t)j * rb_a + pa : kOob;
      v1 = row_ok && pa + 64 < lim_a ? (uint32_t)j * rb_a + pa + 64 : kOob;
      v2 = row_ok && pa + 128 < lim_a ? (uint32_t)j * rb_a + pa + 128 : kOob;
    }
    dst.c0 = ld4(r01, v0, s01);
    dst.c1 = ld4(r01, v1, s01);
    if constexpr (!I4) dst.c2 = ld4(r2, v2, s2);
  };

  // ---- prologue loads: x (16 bytes per item), anchor mask, anchor indices ----
  const int n_items = B * G * 4;  // (b, group, quarter)
  const auto r_x = rsrc(a.x, (uint32_t)((size_t)B * ldk * 2));
  const auto r_mask = rsrc(M.mask, M.mask ? (uint32_t)G * 4 : 0u);
  const auto r_idx = rsrc(M.idx, (uint32_t)M.n_out * 4);
  u32x4 xv[XI];
  uint32_t mk[XI];
  const bool has_mask = !I4 && M.mask != nullptr;
#pragma unroll
  for (int q = 0; q < XI; ++q) {
    xv[q] = u32x4{0, 0, 0, 0};
    mk[q] = 0;
    if (q * NT < n_items) {  // uniform; these are the wave's first loads
      const int it = q * NT + tid;
      const bool ok = it < n_items;
      const int bg = it >> 2, qt = it & 3;
      int b = 0;
#pragma unroll
      for (int t = 1; t < B; ++t) b += bg >= t * G;
      const int gr = bg - b * G;
      const uint32_t xoff = ok ? (uint32_t)((b * ldk + kbase + gr * 32 + qt * 8) * 2) : kOob;
      xv[q] = XC ? ld4_coherent(r_x, xoff, 0) : ld4(r_x, xoff, 0);
      if (has_mask) mk[q] = ld1(r_mask, ok ? (uint32_t)gr * 4 : kOob, 0);
    }
  }
  uint32_t aidx[IX];  // valid where q * NT + tid < n_out
#pragma unroll
  for (int q = 0; q < IX; ++q) {
    aidx[q] = 0;
    if (q * NT < M.n_out) {  // uniform
      const int o = q * NT + tid;
      // INT4: the anchors are the first n_out positions of x
      aidx[q] = I4 ? (uint32_t)o : ld1(r_idx, o < M.n_out ? (uint32_t)o * 4 : kOob, 0);
    }
  }
  // ---- weight prefetch: the first P steps (every ring load is
  //      unconditional, so the waits below count exactly) ----
  SlotT ring[P];
  Cursor cl = st.start(wave);
  __builtin_amdgcn_sched_barrier(0);
  constexpr int E = kEarly < P ? kEarly : P;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    issue(ring[i], cl);
    st.advance(cl);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- x preparation: limbs, coefficients, raw copy ----
  {
    const float C0 = -1.52f, C1 = -0.45f, C2 = 0.45f;
    const float d1 = C1 - C0, d3 = (C2 - C0) - 2.0f * d1;
#pragma unroll
    for (int q = 0; q < XI; ++q) {
      if (q * NT < n_items) {  // uniform: whole quads stay together
        const int it = q * NT + tid;
        const bool ok = it < n_items;
        const int bg = it >> 2, qt = it & 3;
        int b = 0;
#pragma unroll
      for (int t = 1; t < B; ++t) b += bg >= t * G;
      const int gr = bg - b * G;
        // channels read as zero: the anchors (their code is the zero level
        // for INT4, so zeroing them there changes no product)
        uint32_t om;
        if constexpr (I4) {
          const int na = M.n_out - (gr * 32 + qt * 8);  // INT4 launches are unsplit
          om = na >= 8 ? 0xFFu : (na <= 0 ? 0u : (1u << na) - 1u);
        } else {
          om = (mk[q] >> (qt * 8)) & 0xFFu;
        }
        uint32_t d[4] = {xv[q][0], xv[q][1], xv[q][2], xv[q][3]};
        if (ok && XR) {
          uint32_t *raw = reinterpret_cast<uint32_t *>(xraw + (size_t)b * KX + gr * 32 + qt * 8);
#pragma unroll
          for (int i = 0; i < 4; ++i) raw[i] = d[i];
        }
        float xf[8];
        float amax = 0.0f, xs = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t h = (d[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
          xf[i] = ((om >> i) & 1u) ? 0.0f : h2f(h);
          amax = fmaxf(amax, fabsf(xf[i]));
          xs += xf[i];
        }
        // the four quarters of a group are lanes 4m..4m+3
        amax = fmaxf(amax, dpp_f<0xB1, 0xF>(amax));
        amax = fmaxf(amax, dpp_f<0x4E, 0xF>(amax));
        xs += dpp_f<0xB1, 0xF>(xs);
        xs += dpp_f<0x4E, 0xF>(xs);
        const int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 8;
        const int sh = 8 - e;  // amax * 2^sh in [128, 256)
        float r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = __builtin_ldexpf(xf[i], sh);
        if constexpr (I4) {
          // element order: element 8qt+i at byte 8(qt&1)+i of half qt/2
          uint8_t *hb = limbs + ((size_t)(b * G + gr) * 3) * 32 + (qt >> 1) * 16 + 8 * (qt & 1);
#pragma unroll
          for (int lb = 0; lb < 3; ++lb) {
            const uint32_t w0 = to_fp8x4(r[0], r[1], r[2], r[3]);
            const uint32_t w1 = to_fp8x4(r[4], r[5], r[6], r[7]);
            if (ok) *reinterpret_cast<u32x2 *>(hb + lb * 32) = u32x2{w0, w1};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              r[i] -= fp8_at(w0, i);
              r[4 + i] -= fp8_at(w1, i);
            }
          }
          if (ok && qt == 0) {
            // sum x q = 2 (P_lo + 4 P_hi) - 8 X_g, P in units of 2^-sh
            const float inv = __builtin_ldexpf(1.0f, -sh);
            coef[b * G + gr] = make_float4(2.0f * inv, 0.0f, -8.0f * xs, xs);
          }
          continue;
        }
        // element 8qt+i sits in half qt/2 at byte (i even) 4(qt&1)+i/2 or
        // (i odd) 8+4(qt&1)+i/2
        uint8_t *hb = limbs + ((size_t)(b * G + gr) * 3) * 32 + (qt >> 1) * 16 + 4 * (qt & 1);
#pragma unroll
        for (int lb = 0; lb < 3; ++lb) {
          const uint32_t ev = to_fp8x4(r[0], r[2], r[4], r[6]);
          const uint32_t od = to_fp8x4(r[1], r[3], r[5], r[7]);
          if (ok) {
            *reinterpret_cast<uint32_t *>(hb + lb * 32) = ev;
            *reinterpret_cast<uint32_t *>(hb + lb * 32 + 8) = od;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            r[2 * i] -= fp8_at(ev, i);
            r[2 * i + 1] -= fp8_at(od, i);
          }
        }
        if (ok && qt == 0) {
          const float inv = __builtin_ldexpf(1.0f, -sh);
          coef[b * G + gr] = make_float4(2.0f * d1 * inv, d3 * inv, C0 * xs, xs);
        }
      }
    }
    if (tid < 8) reinterpret_cast<uint32_t *>(zero)[tid] = 0u;
    if (XR && tid < 8 * B) xraw[(tid >> 3) * KX + K + (tid & 7)] = 0;
#pragma unroll
    for (int q = 0; q < IX; ++q) {
      const int o = q * NT + tid;
      if (q * NT < a.xo_len && o < a.xo_len) aidx_l[o] = (int)aidx[q];
    }
  }
  // LDS-only barrier: the weight prefetch stays in flight
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
  for (int i = E; i < P; ++i) {
    issue(ring[i], cl);
    st.advance(cl);
  }

  // anchor x gathered once (zero past n_out; indices clamped to the zeros
  // at K), then a second LDS-only barrier (none without anchors)
  if (a.xo_len > 0) {  // uniform
    for (int o = tid; o < a.xo_len; o += NT) {
      // XR only for unsplit launches (ldk == K)
      const uint32_t ci = o < M.n_out ? min((uint32_t)aidx_l[o], (uint32_t)ldk) : (uint32_t)ldk;
      if (XR) {
#pragma unroll
        for (int b = 0; b < B; ++b) xo[b * a.xo_len + o] = xraw[(size_t)b * KX + ci];
      } else {
        // from global x: one 2-byte load per (row, anchor), all in flight;
        // past n_out an out-of-range offset reads zero
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const uint32_t off = ci < (uint32_t)ldk ? (uint32_t)(b * ldk + (int)ci) * 2u : kOob;
          xo[b * a.xo_len + o] =
              (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r_x, (int)off, 0, XC ? kCoherent : 0);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }

  // ---- per-lane A-operand addresses ----
  const int s_a = j >> 2, limb = j & 3;
  const bool a_ok = limb < 3 && ((g >> 1) == (s_a & 1));
  const int a_lane = (4 * s_a) * 96 + limb * 32 + (g & 1) * 16;  // plus 96 * chunk group
  const bool a_hi = (s_a >> 1) != 0;

  float acc[B];
#pragma unroll
  for (int b = 0; b < B; ++b) acc[b] = 0.0f;

  auto finish_unit = [&](int u) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      float v = acc[b];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane < 16) parts[((size_t)u * 16 + j) * B + b] = v;
      acc[b] = 0.0f;
    }
  };

  auto compute = [&](const SlotT &src, const Cursor &c) __attribute__((always_inline)) {
    const int split = c.split;
    if constexpr (I4) {
      if (c.step < L) {
        const int sc = split * L + c.step;
        // chunk ch: this lane's group 16 sc + 4g + ch (code words c_ch), its
        // nibbles split into the two e2m1 operands; chunks outermost, so
        // only one chunk's operands are live
        const uint8_t *p_lo = a_ok && !a_hi ? limbs + (size_t)(16 * sc) * 96 + a_lane : zero;
        const uint8_t *p_hi = a_ok && a_hi ? limbs + (size_t)(16 * sc) * 96 + a_lane : zero;
        const int st_lo = a_ok && !a_hi ? 96 : 0, st_hi = a_ok && a_hi ? 96 : 0;
        const int bst_lo = a_ok && !a_hi ? G * 96 : 0, bst_hi = a_ok && a_hi ? G * 96 : 0;
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
          const u32x4 cw = ch == 0 ? src.c0 : (ch == 1 ? src.c1 : (ch == 2 ? src.c2 : src.c3));
          const uint32_t w0 = cw[0], w1 = cw[1], w2 = cw[2], w3 = cw[3];
          const v8i blo = {(int)(w0 & 0x33333333u), (int)(w1 & 0x33333333u), (int)(w2 & 0x33333333u),
                           (int)(w3 & 0x33333333u), 0, 0, 0, 0};
          const v8i bhi = {(int)((w0 >> 2) & 0x33333333u), (int)((w1 >> 2) & 0x33333333u),
                           (int)((w2 >> 2) & 0x33333333u), (int)((w3 >> 2) & 0x33333333u), 0, 0, 0, 0};
          const uint32_t sw = src.sz[ch >> 1];
          const float S = h2f((ch & 1) ? (sw >> 16) : (sw & 0xFFFFu));
#pragma unroll
          for (int b = 0; b < B; ++b) {
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(p_lo + b * bst_lo + ch * st_lo);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(p_hi + b * bst_hi + ch * st_hi);
            const v8i A = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                           (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            const float4 cf = coef[b * G + 16 * sc + ch + 4 * g];
            v4f d = mfma_x_codes(A, blo);
            d = mfma_x_codes(A, bhi, d, 0x81);  // 2^2
            const float pu = (d[0] + d[1]) + d[2];
            acc[b] = __builtin_fmaf(S, __builtin_fmaf(pu, cf.x, cf.z), acc[b]);
          }
        }
        return;
      }
    }
    if (!I4 && c.step < L) {
      const int sc = split * L + c.step;
      // chunk ch covers groups 16 sc + ch + 4 s of slots s = 0..3; this
      // lane's codes and S/Z are those of slot g
      v8i bq[4], bh[4];
      float S[4], Z[4];
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        const u32x4 &cw = (ch >> 1) ? src.c1 : src.c0;
        const uint32_t c0 = cw[(ch & 1) * 2], c1 = cw[(ch & 1) * 2 + 1];
        const uint32_t c0s = c0 >> 2, c1s = c1 >> 2;
        bq[ch] = v8i{(int)(c0 & 0x33333333u), (int)(c0s & 0x33333333u),
                     (int)(c1 & 0x33333333u), (int)(c1s & 0x33333333u), 0, 0, 0, 0};
        bh[ch] = v8i{(int)(c0 & 0x22222222u), (int)(c0s & 0x22222222u),
                     (int)(c1 & 0x22222222u), (int)(c1s & 0x22222222u), 0, 0, 0, 0};
        const uint32_t szw = src.c2[ch];
        S[ch] = h2f(szw & 0xFFFFu);
        Z[ch] = h2f(szw >> 16);
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        // all operand and coefficient reads first, then the eight products,
        // then the epilogues: LDS and matrix-core latencies overlap
        const int gb = b * G + 16 * sc;
        const uint8_t *pa = limbs + (size_t)gb * 96 + a_lane;
        const uint8_t *p_lo = a_ok && !a_hi ? pa : zero;
        const uint8_t *p_hi = a_ok && a_hi ? pa : zero;
        const int st_lo = a_ok && !a_hi ? 96 : 0, st_hi = a_ok && a_hi ? 96 : 0;
        u32x4 lo[4], hi[4];
        float4 cf[4];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
          lo[ch] = *reinterpret_cast<const u32x4 *>(p_lo + ch * st_lo);
          hi[ch] = *reinterpret_cast<const u32x4 *>(p_hi + ch * st_hi);
        }
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) cf[ch] = coef[gb + ch + 4 * g];
        v4f dq[4], dh[4];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
          const v8i A = {(int)lo[ch][0], (int)lo[ch][1], (int)lo[ch][2], (int)lo[ch][3],
                         (int)hi[ch][0], (int)hi[ch][1], (int)hi[ch][2], (int)hi[ch][3]};
          dq[ch] = mfma_x_codes(A, bq[ch]);
          dh[ch] = mfma_x_codes(A, bh[ch]);
        }
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
          const float pq = (dq[ch][0] + dq[ch][1]) + dq[ch][2];
          const float ph = (dh[ch][0] + dh[ch][1]) + dh[ch][2];
          const float t = __builtin_fmaf(pq, cf[ch].x, __builtin_fmaf(ph, cf[ch].y, cf[ch].z));
          acc[b] = __builtin_fmaf(S[ch], t, acc[b]);
          acc[b] = __builtin_fmaf(Z[ch], cf[ch].w, acc[b]);
        }
      }
    } else {
      const int an = split + W * (c.step - L);
      // pieces taken field by field (a copy of part of the slot into an
      // array keeps the whole ring in private memory)
      auto piece = [&](const u32x4 pc, int i) __attribute__((always_inline)) {
        const int o = an * kAnchorChunk + 8 * (g + 4 * i);
        // o + 8 <= xo_len always (xo_len is a multiple of 96)
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const u32x4 xv4 = *reinterpret_cast<const u32x4 *>(xo + b * a.xo_len + o);
#pragma unroll
          for (int p = 0; p < 4; ++p) acc[b] = dot2(xv4[p], pc[p], acc[b]);
        }
      };
      piece(src.c0, 0);
      piece(src.c1, 1);
      piece(src.c2, 2);
    }
  };

  // Rounds of P steps: every round but the last refills each slot after
  // consuming it (unconditionally, so the waits count exactly; a refill past
  // the end reads through a zero-size descriptor); the last round only
  // drains the ring, so at most P - 1 refills per wave are dead.
  int n_steps = 0;
  for (int u = wave; u < n_units; u += NW) n_steps += st.unit_len(u % st.W);
  const int n_rounds = (n_steps + P - 1) / P;
  Cursor cc = st.start(wave);
  for (int r = 1; r < n_rounds; ++r) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const bool on = cc.unit < n_units;  // uniform
      const int u = cc.unit;
      const bool last = on && cc.step + 1 >= cc.len;
      if (on) compute(ring[i], cc);
      issue(ring[i], cl);
      st.advance(cl);
      if (on) st.advance(cc);
      if (last) finish_unit(u);
    }
  }
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const bool on = cc.unit < n_units;  // uniform
    const int u = cc.unit;
    const bool last = on && cc.step + 1 >= cc.len;
    if (on) compute(ring[i], cc);
    if (on) st.advance(cc);
    if (last) finish_unit(u);
  }

  // ---- partial row sums of every unit -> y, splits added in order ----
  __syncthreads();
  if (SW) {
    // gate row t0 * 16 + rl pairs with up row I + t0 * 16 + rl
    const int I = H * 16;
    const size_t esz = a.f32out ? 4 : 2;
    for (int t = tid; t < np * 16 * B; t += NT) {
      const int rl = t / B, b = t - rl * B;
      const int tl = rl >> 4, jj = rl & 15;
      float g = 0.0f, u = 0.0f;
      for (int sp = 0; sp < W; ++sp) {
        g += parts[((size_t)(tl * W + sp) * 16 + jj) * B + b];
        u += parts[((size_t)((np + tl) * W + sp) * 16 + jj) * B + b];
      }
      const float v = silu(g) * u;
      const size_t off = (size_t)b * I + t0 * 16 + rl;
      if (XC) {
        const auto ry = rsrc(M.y, (uint32_t)((size_t)B * I * esz));
        if (a.f32out)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ry, (int)(off * 4), 0, kCoherent);
        else
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)v), ry, (int)(off * 2), 0,
                                                kCoherent);
      } else if (a.f32out) {
        reinterpret_cast<float *>(M.y)[off] = v;
      } else {
        reinterpret_cast<_Float16 *>(M.y)[off] = (_Float16)v;
      }
    }
    return;
  }
  const int rows = (t1 - t0) * 16;
  for (int t = tid; t < rows * B; t += NT) {
    const int rl = t / B, b = t - rl * B;
    const int tl = rl >> 4, jj = rl & 15;
    const int row = t0 * 16 + rl;
    if (row >= M.N) continue;
    float v = 0.0f;
    for (int sp = 0; sp < W; ++sp) v += parts[((size_t)(tl * W + sp) * 16 + jj) * B + b];
    const size_t off = (size_t)b * M.N + row;
    if (XC) {  // written through to memory (y is a later stage's x)
      const auto ry = rsrc(M.y, (uint32_t)((size_t)B * M.N * (a.f32out ? 4 : 2)));
      if (a.f32out)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ry, (int)(off * 4), 0, kCoherent);
      else
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (_Float16)v), ry, (int)(off * 2), 0,
                                              kCoherent);
    } else if (a.f32out) {
      reinterpret_cast<float *>(M.y)[off] = v;
    } else {
      reinterpret_cast<_Float16 *>(M.y)[off] = (_Float16)v;
    }
  }
}

template <int B, int P, bool MULTI, bool XR = true, bool SW = false>
__global__ __launch_bounds__(kThreads) void kernel(Args a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  body<B, P, MULTI, false, XR, kThreads, SW>(a, (int)blockIdx.x, lds);
}

// The v3.2 INT4 format on the same body (one matrix, 3-slot ring, unsplit).
template <int B, bool XR>
__global__ __launch_bounds__(kThreads) void kernel_int4(Args a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  body<B, 3, false, false, XR, kThreads, false, true>(a, (int)blockIdx.x, lds);
}

// ---------------------------------------------------------------------------
// Fused decode stack: one persistent launch runs a sequence of grouped
// batch-1 GEMV stages (the projections of a decoder's layers in order), with
// a device-wide barrier between stages instead of a kernel boundary. The
// launch has one workgroup of 1024 threads (16 waves, as many as two
// 512-thread launches put on a CU) per CU, co-resident by cooperative
// launch; each stage is planned for at most one workgroup per CU and runs
// the matrix-core GEMV body.
constexpr int kStackThreads = 1024;

struct Stage {
  Args a;
  int grid;  // workgroups the stage was planned for (<= the launch's)
};

// A barrier wait gives up after this many polls (a quarter of a second or
// more) and sets the error word instead of hanging; the results are then
// invalid, and every later wait of the run returns at once.
constexpr uint32_t kSpinLimit = 1u << 18;

// Sync buffer (uint32): [0] error word, [1..15] unused, [16 + w] the arrival
// flag of workgroup w: the number of barriers it has passed in this run.
constexpr int kSyncFlags = 16;

// Device-wide barrier number `gen` (1, 2, ...) of a run. What crosses stages
// (each stage's y, the next stages' x) is stored and loaded with
// system-coherent buffer accesses (sc0 sc1: write-through to memory, and
// loads that miss every cache), so no cache needs a writeback or
// invalidation: a store is visible to every CU once it has completed, and a
// load issued after the barrier reads memory. Arrival: every thread waits
// until its stores have completed (vmcnt 0), the workgroup synchronizes,
// and one thread stores gen into the workgroup's own flag (a coherent
// store; no two workgroups write the same word, so nothing contends on a
// counter). Wait: wave 0 reads all flags, 64 lanes times four words per
// poll (coalesced), until every flag holds gen or more; the workgroup
// barrier after it releases the other waves.
__device__ inline void grid_sync(uint32_t *sync, uint32_t gen, int n_wg) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  const auto rf = rsrc(sync + kSyncFlags, (uint32_t)n_wg * 4u);
  if (threadIdx.x == 0)
    __builtin_amdgcn_raw_buffer_store_b32(gen, rf, (int)(blockIdx.x * 4u), 0, kCoherent);
  if (threadIdx.x < 64) {
    const uint32_t lane = threadIdx.x;
    const auto re = rsrc(sync, 4u);
    uint32_t n = 0;
    for (;;) {
      // after a timed-out wait (error word set) the run only drains
      const bool err = __builtin_amdgcn_raw_buffer_load_b32(re, 0, 0, kCoherent) != 0u;
      bool arrived = true;  // this lane's flags
      for (int i = 0; i < n_wg; i += 64) {  // uniform trip count
        // flags past n_wg read as 0 through the descriptor: count them as in
        const uint32_t f = __builtin_amdgcn_raw_buffer_load_b32(rf, (int)((i + lane) * 4u), 0, kCoherent);
        arrived = arrived && (f >= gen || i + (int)lane >= n_wg);
      }
      if (__builtin_amdgcn_ballot_w64(!(err || arrived)) == 0) break;  // wave-uniform exit
      if (++n >= kSpinLimit) {
        if (lane == 0)
          __builtin_amdgcn_raw_buffer_store_b32(1u, rsrc(sync, 4u), 0, 0, kCoherent);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
}

__global__ __launch_bounds__(kStackThreads) void stack_kernel(const Stage *__restrict__ stages, int n_stages,
                                                              uint32_t *sync) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int vb = (int)blockIdx.x;  // this workgroup's share of every stage
  for (int s = 0; s < n_stages; ++s) {
    if (vb < stages[s].grid) {
      if (stages[s].a.swiglu)
        body<1, 3, false, true, false, kStackThreads, true>(stages[s].a, vb, lds);
      else
        body<1, 3, true, true, false, kStackThreads>(stages[s].a, vb, lds);
    }
    __syncthreads();  // LDS is reused by the next stage
    grid_sync(sync, (uint32_t)(s + 1), (int)gridDim.x);
  }
}

__global__ void sync_reset_kernel(uint32_t *sync, int words) {
  for (int i = threadIdx.x; i < words; i += blockDim.x) sync[i] = 0u;
}

// ---------------------------------------------------------------------------
// host side

namespace {

template <int B, int P, bool MULTI, bool XR, bool SW = false>
qw_status launch_bpmx(const Args &a, int grid, size_t lds, hipStream_t s) {
  if (lds > 64 * 1024) {
    QW_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(&kernel<B, P, MULTI, XR, SW>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  }
  QW_HIP_TRY(launch(kernel<B, P, MULTI, XR, SW>, grid, kThreads, lds, s, a));
  return QW_OK;
}

// Without the raw x copy: wide batches that fit one pass only so, and every
// K-split launch (a part's LDS holds only its own channels of x).
template <int B, int P, bool MULTI>
qw_status launch_bpm(const Args &a, int grid, size_t lds, hipStream_t s) {
  if (!a.xraw) return launch_bpmx<B, P, MULTI, false>(a, grid, lds, s);
  return launch_bpmx<B, P, MULTI, true>(a, grid, lds, s);
}

template <int B, int P>
qw_status launch_bp(const Args &a, int grid, size_t lds, hipStream_t s) {
  if constexpr (P == 3) {  // the merged gate/up product runs on the 3-slot ring only
    if (a.swiglu)
      return a.xraw ? launch_bpmx<B, P, false, true, true>(a, grid, lds, s)
                    : launch_bpmx<B, P, false, false, true>(a, grid, lds, s);
  }
  return a.count > 1 ? launch_bpm<B, P, true>(a, grid, lds, s) : launch_bpm<B, P, false>(a, grid, lds, s);
}

template <int B>
qw_status launch_int4_b(const Args &a, int grid, size_t lds, hipStream_t s) {
  auto fn = a.xraw ? kernel_int4<B, true> : kernel_int4<B, false>;
  if (lds > 64 * 1024)
    QW_HIP_TRY(hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)lds));
  QW_HIP_TRY(launch(fn, grid, kThreads, lds, s, a));
  return QW_OK;
}

qw_status launch_int4_sel(const Args &a, int B, int grid, size_t lds, hipStream_t s) {
  switch (B) {
    case 1: return launch_int4_b<1>(a, grid, lds, s);
    case 2: return launch_int4_b<2>(a, grid, lds, s);
    case 3: return launch_int4_b<3>(a, grid, lds, s);
    case 4: return launch_int4_b<4>(a, grid, lds, s);
    case 5: return launch_int4_b<5>(a, grid, lds, s);
    case 6: return launch_int4_b<6>(a, grid, lds, s);
    case 7: return launch_int4_b<7>(a, grid, lds, s);
    default: return launch_int4_b<8>(a, grid, lds, s);
  }
}

// Ring depth: 3 slots, or the deep ring (6 slots up to batch 2, 4 beyond).
qw_status launch_b(const Args &a, int B, bool deep, int grid, size_t lds, hipStream_t s) {
  switch (B) {
    case 1: return deep ? launch_bp<1, 6>(a, grid, lds, s) : launch_bp<1, 3>(a, grid, lds, s);
    case 2: return deep ? launch_bp<2, 6>(a, grid, lds, s) : launch_bp<2, 3>(a, grid, lds, s);
    case 3: return deep ? launch_bp<3, 4>(a, grid, lds, s) : launch_bp<3, 3>(a, grid, lds, s);
    case 4: return deep ? launch_bp<4, 4>(a, grid, lds, s) : launch_bp<4, 3>(a, grid, lds, s);
    case 5: return deep ? launch_bp<5, 4>(a, grid, lds, s) : launch_bp<5, 3>(a, grid, lds, s);
    case 6: return deep ? launch_bp<6, 4>(a, grid, lds, s) : launch_bp<6, 3>(a, grid, lds, s);
    case 7: return deep ? launch_bp<7, 4>(a, grid, lds, s) : launch_bp<7, 3>(a, grid, lds, s);
    default: return deep ? launch_bp<8, 4>(a, grid, lds, s) : launch_bp<8, 3>(a, grid, lds, s);
  }
}

// Waves per tile: a divisor of the super-chunk count minimising the time of
// the busiest wave of a workgroup of nw waves holding `tw` tiles, with at
// most max_units units (tw * w) per workgroup.
int pick_splits(int tw, int sc, int nw, long max_units = 1L << 30) {
  int best = 1;
  long best_t = -1;
  for (int w = 1; w <= sc; ++w) {
    if (sc % w) continue;
    const long units = (long)tw * w;
    if (w > 1 && units > max_units) continue;
    const long t = ((units + nw - 1) / nw) * (sc / w);
    if (best_t < 0 || t < best_t) {
      best_t = t;
      best = w;
    }
  }
  return best;
}

}  // namespace

// Plans a grouped launch (Args for the whole batch, its grid); returns
// QW_ERR_UNSUPPORTED when the shape does not fit this kernel. With more
// workgroups wanted than ``budget``, the group's matrices share the budget
// in proportion to their tiles (a matrix alone is never cut).
// swiglu: ws[0] alone is a merged gate/up matrix (N = 2I, I % 16 == 0); its
// I / 16 tile pairs are dealt to up to 2 workgroups per CU (as many as the
// two matrices would take as a grouped launch), within ``budget``.
// batch > 0: a matrix whose whole batch would miss one pass only through
// the LDS buffer of partial row sums (many tiles per workgroup times many K
// splits) gets fewer splits so that it fits: the weights then stream once
// instead of once per batch slice (27648x5120 batch 8: two 4-row passes,
// 54.6 us, against one pass). Each matrix's splits depend on itself and the
// batch only, so grouped and separate launches keep giving the same bits.
static bool fits_whole(int B, int K, int xo_len, long units) {
  return (long)B * K <= (long)kXItems * kThreads * 8 &&
         (lds_layout(B, K, xo_len, (int)units, 1).total <= 160 * 1024 ||
          lds_layout(B, K, xo_len, (int)units, 0).total <= 160 * 1024);
}

static qw_status plan(const qw_weight *ws, int count, const uint16_t *x, void *const *ys, bool f32,
                      int cus, Args &a, int &grid, int budget = 1 << 30, int nt = kThreads,
                      bool swiglu = false, int batch = 0) {
  const int K = ws[0].K;
  if (K % 512 != 0 || count > kMats) return QW_ERR_UNSUPPORTED;
  if (swiglu && (count != 1 || ws[0].N % 32 != 0)) return QW_ERR_INVALID_ARG;
  int na_max = 0;
  for (int i = 0; i < count; ++i) {
    const int npad = ws[i].n_out > 0 ? ws[i].n_out_pad : 0;
    if ((size_t)ws[i].N * npad * 2 >= (1ull << 31)) return QW_ERR_UNSUPPORTED;
    na_max = max(na_max, (npad + kAnchorChunk - 1) / kAnchorChunk);
  }
  const int xo_len = na_max * kAnchorChunk;
  // the body gathers up to kIdxItems * kThreads anchors (per thread scaled
  // to the workgroup size)
  if (xo_len > kIdxItems * kThreads) return QW_ERR_UNSUPPORTED;
  const int SC = K / 512;
  a = Args{};
  a.count = count;
  a.x = x;
  a.K = K;
  a.ldk = K;
  a.f32out = f32 ? 1 : 0;
  a.xo_len = xo_len;
  a.xraw = 1;
  a.swiglu = swiglu ? 1 : 0;
  // every matrix is planned as if it were launched alone (its workgroup
  // count, hence its K split and summation order, do not depend on what it
  // is grouped with), so a grouped launch gives the bits of separate ones
  int units_max = 0;
  grid = 0;
  for (int i = 0; i < count; ++i) {
    Mat &m = a.m[i];
    m.codes = reinterpret_cast<const uint32_t *>(ws[i].codes);
    m.sz = reinterpret_cast<const uint32_t *>(ws[i].scales);
    m.mask = ws[i].n_out > 0 ? ws[i].out_mask : nullptr;
    m.idx = ws[i].out_idx;
    m.wo = ws[i].out_w;
    m.y = ys[i];
    m.N = ws[i].N;
    m.n_out = ws[i].n_out;
    m.n_out_pad = ws[i].n_out > 0 ? ws[i].n_out_pad : 0;
    m.ld_a = m.n_out_pad;
    m.tiles = (m.N + 15) / 16;
    m.wg_count = swiglu ? max(1, min(m.tiles / 2, min(2 * cus, budget))) : max(1, min(m.tiles, cus));
  }
  long want = 0, all_tiles = 0;
  for (int i = 0; i < count; ++i) {
    want += a.m[i].wg_count;
    all_tiles += a.m[i].tiles;
  }
  if (count > 1 && want > budget)
    for (int i = 0; i < count; ++i)
      a.m[i].wg_count = (int)max(1L, (long)budget * a.m[i].tiles / all_tiles);
  for (int i = 0; i < count; ++i) {
    Mat &m = a.m[i];
    m.wg_begin = grid;
    grid += m.wg_count;
    // tiles of the busiest workgroup (two per pair with swiglu)
    const int tw = swiglu ? 2 * ((m.tiles / 2 + m.wg_count - 1) / m.wg_count)
                          : (m.tiles + m.wg_count - 1) / m.wg_count;
    m.W = pick_splits(tw, SC, nt / 64);
    if (batch > 0) {
      const int npad = m.n_out_pad;
      const int xo_i = (npad + kAnchorChunk - 1) / kAnchorChunk * kAnchorChunk;
      long cap = (long)tw * m.W;
      if (!fits_whole(batch, K, xo_i, cap)) {
        while (cap > tw && !fits_whole(batch, K, xo_i, cap)) --cap;
        if (fits_whole(batch, K, xo_i, cap)) m.W = pick_splits(tw, SC, nt / 64, cap);
      }
    }
    units_max = max(units_max, tw * m.W);
  }
  a.units_max = units_max;
  for (int i = 0; i < count; ++i)
    if ((long)a.m[i].tiles * (a.m[i].wg_count + 1) >= (1L << 31)) return QW_ERR_UNSUPPORTED;
  return QW_OK;
}

// ---------------------------------------------------------------------------
// K split. A matrix's channels are cut into ks equal parts (whole super-chunks
// of 512) and its anchor chunks into ks runs; each part is one matrix of a
// grouped launch (up to kMats parts per launch, several launches beyond)
// whose rows are fp32 partial sums, written to a workspace; a last kernel
// adds the parts in order into y. It lets batches whose x (limbs for every
// row) does not fit one workgroup's LDS stream the weights once, instead of
// once per batch row through the vector-ALU kernel.

__global__ __launch_bounds__(256) void split_reduce_kernel(const float *parts, int ks, int n, void *y,
                                                           int f32) {
  const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (i >= n) return;
  float v = parts[i];
  for (int p = 1; p < ks; ++p) v += parts[(size_t)p * n + i];
  if (f32)
    reinterpret_cast<float *>(y)[i] = v;
  else
    reinterpret_cast<_Float16 *>(y)[i] = (_Float16)v;
}

namespace {

constexpr int kMaxSplit = 8;

bool fits_one_wg(int b, int K, int xo_len, int units_max, int xr) {
  return (long)b * K <= (long)kXItems * kThreads * 8 &&
         lds_layout(b, K, xo_len, units_max, xr).total <= 160 * 1024;
}

// Batch slices of an unsplit launch planned as `a` (0: none fits), and
// whether they keep the raw x copy. Without the raw x copy the whole batch
// may fit one pass (the weights stream once instead of once per slice); with
// it the anchor gather reads LDS instead of memory, so it is kept whenever
// the batch fits with it. Slices of one row are left to the vector-ALU
// kernel (faster there).
int unsplit_slices(const Args &a, int B, int *xraw, int *bmax_out) {
  int bmax = B;
  *xraw = 1;
  if (!fits_one_wg(B, a.K, a.xo_len, a.units_max, 1) && fits_one_wg(B, a.K, a.xo_len, a.units_max, 0)) {
    *xraw = 0;
  } else {
    while (bmax > 0 && !fits_one_wg(bmax, a.K, a.xo_len, a.units_max, 1)) --bmax;
  }
  *bmax_out = bmax;
  if (bmax < B && bmax < 2) return 0;
  return (B + bmax - 1) / bmax;
}

// Part p of ks: the weight view with its channels and its run of anchor
// chunks, planned alone; its Mat is a.m[0]. The parts of one launch share
// the CUs (each gets cus / parts-in-its-launch workgroups with
// proportionally more tiles), so every workgroup prepares x for its own part
// only; measured on MI355X, giving each part all the CUs instead (one
// workgroup per CU per part) made every launch prepare x parts times over:
// 5120x27648 at batches 2 / 4 / 8 ran 40 / 63 / 128 us against 22 / 30 / 62.
qw_status plan_part(const qw_weight &w, int ks, int p, const uint16_t *x, int cus, Args &a, int &grid) {
  qw_weight pw = w;
  pw.K = w.K / ks;
  void *dummy = nullptr;
  const int share = min(kMats, ks - (p / kMats) * kMats);  // parts in p's launch
  QW_TRY(plan(&pw, 1, x, &dummy, true, max(1, cus / share), a, grid));
  Mat &m = a.m[0];
  const int kp = pw.K;
  m.kbase = p * kp;
  m.codes += (size_t)p * kp / 16;
  m.sz += (size_t)p * kp / 32;
  if (m.mask) m.mask += (size_t)p * kp / 32;
  const int na = (m.ld_a + kAnchorChunk - 1) / kAnchorChunk;
  const int a0 = p * na / ks, a1 = (p + 1) * na / ks;
  m.abase = a0 * kAnchorChunk;
  m.n_out = max(0, min(m.n_out, a1 * kAnchorChunk) - m.abase);
  m.n_out_pad = max(0, min(m.n_out_pad, a1 * kAnchorChunk) - m.abase);
  if (m.n_out == 0) m.n_out_pad = 0;
  m.idx += m.abase;
  m.wo += m.abase;
  a.ldk = w.K;
  a.xraw = 0;
  a.f32out = 1;
  a.xo_len = (m.n_out_pad + kAnchorChunk - 1) / kAnchorChunk * kAnchorChunk;
  return QW_OK;
}

// K parts for one matrix at batch B: 1 = unsplit, 0 = this kernel does not
// take the shape. Measured on MI355X:
//  * the split pays where no unsplit pass of two or more batch rows fits;
//    shapes that fit whole ran as fast or faster whole at batches 2-4 (the
//    parts add a launch and a reduction), and at batch 1 the parts were no
//    faster than the vector-ALU kernel on 5120x27648 (19.2 us in 3 parts);
//  * among the part counts that fit: the fewest launches (kMats parts per
//    launch), then the most parts (5120x27648 batch 2: 21.7 us in 3 parts,
//    26.6 in 2, 30.6 in 6; 8192x28672 batch 8: 71.9 us in 8, 82.2 in 7).
// The test hook QW_TUNE_GEMV2_SPLIT = n forces n parts where n is valid.
int choose_split_uncached(const qw_weight &w, int B, int cus, int forced) {
  const int K = w.K;
  if (K % 512 != 0) return 0;
  Args a;
  int grid = 0;
  void *dummy = nullptr;
  if (plan(&w, 1, nullptr, &dummy, true, cus, a, grid, 1 << 30, kThreads, false, B) != QW_OK) return 0;
  int xr = 1, bmax = 0;
  const int ns = unsplit_slices(a, B, &xr, &bmax);
  if (ns > 0 && forced <= 1) return 1;
  const int SC = K / 512;
  int best = 0;
  for (int ks = 2; ks <= kMaxSplit; ++ks) {
    if (SC % ks != 0) continue;
    // every part must fit (their anchor runs differ by up to one chunk)
    bool fit = true;
    for (int p = 0; p < ks && fit; ++p) {
      Args ap;
      int gp = 0;
      fit = plan_part(w, ks, p, nullptr, cus, ap, gp) == QW_OK &&
            fits_one_wg(B, ap.K, ap.xo_len, ap.units_max, 0);
    }
    if (!fit) continue;
    if (forced == ks) return ks;
    // ks grows: it replaces best unless it needs more launches
    if (best == 0 || (ks + kMats - 1) / kMats == (best + kMats - 1) / kMats) best = ks;
  }
  if (ns > 0) return 1;  // a forced count that does not apply
  return best;
}

// The choice depends on the shape only, so it is planned once per shape
// (a small table, replaced round-robin) instead of on every call.
struct SplitKey {
  int N, K, n_out, n_out_pad, B, cus, forced;
  bool operator==(const SplitKey &o) const {
    return N == o.N && K == o.K && n_out == o.n_out && n_out_pad == o.n_out_pad && B == o.B &&
           cus == o.cus && forced == o.forced;
  }
};
constexpr int kSplitCache = 64;
struct SplitCache {
  std::mutex mu;
  SplitKey key[kSplitCache];
  int ks[kSplitCache];
  int used = 0, next = 0;
};
SplitCache g_split;

int choose_split(const qw_weight &w, int B, int cus) {
  const int forced = tune(QW_TUNE_GEMV2_SPLIT);
  const SplitKey k{w.N, w.K, w.n_out, w.n_out > 0 ? w.n_out_pad : 0, B, cus, forced};
  {
    std::lock_guard<std::mutex> lock(g_split.mu);
    for (int i = 0; i < g_split.used; ++i)
      if (g_split.key[i] == k) return g_split.ks[i];
  }
  const int ks = choose_split_uncached(w, B, cus, forced);
  std::lock_guard<std::mutex> lock(g_split.mu);
  const int slot = g_split.used < kSplitCache ? g_split.used++ : (g_split.next++ % kSplitCache);
  g_split.key[slot] = k;
  g_split.ks[slot] = ks;
  return ks;
}

bool deep_ring() {
  // 3 ring slots per wave: measured on MI355X, the deep ring (6 slots up to
  // batch 2, 4 beyond) is slower with weights coming from HBM even for waves
  // with many steps; the test hook QW_TUNE_GEMV2_DEEP_RING = 1 selects it
  // (tests check both give the same bits)
  return tune(QW_TUNE_GEMV2_DEEP_RING) == 1;
}

// fp32 partial rows of ks parts at batch B
size_t split_bytes(const qw_weight &w, int ks, int B) { return (size_t)ks * B * w.N * sizeof(float); }

// The parts write their fp32 partial rows to ``parts`` (the caller's
// workspace, split_bytes long); the reduction adds them in part order.
qw_status launch_split(const qw_weight &w, int ks, const uint16_t *x, int B, void *y, bool f32, int cus,
                       float *parts, hipStream_t s) {
  const size_t plane = (size_t)B * w.N;
  if (plane > (size_t)INT32_MAX) return QW_ERR_UNSUPPORTED;  // int indices in the reduction
  Args parts_a[kMaxSplit];
  int grid_p[kMaxSplit];
  for (int p = 0; p < ks; ++p) QW_TRY(plan_part(w, ks, p, x, cus, parts_a[p], grid_p[p]));
  const bool deep = deep_ring();
  qw_status st = QW_OK;
  for (int p0 = 0; p0 < ks && st == QW_OK; p0 += kMats) {
    Args a = parts_a[p0];
    a.count = min(kMats, ks - p0);
    int xo_len = 0;
    for (int i = 0; i < a.count; ++i) {
      a.m[i] = parts_a[p0 + i].m[0];
      a.m[i].y = parts + (size_t)(p0 + i) * plane;
      a.m[i].wg_begin = i * grid_p[p0];
      xo_len = max(xo_len, parts_a[p0 + i].xo_len);
    }
    a.xo_len = xo_len;
    const size_t lds = lds_layout(B, a.K, a.xo_len, a.units_max, 0).total;
    st = launch_b(a, B, deep, grid_p[p0] * a.count, lds, s);
  }
  if (st == QW_OK &&
      launch(split_reduce_kernel, (unsigned)((plane + 255) / 256), 256, 0, s, (const float *)parts, ks,
             (int)plane, y, f32 ? 1 : 0) != hipSuccess)
    st = QW_ERR_HIP;
  return st;
}

}  // namespace

// Workspace bytes of a K-split call of w at batch B (0: runs unsplit or not
// on this kernel).
size_t split_workspace_bytes(const qw_weight &w, int B, int cus) {
  if (B < 1 || B > 8) return 0;
  const int ks = choose_split(w, B, cus);
  return ks > 1 ? split_bytes(w, ks, B) : 0;
}

// Returns QW_ERR_UNSUPPORTED (nothing enqueued) when the shape does not fit
// this kernel, or needs K parts and ``work`` (the caller's workspace of
// work_bytes) cannot hold their partial rows; the caller then uses the
// vector-ALU kernel. A grouped call whose matrices would be split alone is
// refused too (the caller then launches them one by one), so that it gives
// the bits of separate calls.
qw_status launch(const qw_weight *ws, int count, const uint16_t *x, int B, void *const *ys,
                 bool f32, int cus, float *work, size_t work_bytes, hipStream_t s) {
  if (B < 1 || B > 8) return QW_ERR_UNSUPPORTED;
  for (int i = 0; i < count; ++i) {
    const int ks = choose_split(ws[i], B, cus);
    if (ks == 0) return QW_ERR_UNSUPPORTED;
    if (ks > 1) {
      if (count != 1 || !work || work_bytes < split_bytes(ws[0], ks, B)) return QW_ERR_UNSUPPORTED;
      return launch_split(ws[0], ks, x, B, ys[0], f32, cus, work, s);
    }
  }
  const int K = ws[0].K;
  Args a;
  int grid = 0;
  QW_TRY(plan(ws, count, x, ys, f32, cus, a, grid, 1 << 30, kThreads, false, B));
  // Widest batch slice whose x (limbs in LDS, raw x in the prologue
  // registers) fits. Batch rows are independent (each is its own row of the
  // product's A operand), so slicing changes no bits.
  int xr = 1, bmax = 0;
  const int n_slices = unsplit_slices(a, B, &xr, &bmax);
  if (n_slices == 0) return QW_ERR_UNSUPPORTED;
  a.xraw = xr;
  const bool deep = deep_ring();
  const size_t esz = f32 ? 4 : 2;
  int b0 = 0;
  for (int sl = 0; sl < n_slices; ++sl) {
    const int bs = (B - b0 + (n_slices - sl) - 1) / (n_slices - sl);  // balanced slices
    Args as = a;
    as.x = x + (size_t)b0 * K;
    for (int i = 0; i < count; ++i)
      as.m[i].y = reinterpret_cast<char *>(ys[i]) + (size_t)b0 * ws[i].N * esz;
    const size_t lds = lds_layout(bs, K, a.xo_len, a.units_max, a.xraw).total;
    QW_TRY(launch_b(as, bs, deep, grid, lds, s));
    b0 += bs;
  }
  return QW_OK;
}

// The merged gate/up product with the gated activation (y: [B][N / 2]):
// unsplit launches only, in balanced batch slices as above. Returns
// QW_ERR_UNSUPPORTED when no slice of two or more rows, nor of one, fits.
qw_status launch_swiglu(const qw_weight &w, const uint16_t *x, int B, void *y, bool f32, int cus,
                        hipStream_t s) {
  if (B < 1 || B > 8) return QW_ERR_UNSUPPORTED;
  const int K = w.K;
  Args a;
  int grid = 0;
  void *ys[1] = {y};
  QW_TRY(plan(&w, 1, x, ys, f32, cus, a, grid, 1 << 30, kThreads, true, B));
  int xr = 1, bmax = 0;
  int n_slices = unsplit_slices(a, B, &xr, &bmax);
  if (n_slices == 0 && bmax == 1) n_slices = B;  // one row at a time
  if (n_slices == 0) return QW_ERR_UNSUPPORTED;
  a.xraw = xr;
  const size_t esz = f32 ? 4 : 2;
  int b0 = 0;
  for (int sl = 0; sl < n_slices; ++sl) {
    const int bs = (B - b0 + (n_slices - sl) - 1) / (n_slices - sl);
    Args as = a;
    as.x = x + (size_t)b0 * K;
    as.m[0].y = reinterpret_cast<char *>(y) + (size_t)b0 * (w.N / 2) * esz;
    const size_t lds = lds_layout(bs, K, a.xo_len, a.units_max, a.xraw).total;
    QW_TRY(launch_b(as, bs, false, grid, lds, s));
    b0 += bs;
  }
  return QW_OK;
}

// The INT4 (v3.2) decode GEMV on the matrix cores (y: [B][N]), unsplit, in
// balanced batch slices as above. Returns QW_ERR_UNSUPPORTED (nothing
// enqueued) when the shape does not fit (K not a multiple of 512, more
// anchors than the gather takes, no slice of two or more rows fits); the
// caller then uses the vector-ALU kernel. The caller has validated the
// view and checked N * K / 2 < 2^31.
qw_status launch_int4(const qw_weight &w, const uint16_t *x, int B, void *y, bool f32, int cus,
                      hipStream_t s) {
  if (B < 1 || B > 8) return QW_ERR_UNSUPPORTED;
  const int K = w.K;
  Args a;
  int grid = 0;
  void *ys[1] = {y};
  QW_TRY(plan(&w, 1, x, ys, f32, cus, a, grid, 1 << 30, kThreads, false, B));
  a.m[0].mask = nullptr;  // anchors: the first n_out positions
  a.m[0].idx = nullptr;
  int xr = 1, bmax = 0;
  const int n_slices = unsplit_slices(a, B, &xr, &bmax);
  if (n_slices == 0) return QW_ERR_UNSUPPORTED;
  a.xraw = xr;
  const size_t esz = f32 ? 4 : 2;
  int b0 = 0;
  for (int sl = 0; sl < n_slices; ++sl) {
    const int bs = (B - b0 + (n_slices - sl) - 1) / (n_slices - sl);
    Args as = a;
    as.x = x + (size_t)b0 * K;
    as.m[0].y = reinterpret_cast<char *>(y) + (size_t)b0 * w.N * esz;
    const size_t lds = lds_layout(bs, K, a.xo_len, a.units_max, a.xraw).total;
    QW_TRY(launch_int4_sel(as, bs, grid, lds, s));
    b0 += bs;
  }
  return QW_OK;
}

}  // namespace gemv2m
}  // namespace qw

// ---------------------------------------------------------------------------
extern "C" {

size_t qw_stack_sync_bytes(const qw_stack *st) {
  if (!st || st->grid < 1) return 0;
  return (size_t)(qw::gemv2m::kSyncFlags + st->grid) * sizeof(uint32_t);
}

size_t qw_stack_plan_bytes(int n_stages) {
  if (n_stages < 1 || n_stages > QW_STACK_MAX_STAGES) return 0;
  return (size_t)n_stages * sizeof(qw::gemv2m::Stage);
}

qw_status qw_stack_prepare(const qw_stack_stage *stages, int n_stages, void *plan, qw_stack *out) {
  using namespace qw;
  using namespace qw::gemv2m;
  if (!stages || !plan || !out || n_stages < 1 || n_stages > QW_STACK_MAX_STAGES) return QW_ERR_INVALID_ARG;
  if (!aligned16(plan)) return QW_ERR_ALIGNMENT;
  int cus = 0;
  QW_TRY(current_device(&cus));
  std::vector<Stage> host((size_t)n_stages);
  size_t lds_max = 0;
  for (int i = 0; i < n_stages; ++i) {
    const qw_stack_stage &sg = stages[i];
    if (sg.count < 1 || sg.count > kMats || !sg.x) return QW_ERR_INVALID_ARG;
    if (sg.swiglu != 0 && sg.swiglu != 1) return QW_ERR_INVALID_ARG;
    if (sg.swiglu && (sg.count != 1 || sg.w[0].N % 32 != 0)) return QW_ERR_INVALID_ARG;
    if (sg.y_dtype != QW_DT_F16 && sg.y_dtype != QW_DT_F32) return QW_ERR_INVALID_ARG;
    if (!aligned16(sg.x)) return QW_ERR_ALIGNMENT;
    for (int m = 0; m < sg.count; ++m) {
      QW_TRY(check_weight_view(&sg.w[m], QW_FMT_2BIT_G32, sg.w[0].K));
      if (!sg.y[m]) return QW_ERR_INVALID_ARG;
      if (!aligned16(sg.y[m])) return QW_ERR_ALIGNMENT;
    }
    int grid = 0;
    QW_TRY(qw::gemv2m::plan(sg.w, sg.count, reinterpret_cast<const uint16_t *>(sg.x), sg.y, sg.y_dtype == QW_DT_F32,
                cus, host[i].a, grid, cus, kStackThreads, sg.swiglu != 0));
    host[i].a.xraw = 0;  // anchors gathered from global x
    const int K = sg.w[0].K;
    if ((long)K > (long)kXItems * kThreads * 8) return QW_ERR_UNSUPPORTED;
    const size_t lds = lds_layout(1, K, host[i].a.xo_len, host[i].a.units_max, 0).total;
    if (lds > 160 * 1024) return QW_ERR_UNSUPPORTED;
    lds_max = max(lds_max, lds);
    host[i].grid = grid;
  }

  QW_HIP_TRY(hipMemcpy(plan, host.data(), host.size() * sizeof(Stage), hipMemcpyHostToDevice));
  out->plan = plan;
  out->n_stages = n_stages;
  out->grid = cus;
  out->lds = (int32_t)lds_max;
  return QW_OK;
}

qw_status qw_stack_run(const qw_stack *st, uint32_t *sync, void *stream) {
  using namespace qw;
  using namespace qw::gemv2m;
  CallScope scope;
  if (!st || !st->plan || !sync || st->n_stages < 1 || st->n_stages > QW_STACK_MAX_STAGES) return QW_ERR_INVALID_ARG;
  if (st->grid < 1 || st->lds < 0 || st->lds > 160 * 1024) return QW_ERR_INVALID_ARG;
  if (!aligned16(sync)) return QW_ERR_ALIGNMENT;
  int cus = 0;
  QW_TRY(current_device(&cus));
  if (st->grid != cus) return QW_ERR_INVALID_ARG;  // prepared for another device
  hipStream_t s = as_stream(stream);
  const void *fn = reinterpret_cast<const void *>(&stack_kernel);
  if (st->lds > 64 * 1024) QW_HIP_TRY(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, st->lds));
  QW_HIP_TRY(launch(sync_reset_kernel, 1, 256, 0, s, sync, kSyncFlags + st->grid));
  const Stage *plan_p = reinterpret_cast<const Stage *>(st->plan);
  int n = st->n_stages;
  uint32_t *sync_p = sync;
  void *args[] = {(void *)&plan_p, (void *)&n, (void *)&sync_p};
  // cooperative: every workgroup resident at once, or the launch fails
  QW_HIP_TRY(launch_cooperative_raw(fn, dim3(st->grid), dim3(kStackThreads), args, (size_t)st->lds, s));
  return QW_OK;
}

}  // extern "C"
