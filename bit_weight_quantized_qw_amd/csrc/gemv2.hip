// Host side of the 2-bit decode GEMV: validation, work split, dispatch.
// The kernel itself (and the decode scheme) is in gemv2_kernel.h.
#include <mutex>

#include "gemv2_kernel.h"

// Scratch of qgemv_2bit_static: the K-split partial rows of callers that
// cannot allocate. Every GPU the library runs on holds its own copy until
// the process ends. In host code this name stands for the array only as a
// symbol: its device address (per device) comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[QW_STATIC_SCRATCH_BYTES];

namespace qw {
namespace gemv2m {
qw_status launch(const qw_weight *ws, int count, const uint16_t *x, int B, void *const *ys,
                 bool f32, int cus, float *work, size_t work_bytes, hipStream_t s);
size_t split_workspace_bytes(const qw_weight &w, int B, int cus);
qw_status launch_swiglu(const qw_weight &w, const uint16_t *x, int B, void *y, bool f32, int cus,
                        hipStream_t s);
}  // namespace gemv2m

namespace gemv2 {
namespace {

int max_uw(int B) { return B == 1 ? 8 : (B == 2 ? 3 : 2); }

// Launch geometry for one batch slice of width Bk.
struct Plan {
  int W, UW, UA, threads, grid;
  size_t lds;
};

// Returns false when this width does not fit (waves or LDS).
bool plan_slice(const qw_weight *ws, int count, int Bk, int cus, Plan *p, int *rows_per_wg_out,
                int *wg_begin_out) {
  const int K = ws[0].K;
  const int KD = K / 16;
  const int U = (KD + 63) / 64;  // 64-lane dword iterations per row
  const int W = (U + max_uw(Bk) - 1) / max_uw(Bk);
  if (W > kMaxWaves) return false;
  const int UW = (U + W - 1) / W;
  long total_rows = 0;
  int ka_max = 0;
  for (int i = 0; i < count; ++i) {
    total_rows += ws[i].N;
    if (ws[i].n_out > 0) ka_max = max(ka_max, ws[i].n_out_pad / 2);
  }
  const int ua_need = (ka_max + 64 * W - 1) / (64 * W);
  if (ua_need > 4) return false;
  const int UA = ua_need == 0 ? 0 : (ua_need <= 2 ? 2 : 4);
  const int V = kMaxWaves / W;
  const int threads = 64 * W * V;
  // one workgroup per CU
  const long target_wgs = max(1L, (long)cus);
  const int rpg = (int)max(1L, (total_rows + target_wgs - 1) / target_wgs);
  int grid = 0;
  for (int i = 0; i < count; ++i) {
    wg_begin_out[i] = grid;
    rows_per_wg_out[i] = rpg;
    grid += (ws[i].N + rpg - 1) / rpg;
  }
  const size_t lds = lds_bytes(Bk, K, rpg, W);
  if (lds > 160 * 1024) return false;
  const int xu = Bk == 1 ? x_units_per_thread<1>() : (Bk == 2 ? x_units_per_thread<2>()
                                                              : x_units_per_thread<4>());
  if (KD > xu * threads) return false;
  *p = Plan{W, UW, UA, threads, grid, lds};
  return true;
}

// One launch for batch width Bk in {1, 2, 4}; x and ys already point at the
// first batch row of this slice (rows keep stride K and N).
qw_status launch_slice(const qw_weight *ws, int count, const uint16_t *x, int Bk,
                       void *const *ys, bool f32, const Plan &p, const int *rows_per_wg,
                       const int *wg_begin, hipStream_t s) {
  Args a{};
  a.count = count;
  a.x = x;
  a.K = ws[0].K;
  a.W = p.W;
  a.f32out = f32 ? 1 : 0;
  for (int i = 0; i < count; ++i) {
    Mat &m = a.m[i];
    m.codes = reinterpret_cast<const uint32_t *>(ws[i].codes);
    m.sz = reinterpret_cast<const uint32_t *>(ws[i].scales);
    m.mask = ws[i].n_out > 0 ? ws[i].out_mask : nullptr;
    m.idx = ws[i].out_idx;
    m.wo = reinterpret_cast<const uint32_t *>(ws[i].out_w);
    m.y = ys[i];
    m.N = ws[i].N;
    m.n_out = ws[i].n_out;
    m.n_out_pad = ws[i].n_out > 0 ? ws[i].n_out_pad : 0;
    m.wg_begin = wg_begin[i];
    m.rows_per_wg = rows_per_wg[i];
  }
  switch (Bk) {
    case 1: return launch_b1(a, p.UW, p.UA, p.grid, p.threads, p.lds, s);
    case 2: return launch_b2(a, p.UW, p.UA, p.grid, p.threads, p.lds, s);
    default: return launch_b4(a, p.UW, p.UA, p.grid, p.threads, p.lds, s);
  }
}

qw_status launch_valu(const qw_weight *ws, int count, const uint16_t *x, int B, void *const *ys,
                      bool f32, int cus, hipStream_t s);

// Argument checks shared by the entry points (and the workspace query).
qw_status check_args(const qw_weight *ws, int count, int B) {
  if (!ws || count < 1 || count > kMaxMats) return QW_ERR_INVALID_ARG;
  if (B < 1 || B > 8) return QW_ERR_INVALID_ARG;
  const int K = ws[0].K;
  for (int i = 0; i < count; ++i) {
    qw_status st = check_weight_view(&ws[i], QW_FMT_2BIT_G32, K);
    if (st != QW_OK) return st;
    // buffer offsets are 32-bit
    if ((size_t)ws[i].N * (ws[i].K / 4) >= (1ull << 31)) return QW_ERR_UNSUPPORTED;
  }
  return QW_OK;
}

// work / work_bytes: the caller's K-split workspace (NULL / 0: none).
qw_status launch(const qw_weight *ws, int count, const void *x, int B, void *const *ys,
                 qw_dtype dt, void *work, size_t work_bytes, hipStream_t s) {
  QW_TRY(check_args(ws, count, B));
  if (!x || !ys) return QW_ERR_INVALID_ARG;
  if (dt != QW_DT_F16 && dt != QW_DT_F32) return QW_ERR_INVALID_ARG;
  if (work_bytes > 0 && !work) return QW_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    if (!ys[i]) return QW_ERR_INVALID_ARG;
    if (!aligned16(ys[i])) return QW_ERR_ALIGNMENT;
  }
  if (!aligned16(x) || !aligned16(work)) return QW_ERR_ALIGNMENT;
  int cus = 0;
  qw_status st = current_device(&cus);
  if (st != QW_OK) return st;
  const int K = ws[0].K;
  const bool f32 = dt == QW_DT_F32;
  // the matrix-core kernel takes the whole batch in one pass when the shape
  // fits it; otherwise batch rows go through vector-ALU kernels of width 4,
  // 2 and 1 (e.g. 7 = 4 + 2 + 1).
  // Path choice (measured on MI355X): the matrix-core kernel for batches of
  // two or more, and at batch 1 for K <= 8192; beyond, at batch 1, for
  // matrices whose 16-row tiles spread evenly over the CUs (at least 3/4 of
  // the slots of the busiest round filled: 4096 or 8192 rows on 256 CUs),
  // the vector-ALU kernel (which splits rows, not tiles) otherwise (5120
  // rows: 320 tiles). The test hook QW_TUNE_GEMV2_PATH = 1 forces the
  // vector-ALU kernel and 0 the matrix-core one where it applies.
  // The choice is made per matrix (a grouped call gives the bits of
  // separate calls): the matrices that take the matrix-core kernel go out as
  // one grouped launch of it (or one by one when the group does not fit it),
  // the rest as grouped launches of the vector-ALU kernel.
  const int force = tune(QW_TUNE_GEMV2_PATH);
  qw_weight mc_w[kMaxMats], va_w[kMaxMats];
  void *mc_y[kMaxMats], *va_y[kMaxMats];
  int n_mc = 0, n_va = 0;
  for (int i = 0; i < count; ++i) {
    const long tiles = (ws[i].N + 15) / 16, wgs = max(1L, min(tiles, (long)cus));
    const long slots = (tiles + wgs - 1) / wgs * wgs;
    const bool balanced = 4 * tiles >= 3 * slots;
    const bool mc = force == 0 || (force < 0 && (B >= 2 || K <= 8192 || balanced));
    if (mc) {
      mc_w[n_mc] = ws[i];
      mc_y[n_mc++] = ys[i];
    } else {
      va_w[n_va] = ws[i];
      va_y[n_va++] = ys[i];
    }
  }
  const uint16_t *xh = reinterpret_cast<const uint16_t *>(x);
  if (n_mc > 0) {
    float *wk = reinterpret_cast<float *>(work);
    st = gemv2m::launch(mc_w, n_mc, xh, B, mc_y, f32, cus, wk, work_bytes, s);
    if (st == QW_ERR_UNSUPPORTED) {
      for (int i = 0; i < n_mc; ++i) {
        st = gemv2m::launch(&mc_w[i], 1, xh, B, &mc_y[i], f32, cus, wk, work_bytes, s);
        if (st == QW_ERR_UNSUPPORTED) {
          va_w[n_va] = mc_w[i];
          va_y[n_va++] = mc_y[i];
        } else if (st != QW_OK) {
          return st;
        }
      }
    } else if (st != QW_OK) {
      return st;
    }
  }
  if (n_va == 0) return QW_OK;
  return launch_valu(va_w, n_va, xh, B, va_y, f32, cus, s);
}

// Vector-ALU kernels over the whole batch: slices of width 4, 2 and 1
// (narrower when the x slice of a wider one does not fit).
qw_status launch_valu(const qw_weight *ws, int count, const uint16_t *x, int B, void *const *ys,
                      bool f32, int cus, hipStream_t s) {
  const int K = ws[0].K;
  const size_t esz = f32 ? 4 : 2;
  qw_status st = QW_OK;
  int b0 = 0;
  while (b0 < B) {
    const int rest = B - b0;
    int Bk = rest >= 4 ? 4 : (rest >= 2 ? 2 : 1);
    Plan p;
    int rpg[kMaxMats], wgb[kMaxMats];
    while (!plan_slice(ws, count, Bk, cus, &p, rpg, wgb)) {
      if (Bk == 1) return QW_ERR_UNSUPPORTED;
      Bk >>= 1;
    }
    void *ysl[kMaxMats];
    for (int i = 0; i < count; ++i)
      ysl[i] = reinterpret_cast<char *>(ys[i]) + (size_t)b0 * ws[i].N * esz;
    st = launch_slice(ws, count, x + (size_t)b0 * K, Bk, ysl, f32, p, rpg, wgb, s);
    if (st != QW_OK) return st;
    b0 += Bk;
  }
  return QW_OK;
}

}  // namespace
}  // namespace gemv2
}  // namespace qw

extern "C" {

qw_status qgemv_2bit(const qw_weight *w, const void *x, int B, void *y, qw_dtype y_dtype,
                     void *stream) {
  qw::CallScope scope;
  void *ys[1] = {y};
  return qw::gemv2::launch(w, 1, x, B, ys, y_dtype, nullptr, 0, qw::as_stream(stream));
}

qw_status qgemv_2bit_ws(const qw_weight *w, const void *x, int B, void *y, qw_dtype y_dtype,
                        void *workspace, size_t workspace_bytes, void *stream) {
  qw::CallScope scope;
  void *ys[1] = {y};
  return qw::gemv2::launch(w, 1, x, B, ys, y_dtype, workspace, workspace_bytes, qw::as_stream(stream));
}

qw_status qgemv_2bit_workspace_bytes(const qw_weight *w, int B, size_t *bytes) {
  using namespace qw;
  if (!bytes) return QW_ERR_INVALID_ARG;
  QW_TRY(gemv2::check_args(w, 1, B));
  int cus = 0;
  QW_TRY(current_device(&cus));
  // the vector-ALU path (forced by the test hook, or K % 512 != 0) needs none
  *bytes = tune(QW_TUNE_GEMV2_PATH) == 1 ? 0 : gemv2m::split_workspace_bytes(*w, B, cus);
  return QW_OK;
}

// Device address of ``scratch`` on the current device, looked up once per
// device (with that device current) and kept.
static qw_status static_scratch(void **out) {
  static std::mutex mu;
  static void *addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return QW_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QW_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return QW_OK;
}

qw_status qgemv_2bit_static(const qw_weight *w, const void *x, int B, void *y, qw_dtype y_dtype,
                            void *stream) {
  using namespace qw;
  CallScope scope;
  size_t need = 0;
  QW_TRY(qgemv_2bit_workspace_bytes(w, B, &need));
  if (need > (size_t)QW_STATIC_SCRATCH_BYTES) return QW_ERR_SCRATCH_LIMIT;
  void *ws = nullptr;
  if (need > 0) QW_TRY(static_scratch(&ws));
  void *ys[1] = {y};
  return gemv2::launch(w, 1, x, B, ys, y_dtype, ws, need, as_stream(stream));
}

qw_status qgemv_2bit_swiglu(const qw_weight *w, const void *x, int B, void *y, qw_dtype y_dtype,
                            void *stream) {
  using namespace qw;
  CallScope scope;
  QW_TRY(gemv2::check_args(w, 1, B));
  if (!x || !y) return QW_ERR_INVALID_ARG;
  if (y_dtype != QW_DT_F16 && y_dtype != QW_DT_F32) return QW_ERR_INVALID_ARG;
  if (w->N % 32 != 0) return QW_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y)) return QW_ERR_ALIGNMENT;
  int cus = 0;
  QW_TRY(current_device(&cus));
  return gemv2m::launch_swiglu(*w, reinterpret_cast<const uint16_t *>(x), B, y, y_dtype == QW_DT_F32, cus,
                               as_stream(stream));
}

qw_status qgemv_2bit_grouped(const qw_weight *ws, int count, const void *x, int B,
                             void *const *ys, qw_dtype y_dtype, void *stream) {
  qw::CallScope scope;
  return qw::gemv2::launch(ws, count, x, B, ys, y_dtype, nullptr, 0, qw::as_stream(stream));
}

}  // extern "C"
