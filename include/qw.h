/*
 * qw.h -- C ABI of libqw: matrix products against block-wise low-bit
 * quantized weights with the dequantization fused into the product, for
 * AMD Instinct MI355X (gfx950).
 *
 * Formats (defined by the pages this library implements):
 *
 *  QW_FMT_2BIT_G32 -- "On-The-Fly Weight Synthesizer (OTF-LLM Engine v4.0)":
 *    adaptive non-uniform 2-bit code. Each weight is one of four Lloyd-Max
 *    Gaussian centroids C = {-1.52, -0.45, +0.45, +1.52} (section 2; fp32
 *    constants), mapped through a per-group scale and offset fitted by
 *    closed-form least squares over groups of 32 along K (section 3):
 *        w_hat[n][k] = S[n][k/32] * C[q[n][k]] + Z[n][k/32].
 *    Four codes per byte ("Key v4.0 Innovations"). Optional FP16 outlier
 *    anchors (section 4): input channels out_idx[0..n_out) whose weights are
 *    kept exactly in fp16; the 2-bit code of those columns is stored but the
 *    products use the anchors instead.
 *  QW_FMT_NF4_B64 -- "AirQuant" README, "Fundamentacao Teorica e
 *    Arquitetura" item 2: NormalFloat4 (QLoRA) with a per-block absmax:
 *        w_hat[n][k] = absmax[n][k/64] * L[q[n][k]],
 *    L = 16 normalised N(0,1) quantiles in [-1, 1] (see qw_nf4_levels).
 *  QW_FMT_INT4_G32 -- the OTF-LLM page's v3.2 INT4 format ("Comparative
 *    Analysis: INT4 (v3.2) vs INT2 Non-Uniform (v4.0)", "Method Comparison
 *    Table"): two 4-bit codes per byte on a uniform symmetric grid with
 *    zero-point 0, a static permutation of the input channels, the top 1%
 *    channels kept in fp16. Channels are stored in permuted order: position
 *    j holds input channel perm[j] (qw_select_perm orders them by descending
 *    outlier score), and the products take activations in that order
 *    (x_p[b][j] = x[b][perm[j]], see qw_permute_cols):
 *        w_hat[n][j] = s[n][j/32] * (u[n][j] - 8),  u in 1..15,
 *    s = fp16(absmax/7) per group of 32 permuted positions; the first n_out
 *    positions are the fp16 anchors (their codes hold the zero level).
 *
 * Memory layout in device memory (all row-major, rows = output features n):
 *  2-bit codes   uint8 [N][K/4]; byte j holds elements 4j..4j+3, element
 *                4j+t in bits 2t..2t+1; code value q indexes C ascending.
 *  2-bit scales  uint16 pairs [N][K/32][2]: [.][.][0] = S, [.][.][1] = Z,
 *                both IEEE fp16 bit patterns.
 *  anchors       out_idx int32 [n_out], strictly ascending, in [0, K);
 *                out_w fp16 [N][n_out_pad], n_out_pad = n_out rounded up to a
 *                multiple of 8, padding zero;
 *                out_mask uint32 [K/32], bit (k % 32) of word k / 32 set iff
 *                channel k is an anchor (derived from out_idx by qw_pack).
 *  NF4 codes     uint8 [N][K/2]; low nibble = element 2j, high = 2j+1.
 *  NF4 scales    float [N][K/64] (absmax per block of 64 along K).
 *  INT4 codes    uint8 [N][K/2]; low nibble = permuted position 2j, high =
 *                2j+1; nibble u = q + 8 with q in -7..7.
 *  INT4 scales   fp16 [N][K/32] (one per group of 32 permuted positions).
 *  INT4 anchors  out_w fp16 [N][n_out_pad]: the weights of permuted
 *                positions 0..n_out-1 (padding zero); out_idx int32 [K] is
 *                the permutation (read by qw_pack only); out_mask unused.
 *
 * Conventions for every entry point:
 *  - pointers documented "device" must point to device memory of the
 *    current HIP device; "host" pointers to host memory. The caller owns
 *    and frees all memory it passes; nothing of it is retained after the
 *    call returns. No entry point allocates device memory: scratch space
 *    (the selectors' scores, the partial rows of a K-split GEMV) is a
 *    caller-owned workspace argument whose size a query function gives.
 *  - ``stream`` is a hipStream_t passed as void* (NULL = default stream).
 *    Device work is only enqueued; no entry point synchronizes.
 *  - arguments are validated on the host before anything is enqueued; on
 *    any error nothing is enqueued and the status says why. A failed launch
 *    returns QW_ERR_HIP. No entry point aborts or throws.
 *  - results are deterministic: the same inputs give the same bits.
 *  - device base pointers must be 16-byte aligned (QW_ERR_ALIGNMENT).
 */
#ifndef QW_H_
#define QW_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QW_ABI_VERSION 2

typedef enum {
  QW_OK = 0,
  QW_ERR_INVALID_ARG = 1, /* a size, count, enum or pointer is out of range */
  QW_ERR_ALIGNMENT = 2,   /* a device pointer is not 16-byte aligned */
  QW_ERR_UNSUPPORTED = 3, /* valid request this build does not implement */
  QW_ERR_HIP = 4,         /* a HIP runtime call or launch failed */
  QW_ERR_NO_DEVICE = 5,   /* no gfx950 device is current */
  QW_ERR_SCRATCH_LIMIT = 6 /* the call needs more scratch than the library's
                              static array holds (qgemv_2bit_static) */
} qw_status;

typedef enum { QW_FMT_2BIT_G32 = 1, QW_FMT_NF4_B64 = 2, QW_FMT_INT4_G32 = 3 } qw_format;
typedef enum { QW_DT_F16 = 1, QW_DT_BF16 = 2, QW_DT_F32 = 3 } qw_dtype;

/* Outlier channel score ("Profile-Guided Activation Outliers", section 4):
 * MEANABS = mean_n |W[n][c]| * mean_p |X[p][c]| (the |W| x |X| shorthand of
 * the page's title and feature list); L2 = ||W[:,c]||_2 * mean_p |X[p][c]|
 * (the section-4 equation). */
typedef enum { QW_SCORE_MEANABS = 1, QW_SCORE_L2 = 2 } qw_score;

/* Non-owning view of one packed weight matrix. All pointers are device
 * pointers owned by the caller. For NF4, out_idx/out_w are unused and n_out
 * must be 0. For INT4, out_idx is the channel permutation [K] (needed by
 * qw_pack only), out_w the anchors [N][n_out_pad], out_mask unused. */
typedef struct {
  int32_t format;     /* qw_format */
  int32_t N, K;       /* output features, input features */
  int32_t n_out;      /* number of fp16 anchor channels (2-bit only) */
  int32_t n_out_pad;  /* row stride of out_w in elements (multiple of 8) */
  uint8_t *codes;     /* see layout above */
  void *scales;       /* 2-bit: uint16 [N][K/32][2]; NF4: float [N][K/64] */
  int32_t *out_idx;   /* [n_out] or NULL when n_out == 0; INT4: perm [K] */
  uint16_t *out_w;    /* fp16 [N][n_out_pad] or NULL when n_out == 0 */
  uint32_t *out_mask; /* [K/32] or NULL when n_out == 0 */
} qw_weight;

/* Byte counts of the buffers of one packed matrix (0 when unused). */
typedef struct {
  size_t codes, scales, out_idx, out_w, out_mask;
  int32_t n_out_pad;
} qw_sizes;

/* Version of this ABI (QW_ABI_VERSION). */
int qw_abi_version(void);

/* Static text for a status code. Never NULL. */
const char *qw_status_str(qw_status s);

/* Kernel timing without launch gaps, for benchmarks and profilers. Arms the
 * next call of qw_select_outliers, qw_pack, qgemv_2bit, qgemv_nf4,
 * qgemv_2bit_grouped or qgemm_prefill made on the calling host thread: the
 * first kernel that call dispatches records start_event when it begins
 * executing, and each of its kernels records stop_event when it ends, so
 * after the call the pair brackets exactly the device execution of its
 * kernels (hipExtLaunchKernel semantics). Both are hipEvent_t passed as
 * void*, created by the caller on the current device; either may be NULL.
 * The pair is consumed by that next call even when it returns an error
 * before launching anything (then neither event is recorded).
 * qw_time_next_call(NULL, NULL) disarms. Host only; returns QW_OK. */
qw_status qw_time_next_call(void *start_event, void *stop_event);

/* Bytes the caller must allocate for each buffer of a packed matrix of the
 * given format and shape, and the anchor row stride, into host struct *out:
 * four 2-bit codes per byte ("Key v4.0 Innovations" of the OTF-LLM page),
 * one fp16 (S, Z) pair per group of 32 (its section 3), n_out fp16 anchor
 * weights per row (its section 4); NF4 two codes per byte and one fp32
 * absmax per block of 64 ("AirQuant" README, item 2); INT4 two codes per
 * byte, one fp16 scale per group of 32, the permutation (K int32) as
 * out_idx and n_out fp16 anchors per row ("Comparative Analysis" of the
 * OTF-LLM page). Host only.
 * Errors: QW_ERR_INVALID_ARG if out is NULL, N, K <= 0, K not a multiple of
 * the group/block size (32 for 2-bit and INT4, 64 for NF4), n_out < 0,
 * n_out >= K, or n_out > 0 for NF4. */
qw_status qw_packed_sizes(qw_format fmt, int N, int K, int n_out, qw_sizes *out);

/* Number of anchor channels for a fraction of K: floor(frac * K) in double
 * precision (section 4 keeps the top 3.5%). Returns -1 if K < 0 or frac is
 * outside [0, 1). Host only. */
int qw_outlier_count(int K, double frac);

/* The four 2-bit centroids (section 2 of the OTF-LLM page) as fp32, into
 * host array out[4]. */
qw_status qw_codebook_2bit(float *out);

/* The 16 NF4 levels the library uses, ascending, as fp32, into host array
 * out[16] ("AirQuant" README, item 2 and "Fontes": NF4 as in QLoRA; the
 * page prints no level, so the construction is this library's reading of
 * QLoRA's). Built on the host at first use from normal quantiles: 8 positive
 * at probabilities evenly spaced from delta down to 1/2 (exclusive), 7
 * negative likewise, plus 0, divided by the largest;
 * delta = 1 - (1/32 + 1/30)/2. */
qw_status qw_nf4_levels(float *out);

/* Bytes of the device workspace the selectors of section 4 (OTF-LLM page:
 * profile-guided outlier channels) and the INT4 permutation need for K
 * channels (K * 20: fp64 scores, profile sums, int32 flags; 0 when K <= 0).
 * Host only. */
size_t qw_select_workspace_bytes(int K);

/* Profile-guided outlier selection (section 4 of the OTF-LLM page).
 *   W      device fp32 [N][K]  weights
 *   X_prof device fp32 [P][K]  calibration activations (P >= 1)
 *   frac   fraction of channels to keep, n = floor(frac*K) (0 <= frac < 1)
 *   out_idx device int32 [n]   receives the n highest-scoring channels in
 *          ascending order; ties in score go to the lower channel.
 *   workspace device scratch of workspace_bytes >= qw_select_workspace_bytes(K)
 *          (16-byte aligned), owned by the caller; its contents on entry do
 *          not matter and are overwritten. Calls that overlap in time must
 *          not share it.
 * Scores are fp64 with sequential sums over rows. Errors: INVALID_ARG for
 * bad sizes, NULL pointers or a workspace that is too small, ALIGNMENT,
 * UNSUPPORTED (W or X_prof of 2 GiB or more), HIP if a launch fails. */
qw_status qw_select_outliers(const float *W, int N, int K, const float *X_prof,
                             int P, double frac, qw_score score,
                             int32_t *out_idx, void *workspace,
                             size_t workspace_bytes, void *stream);

/* The channel permutation of the INT4 format ("Global Static Permutation"
 * of the OTF-LLM page's v3.2 engine): perm_out[j] = the channel of rank j
 * by descending outlier score (the section-4 score of qw_select_outliers,
 * same arguments and arithmetic), ties to the lower channel, so its first
 * floor(0.01 K) entries are the top-1% channels the format keeps in fp16.
 *   W, X_prof, score, workspace: as qw_select_outliers
 *   perm_out device int32 [K]
 * Errors as qw_select_outliers. */
qw_status qw_select_perm(const float *W, int N, int K, const float *X_prof, int P,
                         qw_score score, int32_t *perm_out, void *workspace,
                         size_t workspace_bytes, void *stream);

/* Columns of X in permuted order: X_p[m][j] = X[m][perm[j]] (the order in
 * which the INT4 products take their activations: the OTF-LLM page's
 * "Comparative Analysis" names a global static permutation of the v3.2
 * format; reading it as a reordering of the channel space done once, the
 * activations are gathered with it).
 *   X      device [M][K], elements of dtype (F16, BF16 or F32)
 *   perm   device int32 [K], a permutation of 0..K-1 (not checked; entries
 *          out of range read zero)
 *   X_p    device [M][K] of the same dtype; must not alias X
 * Errors: INVALID_ARG, ALIGNMENT, UNSUPPORTED (X of 2 GiB or more), HIP. */
qw_status qw_permute_cols(const void *X, qw_dtype dtype, int M, int K, const int32_t *perm,
                          void *X_p, void *stream);

/* Quantize and pack fp32 weights into ``dst`` (buffers allocated by the
 * caller with the sizes from qw_packed_sizes; dst->format, N, K, n_out,
 * n_out_pad must describe them).
 *   W        device fp32 [N][K]
 *   dst->out_idx (2-bit, n_out > 0) device int32 [n_out], strictly ascending;
 *            those columns are zeroed before the fit and copied to out_w
 *            rounded to fp16 (nearest-even); out_mask is written from it.
 * 2-bit: per group of 32 along K, in fp64 without fused multiply-add:
 * mean m and population variance v; code q = (w-m >= 0 ? 2 : 1) moved to
 * the outer level (3 or 0) when (w-m)^2 > t^2 v with t = (C[2]+C[3])/2;
 * S = sum (w-m)(c-cbar) / (sum (c-cbar)^2 + 1e-8), Z = m - S cbar
 * (section 3); S and Z rounded once to fp16 (nearest-even, subnormals kept).
 * NF4: per block of 64, absmax a = max |w|; q = number of level midpoints
 * t_j with w > t_j * a (nearest level, ties low); a == 0 gives q = 7.
 * INT4: dst->out_idx holds the permutation (device int32 [K], a
 * permutation of 0..K-1); W stays in its original channel order and is
 * read through it. Positions j < n_out are the anchors: out_w = fp16 of the
 * weight, nearest-even; their codes are the zero level. Per group of 32
 * permuted positions (anchors counted as 0), in fp64: a = max |w|,
 * s = fp16(a / 7) (nearest-even), q = clamp(rint(w / s), -7, 7) with the
 * stored s (rint: nearest, ties to even; s == 0 gives q = 0).
 * The result is bit-identical to the reference quantizer. Errors:
 * INVALID_ARG, ALIGNMENT, HIP. out_idx ordering is not checked here (the
 * Python binding checks it). */
qw_status qw_pack(const float *W, const qw_weight *dst, void *stream);

/* Maximum refine_rounds accepted by qw_pack_ex. */
#define QW_MAX_REFINE_ROUNDS 64

/* qw_pack with a choice of weight storage type and an optional refinement
 * of the 2-bit code.
 *   W        device [N][K] in w_dtype: QW_DT_F32, QW_DT_F16 or QW_DT_BF16;
 *            each weight widens exactly to fp32, so fp16/bf16 weights give
 *            the same result as their fp32 values passed to qw_pack
 *            (anchors: fp16 rounding of that value).
 *   refine_rounds  0..QW_MAX_REFINE_ROUNDS, 2-bit only (0 for NF4):
 *            after the single pass, rounds of
 *              (a) levels l_j = S*C[j] + Z of the unrounded fit (fp64,
 *                  product then sum);
 *              (b) every weight takes the level nearest to it, |w - l_j| in
 *                  fp64, keeping its code when that level is among the
 *                  nearest, else the lowest nearest j;
 *              (c) the section-3 fit redone for the new codes (same mean,
 *                  sums and epsilon as the single pass).
 *            The nearest-centroid rule of section 2 applied to the fitted
 *            levels, alternated with the fit of section 3 as in Lloyd's
 *            method; no round raises the group's squared error (beyond the
 *            epsilon's effect), and S, Z of the last fit are stored.
 * Buffers and other rules as qw_pack, whose result qw_pack_ex(W, QW_DT_F32,
 * 0, dst, stream) is. The result is bit-identical to the reference
 * quantizer run with the same rounds. Errors: INVALID_ARG (dtype, rounds
 * out of range or non-zero for NF4, and the qw_pack checks), ALIGNMENT,
 * HIP. */
qw_status qw_pack_ex(const void *W, qw_dtype w_dtype, int refine_rounds,
                     const qw_weight *dst, void *stream);

/* Calibration statistic of section 4 (the mean activation magnitude of
 * each input channel over a calibration pass), accumulated on the device
 * over any number of batches so the profile never has to be held at once:
 *   abs_sum[c] += |X[0][c]| + |X[1][c]| + ... + |X[M-1][c]|
 * in fp64, rows added in order (so batches given in order sum exactly as
 * one long profile would).
 *   X        device [M][K] in x_dtype (F32, F16 or BF16), M >= 1
 *   abs_sum  device double [K], caller-initialised (zeros before the first
 *            batch); read and written.
 * Errors: INVALID_ARG, ALIGNMENT, HIP. */
qw_status qw_profile_accumulate(const void *X, qw_dtype x_dtype, int M, int K,
                                double *abs_sum, void *stream);

/* qw_select_outliers from accumulated profile sums instead of the profile
 * rows: the mean magnitude of channel c is prof_abs_sum[c] / prof_rows, and
 * W may be fp32, fp16 or bf16 (widened exactly). With sums from
 * qw_profile_accumulate over the same rows, in the same order, the chosen
 * channels are identical to qw_select_outliers on those rows (section 4 of
 * the OTF-LLM page).
 *   prof_abs_sum device double [K]; prof_rows >= 1 rows summed.
 *   workspace    as for qw_select_outliers (qw_select_workspace_bytes(K)).
 * Errors as qw_select_outliers. */
qw_status qw_select_outliers_ex(const void *W, qw_dtype w_dtype, int N, int K,
                                const double *prof_abs_sum, long long prof_rows,
                                double frac, qw_score score, int32_t *out_idx,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/* Decode GEMV for the 2-bit format ("Key v4.0 Innovations" of the OTF-LLM
 * page: the packed codes are dequantized in registers inside the product;
 * section 1: decoding streams every weight once per token; sections 2-4:
 * codebook, per-group S and Z, fp16 anchors):
 *   y[b][n] = sum_k x_R[b][k] w_hat[n][k] + sum_o x[b][out_idx[o]] out_w[n][o]
 * for b < B, where x_R is x with the anchor channels set to zero.
 *   x  device fp16 [B][K], 1 <= B <= 8
 *   y  device [B][N], fp16 (QW_DT_F16, rounded nearest-even) or fp32
 * Accumulation is fp32. Codes are decoded in registers; nothing is
 * materialized. y must not alias x. Needs no workspace: batches whose x
 * does not fit one workgroup whole (e.g. B >= 2 at K = 27648) run one row
 * group at a time on the vector-ALU kernel; qgemv_2bit_ws runs them with
 * the weights streamed once.
 * Errors: INVALID_ARG (format mismatch, B, dtype), ALIGNMENT, UNSUPPORTED,
 * HIP. */
qw_status qgemv_2bit(const qw_weight *w, const void *x, int B, void *y,
                     qw_dtype y_dtype, void *stream);

/* Device workspace bytes qgemv_2bit_ws needs for weight w at batch B (into
 * host *bytes; the K split is this library's, the pages being silent on
 * batched decode): 0 when the call runs without one, else parts * B * N * 4
 * for the fp32 partial rows of its K parts (parts <= 8). Host only; the
 * answer depends on the shape and on the current device. Errors as
 * qgemv_2bit's argument checks. */
qw_status qgemv_2bit_workspace_bytes(const qw_weight *w, int B, size_t *bytes);

/* qgemv_2bit with a caller-owned device workspace (16-byte aligned,
 * workspace_bytes long; may be NULL when workspace_bytes is 0). When the
 * batch's x does not fit one workgroup whole and the workspace holds
 * qgemv_2bit_workspace_bytes(w, B), K is cut into equal parts of whole
 * 512-channel runs whose fp32 partial rows are written to the workspace and
 * then added in part order (deterministic) into y; the weights stream once.
 * With a smaller workspace the call runs as qgemv_2bit does. The
 * workspace's contents on entry do not matter; calls that overlap in time
 * (other streams, graph replays) must not share it. Same results rules and
 * errors as qgemv_2bit. */
qw_status qgemv_2bit_ws(const qw_weight *w, const void *x, int B, void *y,
                        qw_dtype y_dtype, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Bytes of the library's static device scratch array (one per device). */
#define QW_STATIC_SCRATCH_BYTES (8u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * qgemv_2bit_ws with the library's own static device array of
 * QW_STATIC_SCRATCH_BYTES in place of the workspace argument. It allocates
 * nothing: no hipMalloc, no hipFree, no allocating library call. The array
 * is one per device, held until the process ends, and keeps the last call's
 * contents (a call overwrites every byte it reads before reading it, so
 * nothing needs clearing). Calls that overlap in time on one device (other
 * streams, graph replays running at once) share it and race: order them.
 * Results are those of qgemv_2bit_ws with a large enough workspace, bit for
 * bit. Errors: those of qgemv_2bit_ws, and QW_ERR_SCRATCH_LIMIT (nothing
 * enqueued) when qgemv_2bit_workspace_bytes(w, B) exceeds
 * QW_STATIC_SCRATCH_BYTES. */
qw_status qgemv_2bit_static(const qw_weight *w, const void *x, int B, void *y,
                            qw_dtype y_dtype, void *stream);

/* Decode GEMV for the INT4 format (the OTF-LLM page's v3.2 engine,
 * "Comparative Analysis" and "Method Comparison Table"; dequantized in
 * registers inside the product as the 2-bit GEMV):
 *   y[b][n] = sum_j x_p[b][j] w_hat[n][j] + sum_{o < n_out} x_p[b][o] out_w[n][o]
 * with x_p the activations in permuted channel order (qw_permute_cols).
 *   x_p device fp16 [B][K], 1 <= B <= 8
 *   y   device [B][N], fp16 (nearest-even) or fp32
 * fp32 accumulation; no workspace. Where K is a multiple of 512 the
 * products run on the matrix cores (the 2-bit GEMV's scheme: the code bits
 * as fp4 operands against exact fp8 limbs of x), batches in slices whose x
 * fits one workgroup; other shapes on the vector ALUs, in row groups. The
 * results of the two kernels agree within the fp32 bound, not bit for bit.
 * Errors: INVALID_ARG, ALIGNMENT, UNSUPPORTED, HIP. */
qw_status qgemv_int4(const qw_weight *w, const void *x_p, int B, void *y,
                     qw_dtype y_dtype, void *stream);

/* Decode GEMV for NF4 ("AirQuant" README, item 2: NF4 block-wise weights;
 * dequantized in registers, as the 2-bit GEMV):
 *   y[b][n] = sum_k x[b][k] w_hat[n][k].
 * Same argument conventions as qgemv_2bit; needs no workspace. */
qw_status qgemv_nf4(const qw_weight *w, const void *x, int B, void *y,
                    qw_dtype y_dtype, void *stream);

/* Several 2-bit decode GEMVs that share one input x (for example the q, k
 * and v projections of one attention block), in one launch (fewer launches
 * per token for the streaming bound of the OTF-LLM page's section 1; the
 * products are those of qgemv_2bit):
 *   y_i = qgemv_2bit(w_i, x) for i < count (count <= 4), bit for bit.
 * All w_i must have the same K; y_i have their own N_i. Same conventions as
 * qgemv_2bit (no workspace); ws and ys are host arrays of count entries. */
qw_status qgemv_2bit_grouped(const qw_weight *ws, int count, const void *x,
                             int B, void *const *ys, qw_dtype y_dtype,
                             void *stream);

/* The gate and up projections of a gated MLP block with the activation
 * between them and the down projection, in one launch:
 *   y[b][n] = silu(g[b][n]) * u[b][n],   silu(t) = t / (1 + exp(-t)),
 *   g[b][n] = sum_k x[b][k] w_hat[n][k], u[b][n] = sum_k x[b][k] w_hat[I+n][k]
 * for n < I, where w is ONE 2-bit view of N = 2I rows: the gate rows
 * (0..I-1) stacked over the up rows (I..2I-1), packed, with its anchor
 * channels selected, as one matrix (the two share their input). Each
 * output's two sums are accumulated as by qgemv_2bit (fp32), the
 * activation and the product in fp32, then one rounding to y_dtype; y is
 * [B][I] and is the down projection's x when y_dtype is fp16. The pages do
 * not name the activation: SiLU is the one of the decoder shapes they quote
 * (the 32B-class block of hidden 5120 and intermediate 27648), and the
 * fusion serves their per-token streaming argument ("On-The-Fly Weight
 * Synthesizer (OTF-LLM Engine v4.0)", section 1: every weight is fetched
 * once per token, so nothing else should cost a pass).
 * Conventions as qgemv_2bit; needs no workspace. Errors: INVALID_ARG also
 * for N not a multiple of 32; UNSUPPORTED when K % 512 != 0 or the batch's
 * x does not fit a workgroup (no K split and no vector-ALU path here). */
qw_status qgemv_2bit_swiglu(const qw_weight *w, const void *x, int B, void *y,
                            qw_dtype y_dtype, void *stream);

/* Fused decode stack (batch 1): a sequence of grouped 2-bit GEMV stages
 * (for example q/k/v, o, gate/up and down of every layer of a decoder, in
 * order) run by ONE persistent launch, with a device-wide barrier between
 * consecutive stages in place of a kernel boundary, so a stage starts only
 * after every output of the one before is written and visible. Each stage
 * computes what qgemv_2bit_grouped computes for it (the matrix-core GEMV's
 * arithmetic with fp32 accumulation; the persistent launch splits the work
 * its own way, so the last bits can differ from a separate call, and are
 * the same from run to run); a stage with swiglu set computes what
 * qgemv_2bit_swiglu computes (the gated activation feeding the down
 * projection), while the attention steps between projections are not part
 * of it.
 * Intended for decode loops where the per-launch cost of hundreds of small
 * GEMVs per token dominates ("Key v4.0 Innovations" and section 1 of the
 * OTF-LLM page: decoding is bound by streaming every weight once per
 * token). */
#define QW_STACK_MAX_STAGES 4096

typedef struct {
  int32_t count;      /* matrices sharing x: 1..4 */
  qw_weight w[4];     /* 2-bit views (device buffers), equal K, K % 512 == 0 */
  const void *x;      /* device fp16 [K] (batch 1) */
  void *y[4];         /* device [N_i] outputs, fp16 or fp32 per y_dtype */
  int32_t y_dtype;    /* QW_DT_F16 or QW_DT_F32 */
  int32_t swiglu;     /* 0, or 1: count is 1, w[0] is a merged gate/up view
                         (N % 32 == 0) and y[0] gets [N/2] gated values, as
                         qgemv_2bit_swiglu */
} qw_stack_stage;

/* Host handle of a prepared stack, written by qw_stack_prepare. */
typedef struct {
  void *plan;         /* the device plan buffer given to qw_stack_prepare */
  int32_t n_stages;
  int32_t grid;       /* workgroups of the persistent launch (one per CU) */
  int32_t lds;        /* LDS bytes per workgroup */
} qw_stack;

/* Bytes of the device plan buffer for n_stages stages (0 if out of range). */
size_t qw_stack_plan_bytes(int n_stages);

/* Plans every stage (as qgemv_2bit_grouped would for batch 1) and copies the
 * plan to ``plan`` (caller-allocated device memory of qw_stack_plan_bytes,
 * 16-byte aligned). The weights, x and y pointers are baked into the plan:
 * later runs read whatever those buffers hold. Unlike every other entry
 * point this call BLOCKS until the plan is on the device (it copies from
 * host memory). Errors: INVALID_ARG, ALIGNMENT, UNSUPPORTED (a stage does
 * not fit the matrix-core kernel: K % 512, K > 49152, LDS), HIP. */
qw_status qw_stack_prepare(const qw_stack_stage *stages, int n_stages, void *plan,
                           qw_stack *out);

/* Bytes of the sync buffer qw_stack_run needs for a prepared stack (0 for a
 * NULL or unprepared handle): 16 words plus one arrival flag per workgroup
 * of the persistent launch. Host only. */
size_t qw_stack_sync_bytes(const qw_stack *st);

/* Enqueues one run of a prepared stack on ``stream``: a fill kernel clears
 * sync, then one cooperative launch with one workgroup of 1024 threads per
 * CU runs all stages.
 *   sync  device uint32 scratch of qw_stack_sync_bytes(st) bytes, owned by
 *         the caller (16-byte aligned): word 0 is non-zero after the run if
 *         a barrier wait gave up (a second or more per wait; the outputs
 *         are then invalid); the rest holds the workgroups' arrival flags.
 *         Runs that share a sync buffer must not overlap.
 * Errors: INVALID_ARG (also a handle prepared on a device with another CU
 * count), ALIGNMENT, HIP (including a cooperative launch the device
 * refuses). */
qw_status qw_stack_run(const qw_stack *st, uint32_t *sync, void *stream);

/* Prefill GEMM: Y[m][n] = sum_k X[m][k] w_bf16[n][k] with
 * w_bf16 = bf16(fp32(S*C[q]+Z)) (one fused multiply-add, then nearest-even)
 * for 2-bit, bf16(fp32(absmax*L[q])) for NF4, bf16(s*q) for INT4 (exact in
 * fp32, then nearest-even); 2-bit and INT4 anchor columns use bf16(out_w).
 * For INT4, X is given in permuted channel order (qw_permute_cols). The pages are silent on prefill; the dequantization is each
 * format's w_hat (OTF-LLM sections 2-3, AirQuant item 2) rounded to bf16.
 * Without anchors the weights are dequantized in registers by the lanes
 * that feed them to the bf16 matrix-core instructions (X is staged through
 * LDS); with anchors, dequantized tiles of W and X are staged through LDS.
 * Accumulation is fp32.
 *   X  device bf16 [M][K], M >= 1
 *   Y  device [M][N], bf16 (QW_DT_BF16, nearest-even of the fp32 result) or
 *      fp32 (QW_DT_F32)
 * Requires K to be a multiple of 64; needs no workspace. Errors:
 * INVALID_ARG, ALIGNMENT, UNSUPPORTED, HIP. */
qw_status qgemm_prefill(const qw_weight *w, const void *X, int M, void *Y,
                        qw_dtype y_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QW_H_ */
