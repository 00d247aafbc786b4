/*
 * fp8ds.h -- C ABI of the FP8 per-tensor delayed-scaling linear-layer path on AMD MI355X
 * (CDNA4, gfx950).
 *
 * The operations follow three TransformerEngine pull-request pages:
 *   "[PyTorch] Refactor FP8 workspaces in linear modules" (PR 820)      -- cited as [WS]
 *   "[PyTorch] cuda graph support" (PR 575)                             -- cited as [CG]
 *   "[PyTorch] Userbuffers support in operation-based API" (PR 1142)    -- cited as [UB]
 * FP8 bit formats are the OCP OFP8 E4M3 and E5M2 encodings (the pages do not state them).
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless a comment says HOST.  The caller owns every buffer;
 *     outputs go into caller-provided memory (the Float8Tensor "data" / "data_transpose"
 *     buffers of [UB], comment on the data kwargs).  The library never allocates device
 *     memory, frees, copies between host and device or synchronises.
 *   - Every call is asynchronous on `stream` (NULL = the null stream) and may be captured
 *     into a hipGraph: the transposes are ordinary kernels in the captured sequence ([WS]
 *     "grown in scope", first bullet; [CG] feature list, persistent transposes).
 *   - bfloat16 tensors are passed as uint16_t bit patterns, FP8 tensors as uint8_t codes.
 *     2-D tensors are row-major and densely packed unless a leading dimension is given.
 *   - Device pointers must be 16-byte aligned unless a call's comment says otherwise.
 *   - Scales live on the device (float32 scalars), so no call reads them on the host.
 *   - Return value: FP8DS_OK (0) or a negative fp8ds_status.  Arguments are checked on the
 *     host before anything is launched; a rejected call launches nothing.  After launching,
 *     a HIP launch error is reported as FP8DS_ERR_HIP (no synchronisation is done, so faults
 *     inside kernels surface at the caller's next synchronisation).
 *   - Numerical trouble (zero, subnormal, infinite or NaN amax) is not an error: the scale
 *     update guards against it.
 */
#ifndef FP8DS_H
#define FP8DS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8DS_E4M3 = 0, /* 1-4-3, bias 7, max 448, S.1111.111 = NaN, no infinity */
    FP8DS_E5M2 = 1  /* 1-5-2, bias 15, max 57344, IEEE-style inf / NaN      */
} fp8ds_format;

typedef enum {
    FP8DS_OUT_BF16 = 0, /* round-to-nearest-even bfloat16 */
    FP8DS_OUT_FP32 = 1
} fp8ds_out_dtype;

typedef enum {
    FP8DS_OK = 0,
    FP8DS_ERR_NULL = -1,      /* a required pointer is NULL                        */
    FP8DS_ERR_SHAPE = -2,     /* a size is negative or violates a stated multiple  */
    FP8DS_ERR_ALIGN = -3,     /* a pointer or leading dimension is misaligned      */
    FP8DS_ERR_FORMAT = -4,    /* unknown fp8ds_format / fp8ds_out_dtype            */
    FP8DS_ERR_WORKSPACE = -5, /* workspace missing or smaller than required        */
    FP8DS_ERR_HIP = -6,       /* the HIP runtime reported an error                 */
    FP8DS_ERR_ARG = -7,       /* another argument is out of its documented range   */
    FP8DS_ERR_SCRATCH = -8    /* the problem needs more than the static scratch    */
} fp8ds_status;

/* Human-readable name of a status code (static storage; never NULL). */
const char *fp8ds_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fp8ds_version(void);

/*
 * fp8_cast_amax -- cast a bfloat16 tensor to FP8 with amax capture
 * ([CG] transpose-cache thread: Float8Tensor.to_float8; [WS] Motivations, first bullet).
 *
 *   out[i] = encode_fmt( float(x[i]) * (*scale) )   one float32 product, then saturating
 *            round-to-nearest-even FP8 (finite overflow and +-inf give the largest finite
 *            code of that sign, every NaN gives 0x7F);
 *   *amax_slot = max(*amax_slot, max_i |x[i]|)      the unscaled input's amax, folded in
 *            with an atomic max (NaN dominates); so several casts of one tensor within an
 *            iteration reduce into the same history slot ([CG] feature list, amaxes reduced
 *            within the current iteration);
 *   *scale_inv_out = 1.0f / (*scale)                the FP8 tensor's private inverse scale
 *            ([WS] Motivations, first and second bullets), written by the cast itself so no
 *            separate initialisation launch is needed.
 *
 * x: [numel] bfloat16.  out: [numel] codes.  scale: 1 float.  amax_slot: 1 float holding a
 * non-negative value or NaN, typically row 0 of the amax history, or NULL to skip amax
 * capture.  scale_inv_out: 1 float or NULL.  noop: NULL, or 1 float; when *noop == 1.0f at
 * run time the kernel writes nothing at all (the noop flag of [WS] review thread), which lets a
 * captured graph skip the recast of a cached tensor.  numel >= 0 (0 launches nothing).
 */
int fp8_cast_amax(const uint16_t *x, int64_t numel, const float *scale, int fmt,
                  uint8_t *out, float *scale_inv_out, float *amax_slot, const float *noop,
                  hipStream_t stream);

/*
 * fp8_cast_transpose -- cast plus transpose: the row-major FP8 tensor and its transpose
 * cache in one pass ([WS] "grown in scope", first bullet; [CG] DbiasCastTranspose example:
 * cast_transpose creates an FP8 tensor with its transpose cache).
 *
 * x: [rows, cols] bfloat16.  out: [rows, cols] codes, out_t: [cols, rows] codes with
 * out_t[j*rows + i] == out[i*cols + j].  Everything else as fp8_cast_amax (same scale,
 * amax, scale_inv and noop rules).  rows, cols >= 0; any sizes are accepted (ragged edges
 * are handled inside).
 */
int fp8_cast_transpose(const uint16_t *x, int64_t rows, int64_t cols, const float *scale, int fmt,
                       uint8_t *out, uint8_t *out_t, float *scale_inv_out, float *amax_slot,
                       const float *noop, hipStream_t stream);

/*
 * fp8_dbias_workspace_bytes -- HOST-only: workspace size fp8_dbias_cast_transpose needs for
 * a [rows, cols] dy: FP8DS_DBIAS_COUNTER_BYTES of per-strip arrival counters, then the partial
 * column sums of fixed-order row blocks (ceil(rows / 256) * cols float32).  0 for empty inputs.
 */
#define FP8DS_DBIAS_COUNTER_BYTES ((size_t)1024)
size_t fp8_dbias_workspace_bytes(int64_t rows, int64_t cols);

/*
 * fp8_dbias_cast_transpose -- bias gradient plus cast+transpose of dy
 * ([CG] transpose-cache thread, DbiasCastTranspose.backward: db = dy.sum(dim=0) and
 * dx = cast_transpose(dy)).
 *
 *   dbias[j] = sum_i float(dy[i, j])   float32, from the bfloat16 dy before the cast, summed
 *              in a fixed order (deterministic run to run);
 *   out, out_t, amax, scale_inv as fp8_cast_transpose (E5M2 is the usual format for dy).
 *
 * dbias: [cols] float32.  workspace: at least fp8_dbias_workspace_bytes(rows, cols) bytes of
 * device memory, 4-byte aligned.  Its first FP8DS_DBIAS_COUNTER_BYTES must be zero before the
 * first call that uses it (zero-fill a new workspace once, e.g. hipMemset after allocating
 * it); every call leaves them zero again, so the workspace stays valid for later calls and
 * graph replays of any shape.  The rest of it needs no initialisation.  Calls that overlap in
 * time must not share a workspace.  Tensors of whole 256 x 256 tiles that give each CU at most
 * two tiles (or three or four, the same number for every CU, with at least 16 tile columns) run
 * as one launch that finishes dbias itself (through those counters); all others as the tile
 * kernel plus a reduction launch.  No noop flag (dy is new every iteration).
 */
int fp8_dbias_cast_transpose(const uint16_t *dy, int64_t rows, int64_t cols, const float *scale,
                             int fmt, uint8_t *out, uint8_t *out_t, float *scale_inv_out,
                             float *amax_slot, float *dbias, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * fp8_dbias_cast_transpose_noalloc -- fp8_dbias_cast_transpose for callers that cannot
 * allocate device memory or pass a workspace (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and kernels, minus the
 * workspace: the partial column sums go to a static device array of
 * FP8DS_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the process
 * ends (zero when the library is loaded, so its counters start at zero).  Calls nothing that
 * allocates.  Limit: fp8_dbias_workspace_bytes(rows, cols) <= FP8DS_NOALLOC_SCRATCH_BYTES
 * (8 MiB: e.g. [8192, 16384] needs 2 MiB + 1 KiB, and 8192 rows fit up to cols = 65528), else
 * FP8DS_ERR_SCRATCH and nothing is launched.  All calls on one GPU share its array and each
 * call overwrites it, so calls that overlap in time on one GPU (on two streams, or from two
 * host threads) race: serialise them.
 */
#define FP8DS_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int fp8_dbias_cast_transpose_noalloc(const uint16_t *dy, int64_t rows, int64_t cols,
                                     const float *scale, int fmt, uint8_t *out, uint8_t *out_t,
                                     float *scale_inv_out, float *amax_slot, float *dbias,
                                     hipStream_t stream);

/*
 * fp8_scale_update -- one delayed-scaling step for T tensors in one launch ([WS] Motivations,
 * first bullet: the FP8 scale-update kernel, and a fix for amaxes small enough to make the
 * scale infinite; [CG] feature list: amaxes reduced within the current iteration).
 *
 * amax_history: [L][T] float32, row 0 = the current iteration's amaxes (the slots the casts
 * fold into).  scale, scale_inv: [T] float32.  fmts: HOST array [T] of fp8ds_format.
 * For every tensor t:
 *   a = max over rows 0..L-1 of amax_history[.][t]    (NaN dominates)
 *   s = (fp8_max(fmts[t]) / a) * 2^-margin            float32
 *   if a == 0, a is not finite, s is not finite or 1.0f / s is not finite (s == 0, or s
 *   below 2^-128): s = scale[t] (previous kept)
 *   scale[t] = s;  scale_inv[t] = 1.0f / s
 *   history: row i takes row i+1 (i < L-1), row L-1 takes the old row 0, row 0 becomes 0.
 * The FP8 tensors' private inverse scales are NOT touched: they change only when a tensor is
 * recast ([WS] Motivations, first bullet).
 * Limits: L >= 1, 1 <= T <= 4096, -126 <= margin <= 126.
 */
int fp8_scale_update(float *amax_history, int64_t L, int64_t T, float *scale, float *scale_inv,
                     const int32_t *fmts, int32_t margin, hipStream_t stream);

/*
 * fp8_gemm_bias -- FP8 GEMM with inverse-scale dequantisation and bias ([CG] transpose-cache
 * thread: fp8_gemm on FP8 data; [UB] bias-offset fix: each output chunk adds its own chunk of
 * the bias).
 *
 *   D[m, n] = (sum_k A[m, k] * B[n, k]) * (*a_scale_inv) * (*b_scale_inv) + bias[n]
 *
 * A: [M, K] codes of format fa, row stride lda bytes.  B: [N, K] codes of format fb, row
 * stride ldb bytes (both operands K-contiguous).  The products are accumulated in float32
 * on the matrix cores.  bias: [N] bfloat16 or NULL.  D: [M, N] with row stride ldd elements,
 * bfloat16 (out_dtype FP8DS_OUT_BF16, rounded to nearest even) or float32.
 * Requirements: M, N, K >= 0; K % 16 == 0; lda, ldb >= K and % 16 == 0; A and B 16-byte
 * aligned; ldd >= N; D aligned to its element size.  M or N == 0 launches nothing; K == 0
 * gives the bias.
 * The result of every element depends only on its own row of A and row of B, never on the
 * tile it falls in, so an N-chunked call sequence (offset B, bias and D pointers with the
 * full ldd) reproduces the unchunked output bit for bit.  K and the row strides (never M or N)
 * select the matrix-core instruction: 16 x 16 x 128 when K % 256 == 0 and lda, ldb < 8 MiB,
 * 32 x 32 x 64 otherwise; the two can round the float32 sum differently in the last bit, so
 * calls with different K or strides need not agree bit for bit.
 */
int fp8_gemm_bias(const uint8_t *A, int fa, const float *a_scale_inv, int64_t lda,
                  const uint8_t *B, int fb, const float *b_scale_inv, int64_t ldb,
                  const uint16_t *bias, void *D, int64_t ldd, int out_dtype,
                  int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * fp8_gemm_bias_chunked -- the N-chunked form of fp8_gemm_bias ([UB] bias-offset fix: the GEMM
 * is split into output chunks and chunk c uses bias + c*Nc).  Chunk c computes output columns
 * [c*Nc, min(N, (c+1)*Nc)) with Nc = ceil(N / n_chunks) rounded up to a multiple of 16, on
 * chunk_streams[c] (HOST array of n_chunks streams), ordered after the work already queued on
 * `stream` and joined back into `stream` with events, so the whole sequence can be captured
 * from `stream` as one hipGraph.  1 <= n_chunks <= 16.  The output equals fp8_gemm_bias bit for
 * bit.  chunk_streams may be NULL: then all chunks run on `stream` in order.  The fork / join
 * events are the library's own (created once per device, kept for the process); each call
 * enqueues its records and waits under a per-device lock, so several host threads may call
 * this at once.
 */
int fp8_gemm_bias_chunked(const uint8_t *A, int fa, const float *a_scale_inv, int64_t lda,
                          const uint8_t *B, int fb, const float *b_scale_inv, int64_t ldb,
                          const uint16_t *bias, void *D, int64_t ldd, int out_dtype,
                          int64_t M, int64_t N, int64_t K, int n_chunks,
                          const hipStream_t *chunk_streams, hipStream_t stream);

/*
 * fp8_gemm_bias_fp8 -- fp8_gemm_bias whose output is itself an FP8 tensor with its own scale
 * ([CG] transpose-cache thread: FP8Linear.backward passes out=dx._data, so the GEMM writes
 * straight into the data of a Float8Tensor).
 *
 *   v[m, n] = (sum_k A[m, k] * B[n, k]) * (*a_scale_inv) * (*b_scale_inv) + bias[n]   (float32)
 *   D[m, n] = saturating round-to-nearest-even code (format d_fmt) of v[m, n] * (*d_scale)
 *   *d_amax_slot = max(*d_amax_slot, max |v|)          (amax of the output before its scale)
 *   *d_scale_inv_out = 1.0f / (*d_scale)               (the output's private inverse scale)
 *
 * A, B, bias, M, N, K and their requirements are those of fp8_gemm_bias.  D: [M, N] codes with
 * row stride ldd >= N bytes, any alignment (16-byte aligned D with ldd % 16 == 0 takes the
 * vector stores).  d_scale is required; d_scale_inv_out and d_amax_slot may be NULL (not
 * written).  The amax fold is an atomic max, so d_amax_slot may be an amax-history slot that
 * other kernels also fold into.  NaN values give code 0x7F and a NaN amax, as in the casts.
 * With M or N == 0 only *d_scale_inv_out is written.
 */
int fp8_gemm_bias_fp8(const uint8_t *A, int fa, const float *a_scale_inv, int64_t lda,
                      const uint8_t *B, int fb, const float *b_scale_inv, int64_t ldb,
                      const uint16_t *bias, uint8_t *D, int64_t ldd, int d_fmt,
                      const float *d_scale, float *d_scale_inv_out, float *d_amax_slot,
                      int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * fp8_transpose -- transpose cache of an FP8 tensor that already exists ([WS] "grown in scope",
 * first bullet: transpose_2d(cache=True) and lazy transpose caching; [CG] transpose-cache
 * thread: dy.transpose() of an FP8 dy without a cache, and the noop flag in transpose used for
 * weight caching across microbatches).
 *
 *   out_t[j, i] = in[i, j]     in: [rows, cols] codes, out_t: [cols, rows] codes
 *
 * The codes are copied, not re-encoded (the tensor's scale and scale_inv are unchanged).
 * noop: NULL, or a device float; when *noop == 1.0f at run time the kernel writes nothing and
 * the cache keeps its previous contents.  Any alignment is accepted (16-byte aligned buffers
 * with rows and cols multiples of 16 take the vector path).  rows or cols == 0 launches
 * nothing.  in and out_t must not overlap.
 */
int fp8_transpose(const uint8_t *in, int64_t rows, int64_t cols, uint8_t *out_t, const float *noop,
                  hipStream_t stream);

/*
 * fp8_linear_fwd -- forward of the FP8 linear layer y = x W^T + bias ([WS] description: one
 * FP8 weight workspace with its transpose; [CG] feature list: FP8 weight caching).
 * Work enqueued on `stream`, in this order:
 *   1. x8 = cast(x, *x_scale) E4M3 (cast+transpose when x8_t != NULL, else cast only),
 *      amax into *x_amax, *x_scale_inv = 1/(*x_scale);
 *   2. w8, w8_t = cast_transpose(W, *w_scale) E4M3, amax into *w_amax, *w_scale_inv written;
 *      skipped on the device when w_noop != NULL and *w_noop == 1.0f (cached weight);
 *   3. y = gemm_bias(x8, w8) with *x_scale_inv, *w_scale_inv and bias.
 * Steps 1 and 2 are one kernel launch when both tensors take the same cast code path (M and N
 * both multiples of 16 with K a multiple of 8, or neither), else two.  A small layer (x8_t
 * NULL, K = 256, 512 or 1024, N % 16 == 0, at most 256 x 256 / K output blocks of 64 x 64 and
 * fewer than 40 of 256 x 256) runs all three steps as one launch, in which each block casts the x and W rows of
 * its output tile (32 x 32 tiles up to 128 blocks of 64 x 64, 64 x 64 tiles beyond).  The
 * results are those of the separate calls in every case, bit for bit.
 * x: [M, K], W: [N, K], bias: [N] or NULL (bfloat16).  x8: [M, K], x8_t: [K, M] or NULL,
 * w8: [N, K], w8_t: [K, N] codes.  y: [M, N] bfloat16.  K % 16 == 0.
 */
int fp8_linear_fwd(const uint16_t *x, const uint16_t *w, const uint16_t *bias,
                   int64_t M, int64_t N, int64_t K,
                   const float *x_scale, float *x_amax, uint8_t *x8, uint8_t *x8_t, float *x_scale_inv,
                   const float *w_scale, float *w_amax, uint8_t *w8, uint8_t *w8_t, float *w_scale_inv,
                   const float *w_noop, uint16_t *y, hipStream_t stream);

/*
 * fp8_linear_bwd -- backward of the FP8 linear layer ([CG] transpose-cache thread,
 * DbiasCastTranspose.backward and FP8Linear.backward).  Launch sequence on `stream`:
 *   1. dbias, dy8, dy8_t = dbias_cast_transpose(dy, *dy_scale) E5M2, amax into *dy_amax,
 *      *dy_scale_inv = 1/(*dy_scale);
 *   2. dgrad dx[M, K] = gemm(dy8 [M, N] E5M2, w8_t [K, N] E4M3), bfloat16;
 *   3. wgrad dW[N, K] = gemm(dy8_t [N, M] E5M2, x8_t [K, M] E4M3), bfloat16 or float32.
 * dy: [M, N] bfloat16.  dbias: [N] float32 or NULL (then no bias gradient is formed and the
 * plain cast_transpose is used).  workspace: fp8_dbias_workspace_bytes(M, N) bytes when dbias
 * is given, zero-filled before its first use as for fp8_dbias_cast_transpose (every call leaves
 * its counters zero).  x8_t, w8_t and their inverse scales come from the forward.  M % 16 == 0 and
 * N % 16 == 0 (they are the contraction lengths of wgrad and dgrad).
 */
int fp8_linear_bwd(const uint16_t *dy, int64_t M, int64_t N, int64_t K,
                   const float *dy_scale, float *dy_amax, uint8_t *dy8, uint8_t *dy8_t,
                   float *dy_scale_inv, float *dbias, void *workspace, size_t workspace_bytes,
                   const uint8_t *x8_t, const float *x_scale_inv,
                   const uint8_t *w8_t, const float *w_scale_inv,
                   uint16_t *dx, void *dw, int dw_dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8DS_H */
