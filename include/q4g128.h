/*
 * q4g128.h -- C ABI of libq4g128.so: the int4-g128 weight-streaming product
 *
 *     y[M][N] = x[M][K] . dequant(W)[K][N],   1 <= M <= 16
 *
 * on AMD Instinct MI355X (gfx950).  M = 1 is a plain decode step; M = 2..16
 * is a speculative verify step that checks a draft of M - 1 tokens plus the
 * next one in one pass (Token Rush README, steps table rows 13-14 and 28:
 * verifying 7 draft tokens; bw24 article, feature list: draft depths up to
 * 8, i.e. 9 rows).  Decode is bound by streaming
 * the weights (Token Rush README, bandwidth paragraph), so the library reads
 * every weight byte once per call, for all M rows together.
 *
 * Weight format (Token Rush README, weight format paragraph): group-wise
 * asymmetric int4, 128 consecutive weights along K per bf16 scale s and bf16
 * minimum m, w = q*s + m for a 4-bit code q, 4.25 bits per weight.
 *
 * Layouts (all row-major, all DEVICE memory owned by the caller):
 *   x      bf16  [M][K]      activation rows
 *   W      uint32 [N][K/8]   codes of output column n; nibble i (bits 4i..4i+3,
 *                            low nibble first) of word j holds code k = 8j + i
 *   scale  bf16  [N][K/128]  scale of column n, group k/128
 *   min    bf16  [N][K/128]  minimum of column n, group k/128
 *   y      fp32  [M][N]      output, fully overwritten, never accumulated into
 *
 * Arithmetic: fp32 accumulation.  For every (K, N) the library fixes one
 * summation order that is the same for every M and every row, so row m of an
 * M-row call equals the one-row call on x[m] bit for bit (bw24 article,
 * exactness paragraph: a verify pass may only be accepted if it reproduces
 * plain decode exactly, and two reductions that differ only in the order of
 * their additions can already break that).  Results are deterministic run to
 * run; the library uses no atomics on results.
 *
 * Conventions for every call below:
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *     work on it and return without synchronising.
 *   - Argument errors return Q4G128_EINVAL (null pointer, M outside [1, 16],
 *     K <= 0, K > 2^24 or K % 128 != 0, N <= 0 or N > 2^28, splits > 65535,
 *     x or W or w_out not 16-byte aligned,
 *     scale or min not 2-byte aligned, y or workspace not 4-byte aligned,
 *     splits outside [1, K/128]) or Q4G128_EWORKSPACE (workspace too small),
 *     always before anything is enqueued.
 *   - A failed kernel launch returns Q4G128_EHIP; q4g128_last_error() then
 *     holds the HIP error text for the calling thread.  An error left pending
 *     on the thread by an earlier, unrelated HIP call is cleared before this
 *     call's launches, so EHIP always reports this call's own launches.
 *   - Outputs must not alias inputs.  The library allocates no memory and is
 *     safe to call from several threads: its only host-side state is
 *     per-device caches of device properties and kernel attributes, held in
 *     atomics and written with the same value by every thread that fills
 *     them.  A split-K workspace must not be shared by calls in flight at
 *     once.
 */
#ifndef Q4G128_H
#define Q4G128_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4G128_ABI_VERSION 1
#define Q4G128_GROUP 128
#define Q4G128_MAX_M 16
#define Q4G128_QUANT_MAX_CAND 16

typedef enum {
    Q4G128_OK = 0,
    Q4G128_EINVAL = 1,
    Q4G128_EWORKSPACE = 2,
    Q4G128_EHIP = 3
} q4g128_status;

/* The product without splitting K: one kernel launch, y written directly.
 * Best for wide N (N/16 well above the compute-unit count).  Short-N shapes
 * whose one-launch form cuts K into parts (q4g128_gemm_parts > 1) hold only
 * a few rows per launch and run wider M as launches over row blocks, each
 * streaming the weights again (17408 -> 5120: 2 rows per launch); for those
 * at M > 1, q4g128_gemm_splitk with the default split count gives the same
 * bits and streams the weights once.
 * Passages: Token Rush README, bandwidth and weight format paragraphs
 * (decode as one pass over the streamed weights; the format), steps table row
 * 3 (an int4 GEMV with projections fused side by side along N). */
q4g128_status q4g128_gemm(const void *x, int M, int K,
                          const uint32_t *W, const void *scale, const void *min,
                          int N, float *y, void *stream);

/* Bytes of workspace q4g128_gemm_splitk needs: splits * M * N * 4 (fp32
 * partial sums P[s][m][n], one slice per split).  Returns 0 for invalid
 * arguments.  Passage: Token Rush README, steps table rows 8-9 (a split-K
 * GEMV: each K range leaves a partial sum that is added up afterwards). */
size_t q4g128_splitk_workspace_bytes(int M, int N, int splits);

/* Split count the library recommends for a (K, N) shape: a function of K, N
 * and the current device's compute-unit count only (never of M, so rows
 * stay bit-identical across M), always whole blocks of 8 groups.  1 means
 * "do not split"; returns 0 for invalid K or N.  Passages: Token Rush README,
 * steps table rows 8-9 (split-K for the short-N projections) and bandwidth
 * paragraph (decode runs at the rate the weights stream, so a short-N shape
 * is split until every compute unit has enough of them in flight). */
int q4g128_splitk_default_splits(int K, int N);

/* K parts of q4g128_gemm's one-launch form for a (K, N) shape on the
 * current device (1 if that form does not cut K): q4g128_gemm_splitk with
 * this many splits gives the bits of q4g128_gemm, for every M.  A function
 * of K, N and the compute-unit count; 0 for invalid K or N. */
int q4g128_gemm_parts(int K, int N);

/* The product with K cut into `splits` contiguous ranges, 1 <= splits <=
 * K/128.  With nb = ceil(K/1024) blocks of 8 groups and splits <= nb, split s
 * covers blocks [s*nb/splits, (s+1)*nb/splits); with more splits than
 * blocks, split s covers the groups [s*G/splits, (s+1)*G/splits), G = K/128
 * (every split at least one group).  Each range writes fp32 partial sums to
 * the workspace; a second pass sums them in ascending s into y.
 * Deterministic; for splits == 1 it computes exactly what q4g128_gemm
 * computes.  For short N, where one column per lane gives too little
 * parallelism.  Passage: Token Rush README, steps table rows 8-9
 * (a split-K GEMV whose partial sums are added afterwards). */
q4g128_status q4g128_gemm_splitk(const void *x, int M, int K,
                                 const uint32_t *W, const void *scale, const void *min,
                                 int N, float *y, int splits,
                                 float *workspace, size_t workspace_bytes,
                                 void *stream);

/* q4g128_gemm_splitk without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The partial sums go to a
 * scratch array the library holds in device memory: 8 MiB (8388608 bytes)
 * per GPU, allocated when the library's code is loaded on that GPU and held
 * until the process ends.  Same arguments, results and bits as
 * q4g128_gemm_splitk; calls nothing that allocates.  Returns
 * Q4G128_EWORKSPACE (with a q4g128_last_error() text) before anything is
 * enqueued if splits * M * N * 4 exceeds 8 MiB.  Every call on one GPU
 * shares that GPU's scratch: calls that overlap in time on one GPU (other
 * streams, other threads) race on it and must be serialised by the caller;
 * calls in order on one stream are safe.  The scratch keeps the last call's
 * partial sums; nothing in it needs clearing (each call overwrites every
 * partial it reads). */
q4g128_status q4g128_gemm_splitk_noalloc(const void *x, int M, int K,
                                         const uint32_t *W, const void *scale, const void *min,
                                         int N, float *y, int splits, void *stream);

/* Bytes of workspace q4g128_gemm_streamk needs for a (K, N) shape: 2 MiB of
 * partial-sum slots plus 4 * ceil(N/16) bytes of counters, rounded up to
 * 256.  Independent of M.  Returns 0 if the shape is not supported (K not a
 * positive multiple of 1024, N outside [1, 2^28]). */
size_t q4g128_streamk_workspace_bytes(int K, int N);

/* The product with the work spread evenly over the compute units (stream-K):
 * one workgroup per compute unit, each wave an equal contiguous share of the
 * (16-column tile, 1024-k block) units.  A tile split between waves is
 * summed in parts; the last wave to finish it adds the parts in a fixed
 * order (determined by K, N and the device's compute-unit count), so results
 * are deterministic and rows are bit-identical across M, but they differ in
 * rounding from q4g128_gemm.  Passages: Token Rush README, bandwidth
 * paragraph (decode is bound by streaming the weights: every CU must stream
 * its share at full rate) and steps table rows 8-9 (partial sums over K).
 *
 * Requirements beyond the common ones: M <= 8; K % 1024 == 0; scale and min 16-byte
 * aligned; workspace 256-byte aligned, at least
 * q4g128_streamk_workspace_bytes(K, N) bytes, ZERO-FILLED before its first
 * use.  Every call leaves the counters it used at zero again, so a workspace
 * can be reused call after call, but not by two calls in flight at once.
 * Returns Q4G128_EINVAL for an unsupported shape (large K is cut into slices
 * internally; shapes whose slices cannot hold 8 rows of x are rejected). */
q4g128_status q4g128_gemm_streamk(const void *x, int M, int K,
                                  const uint32_t *W, const void *scale, const void *min,
                                  int N, float *y, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* Bytes of workspace q4g128_gemm_swiglu needs for (M, K, N):
 * splits * M * N * 4, splits the larger of q4g128_splitk_default_splits(K, N)
 * and the fused launch's K-part count (the partial sums of the calls the
 * fused launch cannot take).  Returns 0 for invalid arguments (N must be
 * even). */
size_t q4g128_swiglu_workspace_bytes(int M, int K, int N);

/* The product on a fused gate/up matrix followed by the SwiGLU activation:
 * N = 2I, output columns 0..I-1 of W are the gate projection and I..2I-1
 * the up projection (Token Rush README, steps table row 3: projections fused
 * side by side along N), and
 *
 *     act[m][i] = bf16( silu(g) * u ),  silu(g) = g / (1 + exp(-g)),
 *     g = y[m][i], u = y[m][I + i]   (y the fp32 product q4g128_gemm gives),
 *
 * in fp32, rounded once to bf16 (nearest even), act bf16 [M][I] 2-byte
 * aligned.  The activation is the gated MLP of the model family the pages
 * run; the pages do not spell it out.  When the shape allows (K a multiple
 * of 1024, scale and min 16-byte aligned, x small enough for the staging
 * and the LDS), one launch computes each
 * gate tile and its up tile on the same compute unit and applies the
 * activation before anything is stored; otherwise the product's split-K
 * partial sums go to the workspace and a second launch sums them (ascending
 * split order) and applies it.  Both give the same bits, rows are
 * bit-identical across M, and y itself is never written.  The workspace
 * (q4g128_swiglu_workspace_bytes) is required either way and must not be
 * shared by calls in flight. */
q4g128_status q4g128_gemm_swiglu(const void *x, int M, int K,
                                 const uint32_t *W, const void *scale, const void *min,
                                 int N, void *act, float *workspace, size_t workspace_bytes,
                                 void *stream);

/* Bytes of workspace q4g128_gemm_rmsnorm needs: 256 (a control block) +
 * q4g128_splitk_workspace_bytes(M, N, splits).  Returns 0 for invalid
 * arguments. */
size_t q4g128_rmsnorm_workspace_bytes(int M, int N, int splits);

/* The product followed by a residual add and RMSNorm, with the split-K
 * partial sums added inside the norm (Token Rush README, steps table rows
 * 8-9: a split-K GEMV whose partials are summed in the norm):
 *
 *     h[m][n]     = residual[m][n] + y[m][n]                    (fp32)
 *     x_out[m][n] = bf16( h[m][n] * inv[m] * gamma[n] ),
 *     inv[m]      = 1 / sqrt( (sum over n of h[m][n]^2) / N + eps )
 *
 * y is the product with K cut into `splits` ranges exactly as in
 * q4g128_gemm_splitk (splits == 1: not cut), its partials summed in
 * ascending split order, so h equals fp32(residual + y_splitk) bit for bit.
 * The sum of squares is taken in a fixed order: 256 partial sums, partial p
 * the fused multiply-add chain over the columns n = p, p+256, p+512, ...
 * (n < N) in ascending n; then a fixed tree over the 256.  The square root and division are correctly rounded.
 * residual and h fp32 [M][N] (h may be the residual itself, updated in
 * place; 4-byte aligned); gamma bf16 [N]; x_out bf16 [M][N] (the next
 * product's input; 2-byte aligned); eps >= 0.  x_out == NULL: the residual
 * add alone (h only; gamma and eps are not read), for a caller that lets the
 * next product normalise h itself (q4g128_gemm_prenorm).  The RMSNorm
 * formula is the usual one of the model family the pages run; the pages do
 * not spell it out.  Rows are bit-identical across M; results deterministic.
 *
 * When `splits` equals q4g128_gemm_parts(K, N) > 1 and the M rows fit that
 * launch's LDS (M <= 8; x for all of K is held there, so 17408 -> 5120 takes
 * one row), the whole call is one launch: each workgroup adds the
 * residual to its own columns, and the workgroup that finishes last (found
 * by a counter) normalises the rows.  Otherwise the partials go to the
 * workspace and a second launch sums them and normalises.  Both give the
 * same bits.  (The last workgroup's pass over the rows costs about 3 us on
 * 17408 -> 5120; moving the norm into the next product, q4g128_gemm_prenorm
 * with x_out == NULL here, costs about 0.1 us here.)
 *
 * Workspace: at least q4g128_rmsnorm_workspace_bytes(M, N, splits) bytes,
 * 4-byte aligned.  Its first 256 bytes are a control block that must hold
 * zeros when the workspace is first given to this function (clear it once,
 * e.g. with hipMemset); every call that completes leaves them zero again.
 * No other call may write them in between, and calls in flight must not
 * share a workspace. */
q4g128_status q4g128_gemm_rmsnorm(const void *x, int M, int K,
                                  const uint32_t *W, const void *scale, const void *min,
                                  int N, const float *residual, const void *gamma, float eps,
                                  float *h, void *x_out, int splits,
                                  float *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace q4g128_gemm_prenorm (swiglu == 0) or
 * q4g128_gemm_swiglu_prenorm (swiglu != 0) needs: M*K*2 rounded up to 256
 * (x, when it is made in a launch of its own), plus for swiglu
 * q4g128_swiglu_workspace_bytes(M, K, N).  Returns 0 for invalid arguments. */
size_t q4g128_prenorm_workspace_bytes(int M, int K, int N, int swiglu);

/* The product of a normalised input: with fp32 rows h [M][K],
 *
 *     x[m][k] = bf16( h[m][k] * inv[m] * gamma[k] ),
 *     inv[m]  = 1 / sqrt( (sum over k of h[m][k]^2) / K + eps ),
 *     y       = x . dequant(W)                          (as q4g128_gemm)
 *
 * x is bit for bit the x_out q4g128_gemm_rmsnorm gives for rows h (same sum
 * of squares order), and y bit for bit q4g128_gemm on that x.  This is the
 * decoder's pre-norm: the residual stream h (q4g128_gemm_rmsnorm with
 * x_out == NULL keeps it) is normalised inside the product that consumes it
 * (the q/k/v projection, the gate/up projection, the output head) instead of
 * in a launch of its own (Token Rush README, steps table: norm, then the
 * projections).  One launch when the shape's one-launch plan takes it (M <=
 * 6; h and gamma 16-byte aligned, scale and min too): every workgroup reads
 * the whole rows of h and gamma while it stages x.  Otherwise x goes to the
 * workspace first (from 7 rows that pair of launches is the faster).  h fp32 [M][K] (4-byte aligned), gamma bf16 [K] (2-byte
 * aligned), eps >= 0, y fp32 [M][N]; workspace: at least
 * q4g128_prenorm_workspace_bytes(M, K, N, 0) bytes, 256-byte aligned, not
 * shared by calls in flight.  Other requirements as q4g128_gemm. */
q4g128_status q4g128_gemm_prenorm(const float *h, const void *gamma, float eps, int M, int K,
                                  const uint32_t *W, const void *scale, const void *min,
                                  int N, float *y, float *workspace, size_t workspace_bytes,
                                  void *stream);

/* q4g128_gemm_swiglu on x = the normalised h above: act [M][N/2] =
 * bf16(silu(gate) * up), bit for bit q4g128_gemm_swiglu on that x.
 * Workspace: q4g128_prenorm_workspace_bytes(M, K, N, 1). */
q4g128_status q4g128_gemm_swiglu_prenorm(const float *h, const void *gamma, float eps, int M, int K,
                                         const uint32_t *W, const void *scale, const void *min,
                                         int N, void *act, float *workspace, size_t workspace_bytes,
                                         void *stream);

/* Decoded weights w_out[n][k] = fp32(q*s + m), rounded once (fma), laid out
 * fp32 [N][K].  Uses the same device unpacking as the product; it exists so
 * tests can compare the unpack and dequant bit for bit.  Passage: Token Rush
 * README, weight format paragraph. */
q4g128_status q4g128_dequant(const uint32_t *W, const void *scale, const void *min,
                             int K, int N, float *w_out, void *stream);

/* Quantize bf16 weights into the format above.  w is bf16 [N][K] (row n
 * holds the K weights of output column n, K a multiple of 128); the outputs
 * W [N][K/8], scale and min [N][K/128] are the layouts the product reads,
 * and err [N][K/128] fp64 (may be NULL) receives each group's squared
 * dequantisation error sum_k (q*s + m - w)^2.
 *
 * Per group the codes come from a search over clipped ranges scored by
 * squared error (Token Rush README, quantization section: narrowing a
 * group's range past its extremes buys a finer step for the other weights).
 * With
 * lo, hi the group's extremes and c their midpoint, candidate (i, j),
 * 0 <= i, j < ncand, taken in the order i*ncand + j, uses the range
 * [lo + (i/20)(c - lo), hi - (j/20)(hi - c)], scale s = (range width)/15 and
 * minimum = the range's low end, each rounded fp64 -> fp32 -> bf16 (nearest
 * even), codes clamp(rint((w - min)/s), 0, 15) (all 0 if s rounds to 0); the
 * first candidate with the smallest error wins.  ncand = 1 is plain
 * round-to-nearest over the full range.  All arithmetic is fp64 with no
 * fused multiply-adds, so the result is deterministic and bit-reproducible.
 *
 * Requirements beyond the common ones: 1 <= ncand <= 16; w and W 16-byte
 * aligned, scale and min 2-byte aligned, err 8-byte aligned.  A group that
 * holds a NaN or an infinity gets codes 0, scale 0, min 0 and err NaN (the
 * call itself succeeds: check err when the input may hold such values). */
q4g128_status q4g128_quantize(const void *w, int K, int N, int ncand, uint32_t *W, void *scale, void *min,
                              double *err, void *stream);

/* Static text for a status code. */
const char *q4g128_status_string(q4g128_status s);

/* Last HIP error text recorded on the calling thread ("" if none). */
const char *q4g128_last_error(void);

/* Q4G128_ABI_VERSION of the loaded library. */
int q4g128_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4G128_H */
