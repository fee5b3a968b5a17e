/*
 * ttt.h -- C ABI of libttt.so, the MI355X (gfx950) large-chunk test-time-training
 * (LaCT) layer: ShortConv2D on V, the fast-weight update, and apply.
 *
 * Sources (page title, then section / equation):
 *   [Scal3R]  "Scal3R: Scalable Test-Time Training for Large-Scale 3D Reconstruction"
 *             -- 一.2 eqs. (3) update, (4) apply; 三 方案1 eq. (9) dot-product loss.
 *   [tttLRM]  "tttLRM: Test-Time Training for Long Context and Autoregressive 3D
 *             Reconstruction" -- 方法步骤详情: W = Update({T_i}), T_i = Apply(W, T_i),
 *             query-only virtual tokens.
 *   [VGG-T3]  "VGG-T3: Offline Feed-Forward 3D Reconstruction at Scale" -- 关键设计 2
 *             (ShortConv2D V -> V'), 关键设计 3 (two inner steps), 损失函数与训练.
 *   [ZipMap]  "ZipMap: Linear-Time Stateful 3D Reconstruction via Test-Time Training"
 *             -- 关键设计 1 (f_W, loss, one-pass gradient with per-token eta_i,
 *             apply), 关键设计 3 (Newton-Schulz), 关键设计 4 (streaming TTTUpdate).
 *   [LoGeR]   "LoGeR: Long-Context Geometric Reconstruction with Hybrid Memory" --
 *             方法概览 (fast weights updated per chunk, carried to later chunks).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Shapes.  H heads, per-head width d, SwiGLU hidden width m.  Supported: d a
 *   multiple of 64 in [64, 1024], m a positive multiple of 64 (the 64-wide MFMA
 *   tile); anything else returns TTT_EUNSUPPORTED.  Kernel choice (results agree
 *   within the bf16 tolerance either way): bf16 tokens with d in {64, 128, 256} run
 *   the fused fast kernels; bf16 with d in {512, 768, 1024} and m % 256 == 0 run the
 *   wide-head kernels (the gradient and apply split at the hidden layer into dense
 *   products); every other shape, and fp32 tokens, run the general kernels, which
 *   read their operands from L1/L2 and are roughly 20-40x slower than the fast or
 *   wide kernels on the same work (about 20 TFLOP/s at d = 1024, m = 2048).
 * Fast weights, always fp32, caller-owned DEVICE memory, contiguous:
 *   w1, w3: [H][m][d]   (row j of head h multiplies the key: z = W1 k)
 *   w2:     [H][d][m]   (f_W(x) = W2 (SiLU(W1 x) o (W3 x)))
 * Token rows (K, V, V', Q, O), caller-owned DEVICE memory, row-major [rows][ld]
 *   elements with ld >= H*d; head h uses columns [h*d, (h+1)*d).  Element type
 *   is `dtype` (TTT_F32 or TTT_BF16, bf16 = IEEE binary32 upper half, RNE).
 *   Rows must start on 16-byte boundaries: (ld * element size) % 16 == 0 and
 *   the base pointer 16-byte aligned.
 * Per-token rates eta: fp32 DEVICE memory, eta[h * eta_head_stride + i];
 *   eta_head_stride = 0 shares one rate per token across heads.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = default stream).
 *   Every call is asynchronous on that stream; the caller synchronises.
 * Workspace.  The library allocates no device memory.  Entry points that need
 *   scratch take a caller-owned DEVICE buffer of at least the size reported
 *   by the matching *_workspace_bytes query (256-byte aligned).
 * Errors.  Every function returns a ttt_status.  Nothing is launched when the
 *   return is TTT_EINVAL / TTT_EUNSUPPORTED / TTT_EWORKSPACE.  TTT_EHIP means a
 *   HIP launch failed; ttt_last_error() then holds hipGetErrorString's text.
 *   No exception crosses this boundary.
 */
#ifndef TTT_H_
#define TTT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TTT_OK = 0,
  TTT_EINVAL = -1,        /* null pointer, negative size, ld too small, steps < 1, ... */
  TTT_EUNSUPPORTED = -2,  /* d or m outside the supported set, unknown dtype */
  TTT_EWORKSPACE = -3,    /* workspace missing or smaller than the query says */
  TTT_EHIP = -4           /* a HIP call failed (message in ttt_last_error) */
} ttt_status;

typedef enum { TTT_F32 = 0, TTT_BF16 = 1 } ttt_dtype;

/* Thread-local text describing the last non-zero status on this thread. */
const char *ttt_last_error(void);

/* Bytes of workspace ttt_update needs for these shapes (0 is never returned). */
int ttt_update_workspace_bytes(int32_t heads, int32_t d, int32_t m, int64_t n,
                               int32_t dtype, size_t *bytes);

/* Bytes of workspace ttt_apply needs (0 in fp32 mode: it reads W directly). */
int ttt_apply_workspace_bytes(int32_t heads, int32_t d, int32_t m, int64_t nq,
                              int32_t dtype, size_t *bytes);

/*
 * ttt_update -- the chunk-wise fast-weight update, repeated `steps` times.
 *
 * [Scal3R] 方案1 and [ZipMap] 关键设计 1: one gradient over every token,
 *   G = grad_W sum_i eta_i * (-f_W(k_i)^T v_i),
 * [ZipMap] 关键设计 3: orthogonalise each of G1, G3, G2 with Muon's quintic
 *   Newton-Schulz (a, b, c) = (3.4445, -4.7750, 2.0315), 5 iterations, on
 *   G / (||G||_F + 1e-7), transposed while it has more rows than columns,
 * then W <- W - lr * NS(G) for W1, W3, W2 simultaneously; [VGG-T3] 关键设计 3:
 *   steps = 2 recomputes G at the new W on the same tokens.
 *
 * w1, w3, w2      : input fast weights (fp32, device, layout above).
 * w1_out..w2_out  : output fast weights; each may equal its input pointer
 *                   (in-place update) or must not overlap it at all.
 * k, v            : [n][ld_kv] keys and (already conv-mixed) values, `dtype`.
 * eta             : per-token rates, see conventions.
 * n               : tokens (>= 0; n = 0 gives G = 0, NS(G) = 0, W unchanged).
 *                   At most 2^31 - 65 per call, and 32 rows of ld_kv must span
 *                   < 2 GiB (TTT_EUNSUPPORTED otherwise; ttt_stream applies the
 *                   limit per chunk).
 * lr              : step size (lr = 0 leaves W bit-identical).
 * steps           : inner steps, >= 1.
 * grad_out, ns_out: optional (NULL to skip), 3*H*m*d floats each, device:
 *                   the last step's G and NS(G) packed as [G1 | G3 | G2] with
 *                   the shapes of w1, w3, w2.
 * workspace       : >= ttt_update_workspace_bytes(H, d, m, n, dtype).
 * The result is deterministic: the same inputs give the same bits.
 */
int ttt_update(int32_t heads, int32_t d, int32_t m,
               const float *w1, const float *w3, const float *w2,
               float *w1_out, float *w3_out, float *w2_out,
               const void *k, const void *v, int64_t ld_kv,
               const float *eta, int64_t eta_head_stride,
               int64_t n, float lr, int32_t steps, int32_t dtype,
               float *grad_out, float *ns_out,
               void *workspace, size_t workspace_bytes, void *stream);

/*
 * ttt_update_ex -- ttt_update with option flags (ttt_update is flags = 0).
 *
 * TTT_NORM_PRESERVE: [ZipMap] 关键设计 3's norm-preserving step.  Each step
 *   replaces W <- W - lr * NS(G) by
 *     W <- ||W||_F * (W - lr * NS(G)) / ||W - lr * NS(G)||_F
 *   for every weight matrix of every head separately (Frobenius norms, ||W||
 *   taken before the step; lr = 1 is the page's form with Delta = NS(g)).  If
 *   W - lr * NS(G) is exactly zero the matrix becomes zero.  The norms are fp32
 *   sums of squares in a fixed order, so results stay deterministic.
 * Other bits are reserved: TTT_EINVAL.  Every other argument is as in ttt_update;
 * the workspace size is the same.
 */
enum { TTT_NORM_PRESERVE = 1 };
int ttt_update_ex(int32_t heads, int32_t d, int32_t m,
                  const float *w1, const float *w3, const float *w2,
                  float *w1_out, float *w3_out, float *w2_out,
                  const void *k, const void *v, int64_t ld_kv,
                  const float *eta, int64_t eta_head_stride,
                  int64_t n, float lr, int32_t steps, int32_t dtype, uint32_t flags,
                  float *grad_out, float *ns_out,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * ttt_update_noalloc -- ttt_update_ex without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The call itself allocates nothing (no hipMalloc,
 * hipFree or allocating library routine, no timing events even when
 * ttt_profile_enable is on); it takes its scratch from a library-owned device array of
 * ttt_noalloc_scratch_bytes() bytes (128 MiB), which every GPU that runs the library
 * holds from the first call on that device until the process ends.
 *
 * Every argument means what it means for ttt_update_ex, and the kernels and the
 * result are the same: bit-identical to ttt_update_ex on the same inputs.
 * Limit: the update's scratch (ttt_update_workspace_bytes for the same shapes) must
 *   fit the array: about 87 MiB for 4 heads of 256 with hidden 512 (any n), 1.4 MiB
 *   for one 64/128 head.  The wide-head path's intermediates grow with n and do not
 *   fit at large n.  A larger need returns TTT_EWORKSPACE before anything runs.
 * Sharing: every call on one GPU uses that GPU's one array, and the array keeps the
 *   last call's contents (each call clears what it needs at zero).  Calls that may
 *   overlap on one GPU (other host threads, other streams) race on it: the caller
 *   must serialise them.
 */
int ttt_update_noalloc(int32_t heads, int32_t d, int32_t m,
                       const float *w1, const float *w3, const float *w2,
                       float *w1_out, float *w3_out, float *w2_out,
                       const void *k, const void *v, int64_t ld_kv,
                       const float *eta, int64_t eta_head_stride,
                       int64_t n, float lr, int32_t steps, int32_t dtype, uint32_t flags,
                       float *grad_out, float *ns_out, void *stream);
/* Size of the array ttt_update_noalloc works in (bytes). */
int ttt_noalloc_scratch_bytes(size_t *bytes);

/*
 * ttt_update_host -- ttt_update_ex with K, V and eta in HOST memory, streamed to
 * the GPU in batches of `batch` tokens ([VGG-T3] 关键发现 2 and 亮点 2: the TTT
 * objective is a sum over tokens, so the gradient of any token set is the sum of
 * its minibatches' gradients, and sets larger than device memory can be
 * processed with the minibatches offloaded to the CPU).
 *
 * For each inner step, every batch is copied host -> device into one of two
 * staging slots of the workspace (on a copy stream the library creates once per
 * device, default priority) while the previous batch's gradient runs on `stream`;
 * each batch's gradient is added to a running fp32 G in a fixed order, and the
 * optimiser step (Newton-Schulz, W update, TTT_NORM_PRESERVE) then runs on G as in
 * ttt_update_ex.  steps = 2 streams the tokens twice.  The result equals
 * ttt_update_ex on the same tokens up to the fp32 order of the sum over tokens;
 * it is deterministic for a given batch.
 *
 * k, v      : HOST rows [n][ld_kv] (`dtype`); (ld_kv * element size) % 16 == 0.
 *             Page-locked memory (hipHostMalloc) lets the copies overlap the
 *             kernels; pageable memory works but copies synchronously.
 * eta       : HOST rates, eta[h * eta_head_stride + i] (stride 0: shared).
 * w*, w*_out: DEVICE fast weights as in ttt_update_ex.
 * batch     : tokens per staged batch (>= 1; the limits of ttt_update apply to it).
 * workspace : DEVICE, >= ttt_update_host_workspace_bytes(H, d, m, batch, ld_kv, dtype).
 * Host buffers must stay unchanged until the work on `stream` has completed.
 */
int ttt_update_host_workspace_bytes(int32_t heads, int32_t d, int32_t m, int64_t batch, int64_t ld_kv,
                                    int32_t dtype, size_t *bytes);
int ttt_update_host(int32_t heads, int32_t d, int32_t m,
                    const float *w1, const float *w3, const float *w2,
                    float *w1_out, float *w3_out, float *w2_out,
                    const void *k, const void *v, int64_t ld_kv,
                    const float *eta, int64_t eta_head_stride,
                    int64_t n, int64_t batch, float lr, int32_t steps, int32_t dtype, uint32_t flags,
                    float *grad_out, float *ns_out,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * ttt_apply -- o_i = f_W(q_i) for every row ([Scal3R] eq. (4); [ZipMap]
 * 关键设计 1; [tttLRM] query-only tokens use the same call).
 *
 * q : [nq][ld_q] queries, `dtype`.   o : [nq][ld_o] outputs, `dtype`;
 * q and o must not overlap.  workspace: >= ttt_apply_workspace_bytes(...)
 * (may be NULL when that is 0).
 */
int ttt_apply(int32_t heads, int32_t d, int32_t m,
              const float *w1, const float *w3, const float *w2,
              const void *q, int64_t ld_q, void *o, int64_t ld_o,
              int64_t nq, int32_t dtype,
              void *workspace, size_t workspace_bytes, void *stream);

/*
 * ttt_shortconv2d -- V' = ShortConv2D(V), [VGG-T3] 关键设计 2: every frame's
 * grid_h x grid_w patch tokens (row-major, after its n_special leading tokens)
 * form an image with `channels` channels; each channel is cross-correlated with
 * its own 3x3 taps, zero padding 1, stride 1, no bias:
 *   V'[y,x,c] = sum_{dy,dx in -1..1} wconv[c][dy+1][dx+1] * V[y+dy, x+dx, c].
 * The n_special tokens are copied unchanged.
 *
 * v, v_out : [frames*tokens_per_frame][ld] device rows, `dtype`; must not overlap.
 * wconv    : [channels][3][3] fp32, device.
 * Requires tokens_per_frame == n_special + grid_h*grid_w, channels % 8 == 0,
 * channels <= ld.
 */
int ttt_shortconv2d(const void *v, void *v_out, int64_t ld, const float *wconv,
                    int32_t frames, int32_t tokens_per_frame, int32_t n_special,
                    int32_t grid_h, int32_t grid_w, int32_t channels,
                    int32_t dtype, void *stream);

/*
 * ttt_output_gate -- [ZipMap] 关键设计 3's gated output unit, applied to the
 * output rows o'_i of ttt_apply:
 *   o_i = RMSNorm(o'_i) * SiLU(W_g o'_i),
 *   RMSNorm(x)[c] = gamma[c] * x[c] / sqrt(mean_c'(x[c']^2) + eps),
 *   (W_g x)[c]    = sum_c' wg[c][c'] * x[c'],   SiLU(z) = z / (1 + e^-z).
 * A row is the whole C = `channels` wide output (all heads), the mean runs over
 * those C channels, and there is no bias.
 *
 * o_in, o_out : [n][ld_in] / [n][ld_out] device rows, `dtype`, columns [0, C)
 *               used; must not overlap each other or wg.
 * wg          : [C][C] row-major, `dtype`, device, 16-byte aligned.
 * gamma       : [C] fp32, device, 16-byte aligned.
 * eps         : >= 0, finite.
 * Requires C >= 64, C % 64 == 0, C <= ld_in, C <= ld_out, and the row
 * alignment of the conventions above.  n = 0 launches nothing.  The products
 * accumulate in fp32 (bf16 or fp32 MFMA operands, as `dtype`).
 */
int ttt_output_gate(int32_t channels, const void *o_in, int64_t ld_in, const void *wg, const float *gamma,
                    float eps, void *o_out, int64_t ld_out, int64_t n, int32_t dtype, void *stream);

/* Bytes of workspace ttt_stream needs for chunks of `chunk` tokens. */
int ttt_stream_workspace_bytes(int32_t heads, int32_t d, int32_t m, int64_t chunk,
                               int32_t dtype, size_t *bytes);

/*
 * ttt_stream -- causal chunked processing, [ZipMap] 关键设计 4 and [LoGeR]
 * 方法概览: for each chunk c of `chunk` consecutive tokens (the last may be
 * shorter):  O_c = f_W(Q_c);  then  W <- update(W, K_c, V_c, eta_c, lr, steps).
 * w1, w3, w2 are updated in place and hold the final state on return.
 * q, o: [n][ld_q] / [n][ld_o]; k, v: [n][ld_kv]; eta as in ttt_update with
 * token index i counted over the whole stream.
 * With bf16 tokens of d in {64, 128, 256}, each chunk's apply runs on a
 * library-owned side stream beside that chunk's first optimiser step (both read only
 * the chunk's starting weights); every piece of that work is ordered before any
 * work the caller enqueues on `stream` afterwards, and the results are those of
 * the sequential order, bit for bit.
 */
int ttt_stream(int32_t heads, int32_t d, int32_t m,
               float *w1, float *w3, float *w2,
               const void *k, const void *v, int64_t ld_kv,
               const float *eta, int64_t eta_head_stride,
               const void *q, int64_t ld_q, void *o, int64_t ld_o,
               int64_t n, int64_t chunk, float lr, int32_t steps, int32_t dtype,
               void *workspace, size_t workspace_bytes, void *stream);

/* ttt_stream with the flags of ttt_update_ex applied to every chunk's update. */
int ttt_stream_ex(int32_t heads, int32_t d, int32_t m,
                  float *w1, float *w3, float *w2,
                  const void *k, const void *v, int64_t ld_kv,
                  const float *eta, int64_t eta_head_stride,
                  const void *q, int64_t ld_q, void *o, int64_t ld_o,
                  int64_t n, int64_t chunk, float lr, int32_t steps, int32_t dtype, uint32_t flags,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Process-wide tuning / testing switches.
 *   TTT_OPT_FORCE_GENERAL: value != 0 routes every call through the general
 *     kernels (any d, both dtypes) instead of the d <= 256 bf16 fast kernels; the
 *     results agree within the bf16 tolerance.  Default 0.
 *   TTT_OPT_SPLITS: value > 0 fixes the number of token ranges the gradient is
 *     split into (0 = automatic, sized to fill the GPU).  Affects workspace size.
 *   TTT_OPT_NS_UNFUSED: value != 0 runs the split-K reduction, the Frobenius
 *     normalisation, each Newton-Schulz product, the weight step and the operand
 *     casts as separate kernels, instead of folding the normalisation, the step
 *     and the casts into the product kernels.  Same mathematics, different fp32
 *     rounding order; default 0 (folded).
 */
typedef enum { TTT_OPT_FORCE_GENERAL = 0, TTT_OPT_SPLITS = 1, TTT_OPT_NS_UNFUSED = 2 } ttt_option;
int ttt_set_option(int32_t option, int64_t value);

/*
 * Kernel timing (instrumentation, no effect on results).  When enabled, every
 * kernel the library launches is bracketed by hipEvents on its stream;
 * ttt_profile_read synchronises those events and returns, per kernel kind, the
 * summed milliseconds and the number of launches since the last reset.
 */
typedef enum {
  TTT_K_CONV = 0, TTT_K_CAST = 1, TTT_K_GRAD = 2, TTT_K_REDUCE = 3,
  TTT_K_NS = 4, TTT_K_APPLY = 5, TTT_K_GATE = 6, TTT_K_COUNT = 7
} ttt_kernel_kind;
int ttt_profile_enable(int32_t on);
int ttt_profile_reset(void);
int ttt_profile_read(int32_t kind, double *total_ms, int64_t *launches);

/*
 * ttt_mfma_rate_probe -- a measurement aid, not a step of the layer: launches, on
 * `stream`, one kernel in which every wave of two per SIMD on every compute unit
 * runs `iters` rounds of 8 independent 16x16x32 bf16 MFMA chains on register
 * operands (no memory traffic).  *flop (HOST) receives the launch's FLOP count
 * (2 x multiply-adds); the caller times the launch (e.g. with events on `stream`)
 * to get the matrix cores' sustained dense bf16 rate at the clock the chip keeps
 * under that load.  iters < 1 or flop == NULL: TTT_EINVAL, nothing launched.
 */
int ttt_mfma_rate_probe(int32_t iters, void *stream, double *flop);

#ifdef __cplusplus
}
#endif
#endif /* TTT_H_ */
