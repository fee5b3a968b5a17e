// Host-side declarations of the kernel launchers (one per .hip file).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ttt {

// Token blocks of the gradient kernels: 32 tokens (one bf16 MFMA reduction step).
constexpr int kTokBlock = 32;
// Hidden units per gradient workgroup (4 waves x 16).
constexpr int kHidTile = 64;

struct GradParams {
  const void *k, *v;         // [n][ld] token rows
  int64_t ld;
  const float *eta;          // eta[h * eta_hs + i]
  int64_t eta_hs;
  const void *w1, *w3;       // [H][m][d] operand-type copies (or fp32 master)
  const void *w2t;           // [H][m][d] transposed W2
  float *part;               // [splits][3][H][m*d] fp32 partial gradients
  int64_t n, nblk;           // tokens, ceil(n / kTokBlock)
  int heads, d, m, splits, dchunks, xcd_map;
  unsigned *group_sync;      // fast kernel: [H * splits] progress counters, zero at launch (or null)
};

struct ApplyParams {
  const void *q;
  int64_t ldq;
  void *o;
  int64_t ldo;
  const void *w1, *w3;       // [H][m][d]
  const void *w2;            // [H][d][m] (general kernels)
  const void *w2t;           // [H][m][d] transposed W2 (fast kernel)
  int64_t nq;
  int heads, d, m, dchunks;
};

// Kernel families.  `fast` variants: bf16 tokens with d in {64, 128, 256}
// (LDS-staged, register-resident weights); `general` variants: any supported d
// (a multiple of 64 up to 1024), fp32 or bf16.
bool grad_fast_supported(int d, bool bf16);
int grad_general_dc(int d, bool bf16);      // output d-chunk width of the general kernel
hipError_t launch_grad(const GradParams &p, int d, bool bf16, bool fast, int grid, hipStream_t s);
// Zeroes n 32-bit words (a kernel, not a memset, so that it can sit in a captured graph).
hipError_t launch_zero_u32(unsigned *p, int n, hipStream_t s);

bool apply_fast_supported(int d, bool bf16);
int apply_general_dc(int d, bool bf16);
hipError_t launch_apply(const ApplyParams &p, int d, bool bf16, bool fast, hipStream_t s);

// fp32 master W -> operand copies.  w1o/w3o: [H][m][d]; w2to: [H][m][d] (transposed W2);
// w2o: [H][d][m].  Any output may be null.  bf16 selects the output type.
// Dense bf16 MFMA rate probe: one launch of `iters` rounds on every compute unit;
// *flop receives the launch's multiply-add count x 2.
hipError_t launch_mfma_probe(int iters, hipStream_t s, double *flop);

hipError_t launch_cast(const float *w1, const float *w3, const float *w2, void *w1o, void *w3o,
                       void *w2to, void *w2o, int heads, int d, int m, bool bf16, hipStream_t s);

// Sum of split partials in fixed split order; also per-4096-element sums of squares.
hipError_t launch_reduce(const float *part, int splits, int64_t per_split, float *g, float *g_copy,
                         float *sumsq, hipStream_t s);

struct NsShape {
  int heads, d, m;           // matrices: 3*heads, G1/G3 [m][d], G2 [d][m]
};
// X = G / (||G||_F + eps), transposed to [min][max] where needed.
hipError_t launch_ns_normalize(const float *g, const float *sumsq, float *x, const NsShape &sh,
                               float eps, hipStream_t s);
// Batched C = alpha * A * op(B) + beta * D over `batch` matrices (fp32 MFMA).
struct GemmBatch {
  const float *a, *b, *dm;
  float *c;
  int M, N, K, lda, ldb, ldd, ldc, b_trans;
  int64_t sa, sb, sd, sc;
  float alpha, beta;
  int batch;
};
hipError_t launch_gemm_f32(const GemmBatch &g, hipStream_t s);
// W_out = W_src - lr * NS (NS taken from X, undoing the transpose); optional ns copy.
hipError_t launch_ns_step(const float *x, const float *w1, const float *w3, const float *w2, float *w1o,
                          float *w3o, float *w2o, float *ns_out, float lr, const NsShape &sh,
                          hipStream_t s);

// The optimiser step in 1 + 3*iters launches: reduce the split partials,
// Newton-Schulz with the Frobenius scale folded in, and W_out = W - lr * NS(G).
// Writes grad_out / ns_out ([3][H] matrices in G's layout) when non-null and the
// operand copies op1, op3 ([H][m][d]) and op2t (W2^T, [H][m][d]) when non-null
// (element type: bf16 when the launcher's bf16 flag is set, else fp32).
struct NsStepParams {
  const float *part;         // [splits][3][H][m*d]
  int splits;
  int64_t per_split;         // 3*H*m*d
  float *grad_out, *ns_out;
  float *sumsq;              // [3H][(m/64)(d/64)] tile sums of squares
  float *x[2], *xt[2];       // [3H][r][c] iterates and their transposes [3H][c][r]
  float *am, *bm;            // [3H][r][r]
  const float *w1, *w3, *w2;
  float *w1o, *w3o, *w2o;
  void *op1v, *op3v, *op2tv;
  float lr, eps, a_coef, b_coef, c_coef;
  int iters, heads, d, m, r, c;
  // Norm-preserving form: the last product writes the unscaled W - lr NS(G) and
  // per-tile sums of squares of W and of that result into wsq (layout of
  // launch_norm_rescale, (d/64)(m/64) slots per matrix) instead of operand copies.
  int norm_preserve;
  float *wsq;
};
// before_last (optional): an event the stream waits for before the last product, the
// one that writes W_out and the operand copies (so that work on another stream may
// read the old copies until then).
hipError_t launch_ns_optimiser(const NsStepParams &p, bool bf16, hipStream_t s, hipEvent_t before_last = nullptr);

// acc = (first ? 0 : acc) + sum_s part[s * per_split ..] (per_split % 4 == 0), fixed order.
hipError_t launch_accumulate(float *acc, const float *part, int splits, int64_t per_split, bool first,
                             hipStream_t s);

// Per-4096-element sums of squares of W1, W3, W2 in matrix order [3][H] (d*m/4096
// slots per matrix), written to out[0 .. 3H * slots).
hipError_t launch_weight_sumsq(const float *w1, const float *w3, const float *w2, float *out, int heads, int d,
                               int m, hipStream_t s);
// Norm-preserving rescale of each matrix b of W_out ([3][H] order):
//   W_out <- W_out * sqrt(sum wsq[b*slots ..]) / sqrt(sum wsq[(3H + b)*slots ..])
// (zero when the second sum is zero), then the operand copies op1, op3 ([H][m][d])
// and op2t (W2^T, [H][m][d]) of the result, each when non-null.
hipError_t launch_norm_rescale(float *w1o, float *w3o, float *w2o, const float *wsq, int slots, void *op1,
                               void *op3, void *op2t, int heads, int d, int m, bool bf16, hipStream_t s);

// Gated output o = gamma * o' / sqrt(mean(o'^2) + eps) * SiLU(W_g o') over rows of
// `channels` elements (channels % 64 == 0); W_g is [channels][channels], row = output.
struct GateParams {
  const void *o_in;
  int64_t ld_in;
  const void *wg;
  const float *gamma;
  float eps;
  void *o_out;
  int64_t ld_out;
  int64_t n;
  int channels;
  int64_t tiles_n;           // gate_tiles(n)
};
int64_t gate_tiles(int64_t n);
hipError_t launch_gate(const GateParams &p, bool bf16, hipStream_t s);

// Wide heads (bf16, d a multiple of 256 from 512 to 1024, m % 256 == 0): the
// update and apply split at the hidden layer into dense contractions (bigd.hip).
bool big_supported(int d, int m, bool bf16);
int64_t big_pad_tokens(int64_t n);          // token rows of the intermediates (multiple of 768)
int big_contract_tiles(int d, int m, int mode);
struct BigFwdParams {                       // dZ1, dZ3, H' = SwiGLU backward of K, V against W
  const void *k, *v;                        // [n][ld] bf16 token rows
  int64_t ld;
  const float *eta;
  int64_t eta_hs;
  const void *w1, *w3, *w2t;                // [H][m][d] bf16
  void *out;                                // 3 x [H][n_pad][m] bf16: dZ1 | dZ3 | H'
  int64_t n, n_pad;
  int heads, d, m;
};
hipError_t launch_big_fwd(const BigFwdParams &p, hipStream_t s);
struct BigCtrParams {                       // split partials of G1 = dZ1^T K, G3 = dZ3^T K, G2 = V^T H'
  const void *k, *v;
  int64_t ld;
  const void *inter;                        // the forward's output
  float *part;                              // [splits][3][H][m d]
  int64_t n, n_pad;
  int heads, d, m, splits;
};
hipError_t launch_big_contract(const BigCtrParams &p, hipStream_t s);
struct BigApplyParams {                     // H = SiLU(Q W1^T) o (Q W3^T); O = H W2^T
  const void *q;
  int64_t ldq;
  void *o;
  int64_t ldo;
  const void *w1, *w3;                      // [H][m][d] bf16
  const void *w2;                           // [H][d][m] bf16
  void *hbuf;                               // [H][nq_pad][m] bf16
  int64_t nq, nq_pad;
  int heads, d, m;
};
hipError_t launch_big_apply(const BigApplyParams &p, hipStream_t s);

hipError_t launch_conv(const void *v, void *out, int64_t ld, const float *w, int frames, int tpf,
                       int nsp, int gh, int gw, int channels, bool bf16, hipStream_t s);

}  // namespace ttt
