// Split-K reduction of the gradient partials, Muon's Newton-Schulz
// orthogonalisation and the step W <- W - lr * NS(G), plus the fp32 -> operand
// weight copies.
//
// Newton-Schulz (ZipMap 关键设计 3: Delta <- NewtonSchulz(g); VGG-T3 and tttLRM
// name the Muon optimiser): X = G / (||G||_F + eps), transposed while it has more
// rows than columns, then five times  A = X X^T,  B = b A + c A A,  X = a X + B X
// with Muon's quintic coefficients (a, b, c) = (3.4445, -4.7750, 2.0315).  The
// iterates and every product's accumulation are fp32.  In fp32 token mode the
// products run on fp32 MFMA; in bf16 token mode each fp32 operand is split into
// bf16 hi + lo parts and the products hi*hi + hi*lo + lo*hi run on bf16 MFMA with
// fp32 accumulation (about 16 significant bits per operand).  Every product is
// batched over the 3*H gradient matrices.
#include "common.h"
#include "kernels.h"

namespace ttt {
namespace {

constexpr int kRedBlock = 4096;   // elements per reduction workgroup (256 threads x 16)

__global__ __launch_bounds__(256) void reduce_kernel(const float *__restrict__ part, int splits,
                                                     int64_t per_split, float *__restrict__ g,
                                                     float *__restrict__ g_copy, float *__restrict__ sumsq) {
  __shared__ float red[256];
  const int64_t base = (int64_t)blockIdx.x * kRedBlock;
  float ss = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t i = base + (int64_t)(q * 256 + threadIdx.x) * 4;
    f32x4 acc = *reinterpret_cast<const f32x4 *>(part + i);
    for (int s = 1; s < splits; ++s) acc += *reinterpret_cast<const f32x4 *>(part + (int64_t)s * per_split + i);
    *reinterpret_cast<f32x4 *>(g + i) = acc;
    if (g_copy) *reinterpret_cast<f32x4 *>(g_copy + i) = acc;
    ss += acc[0] * acc[0] + acc[1] * acc[1] + acc[2] * acc[2] + acc[3] * acc[3];
  }
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) sumsq[blockIdx.x] = red[0];
}

// acc = (first ? 0 : acc) + sum over splits of part, in split order (deterministic).
__global__ __launch_bounds__(256) void accumulate_kernel(float *__restrict__ acc, const float *__restrict__ part,
                                                         int splits, int64_t per_split, int first) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= per_split) return;
  f32x4 v = first ? f32x4{0, 0, 0, 0} : *reinterpret_cast<const f32x4 *>(acc + i);
  for (int s = 0; s < splits; ++s) v += *reinterpret_cast<const f32x4 *>(part + (int64_t)s * per_split + i);
  *reinterpret_cast<f32x4 *>(acc + i) = v;
}

// Matrix b (0 .. 3H-1): j = b / H selects G1, G3, G2; G1/G3 are [m][d], G2 [d][m].
// X_b is [r][c] with r = min(d, m), c = max(d, m): the transpose of G_b when G_b
// has more rows than columns.
__device__ __forceinline__ bool ns_transposed(int j, int d, int m) { return j < 2 ? (m > d) : (d > m); }

__global__ __launch_bounds__(256) void ns_normalize_kernel(const float *__restrict__ g, const float *__restrict__ sumsq,
                                                           float *__restrict__ x, int heads, int d, int m, float eps) {
  const int64_t mat = (int64_t)d * m;
  const int per = (int)(mat / kRedBlock);
  const int64_t e0 = (int64_t)blockIdx.x * kRedBlock;
  const int b = (int)(e0 / mat);
  const int j = b / heads;
  float ss = 0.0f;
  for (int i = 0; i < per; ++i) ss += sumsq[(int64_t)b * per + i];
  const float scale = 1.0f / (sqrtf(ss) + eps);
  const bool tr = ns_transposed(j, d, m);
  const int rows = j < 2 ? m : d, cols = j < 2 ? d : m;     // shape of G_b
  const float *G = g + (int64_t)b * mat;
  float *X = x + (int64_t)b * mat;
  for (int q = threadIdx.x; q < kRedBlock; q += 256) {
    const int64_t e = e0 + q - (int64_t)b * mat;            // index inside X_b
    float val;
    if (tr) {                                               // X = G^T: [cols][rows]
      const int64_t xr = e / rows, xc = e % rows;
      val = G[xc * cols + xr];
    } else {
      val = G[e];
    }
    X[e] = val * scale;
  }
}

// 32x32 output tile per single-wave workgroup, K staged through LDS 32 at a time.
__global__ __launch_bounds__(64) void gemm_f32_kernel(GemmBatch p) {
  __shared__ __attribute__((aligned(16))) float as[32][36];
  __shared__ __attribute__((aligned(16))) float bs[32][36];   // [n][k]
  const int bz = blockIdx.z;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const float *A = p.a + bz * p.sa;
  const float *B = p.b + bz * p.sb;
  const int l = threadIdx.x, g = l >> 4, li = l & 15;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a) acc[a][0] = acc[a][1] = f32x4{0, 0, 0, 0};

  for (int k0 = 0; k0 < p.K; k0 += 32) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = (l >> 3) + 8 * q, c4 = (l & 7) * 4;
      *reinterpret_cast<f32x4 *>(&as[r][c4]) = *reinterpret_cast<const f32x4 *>(A + (int64_t)(i0 + r) * p.lda + k0 + c4);
      if (p.b_trans) {
        *reinterpret_cast<f32x4 *>(&bs[r][c4]) = *reinterpret_cast<const f32x4 *>(B + (int64_t)(j0 + r) * p.ldb + k0 + c4);
      } else {   // B is [K][N]: row k0 + r, columns j0 + c4 .. +4 -> bs[n][k]
        const f32x4 v = *reinterpret_cast<const f32x4 *>(B + (int64_t)(k0 + r) * p.ldb + j0 + c4);
#pragma unroll
        for (int t = 0; t < 4; ++t) bs[c4 + t][r] = v[t];
      }
    }
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const f32x8 af = ld8(&as[16 * mt + li][8 * g]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mma(af, ld8(&bs[16 * nt + li][8 * g]), acc[mt][nt]);
    }
    __syncthreads();
  }
  float *C = p.c + bz * p.sc;
  const float *Dm = p.dm ? p.dm + bz * p.sd : nullptr;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 16 * mt + 4 * g + r, j = j0 + 16 * nt + li;
        float v = p.alpha * acc[mt][nt][r];
        if (Dm) v += p.beta * Dm[(int64_t)i * p.ldd + j];
        C[(int64_t)i * p.ldc + j] = v;
      }
}

__global__ __launch_bounds__(256) void ns_step_kernel(const float *__restrict__ x, const float *w1, const float *w3,
                                                      const float *w2, float *w1o, float *w3o, float *w2o,
                                                      float *__restrict__ ns_out, float lr, int heads, int d, int m) {
  const int64_t mat = (int64_t)d * m;
  const int64_t total = 3 * heads * mat;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t b = e / mat, off = e % mat;
    const int j = (int)(b / heads), h = (int)(b % heads);
    const int rows = j < 2 ? m : d, cols = j < 2 ? d : m;
    float ns;
    if (ns_transposed(j, d, m)) {      // X_b = G_b^T is [cols][rows]
      const int64_t r = off / cols, c = off % cols;
      ns = x[b * mat + c * rows + r];
    } else {
      ns = x[e];
    }
    const float *src = j == 0 ? w1 : (j == 1 ? w3 : w2);
    float *dst = j == 0 ? w1o : (j == 1 ? w3o : w2o);
    const int64_t wi = (int64_t)h * mat + off;
    dst[wi] = src[wi] - lr * ns;
    if (ns_out) ns_out[e] = ns;
  }
}

// Weight copies in one launch: W1, W3 (and W2 when asked) cast row for row, 2048
// elements per workgroup, then W2 [H][d][m] -> W2^T [H][m][d] through 32x32 LDS tiles.
// A null output skips its part (its workgroups return at once).
template <typename T>
struct CastJob {
  const float *src[3];
  T *dst[3];            // W1, W3, W2 copies in their own layout
  T *w2t;               // W2^T copy
  int64_t n;            // elements per matrix (H d m, a multiple of 2048)
  int row_blocks;       // n / 2048
  int heads, d, m;
};
constexpr int kCastChunk = 2048;

template <typename T>
__global__ __launch_bounds__(256) void cast_kernel(CastJob<T> p) {
  __shared__ float tile[32][33];
  int blk = blockIdx.x;
  if (blk < 3 * p.row_blocks) {
    const int j = blk / p.row_blocks;
    T *o = p.dst[j];
    if (o == nullptr) return;
    const int64_t e = (int64_t)(blk % p.row_blocks) * kCastChunk + threadIdx.x * 8;
    const float *w = p.src[j] + e;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(w), b = *reinterpret_cast<const f32x4 *>(w + 4);
    if constexpr (sizeof(T) == 2) {
      bf16x8 v;
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        v[z] = (__bf16)a[z];
        v[4 + z] = (__bf16)b[z];
      }
      *reinterpret_cast<bf16x8 *>(o + e) = v;
    } else {
      *reinterpret_cast<f32x4 *>(o + e) = a;
      *reinterpret_cast<f32x4 *>(o + e + 4) = b;
    }
    return;
  }
  if (p.w2t == nullptr) return;
  blk -= 3 * p.row_blocks;
  const int tc = p.m / 32, tr = p.d / 32;
  const int h = blk / (tr * tc), rem = blk % (tr * tc);
  const int r0 = (rem / tc) * 32, c0 = (rem % tc) * 32;    // rows of W2 (d), cols (m)
  const float *src = p.src[2] + (int64_t)h * p.d * p.m;
  T *dst = p.w2t + (int64_t)h * p.d * p.m;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) tile[r][tx] = src[(int64_t)(r0 + r) * p.m + c0 + tx];
  __syncthreads();
  for (int r = ty; r < 32; r += 8) dst[(int64_t)(c0 + r) * p.d + r0 + tx] = from_f32<T>(tile[tx][r]);
}

template <typename T>
hipError_t cast_impl(const float *w1, const float *w3, const float *w2, void *w1o, void *w3o, void *w2to,
                     void *w2o, int heads, int d, int m, hipStream_t s) {
  CastJob<T> p{};
  p.src[0] = w1, p.src[1] = w3, p.src[2] = w2;
  p.dst[0] = static_cast<T *>(w1o), p.dst[1] = static_cast<T *>(w3o), p.dst[2] = static_cast<T *>(w2o);
  p.w2t = static_cast<T *>(w2to);
  p.n = (int64_t)heads * d * m;
  p.row_blocks = (int)(p.n / kCastChunk);
  p.heads = heads, p.d = d, p.m = m;
  const int64_t blocks = 3LL * p.row_blocks + (w2to ? (int64_t)heads * (d / 32) * (m / 32) : 0);
  hipLaunchKernelGGL(cast_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}


// ---------------------------------------------------------------- optimiser step
// The optimiser step as 16 launches: a preparation kernel (split-K sum of the
// gradient partials in fixed order, G and G^T copies, per-tile sums of squares)
// and one tile kernel per Newton-Schulz product.  The scale s = 1 / (||G|| + eps)
// is folded into the first iteration's coefficients (A = s^2 G G^T,
// X' = a s G + B (s G)), and the last product's epilogue writes W_out, the
// optional NS copy and the operand copies that the next gradient pass and the
// apply kernel read, so neither a normalisation nor a step nor a cast kernel runs.
//
// Every product is an "NT" product C[i][j] = sum_k P[i][k] Q[j][k] of row panels:
//   A = X X^T           (P = Q = X,  K = c)
//   A A                 (P = Q = A,  K = r; A is symmetric)
//   B X                 (P = B, Q = X^T, K = r; X^T is kept alongside X)
// on 64x64 output tiles, 4 waves of 32x32, K staged through LDS 64 at a time
// with the next chunk's loads in flight.

constexpr int kT = 64;        // output tile
constexpr int kKc = 64;       // K chunk
constexpr int kLdsW = kKc + 4;

constexpr int kLdsH = kKc;       // bf16 row of a split tile: 128 bytes, chunks swizzled (ns_at)

struct NsSmem {
  union {
    struct {
      float a[2][kT][kLdsW];
      float b[2][kT][kLdsW];
    } g;
    struct {                     // bf16 hi / lo parts of the same chunks
      __bf16 ah[2][kT][kLdsH], al[2][kT][kLdsH];
      __bf16 bh[2][kT][kLdsH], bl[2][kT][kLdsH];
    } h;
    float tr[kT][kT + 1];
  };
  float red[256];
};

// acc (per wave: 2x2 blocks of 16x16) = P[0 .. 63][0..K) Q[0 .. 63][0..K)^T
__device__ __forceinline__ void tile_nt(const float *__restrict__ P, int ldp, const float *__restrict__ Q, int ldq,
                                        int K, NsSmem &sm, f32x4 acc[2][2]) {
  const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, li = l & 15;
  const int lr = t >> 4, lc = (t & 15) * 4;         // loader: rows lr + 16 u; 4 floats at lc
#pragma unroll
  for (int a = 0; a < 2; ++a) acc[a][0] = acc[a][1] = f32x4{0, 0, 0, 0};
  f32x4 pa[4], pb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    pa[u] = *reinterpret_cast<const f32x4 *>(P + (int64_t)(lr + 16 * u) * ldp + lc);
    pb[u] = *reinterpret_cast<const f32x4 *>(Q + (int64_t)(lr + 16 * u) * ldq + lc);
  }
  const int nk = K / kKc;
  for (int kc = 0; kc < nk; ++kc) {
    const int buf = kc & 1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<f32x4 *>(&sm.g.a[buf][lr + 16 * u][lc]) = pa[u];
      *reinterpret_cast<f32x4 *>(&sm.g.b[buf][lr + 16 * u][lc]) = pb[u];
    }
    __syncthreads();
    if (kc + 1 < nk) {
      const int k0 = (kc + 1) * kKc;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pa[u] = *reinterpret_cast<const f32x4 *>(P + (int64_t)(lr + 16 * u) * ldp + k0 + lc);
        pb[u] = *reinterpret_cast<const f32x4 *>(Q + (int64_t)(lr + 16 * u) * ldq + k0 + lc);
      }
    }
    const int ra = (w >> 1) * 32 + li, rb = (w & 1) * 32 + li;
#pragma unroll
    for (int kk = 0; kk < kKc; kk += 32) {
      const f32x8 a0 = ld8(&sm.g.a[buf][ra][kk + 8 * g]), a1 = ld8(&sm.g.a[buf][ra + 16][kk + 8 * g]);
      const f32x8 b0 = ld8(&sm.g.b[buf][rb][kk + 8 * g]), b1 = ld8(&sm.g.b[buf][rb + 16][kk + 8 * g]);
      acc[0][0] = mma(a0, b0, acc[0][0]);
      acc[0][1] = mma(a0, b1, acc[0][1]);
      acc[1][0] = mma(a1, b0, acc[1][0]);
      acc[1][1] = mma(a1, b1, acc[1][1]);
    }
  }
}

// tile_nt with each fp32 operand split into bf16 hi + lo (x = hi + lo to about 16
// significant bits) and the product taken as hi*hi + hi*lo + lo*hi on bf16 MFMA,
// fp32 accumulation: about 2e-5 relative error on Newton-Schulz's output (fp32
// products give 2e-6) for a fifth of the fp32-MFMA cycles.  The global loads run
// two K chunks ahead (two register sets, one per LDS buffer).
__device__ __forceinline__ void split4(const f32x4 v, __bf16 *hi, __bf16 *lo) {
  bf16x4 h, l;
#pragma unroll
  for (int z = 0; z < 4; ++z) {
    h[z] = (__bf16)v[z];
    l[z] = (__bf16)(v[z] - (float)h[z]);
  }
  *reinterpret_cast<bf16x4 *>(hi) = h;
  *reinterpret_cast<bf16x4 *>(lo) = l;
}
// Element (r, c) of a split tile: 128-byte rows, 16-byte chunk c / 8 at (c / 8) ^ sw(r)
// with sw flipping chunk bits 0 and 1 with row bit 1 and bit 2 with row bit 2.  A
// ds_read_b128 of rows R + (0..15) at chunk 4h + g is served 8 rows of two lane groups
// at a time on gfx950; under this map each such half meets 16 distinct 16-byte bank
// groups (the former 144-byte padded rows did not: measured conflicts, 5% slower at
// 768 x 768).
__device__ __forceinline__ __bf16 *ns_at(__bf16 (*tile)[kLdsH], int r, int c) {
  const int sw = 3 * ((r >> 1) & 1) | (((r >> 2) & 1) << 2);
  return reinterpret_cast<__bf16 *>(reinterpret_cast<unsigned char *>(tile) + r * 128 + ((((c >> 3) ^ sw)) << 4) +
                                    ((c & 7) << 1));
}
__device__ __forceinline__ void tile_nt_split(const float *__restrict__ P, int ldp, const float *__restrict__ Q,
                                              int ldq, int K, NsSmem &sm, f32x4 acc[2][2]) {
  const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, li = l & 15;
  const int lr = t >> 4, lc = (t & 15) * 4;
#pragma unroll
  for (int a = 0; a < 2; ++a) acc[a][0] = acc[a][1] = f32x4{0, 0, 0, 0};
  f32x4 pa[2][4], pb[2][4];
  auto load = [&](int kc, int s) {
    const int k0 = kc * kKc;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      pa[s][u] = *reinterpret_cast<const f32x4 *>(P + (int64_t)(lr + 16 * u) * ldp + k0 + lc);
      pb[s][u] = *reinterpret_cast<const f32x4 *>(Q + (int64_t)(lr + 16 * u) * ldq + k0 + lc);
    }
  };
  const int nk = K / kKc;
  load(0, 0);
  if (nk > 1) load(1, 1);
  auto chunk = [&](int kc, int s) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      split4(pa[s][u], ns_at(sm.h.ah[s], lr + 16 * u, lc), ns_at(sm.h.al[s], lr + 16 * u, lc));
      split4(pb[s][u], ns_at(sm.h.bh[s], lr + 16 * u, lc), ns_at(sm.h.bl[s], lr + 16 * u, lc));
    }
    __syncthreads();
    if (kc + 2 < nk) load(kc + 2, s);
    const int ra = (w >> 1) * 32 + li, rb = (w & 1) * 32 + li;
#pragma unroll
    for (int kk = 0; kk < kKc; kk += 32) {
      bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ah[i] = ld8(ns_at(sm.h.ah[s], ra + 16 * i, kk + 8 * g));
        al[i] = ld8(ns_at(sm.h.al[s], ra + 16 * i, kk + 8 * g));
        bh[i] = ld8(ns_at(sm.h.bh[s], rb + 16 * i, kk + 8 * g));
        bl[i] = ld8(ns_at(sm.h.bl[s], rb + 16 * i, kk + 8 * g));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = mma(al[i], bh[j], acc[i][j]);
          acc[i][j] = mma(ah[i], bl[j], acc[i][j]);
          acc[i][j] = mma(ah[i], bh[j], acc[i][j]);
        }
    }
  };
  int kc = 0;
  for (; kc + 2 <= nk; kc += 2) {
    chunk(kc, 0);
    chunk(kc + 1, 1);
  }
  if (kc < nk) chunk(kc, 0);
}

// Deterministic block sum (every workgroup computes the same value the same way).
__device__ __forceinline__ float block_sum(float v, NsSmem &sm) {
  sm.red[threadIdx.x] = v;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) sm.red[threadIdx.x] += sm.red[threadIdx.x + w];
    __syncthreads();
  }
  const float r = sm.red[0];
  __syncthreads();
  return r;
}

// s_b = 1 / (||G_b||_F + eps) from the tile sums of squares, the same in every workgroup
__device__ __forceinline__ float ns_scale(const NsStepParams &p, int b, NsSmem &sm) {
  const int tiles_g = (p.m / kT) * (p.d / kT);
  float v = 0.0f;
  for (int i = threadIdx.x; i < tiles_g; i += 256) v += p.sumsq[(int64_t)b * tiles_g + i];
  return 1.0f / (sqrtf(block_sum(v, sm)) + p.eps);
}

// Launch-order block id -> work item, so that consecutive items (tiles of one
// matrix, which read the same panels) run on one XCD (blocks go round-robin
// over the 8 XCDs).
__device__ __forceinline__ int xcd_item() {
  const int n = gridDim.x, b = blockIdx.x;
  return n % 8 == 0 ? (b & 7) * (n >> 3) + (b >> 3) : b;
}

__global__ __launch_bounds__(256) void ns_prep_kernel(NsStepParams p) {
  __shared__ NsSmem sm;
  const int H = p.heads, d = p.d, m = p.m;
  const int64_t mat = (int64_t)d * m;
  const int t = threadIdx.x;
  const int tiles_g = (m / kT) * (d / kT);
  const int tile = xcd_item();
  const int b = tile / tiles_g, tt = tile % tiles_g;
  const int j = b / H;
  const int rows = j < 2 ? m : d, cols = j < 2 ? d : m;    // G_b is [rows][cols]
  const int ct = cols / kT;
  const int r0 = (tt / ct) * kT, c0 = (tt % ct) * kT;
  const bool tr = rows > cols;                             // X_b = G_b^T
  float *gl = (tr ? p.xt[0] : p.x[0]) + (int64_t)b * mat;  // buffer in G's layout
  float *gt = (tr ? p.x[0] : p.xt[0]) + (int64_t)b * mat;  // buffer in G^T's layout
  float ss = 0.0f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = t + 256 * u, rr = q >> 4, cc = (q & 15) * 4;
    const int64_t e = (int64_t)b * mat + (int64_t)(r0 + rr) * cols + c0 + cc;
    f32x4 acc = *reinterpret_cast<const f32x4 *>(p.part + e);
    for (int s = 1; s < p.splits; ++s) acc += *reinterpret_cast<const f32x4 *>(p.part + (int64_t)s * p.per_split + e);
    if (p.grad_out) *reinterpret_cast<f32x4 *>(p.grad_out + e) = acc;
    *reinterpret_cast<f32x4 *>(gl + (int64_t)(r0 + rr) * cols + c0 + cc) = acc;
#pragma unroll
    for (int z = 0; z < 4; ++z) sm.tr[rr][cc + z] = acc[z];
    ss += acc[0] * acc[0] + acc[1] * acc[1] + acc[2] * acc[2] + acc[3] * acc[3];
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {        // G^T tile: row c0 + rr, columns r0 + cc ..
    const int q = t + 256 * u, rr = q >> 4, cc = (q & 15) * 4;
    const f32x4 v{sm.tr[cc][rr], sm.tr[cc + 1][rr], sm.tr[cc + 2][rr], sm.tr[cc + 3][rr]};
    *reinterpret_cast<f32x4 *>(gt + (int64_t)(c0 + rr) * rows + r0 + cc) = v;
  }
  const float tot = block_sum(ss, sm);
  if (t == 0) p.sumsq[tile] = tot;
}

// PH 0: A = X X^T; 1: B = b A + c A A; 2: X' = a X + B X; 3: the last X' as the step.
template <typename T, int PH>
__global__ __launch_bounds__(256) void ns_tile_kernel(NsStepParams p, int cur, int first) {
  __shared__ NsSmem sm;
  const int H = p.heads, d = p.d, m = p.m, r = p.r, c = p.c;
  const int64_t mat = (int64_t)d * m, srr = (int64_t)r * r;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, li = l & 15;
  // A = X X^T and B = b A + c A A are symmetric: PH 0 and 1 compute the upper-triangle
  // tiles (ti <= tj) only and write each off-diagonal one mirrored as well.  PH 2 and 3
  // cover all rt x (c / kT) tiles of X'.
  const int rt = r / kT, nt = PH < 2 ? rt : c / kT;
  const int per_mat = PH < 2 ? rt * (rt + 1) / 2 : rt * nt;
  const int tile = xcd_item();
  const int b = tile / per_mat;
  int ti, tj;
  if (PH < 2) {
    int k = tile % per_mat;
    ti = 0;
    while (k >= rt - ti) {
      k -= rt - ti;
      ++ti;
    }
    tj = ti + k;
  } else {
    ti = (tile % per_mat) / nt;
    tj = tile % nt;
  }
  const bool mirror = PH < 2 && ti != tj;
  const float *X = p.x[cur] + (int64_t)b * mat, *XT = p.xt[cur] + (int64_t)b * mat;
  const float *A = p.am + b * srr;
  float *Bm = p.bm + b * srr;
  float alpha = 1.0f;
  if (first && (PH == 0 || PH >= 2)) {
    const float s = ns_scale(p, b, sm);
    alpha = PH == 0 ? s * s : s;
  }
  f32x4 acc[2][2];
  // bf16 mode: split-bf16 products; fp32 mode: fp32 MFMA
  constexpr bool split = sizeof(T) == 2;
  auto prod = [&](const float *P, int ldp, const float *Q, int ldq, int K) __attribute__((always_inline)) {
    if constexpr (split)
      tile_nt_split(P, ldp, Q, ldq, K, sm, acc);
    else
      tile_nt(P, ldp, Q, ldq, K, sm, acc);
  };
  if (PH == 0) prod(X + (int64_t)ti * kT * c, c, X + (int64_t)tj * kT * c, c, c);
  if (PH == 1) prod(A + (int64_t)ti * kT * r, r, A + (int64_t)tj * kT * r, r, r);
  if (PH >= 2) prod(Bm + (int64_t)ti * kT * r, r, XT + (int64_t)tj * kT * r, r, r);
  const int hj = b / H, h = b % H;
  const bool tr = (hj < 2 ? m : d) > (hj < 2 ? d : m);
  float ssw = 0.0f, ssd = 0.0f;      // norm-preserving form: sums of squares of W and W - lr NS
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = ti * kT + (w >> 1) * 32 + 16 * a + 4 * g, jj = tj * kT + (w & 1) * 32 + 16 * e + li;
      if (PH == 0) {
        f32x4 v;
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          v[z] = alpha * acc[a][e][z];
          p.am[b * srr + (int64_t)(i + z) * r + jj] = v[z];
        }
        if (mirror) *reinterpret_cast<f32x4 *>(p.am + b * srr + (int64_t)jj * r + i) = v;
      } else if (PH == 1) {
        f32x4 v;
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          const int64_t o = (int64_t)(i + z) * r + jj;
          v[z] = p.c_coef * acc[a][e][z] + p.b_coef * A[o];
          Bm[o] = v[z];
        }
        if (mirror) *reinterpret_cast<f32x4 *>(Bm + (int64_t)jj * r + i) = v;
      } else {
        // X[i .. i+3][jj] is the contiguous X^T[jj][i .. i+3]
        const f32x4 xo = *reinterpret_cast<const f32x4 *>(XT + (int64_t)jj * r + i);
        const float beta = p.a_coef * alpha;
        f32x4 v;
#pragma unroll
        for (int z = 0; z < 4; ++z) v[z] = alpha * acc[a][e][z] + beta * xo[z];
        if (PH == 2) {
          float *Xo = p.x[cur ^ 1] + (int64_t)b * mat;
#pragma unroll
          for (int z = 0; z < 4; ++z) Xo[(int64_t)(i + z) * c + jj] = v[z];
          *reinterpret_cast<f32x4 *>(p.xt[cur ^ 1] + (int64_t)b * mat + (int64_t)jj * r + i) = v;
        } else {
          // X_b[i][jj] is NS(G_b) at (i, jj), or at (jj, i) when X_b = G_b^T
          const float *W = hj == 0 ? p.w1 : (hj == 1 ? p.w3 : p.w2);
          float *Wo = hj == 0 ? p.w1o : (hj == 1 ? p.w3o : p.w2o);
          const int gcols = hj < 2 ? d : m;
          T *op = p.norm_preserve ? nullptr : static_cast<T *>(hj == 0 ? p.op1v : (hj == 1 ? p.op3v : p.op2tv));
#pragma unroll
          for (int z = 0; z < 4; ++z) {
            const int gr = tr ? jj : i + z, gc = tr ? i + z : jj;
            const int64_t ew = (int64_t)h * mat + (int64_t)gr * gcols + gc;
            const float w0 = W[ew];
            const float nw = w0 - p.lr * v[z];
            Wo[ew] = nw;
            ssw += w0 * w0;
            ssd += nw * nw;
            if (p.ns_out) p.ns_out[(int64_t)b * mat + (int64_t)gr * gcols + gc] = v[z];
            if (op) {
              // W1/W3 copies keep G's [m][d] layout; W2 [d][m] is copied transposed
              const int64_t oe = hj < 2 ? ew : (int64_t)h * mat + (int64_t)gc * d + gr;
              op[oe] = from_f32<T>(nw);
            }
          }
        }
      }
    }
  if (PH == 3 && p.norm_preserve) {
    const float sw = block_sum(ssw, sm), sd = block_sum(ssd, sm);
    if (t == 0) {
      p.wsq[tile] = sw;
      p.wsq[(int64_t)gridDim.x + tile] = sd;
    }
  }
}

// ---------------------------------------------------- norm-preserving step
// ZipMap 关键设计 3 keeps the Frobenius norm of each fast-weight matrix across the
// step: W^ = ||W|| (W - Delta) / ||W - Delta||.  The step kernels leave W - Delta
// in W_out and per-tile sums of squares of W and of W - Delta; the rescale sums
// them in fixed order (the same in every workgroup) and scales W_out in place.

__global__ __launch_bounds__(256) void weight_sumsq_kernel(const float *__restrict__ w1, const float *__restrict__ w3,
                                                           const float *__restrict__ w2, float *__restrict__ out,
                                                           int heads, int64_t mat) {
  __shared__ NsSmem sm;
  const int64_t e0 = (int64_t)blockIdx.x * kRedBlock;
  const int64_t b = e0 / mat;
  const int j = (int)(b / heads), h = (int)(b % heads);
  const float *src = (j == 0 ? w1 : (j == 1 ? w3 : w2)) + (int64_t)h * mat + (e0 - b * mat);
  float ss = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(src + (q * 256 + threadIdx.x) * 4);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  const float tot = block_sum(ss, sm);
  if (threadIdx.x == 0) out[blockIdx.x] = tot;
}

// One 64x64 tile of matrix b in W's own layout per workgroup.
template <typename T>
__global__ __launch_bounds__(256) void norm_rescale_kernel(float *w1o, float *w3o, float *w2o,
                                                           const float *__restrict__ wsq, int slots, T *op1, T *op3,
                                                           T *op2t, int heads, int d, int m) {
  __shared__ NsSmem sm;
  const int t = threadIdx.x;
  const int64_t mat = (int64_t)d * m;
  const int tiles = (int)(mat / (kT * kT));
  const int b = blockIdx.x / tiles, tt = blockIdx.x % tiles;
  const int j = b / heads, h = b % heads;
  const int B = 3 * heads;
  float sw = 0.0f, sd = 0.0f;
  for (int i = t; i < slots; i += 256) {
    sw += wsq[(int64_t)b * slots + i];
    sd += wsq[(int64_t)(B + b) * slots + i];
  }
  sw = block_sum(sw, sm);
  sd = block_sum(sd, sm);
  const float scale = sd > 0.0f ? sqrtf(sw) / sqrtf(sd) : 0.0f;
  const int rows = j < 2 ? m : d, cols = j < 2 ? d : m;
  const int ct = cols / kT;
  const int r0 = (tt / ct) * kT, c0 = (tt % ct) * kT;
  float *W = (j == 0 ? w1o : (j == 1 ? w3o : w2o)) + (int64_t)h * mat;
  T *op = j == 0 ? op1 : (j == 1 ? op3 : nullptr);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = t + 256 * u, rr = q >> 4, cc = (q & 15) * 4;
    f32x4 *pw = reinterpret_cast<f32x4 *>(W + (int64_t)(r0 + rr) * cols + c0 + cc);
    const f32x4 v = *pw * scale;
    *pw = v;
    if (op) {
#pragma unroll
      for (int z = 0; z < 4; ++z) op[(int64_t)h * mat + (int64_t)(r0 + rr) * cols + c0 + cc + z] = from_f32<T>(v[z]);
    }
    if (j == 2) {
#pragma unroll
      for (int z = 0; z < 4; ++z) sm.tr[rr][cc + z] = v[z];
    }
  }
  if (j == 2 && op2t) {               // W2 [d][m] tile -> W2^T [m][d]
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = t + 256 * u, rr = q >> 4, cc = (q & 15) * 4;
#pragma unroll
      for (int z = 0; z < 4; ++z)
        op2t[(int64_t)h * mat + (int64_t)(c0 + rr) * d + r0 + cc + z] = from_f32<T>(sm.tr[cc + z][rr]);
    }
  }
}

template <typename T>
hipError_t rescale_impl(float *w1o, float *w3o, float *w2o, const float *wsq, int slots, void *op1, void *op3,
                        void *op2t, int heads, int d, int m, hipStream_t s) {
  const int blocks = 3 * heads * (d / kT) * (m / kT);
  hipLaunchKernelGGL(norm_rescale_kernel<T>, dim3(blocks), dim3(256), 0, s, w1o, w3o, w2o, wsq, slots,
                     static_cast<T *>(op1), static_cast<T *>(op3), static_cast<T *>(op2t), heads, d, m);
  return hipGetLastError();
}

template <typename T>
hipError_t ns_optimiser_impl(const NsStepParams &p, hipStream_t s, hipEvent_t before_last) {
  const int B = 3 * p.heads, rt = p.r / kT, ct = p.c / kT;
  hipLaunchKernelGGL(ns_prep_kernel, dim3(B * rt * ct), dim3(256), 0, s, p);
  int cur = 0;
  for (int it = 0; it < p.iters; ++it) {
    const int first = it == 0;
    const int tri = B * rt * (rt + 1) / 2;      // upper-triangle tiles of the symmetric products
    hipLaunchKernelGGL((ns_tile_kernel<T, 0>), dim3(tri), dim3(256), 0, s, p, cur, first);
    hipLaunchKernelGGL((ns_tile_kernel<T, 1>), dim3(tri), dim3(256), 0, s, p, cur, first);
    if (it + 1 < p.iters) {
      hipLaunchKernelGGL((ns_tile_kernel<T, 2>), dim3(B * rt * ct), dim3(256), 0, s, p, cur, first);
    } else {
      if (before_last) {
        const hipError_t e = hipStreamWaitEvent(s, before_last, 0);
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL((ns_tile_kernel<T, 3>), dim3(B * rt * ct), dim3(256), 0, s, p, cur, first);
    }
    cur ^= 1;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_ns_optimiser(const NsStepParams &p, bool bf16, hipStream_t s, hipEvent_t before_last) {
  return bf16 ? ns_optimiser_impl<__bf16>(p, s, before_last) : ns_optimiser_impl<float>(p, s, before_last);
}

hipError_t launch_accumulate(float *acc, const float *part, int splits, int64_t per_split, bool first,
                             hipStream_t s) {
  const int64_t blocks = (per_split / 4 + 255) / 256;
  hipLaunchKernelGGL(accumulate_kernel, dim3((unsigned)blocks), dim3(256), 0, s, acc, part, splits, per_split,
                     first ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_weight_sumsq(const float *w1, const float *w3, const float *w2, float *out, int heads, int d,
                               int m, hipStream_t s) {
  const int64_t mat = (int64_t)d * m;
  hipLaunchKernelGGL(weight_sumsq_kernel, dim3((unsigned)(3 * heads * mat / kRedBlock)), dim3(256), 0, s, w1, w3, w2,
                     out, heads, mat);
  return hipGetLastError();
}

hipError_t launch_norm_rescale(float *w1o, float *w3o, float *w2o, const float *wsq, int slots, void *op1,
                               void *op3, void *op2t, int heads, int d, int m, bool bf16, hipStream_t s) {
  return bf16 ? rescale_impl<__bf16>(w1o, w3o, w2o, wsq, slots, op1, op3, op2t, heads, d, m, s)
              : rescale_impl<float>(w1o, w3o, w2o, wsq, slots, op1, op3, op2t, heads, d, m, s);
}

hipError_t launch_cast(const float *w1, const float *w3, const float *w2, void *w1o, void *w3o, void *w2to,
                       void *w2o, int heads, int d, int m, bool bf16, hipStream_t s) {
  return bf16 ? cast_impl<__bf16>(w1, w3, w2, w1o, w3o, w2to, w2o, heads, d, m, s)
              : cast_impl<float>(w1, w3, w2, w1o, w3o, w2to, w2o, heads, d, m, s);
}

hipError_t launch_reduce(const float *part, int splits, int64_t per_split, float *g, float *g_copy, float *sumsq,
                         hipStream_t s) {
  const int64_t blocks = per_split / kRedBlock;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, part, splits, per_split, g, g_copy, sumsq);
  return hipGetLastError();
}

hipError_t launch_ns_normalize(const float *g, const float *sumsq, float *x, const NsShape &sh, float eps,
                               hipStream_t s) {
  const int64_t blocks = 3LL * sh.heads * sh.d * sh.m / kRedBlock;
  hipLaunchKernelGGL(ns_normalize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, g, sumsq, x, sh.heads, sh.d, sh.m,
                     eps);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmBatch &g, hipStream_t s) {
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(g.N / 32, g.M / 32, g.batch), dim3(64), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_ns_step(const float *x, const float *w1, const float *w3, const float *w2, float *w1o, float *w3o,
                          float *w2o, float *ns_out, float lr, const NsShape &sh, hipStream_t s) {
  const int64_t total = 3LL * sh.heads * sh.d * sh.m;
  const int grid = (int)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
  hipLaunchKernelGGL(ns_step_kernel, dim3(grid), dim3(256), 0, s, x, w1, w3, w2, w1o, w3o, w2o, ns_out, lr, sh.heads,
                     sh.d, sh.m);
  return hipGetLastError();
}

}  // namespace ttt
