// Gated TTT output, ZipMap 关键设计 3: o_i = RMSNorm(o'_i) * SiLU(W_g o'_i) over
// whole rows o'_i of C channels, RMSNorm(x) = gamma * x / sqrt(mean(x^2) + eps).
//
// One fused kernel: the gate pre-activation O' W_g^T is a dense contraction
// (n x C x C) on bf16 (or fp32) MFMA; the row sums of squares for the RMS are
// taken from the same O' pieces as they pass through registers on their way to
// LDS, and the epilogue multiplies the normalised input by SiLU of the product,
// so neither the pre-activation nor the norm ever goes to HBM.
//
// Workgroup: 8 waves, a 256-token x 128-channel output tile; wave w owns tokens
// 64 (w % 4) .. +64 and channels 64 (w / 4) .. +64 (4 x 4 MFMA 16x16 tiles).
// The reduction runs over C in chunks of 128 bytes per row (64 bf16 / 32 fp32),
// double-buffered in LDS with the next chunk's global loads in flight.
#include "common.h"
#include "kernels.h"

namespace ttt {
namespace {

constexpr int kGateTok = 256;     // tokens per workgroup
constexpr int kGateCh = 128;      // output channels per workgroup
constexpr int kRowB = 128;        // bytes of one row of a staged chunk

struct GateSmem {
  unsigned char a[2][kGateTok * kRowB];
  unsigned char b[2][kGateCh * kRowB];
  float rinv[kGateTok];
};

// 16-byte piece c (0..7) of staged row r.  Fragment reads take 16 rows at one
// piece (16 lanes per LDS cycle for 16-byte reads): rows r and r + 2q land on
// the same banks without a swizzle, so the piece index is XORed with r / 2.
__device__ __forceinline__ int gate_slot(int r, int c) { return r * kRowB + ((c ^ ((r >> 1) & 7)) << 4); }

template <typename T> __device__ __forceinline__ typename FragOf<T>::type gate_frag(const unsigned char *s, int r,
                                                                                   int piece);
template <> __device__ __forceinline__ bf16x8 gate_frag<__bf16>(const unsigned char *s, int r, int piece) {
  return *reinterpret_cast<const bf16x8 *>(s + gate_slot(r, piece));
}
template <> __device__ __forceinline__ f32x8 gate_frag<float>(const unsigned char *s, int r, int piece) {
  const f32x4 lo = *reinterpret_cast<const f32x4 *>(s + gate_slot(r, piece));
  const f32x4 hi = *reinterpret_cast<const f32x4 *>(s + gate_slot(r, piece + 1));
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ float piece_sumsq(u32x4 raw, __bf16) {
  const bf16x8 v = __builtin_bit_cast(bf16x8, raw);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += (float)v[i] * (float)v[i];
  return s;
}
__device__ __forceinline__ float piece_sumsq(u32x4 raw, float) {
  const f32x4 v = __builtin_bit_cast(f32x4, raw);
  return v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
}

template <typename T>
__global__ __launch_bounds__(512) void gate_kernel(GateParams p) {
  __shared__ __attribute__((aligned(16))) GateSmem sm;
  constexpr int E = 16 / (int)sizeof(T);          // elements per 16-byte piece
  constexpr int KS = E / 4;                       // 32-element MFMA steps per 128-byte chunk
  const int t = threadIdx.x;
  const int C = p.channels;
  const int tiles_c = (C + kGateCh - 1) / kGateCh;
  const int64_t total = p.tiles_n * tiles_c;
  // consecutive work items (the channel tiles of one token tile, which read the
  // same O' rows) go to one XCD: launch-order blocks cycle over the 8 XCDs
  const int64_t per_xcd = (total + 7) >> 3;
  const int64_t item = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= total) return;
  const int64_t tok0 = (item / tiles_c) * kGateTok;
  const int j0 = (int)(item % tiles_c) * kGateCh;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, g = l >> 4, li = l & 15;
  const int wr = w & 3, wc = w >> 2;
  const bool active = j0 + 64 * wc < C;           // wave-uniform: this wave's channels exist

  const T *oin = static_cast<const T *>(p.o_in);
  const T *wg = static_cast<const T *>(p.wg);
  const int pc = t & 7;                           // piece column of this thread's loads
  const int lrow = t >> 3;                        // rows lrow + 64 u
  const T *asrc[4];
  const T *bsrc[2];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int64_t tok = tok0 + lrow + 64 * u;
    if (tok >= p.n) tok = p.n - 1;
    asrc[u] = oin + tok * p.ld_in + pc * E;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    int ch = j0 + lrow + 64 * u;
    if (ch >= C) ch = C - 1;
    bsrc[u] = wg + (int64_t)ch * C + pc * E;
  }
  u32x4 ra[4], rb[2];
#pragma unroll
  for (int u = 0; u < 4; ++u) ra[u] = *reinterpret_cast<const u32x4 *>(asrc[u]);
#pragma unroll
  for (int u = 0; u < 2; ++u) rb[u] = *reinterpret_cast<const u32x4 *>(bsrc[u]);

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[a][e] = f32x4{0, 0, 0, 0};
  float ss[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  const int nk = C / (8 * E);
  for (int kc = 0; kc < nk; ++kc) {
    const int buf = kc & 1;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<u32x4 *>(sm.a[buf] + gate_slot(lrow + 64 * u, pc)) = ra[u];
      ss[u] += piece_sumsq(ra[u], T{});
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) *reinterpret_cast<u32x4 *>(sm.b[buf] + gate_slot(lrow + 64 * u, pc)) = rb[u];
    __syncthreads();
    if (kc + 1 < nk) {
      const int64_t k1 = (int64_t)(kc + 1) * 8 * E;
#pragma unroll
      for (int u = 0; u < 4; ++u) ra[u] = *reinterpret_cast<const u32x4 *>(asrc[u] + k1);
#pragma unroll
      for (int u = 0; u < 2; ++u) rb[u] = *reinterpret_cast<const u32x4 *>(bsrc[u] + k1);
    }
    if (active) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        // lane group g takes elements 32 ks + 8 g .. +8 of the chunk
        const int piece = (32 * ks + 8 * g) * (int)sizeof(T) / 16;
        typename FragOf<T>::type fa[4], fb[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) fa[a] = gate_frag<T>(sm.a[buf], 64 * wr + 16 * a + li, piece);
#pragma unroll
        for (int e = 0; e < 4; ++e) fb[e] = gate_frag<T>(sm.b[buf], 64 * wc + 16 * e + li, piece);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[a][e] = mma(fa[a], fb[e], acc[a][e]);
      }
    }
  }

  // row sums of squares: the 8 threads of a row are 8 consecutive lanes
  const float invc = 1.0f / (float)C;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float s = ss[u];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if (pc == 0) sm.rinv[lrow + 64 * u] = 1.0f / sqrtf(s * invc + p.eps);
  }
  __syncthreads();
  if (!active) return;

  T *out = static_cast<T *>(p.o_out);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int ch = j0 + 64 * wc + 16 * e + li;
    if (ch >= C) continue;
    const float gam = p.gamma[ch];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        const int row = 64 * wr + 16 * a + 4 * g + z;
        const int64_t tok = tok0 + row;
        if (tok >= p.n) continue;
        const float x = to_f32(oin[tok * p.ld_in + ch]);
        const float zg = acc[a][e][z];
        out[tok * p.ld_out + ch] = from_f32<T>(gam * x * sm.rinv[row] * (zg * sigmoid_fast(zg)));
      }
  }
}

}  // namespace

hipError_t launch_gate(const GateParams &p, bool bf16, hipStream_t s) {
  const int64_t tiles_c = (p.channels + kGateCh - 1) / kGateCh;
  const int64_t blocks = (p.tiles_n * tiles_c + 7) / 8 * 8;
  if (bf16)
    hipLaunchKernelGGL(gate_kernel<__bf16>, dim3((unsigned)blocks), dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL(gate_kernel<float>, dim3((unsigned)blocks), dim3(512), 0, s, p);
  return hipGetLastError();
}

int64_t gate_tiles(int64_t n) { return (n + kGateTok - 1) / kGateTok; }

}  // namespace ttt
