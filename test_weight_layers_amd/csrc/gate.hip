// Gated TTT output, ZipMap 关键设计 3: o_i = RMSNorm(o'_i) * SiLU(W_g o'_i) over
// whole rows o'_i of C channels, RMSNorm(x) = gamma * x / sqrt(mean(x^2) + eps).
//
// One fused kernel: the gate pre-activation O' W_g^T is a dense contraction
// (n x C x C) on bf16 (or fp32) MFMA; the row sums of squares for the RMS are
// taken from the O' operand fragments of the product, and the epilogue
// multiplies the normalised input by SiLU of the product, so neither the
// pre-activation nor the norm ever goes to HBM.
//
// Workgroup: 8 waves, a 256-token x 256-channel output tile; wave w owns tokens
// 64 (w % 4) .. +64 and channels 128 (w / 4) .. +128 (4 x 8 MFMA 16x16 tiles),
// so every staged byte feeds 128 multiply-adds: the L2 -> LDS supply of about
// 12-18 bytes per clock per CU, not the MFMA rate, is what a narrower tile hits.
// The reduction runs over C in chunks of 128 bytes per row (64 bf16 / 32 fp32),
// DMA'd from global memory straight into two 64 KB LDS stages, one chunk ahead
// of the one being multiplied.  The RMS sums of
// squares come from the O' fragments the channel-0 waves already hold.
#include "common.h"
#include "kernels.h"

namespace ttt {
namespace {

constexpr int kGateTok = 256;     // tokens per workgroup
constexpr int kGateCh = 256;      // output channels per workgroup

template <typename T> struct GateGeo {
  static constexpr int kRowB = 128;                     // one chunk of a row: a whole cache line
  static constexpr int kEpc = kRowB / (int)sizeof(T);   // reduction elements per chunk: 64 / 32
  static constexpr int kKs = kEpc / 32;                 // MFMA k-steps per chunk
  static constexpr int kPieces = kRowB / 16;            // 16-byte pieces per row
  static constexpr int kRowsPerKb = 1024 / kRowB;       // rows per 1 KB DMA piece
  static constexpr int kStageA = kGateTok * kRowB;
  static constexpr int kStage = kStageA + kGateCh * kRowB;
  static constexpr int kNst = 2;                        // ring depth
  static constexpr int kDmaA = kStageA / 1024 / 8;      // 1 KB DMAs per wave per stage (A part)
  static constexpr int kDmaB = kGateCh * kRowB / 1024 / 8;
  static constexpr int kDma = kDmaA + kDmaB;
};

// Piece c of staged row r sits at position c ^ swizzle(r).  Fragment reads take
// 16 consecutive rows at one piece (16 lanes per LDS cycle for 16-byte reads);
// with 128-byte rows, rows r and r + 2q collide without a swizzle, so the piece
// index is XORed with r / 2.  Whole 128-byte rows per chunk make every DMA
// instruction fetch 8 full cache lines (64-byte halves would touch 16).
template <typename T> __device__ __forceinline__ int gate_swz(int r) { return (r >> 1) & 7; }
template <typename T> __device__ __forceinline__ int gate_slot(int r, int c) {
  return r * GateGeo<T>::kRowB + ((c ^ gate_swz<T>(r)) << 4);
}

// lane group g's 8 reduction elements 32 ks + 8g .. +8 of staged row r
template <typename T> __device__ __forceinline__ typename FragOf<T>::type gate_frag(const unsigned char *s, int r,
                                                                                   int ks, int g);
template <> __device__ __forceinline__ bf16x8 gate_frag<__bf16>(const unsigned char *s, int r, int ks, int g) {
  return *reinterpret_cast<const bf16x8 *>(s + gate_slot<__bf16>(r, 4 * ks + g));
}
template <> __device__ __forceinline__ f32x8 gate_frag<float>(const unsigned char *s, int r, int ks, int g) {
  const f32x4 lo = *reinterpret_cast<const f32x4 *>(s + gate_slot<float>(r, 8 * ks + 2 * g));
  const f32x4 hi = *reinterpret_cast<const f32x4 *>(s + gate_slot<float>(r, 8 * ks + 2 * g + 1));
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// sum of squares of 8 bf16 values with four bf16 dot2 instructions (x0^2 + x1^2 + acc,
// exact products, fp32 sums) instead of eight conversions and eight FMAs
__device__ __forceinline__ float frag_sumsq(const bf16x8 v, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {v[2 * i], v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float frag_sumsq(const f32x8 v, float acc) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc += v[i] * v[i];
  return acc;
}


template <typename T>
__global__ __launch_bounds__(512) void gate_kernel(GateParams p) {
  using G = GateGeo<T>;
  constexpr int NST = G::kNst;
  // the ring's stages are separate arrays so that the compiler can tell the
  // stage being read from the ones the DMAs are filling
  __shared__ __attribute__((aligned(1024))) unsigned char st0[G::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[G::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[NST > 2 ? G::kStage : 16];
  __shared__ __attribute__((aligned(1024))) unsigned char st3[NST > 3 ? G::kStage : 16];
  __shared__ float rinv[kGateTok];
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
  const bool active = j0 + 128 * wc < C;          // wave-uniform: this wave's channels exist

  const T *oin = static_cast<const T *>(p.o_in);
  const T *wg = static_cast<const T *>(p.wg);
  // DMA sources.  1 KB piece b of a stage's A part holds rows kRowsPerKb * b ..
  // (wave w fills b = kDmaA w ..), of its B part likewise; lane l writes row
  // kRowsPerKb b + l / kPieces at position l % kPieces, which holds the row's
  // piece (l % kPieces) ^ swizzle.  Each lane's source offset inside the tile's rows
  // is fixed (rows past n read row n - 1, channels past C channel C - 1); the chunk
  // advances by a wave-uniform offset, so a copy needs no address arithmetic.
  const int64_t a_rows = p.n - tok0 < kGateTok ? p.n - tok0 : kGateTok;
  const __amdgpu_buffer_rsrc_t arsrc = buffer_view(oin + tok0 * p.ld_in, (unsigned)(a_rows * p.ld_in * sizeof(T)));
  const __amdgpu_buffer_rsrc_t brsrc = buffer_view(wg + (int64_t)j0 * C,
                                                   (unsigned)((C - j0 < kGateCh ? C - j0 : kGateCh) * C * sizeof(T)));
  unsigned aoff[G::kDmaA], boff[G::kDmaB];
#pragma unroll
  for (int j = 0; j < G::kDmaA; ++j) {
    const int r = G::kRowsPerKb * (G::kDmaA * w + j) + l / G::kPieces;
    const int rr = r < a_rows ? r : (int)a_rows - 1;
    aoff[j] = (unsigned)((int64_t)rr * p.ld_in * sizeof(T)) + 16u * (unsigned)((l % G::kPieces) ^ gate_swz<T>(r));
  }
#pragma unroll
  for (int j = 0; j < G::kDmaB; ++j) {
    const int r = G::kRowsPerKb * (G::kDmaB * w + j) + l / G::kPieces;
    const int rr = j0 + r < C ? r : C - 1 - j0;
    boff[j] = (unsigned)((int64_t)rr * C * sizeof(T)) + 16u * (unsigned)((l % G::kPieces) ^ gate_swz<T>(r));
  }
  auto issue = [&](int kc, unsigned char *dst) __attribute__((always_inline)) {
    const unsigned kb = (unsigned)kc * G::kRowB;
#pragma unroll
    for (int j = 0; j < G::kDmaA; ++j) copy16_to_lds(arsrc, aoff[j], kb, dst + (G::kDmaA * w + j) * 1024);
#pragma unroll
    for (int j = 0; j < G::kDmaB; ++j) copy16_to_lds(brsrc, boff[j], kb, dst + G::kStageA + (G::kDmaB * w + j) * 1024);
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[a][e] = f32x4{0, 0, 0, 0};
  float ss[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  // copy j (of kDma) of this wave's share of chunk kc into dst
  auto issue_one = [&](int kc, unsigned char *dst, int j) __attribute__((always_inline)) {
    const unsigned kb = (unsigned)kc * G::kRowB;
    if (j < G::kDmaA)
      copy16_to_lds(arsrc, aoff[j], kb, dst + (G::kDmaA * w + j) * 1024);
    else
      copy16_to_lds(brsrc, boff[j - G::kDmaA], kb, dst + G::kStageA + (G::kDmaB * w + j - G::kDmaA) * 1024);
  };
  // products of the stage; between(e) runs after column tile e of the first k-step
  auto compute = [&](const unsigned char *stage, auto &&between) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < G::kKs; ++ks) {
      typename FragOf<T>::type fa[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) fa[a] = gate_frag<T>(stage, 64 * wr + 16 * a + li, ks, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const typename FragOf<T>::type fb = gate_frag<T>(stage + G::kStageA, 128 * wc + 16 * e + li, ks, g);
#pragma unroll
        for (int a = 0; a < 4; ++a) acc[a][e] = mma(fa[a], fb, acc[a][e]);
        if (ks == 0) between(e);
      }
      if (wc == 0) {
#pragma unroll
        for (int a = 0; a < 4; ++a) ss[a] = frag_sumsq(fa[a], ss[a]);
      }
    }
  };
  const int nk = C / G::kEpc;
  // one chunk: wait for its stage (the later chunks' DMAs may stay in flight),
  // barrier, multiply, refilling the stage read one chunk ago with chunk kc + NST - 1
  // (its copies spread over the first k-step's column tiles: issued all after the
  // barrier they held every wave at once, 4% slower)
  auto step = [&](int kc, const unsigned char *cur, unsigned char *refill) __attribute__((always_inline)) {
    const int later = nk - 1 - kc;                // chunks after kc already issued: min(later, NST - 2)
    if (NST > 3 && later >= 2)
      wait_vmcnt<2 * G::kDma>();
    else if (NST > 2 && later >= 1)
      wait_vmcnt<G::kDma>();
    else
      wait_vmcnt<0>();
    bare_barrier();
    const bool more = kc + NST - 1 < nk;          // wave-uniform
    if (!active) {                                // no products: copy at once
      if (more) issue(kc + NST - 1, refill);
      return;
    }
    // the copies of chunk kc + NST - 1 go out spread over the first k-step's column tiles
    compute(cur, [&](int e) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < G::kDma; ++j)
        if (more && j * 8 / G::kDma == e) issue_one(kc + NST - 1, refill, j);
    });
  };
  unsigned char *const ring[4] = {st0, st1, st2, st3};
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < nk) issue(s, ring[s]);
  for (int kc = 0; kc < nk; kc += NST) {
    step(kc, st0, ring[NST - 1]);
    if (kc + 1 < nk) step(kc + 1, st1, st0);
    if (NST > 2 && kc + 2 < nk) step(kc + 2, st2, st1);
    if (NST > 3 && kc + 3 < nk) step(kc + 3, st3, st2);
  }

  // The epilogue's O' loads (16 rows of 8 channels per thread, rows past n read row
  // n - 1) are issued first, so that their latency overlaps the RMS and SiLU work.
  bf16x8 xs[16];
  f32x4 g0 = f32x4{0, 0, 0, 0}, g1 = g0;
  if constexpr (sizeof(T) == 2) {
    const int ch = j0 + 8 * (t & 31);
    if (ch < C) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        int64_t tok = tok0 + 16 * i + (t >> 5);
        if (tok >= p.n) tok = p.n - 1;
        xs[i] = *reinterpret_cast<const bf16x8 *>(oin + tok * p.ld_in + ch);
      }
      g0 = *reinterpret_cast<const f32x4 *>(p.gamma + ch);
      g1 = *reinterpret_cast<const f32x4 *>(p.gamma + ch + 4);
    }
  }
  // row sums of squares: lanes li, li+16, li+32, li+48 of a channel-0 wave hold
  // the four element groups of row 64 wr + 16 a + li
  if (wc == 0) {
    const float invc = 1.0f / (float)C;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float s = ss[a];
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      if (g == 0) rinv[64 * wr + 16 * a + li] = 1.0f / sqrtf(s * invc + p.eps);
    }
  }
  T *out = static_cast<T *>(p.o_out);
  if constexpr (sizeof(T) == 2) {
    // bf16: SiLU(z) goes through LDS (the ring is free now) as a 256 x 256 bf16
    // tile, rows 64 b .. 64 b + 63 in stage b; then every thread finishes 8
    // consecutive channels of a row with 16-byte loads of O' and 16-byte stores.
    // Tile column c of row r sits at c ^ (16 ((r / 4) % 4)), so the four row
    // groups of a 2-byte store wave land on distinct banks.
    auto zrow = [&](int blk) __attribute__((always_inline)) -> __bf16 * {   // 64 rows of 512 bytes
      return reinterpret_cast<__bf16 *>((blk < 2 ? st0 : st1) + (blk & 1) * 64 * 512);
    };
    __syncthreads();                  // every wave is done with the ring
    if (active) {
      __bf16 *zt = zrow(wr);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          const int r = 16 * a + 4 * g + z;                        // row inside the block
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float zg = acc[a][e][z];
            const int c = (128 * wc + 16 * e + li) ^ (16 * g);     // (r / 4) % 4 == g
            zt[r * kGateCh + c] = (__bf16)(zg * sigmoid_fast(zg));
          }
        }
    }
    __syncthreads();
    const int cv = t & 31;                      // 8-channel group of the tile
    const int ch = j0 + 8 * cv;
    if (ch >= C) return;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 16 * i + (t >> 5);
      const int64_t tok = tok0 + row;
      const int r = row & 63;
      const bf16x8 sz = *reinterpret_cast<const bf16x8 *>(zrow(i >> 2) + r * kGateCh + ((8 * cv) ^ (16 * ((r >> 2) & 3))));
      const float ri = rinv[row];
      bf16x8 y;
#pragma unroll
      for (int u = 0; u < 8; ++u) y[u] = (__bf16)((u < 4 ? g0[u] : g1[u - 4]) * (float)xs[i][u] * ri * (float)sz[u]);
      // the gated rows are not read again here: streaming (non-temporal) stores
      if (tok < p.n) __builtin_nontemporal_store(y, reinterpret_cast<bf16x8 *>(out + tok * p.ld_out + ch));
    }
  } else {
    __syncthreads();
    if (!active) return;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ch = j0 + 128 * wc + 16 * e + li;
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
          out[tok * p.ld_out + ch] = from_f32<T>(gam * x * rinv[row] * (zg * sigmoid_fast(zg)));
        }
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
