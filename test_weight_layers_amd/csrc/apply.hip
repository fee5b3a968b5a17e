// Apply: o = f_W(q) = W2 (SiLU(W1 q) o (W3 q)) for every query row
// (Scal3R eq. (4); ZipMap 关键设计 1; tttLRM query-only tokens use the same pass).
//
// Two back-to-back contractions per head: Z = W1 Q^T, W3 Q^T over d (computed
// transposed, hidden units as MFMA rows), the SiLU-gate in registers, then
// O^T += W2 H^T over the hidden units.  The hidden rows of each 32-unit chunk
// are permuted (perm_row) so that the accumulator layout of the first product
// is the operand layout of the second; H never leaves registers.
#include "common.h"
#include "kernels.h"

namespace ttt {
namespace {

constexpr int kHidChunk = 32;
#ifndef APPLY_WAVES
#define APPLY_WAVES 8
#endif
constexpr int kApplyWaves = APPLY_WAVES;   // waves (of 32 tokens) per fast workgroup

// ---------------------------------------------------------------- fast path
// bf16, D <= 256.  A workgroup owns 32 WV tokens of one head (32 per wave, WV
// waves, two per SIMD when WV = 8); each wave keeps its Q fragments and its O^T
// accumulators in registers.  The head's weights stream through LDS 32 hidden
// units at a time: W1 and W3 rows and W2^T rows ([hidden][d], so the second
// product reads them with the transposing load), DMA'd into one of two separate
// stage arrays while the other is consumed.  Every weight byte fetched serves
// 32 WV tokens, so the tile is as tall as the register file allows.
template <int D>
struct ApplyLayout {
  static constexpr int kChunks = D / 8;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTile = kHidChunk * kRowBytes;   // one [32][D] tile
  static constexpr int kStage = 3 * kTile;              // W1, W3, W2^T
};

template <int D, int WV>
__global__ __launch_bounds__(64 * WV, 1) void apply_fast_kernel(ApplyParams p) {
  using L = ApplyLayout<D>;
  constexpr int KC = D / 32, DT = D / 16;
  constexpr int NPIECE = L::kStage / 1024, PPW = (NPIECE + WV - 1) / WV, kRowsPer = 1024 / L::kRowBytes;
  constexpr int PPT = NPIECE / 3;                        // 1 KB pieces per tile
  __shared__ __attribute__((aligned(16))) unsigned char sa[L::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char sb[L::kStage];

  const int h = blockIdx.x % p.heads;
  const int64_t tile = blockIdx.x / p.heads;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, g = l >> 4, li = l & 15;
  const int64_t tok0 = tile * (32 * WV) + 32 * w;

  // Q^T fragments (B operand): token tok0 + 16t + li, d = 32 kc + 8g .. +8
  bf16x8 qf[2][KC];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t tok = tok0 + 16 * t + li;
    const __bf16 *Q = static_cast<const __bf16 *>(p.q) + (tok < p.nq ? tok : 0) * p.ldq + (int64_t)h * D + 8 * g;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const bf16x8 x = ld8(Q + 32 * kc);
      qf[t][kc] = (tok < p.nq) ? x : zero8<__bf16>();
    }
  }
  f32x4 acc[DT][2];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i][0] = acc[i][1] = f32x4{0, 0, 0, 0};

  // DMA: piece b of a stage is tile b / PPT, rows kRowsPer * (b % PPT) ..; lane l
  // fills row r at physical chunk l % kChunks = logical chunk ^ swizzle(tile, r).
  const char *wsrc[3] = {static_cast<const char *>(p.w1), static_cast<const char *>(p.w3),
                         static_cast<const char *>(p.w2t)};
  // offset of piece q in a chunk, formed at each use (the lane index passes through
  // an empty asm) rather than held in registers
  auto piece_off = [&](int q) {
    int lw = l;
    asm volatile("" : "+v"(lw));
    const int piece = w * PPW + q, mat = piece < NPIECE ? piece / PPT : 0;
    const int r = kRowsPer * (piece % PPT) + lw / L::kChunks;
    const int sw = (mat < 2 ? swz_rows_b128(r) : swz_rows(r)) & (L::kChunks - 1);
    return (r * D + 8 * ((lw % L::kChunks) ^ sw)) * 2;
  };
  const int64_t head_off = (int64_t)h * p.m * D * 2;
  auto stage_chunk = [&](int hc, unsigned char *dst) {
    const int64_t base = head_off + (int64_t)hc * kHidChunk * D * 2;   // wave-uniform
#pragma unroll
    for (int q = 0; q < PPW; ++q) {
      const int piece = w * PPW + q;
      if (NPIECE % WV != 0 && piece >= NPIECE) break;     // wave-uniform
      copy16_to_lds(wsrc[piece / PPT] + base + piece_off(q), dst + piece * 1024);
    }
  };

  // W1 / W3 reads: row perm_row(u, li), chunk 4kc + g  ->  base ^ 64 kc
  int base_a[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int rw = perm_row(u, li);
    base_a[u] = rw * L::kRowBytes + 16 * (g ^ (swz_rows_b128(rw) & (L::kChunks - 1)));
  }
  // W2^T transposed reads: lane supplies row 8g + 4q + li/4, column 16 dt + 4 (li % 4)
  // and receives hidden rows 8g + 4q .. +3 of d column 16 dt + li  ->  base ^ 32 dt
  int base_b[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 8 * g + 4 * q + (li >> 2);
    base_b[q] = 2 * L::kTile + row * L::kRowBytes + 16 * (((li & 3) >> 1) ^ (swz_rows(row) & (L::kChunks - 1))) +
                8 * (li & 1);
  }

  auto compute = [&](const unsigned char *base) {
    // Z^T rows = hidden perm_row(u, li) of the chunk, cols = tokens
    f32x4 z1[2][2], z3[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int t = 0; t < 2; ++t) z1[u][t] = z3[u][t] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        int ba = base_a[u];                 // one XOR per read rather than held addresses
        asm volatile("" : "+v"(ba));
        const unsigned char *pa = base + (ba ^ (64 * kc));
        const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(pa);
        const bf16x8 a3 = *reinterpret_cast<const bf16x8 *>(pa + L::kTile);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          z1[u][t] = mma(a1, qf[t][kc], z1[u][t]);
          z3[u][t] = mma(a3, qf[t][kc], z3[u][t]);
        }
      }
    }
    // H = SiLU(z1) o z3; element v = 4u + r is hidden 8g + v of the chunk
    bf16x8 hf[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float hv[8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float z = z1[u][t][r];
          hv[4 * u + r] = z * sigmoid_fast(z) * z3[u][t][r];
        }
      hf[t] = pack8<__bf16>(hv);
    }
    // O^T[d][tok] += W2[d][chunk] H^T
    // the transposing reads run kRing column blocks ahead of their MFMAs (a read's
    // latency is longer than the two MFMAs it feeds)
    constexpr int kRing = 8;
    bf16x4 wlo[kRing], whi[kRing];
    auto rd_w2 = [&](int dt) __attribute__((always_inline)) {
      int b0 = base_b[0], b1 = base_b[1];
      asm volatile("" : "+v"(b0), "+v"(b1));
      wlo[dt % kRing] = lds_read_tr16(base + (b0 ^ (32 * dt)));
      whi[dt % kRing] = lds_read_tr16(base + (b1 ^ (32 * dt)));
    };
#pragma unroll
    for (int q = 0; q < kRing - 1 && q < DT; ++q) rd_w2(q);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      if (dt + kRing - 1 < DT) rd_w2(dt + kRing - 1);
      const bf16x8 w2f = cat8(wlo[dt % kRing], whi[dt % kRing]);
      acc[dt][0] = mma(w2f, hf[0], acc[dt][0]);
      acc[dt][1] = mma(w2f, hf[1], acc[dt][1]);
    }
  };

  const int nch = p.m / kHidChunk;
  stage_chunk(0, sa);
  wait_all_memory();
  __syncthreads();
  for (int hc = 0; hc < nch; hc += 2) {
    if (hc + 1 < nch) stage_chunk(hc + 1, sb);
    compute(sa);
    wait_all_memory();
    __syncthreads();
    if (hc + 1 < nch) {
      if (hc + 2 < nch) stage_chunk(hc + 2, sa);
      compute(sb);
      wait_all_memory();
      __syncthreads();
    }
  }

  // O[tok][16 dt + 4g + r] for r = 0..3: one 8-byte store per (dt, t)
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t tok = tok0 + 16 * t + li;
    if (tok >= p.nq) continue;
    __bf16 *O = static_cast<__bf16 *>(p.o) + tok * p.ldo + (int64_t)h * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (__bf16)acc[dt][t][r];
      *reinterpret_cast<bf16x4 *>(O + 16 * dt) = v;
    }
  }
}

// ------------------------------------------------------------- general path
// Any supported d, fp32 or bf16: 16 tokens per wave, 64 per workgroup, one
// output d-chunk of DC columns per workgroup; operands read from global
// memory (L1/L2 resident).  The first contraction is recomputed per d-chunk.
template <typename T, int D, int DC>
__global__ __launch_bounds__(256) void apply_general_kernel(ApplyParams p) {
  using F = typename FragOf<T>::type;
  constexpr int KC = D / 32, DT = DC / 16;
  const int h = blockIdx.x % p.heads;
  int64_t rest = blockIdx.x / p.heads;
  const int dc = rest % p.dchunks;
  const int64_t tile = rest / p.dchunks;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
  const int64_t tok = tile * 64 + 16 * w + li;
  const bool ok = tok < p.nq;
  const int d0 = dc * DC;

  const T *Q = static_cast<const T *>(p.q) + (ok ? tok : 0) * p.ldq + (int64_t)h * D + 8 * g;
  const T *W1 = static_cast<const T *>(p.w1) + (int64_t)h * p.m * D;
  const T *W3 = static_cast<const T *>(p.w3) + (int64_t)h * p.m * D;
  const T *W2 = static_cast<const T *>(p.w2) + (int64_t)h * D * p.m;

  f32x4 acc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc[i] = f32x4{0, 0, 0, 0};

  for (int hc = 0; hc < p.m / kHidChunk; ++hc) {
    f32x4 z1[2], z3[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      z1[u] = z3[u] = f32x4{0, 0, 0, 0};
      const int64_t row = (int64_t)(hc * kHidChunk + perm_row(u, li)) * D + 8 * g;
#pragma unroll 2
      for (int kc = 0; kc < KC; ++kc) {
        const F qf = ok ? ld8(Q + 32 * kc) : zero8<T>();
        z1[u] = mma(ld8(W1 + row + 32 * kc), qf, z1[u]);
        z3[u] = mma(ld8(W3 + row + 32 * kc), qf, z3[u]);
      }
    }
    float hv[8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float z = z1[u][r];
        hv[4 * u + r] = z * sigmoid_fast(z) * z3[u][r];
      }
    const F hf = pack8<T>(hv);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const F w2f = ld8(W2 + (int64_t)(d0 + 16 * dt + li) * p.m + hc * kHidChunk + 8 * g);
      acc[dt] = mma(w2f, hf, acc[dt]);
    }
  }
  if (!ok) return;
  T *O = static_cast<T *>(p.o) + tok * p.ldo + (int64_t)h * D + d0 + 4 * g;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) O[16 * dt + r] = from_f32<T>(acc[dt][r]);
}

template <typename T, int D>
hipError_t launch_general(const ApplyParams &p, hipStream_t s) {
  constexpr int DC = (D < 128) ? D : 128;
  const int64_t tiles = (p.nq + 63) / 64;
  const int64_t grid = tiles * p.heads * p.dchunks;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((apply_general_kernel<T, D, DC>), dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_general_d(const ApplyParams &p, int d, hipStream_t s) {
  switch (d) {
    case 64: return launch_general<T, 64>(p, s);
    case 128: return launch_general<T, 128>(p, s);
    case 256: return launch_general<T, 256>(p, s);
    case 512: return launch_general<T, 512>(p, s);
    case 768: return launch_general<T, 768>(p, s);
    case 1024: return launch_general<T, 1024>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool apply_fast_supported(int d, bool bf16) { return bf16 && (d == 64 || d == 128 || d == 256); }
int apply_general_dc(int d, bool) { return d < 128 ? d : 128; }

hipError_t launch_apply(const ApplyParams &p, int d, bool bf16, bool fast, hipStream_t s) {
  if (fast) {
    const int64_t grid = (p.nq + 32 * kApplyWaves - 1) / (32 * kApplyWaves) * p.heads;
    if (grid == 0) return hipSuccess;
    switch (d) {
      case 64: hipLaunchKernelGGL((apply_fast_kernel<64, kApplyWaves>), dim3((unsigned)grid), dim3(64 * kApplyWaves), 0, s, p); break;
      case 128: hipLaunchKernelGGL((apply_fast_kernel<128, kApplyWaves>), dim3((unsigned)grid), dim3(64 * kApplyWaves), 0, s, p); break;
      case 256: hipLaunchKernelGGL((apply_fast_kernel<256, kApplyWaves>), dim3((unsigned)grid), dim3(64 * kApplyWaves), 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  return bf16 ? launch_general_d<__bf16>(p, d, s) : launch_general_d<float>(p, d, s);
}

}  // namespace ttt
