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
constexpr int kApplyWaves = 8;   // waves (of 32 tokens) per fast workgroup

// ---------------------------------------------------------------- fast path
// bf16, D <= 256.  A workgroup owns 32 WV tokens of one head (32 per wave, WV
// waves, two per SIMD when WV = 8); each wave keeps its Q fragments and its O^T
// accumulators in registers.  The head's weights stream through LDS 32 hidden
// units at a time: W1 and W3 rows and W2^T rows ([hidden][d], so the second
// product reads them with the transposing load), DMA'd into a ring of three
// separate stage arrays.  Every weight byte fetched serves 32 WV tokens, so the
// tile is as tall as the register file allows.  The chunks run as a software
// pipeline (see the loop) so that each wave's SiLU-gate VALU work issues between
// its own MFMAs, and O leaves through LDS as whole rows.
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
  static_assert(WV <= 9, "the O staging puts three waves' rows in each stage array");
  __shared__ __attribute__((aligned(16))) unsigned char sa[L::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char sb[L::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char sc[L::kStage];

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

  // DMA: piece b of a stage is tile b / PPT (W1, W3, W2^T), rows kRowsPer * (b % PPT)
  // + lr with lr = lane / kChunks; lane l fills row r at physical chunk l % kChunks,
  // which holds the logical chunk (l % kChunks) ^ swizzle(tile, r).  Both swizzles
  // copy row bits onto chunk bits one by one, so swizzle(kRowsPer p + lr) =
  // swizzle(kRowsPer p) ^ swizzle(lr): a lane's source offset is its own constant
  // (held, one per swizzle) XORed with a wave-uniform one, plus 1 KB per piece.
  auto lane_part = [&](bool b128) {
    const int lr = l / L::kChunks;
    const int sw = (b128 ? swz_rows_b128(lr) : swz_rows(lr)) & (L::kChunks - 1);
    return (unsigned)(lr * L::kRowBytes + 16 * ((l % L::kChunks) ^ sw));
  };
  const unsigned lane_b128 = lane_part(true), lane_rows = lane_part(false);
  const char *wsrc[3] = {static_cast<const char *>(p.w1), static_cast<const char *>(p.w3),
                         static_cast<const char *>(p.w2t)};
  const int64_t head_off = (int64_t)h * p.m * D * 2;
  // piece q (of PPW) of this wave's share of chunk hc's copy into dst
  auto stage_piece = [&](int hc, unsigned char *dst, int q) __attribute__((always_inline)) {
    const int64_t base = head_off + (int64_t)hc * kHidChunk * D * 2;   // wave-uniform
    const int piece = w * PPW + q;
    if (NPIECE % WV != 0 && piece >= NPIECE) return;     // wave-uniform
    const int mat = piece / PPT, pr = piece % PPT;
    const int r0 = kRowsPer * pr;
    const unsigned s = 16u * (unsigned)((mat < 2 ? swz_rows_b128(r0) : swz_rows(r0)) & (L::kChunks - 1));
    const __amdgpu_buffer_rsrc_t rs = buffer_view(wsrc[mat] + base, L::kTile);
    copy16_to_lds(rs, xor_scalar_here(mat < 2 ? lane_b128 : lane_rows, s), 1024u * (unsigned)pr,
                  dst + piece * 1024);
  };
  auto stage_chunk = [&](int hc, unsigned char *dst) {
#pragma unroll
    for (int q = 0; q < PPW; ++q) stage_piece(hc, dst, q);
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

  // First product for hidden half u (tile rows perm_row(u, .)) of the chunk staged at
  // `base`: z1, z3 for the two token tiles, over d in KC steps; the W1 / W3 fragment
  // reads run one step ahead (a deeper ring does not fit the register file).
  // gate(kc) runs after the MFMAs of step kc, so that the SiLU-gate VALU work it is
  // given issues between this wave's MFMAs.
  auto first_half = [&](const unsigned char *base, int u, f32x4(&z1)[2], f32x4(&z3)[2], auto &&gate)
                        __attribute__((always_inline)) {
    constexpr int RA = 2;
    bf16x8 ra1[RA], ra3[RA];
    auto rd = [&](int kc, int slot) __attribute__((always_inline)) {
      const unsigned char *pa = base + xor_here(base_a[u], 64 * kc);
      ra1[slot] = *reinterpret_cast<const bf16x8 *>(pa);
      ra3[slot] = *reinterpret_cast<const bf16x8 *>(pa + L::kTile);
    };
#pragma unroll
    for (int t = 0; t < 2; ++t) z1[t] = z3[t] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < RA - 1 && q < KC; ++q) rd(q, q);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if (kc + RA - 1 < KC) rd(kc + RA - 1, (kc + RA - 1) % RA);
      const int sl = kc % RA;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        z1[t] = mma(ra1[sl], qf[t][kc], z1[t]);
        z3[t] = mma(ra3[sl], qf[t][kc], z3[t]);
      }
      gate(kc);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // H of one hidden half: h[t][r] = SiLU(z1) z3 of hidden 8g + 4u + r, token 16t + li.
  // The 8 elements per lane are spread over the KC steps of the product that hides them.
  auto gate_part = [&](int kc, const f32x4(&z1)[2], const f32x4(&z3)[2], bf16x4(&h)[2])
                       __attribute__((always_inline)) {
    constexpr int EPS = 8 / KC;   // elements per step
#pragma unroll
    for (int e = EPS * kc; e < EPS * (kc + 1); ++e) {
      const int t = e >> 2, r = e & 3;
      const float z = z1[t][r];
      h[t][r] = (__bf16)(z * sigmoid_fast(z) * z3[t][r]);
    }
  };
  // O^T[d][tok] += W2[d][chunk] H^T for the chunk staged at `base`; the transposing
  // reads run kRing column blocks ahead of their MFMAs, and between(dt) runs after
  // column block dt's products.
  auto second = [&](const unsigned char *base, const bf16x4(&h0)[2], const bf16x4(&h1)[2], auto &&between)
                    __attribute__((always_inline)) {
    const bf16x8 hf0 = cat8(h0[0], h1[0]), hf1 = cat8(h0[1], h1[1]);
    constexpr int kRing = 6;
    bf16x4 wlo[kRing], whi[kRing];
    auto rd_w2 = [&](int dt) __attribute__((always_inline)) {
      wlo[dt % kRing] = lds_read_tr16(base + xor_here(base_b[0], 32 * dt));
      whi[dt % kRing] = lds_read_tr16(base + xor_here(base_b[1], 32 * dt));
    };
#pragma unroll
    for (int q = 0; q < kRing - 1 && q < DT; ++q) rd_w2(q);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      if (dt + kRing - 1 < DT) rd_w2(dt + kRing - 1);
      const bf16x8 w2f = cat8(wlo[dt % kRing], whi[dt % kRing]);
      acc[dt][0] = mma(w2f, hf0, acc[dt][0]);
      acc[dt][1] = mma(w2f, hf1, acc[dt][1]);
      between(dt);
    }
  };

  // Software pipeline over the 32-unit chunks, three stages: iteration c runs
  //   A: first product of half 0 of chunk c, hiding the gate of half 1 of chunk c - 1;
  //   B: the second product of chunk c - 1 (its W2^T still in the previous stage);
  //   C: first product of half 1 of chunk c, hiding the gate of half 0 of chunk c;
  // and the DMA of chunk c + 1 into the stage chunk c - 2 left, its copies spread over
  // B's products (issued all at the start of A, they held both waves of a SIMD at
  // once: 2% slower).
  const int nch = p.m / kHidChunk;
  f32x4 za1[2], za3[2];   // half 0 of chunk c (made in A, gated in C)
  f32x4 zb1[2], zb3[2];   // half 1 of chunk c (made in C, gated in A of the next chunk)
  bf16x4 h0[2], h1[2];    // H of the chunk waiting for its second product
  auto no_gate = [](int) __attribute__((always_inline)) {};
  auto iter = [&](int c, const unsigned char *cur, const unsigned char *prev, unsigned char *next)
                  __attribute__((always_inline)) {
    const bool more = c + 1 < nch;
    first_half(cur, 0, za1, za3, [&](int kc) __attribute__((always_inline)) { gate_part(kc, zb1, zb3, h1); });
    // the copies of chunk c + 1 go out spread over the second product
    second(prev, h0, h1, [&](int dt) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < PPW; ++q)
        if (more && q * DT / PPW == dt) stage_piece(c + 1, next, q);
    });
    first_half(cur, 1, zb1, zb3, [&](int kc) __attribute__((always_inline)) { gate_part(kc, za1, za3, h0); });
    wait_all_memory();
    __syncthreads();
  };
  stage_chunk(0, sa);
  wait_all_memory();
  __syncthreads();
  if (nch > 1) stage_chunk(1, sb);
  first_half(sa, 0, za1, za3, no_gate);
  first_half(sa, 1, zb1, zb3, [&](int kc) __attribute__((always_inline)) { gate_part(kc, za1, za3, h0); });
  wait_all_memory();
  __syncthreads();
  for (int c = 1; c < nch; c += 3) {
    iter(c, sb, sa, sc);
    if (c + 1 < nch) iter(c + 1, sc, sb, sa);
    if (c + 2 < nch) iter(c + 2, sa, sc, sb);
  }
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) gate_part(kc, zb1, zb3, h1);
  const int last = (nch - 1) % 3;
  second(last == 0 ? sa : last == 1 ? sb : sc, h0, h1, [](int) __attribute__((always_inline)) {});

  // O goes out through LDS: each wave writes its 32 x D bf16 tile (row = token) into a
  // region of its own, then stores whole rows with 16-byte lanes (every store
  // instruction covers 1 KB of consecutive rows).  16-byte chunk c of row r sits at
  // position c ^ (r % 16) of the row (r % NC for rows of fewer than 16 chunks), so
  // the 8-byte writes of 16 rows at one chunk hit distinct banks.
  __syncthreads();   // every wave is done with the stages
  {
    constexpr int RB = 2 * D, NC = D / 8, SW = (NC < 16 ? NC : 16) - 1, RPI = 1024 / RB;
    unsigned char *ot = (w < 3 ? sa : w < 6 ? sb : sc) + (w % 3) * 32 * RB;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r = 16 * t + li;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (__bf16)acc[dt][t][q];
        const int c = 2 * dt + (g >> 1);
        *reinterpret_cast<bf16x4 *>(ot + r * RB + 16 * (c ^ (r & SW)) + 8 * (g & 1)) = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));   // lgkmcnt(0): this wave's tile is in LDS
#pragma unroll
    for (int j = 0; j < 32 / RPI; ++j) {
      const int r = RPI * j + l / NC, c = l % NC;
      const bf16x8 v = *reinterpret_cast<const bf16x8 *>(ot + r * RB + 16 * (c ^ (r & SW)));
      const int64_t tok = tok0 + r;
      if (tok < p.nq)
        *reinterpret_cast<bf16x8 *>(static_cast<__bf16 *>(p.o) + tok * p.ldo + (int64_t)h * D + 8 * c) = v;
    }
  }
}

// ------------------------------------------------------------- general path
// Any supported d (a multiple of 64 up to 1024, taken at run time), fp32 or bf16:
// 16 tokens per wave, 64 per workgroup, one output d-chunk of DC columns per
// workgroup; operands read from global memory (L1/L2 resident).  The first
// contraction is recomputed per d-chunk.
template <typename T, int DC>
__global__ __launch_bounds__(256) void apply_general_kernel(ApplyParams p) {
  using F = typename FragOf<T>::type;
  constexpr int DT = DC / 16;
  const int D = p.d, KC = D / 32;
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

template <typename T>
hipError_t launch_general_d(const ApplyParams &p, int d, hipStream_t s) {
  if (d < 64 || d > 1024 || d % 64 != 0 || p.d != d) return hipErrorInvalidValue;
  const int64_t tiles = (p.nq + 63) / 64;
  const int64_t grid = tiles * p.heads * p.dchunks;
  if (grid == 0) return hipSuccess;
  if (apply_general_dc(d, sizeof(T) == 2) == 128)
    hipLaunchKernelGGL((apply_general_kernel<T, 128>), dim3((unsigned)grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((apply_general_kernel<T, 64>), dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool apply_fast_supported(int d, bool bf16) { return bf16 && (d == 64 || d == 128 || d == 256); }
// output d-chunk of the general kernel: 128 columns where d allows, else 64
int apply_general_dc(int d, bool) { return d % 128 == 0 ? 128 : 64; }

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
