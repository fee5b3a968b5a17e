// Wide-head kernels (bf16, d in {512, 768, 1024}; ZipMap's own state is d = 1024
// with fast-weight hidden 2048, its 损失函数 / 训练策略 section).
//
// At these widths one head's weights (3 m d bf16) and gradient accumulators
// (3 m d fp32) no longer fit on chip next to a token tile, so the fused d <= 256
// kernels do not carry over.  The update and apply are split at the hidden layer
// instead, each half a dense contraction on bf16 MFMA:
//
//   gradient, forward (big_fwd_kernel):   per token tile x hidden tile,
//     z1 = K W1^T, z3 = K W3^T, p = V W2 over d, then the SwiGLU backward of the
//     eta-weighted dot-product loss (ZipMap 关键设计 1) in the epilogue:
//       dZ1 = dH z3 (s + a - a s),  dZ3 = dH a,  H' = -eta a z3,  dH = -eta p
//     written as bf16 token-major [n][m] (the operand precision the fused kernels
//     use for the same quantities);
//   gradient, contractions (big_contract_kernel), split over token ranges:
//     G1 = dZ1^T K, G3 = dZ3^T K (mode 0) and G2 = V^T H' (mode 1) into the fp32
//     split partials the optimiser step already sums;
//   apply (big_hidden_kernel, big_out_kernel):  H = SiLU(Q W1^T) o (Q W3^T) over d,
//     then O = H W2^T over m (Scal3R eq. (4); ZipMap 关键设计 1).
//
// The intermediates cost 2 x 2 B per element of [n][m] (written once, read once),
// under 15% of the MFMA time at these widths.
#include "common.h"
#include "kernels.h"

namespace ttt {
namespace {


// Launch-order block -> work item: blocks go round-robin over the 8 XCDs, so
// item (b % 8) * per + b / 8 puts consecutive items (which share operand rows)
// on one XCD and its L2.
__device__ __forceinline__ int64_t xcd_work_item(int64_t total) {
  const int64_t per = (total + 7) >> 3;
  return (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
}

// copy16_to_lds (global_load_lds_dwordx4) issued through inline asm, so that the
// compiler does not count it: its waits for LDS reads cannot tell which stage a
// pending copy writes once the copies stay in flight across a loop's back edge, and
// it then waits for all of them.  The caller waits for these copies itself
// (s_waitcnt vmcnt) before reading their data.
__device__ __forceinline__ void copy16_to_lds_untracked(const void *gsrc, unsigned char *lds_wave_base) {
  const unsigned m0v = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)lds_wave_base;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(m0v) : "memory");
}

// ------------------------------------------------------------------ NT tiles
// C[i][j] = sum_k A[i][k] B[j][k], every operand row k-contiguous in HBM.  A
// workgroup (WR x WC waves) stages NA "A" operands of TM rows and NB "B" operands
// of TN rows, 32 reduction elements (64 bytes) per row, and multiplies NP (A, B)
// pairs into NP accumulator sets.  Stages are DMA'd 1 KB (16 rows) per wave
// instruction into a ring of NST stages, NST - 1 chunks ahead.  Each MFMA takes the
// B rows as its row operand, so the accumulator of 16 x 16 tile (i, j) holds C^T:
// lane (g, li) has C[16 i + li][16 j + 4 g + r], r = 0..3 (four consecutive
// columns of one row, which the epilogues store as one 8-byte unit).
template <int NA_, int NB_, int TM_, int TN_, int NST_, int WR_ = 4, int WC_ = 2>
struct NtGeo {
  static constexpr int NA = NA_, NB = NB_, TM = TM_, TN = TN_, NST = NST_, WR = WR_, WC = WC_;
  static constexpr int kWaves = WR * WC, kThreads = 64 * kWaves;
  static constexpr int kRows = NA * TM + NB * TN;
  static constexpr int kStage = kRows * 64;
  static constexpr int kPPW = kStage / 1024 / kWaves;  // DMA pieces per wave per stage
  static constexpr int WM = TM / WR, WN = TN / WC;     // wave tile
  static constexpr int FM = WM / 16, FN = WN / 16;     // MFMA tiles per wave
  static_assert((kStage / 1024) % kWaves == 0, "stage must split evenly over the waves");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "tile shape");
};

// 16-byte piece c (0..3) of staged 64-byte row r sits at c ^ swz_64(r), under which
// the fragment reads (rows R..R+15, R % 16 == 0, lane group g at piece g) are
// conflict-free.
__device__ __forceinline__ bf16x8 nt_frag(const unsigned char *stage, int r, int g) {
  return *reinterpret_cast<const bf16x8 *>(stage + r * 64 + ((g ^ swz_64(r)) << 4));
}
// Lane l of DMA piece b fills staged row 16 b + l / 4 at position l % 4, i.e. the
// row's piece (l % 4) ^ swz_64(row).
__device__ __forceinline__ int nt_piece_row(int b, int l) { return 16 * b + (l >> 2); }
__device__ __forceinline__ int nt_piece_off(int row, int l) { return ((l & 3) ^ swz_64(row)) << 4; }

// The mainloop.  src[q]: this lane's source address of its q-th piece at chunk 0
// (chunk kc adds 64 kc bytes).  PA/PB: operand indices of each pair.
template <class G, int NP>
__device__ __forceinline__ void nt_mainloop(f32x4 (&acc)[NP][G::FM][G::FN], const char *const (&src)[G::kPPW],
                                            const int (&pa)[NP], const int (&pb)[NP], int nk, unsigned char *st0,
                                            unsigned char *st1, unsigned char *st2, unsigned char *st3, int w, int g,
                                            int li, int wr, int wc) {
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
      for (int j = 0; j < G::FN; ++j) acc[p][i][j] = f32x4{0, 0, 0, 0};
  auto issue = [&](int kc, unsigned char *dst) __attribute__((always_inline)) {
    const int kb = kc * 64;
#pragma unroll
    for (int q = 0; q < G::kPPW; ++q) copy16_to_lds_untracked(src[q] + kb, dst + (w * G::kPPW + q) * 1024);
  };
  // Products of the stage at `stg`.  The B fragments are read one group (FN x NB
  // groups, each feeding NP products) ahead; after each group's products
  // `between(group)` runs (the next chunk's copies are spread over the groups there,
  // so that the copy path and the matrix cores work at the same time).
  constexpr int NG = G::NB * G::FN;
  auto compute = [&](const unsigned char *stg, auto &&between) __attribute__((always_inline)) {
    bf16x8 fa[G::NA][G::FM];
#pragma unroll
    for (int a = 0; a < G::NA; ++a)
#pragma unroll
      for (int i = 0; i < G::FM; ++i) fa[a][i] = nt_frag(stg, a * G::TM + wr * G::WM + 16 * i + li, g);
    auto rd_b = [&](int gi) __attribute__((always_inline)) {
      const int b = gi / G::FN, j = gi % G::FN;
      return nt_frag(stg, G::NA * G::TM + b * G::TN + wc * G::WN + 16 * j + li, g);
    };
    bf16x8 fb_next = rd_b(0);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const bf16x8 fb = fb_next;
      if (gi + 1 < NG) fb_next = rd_b(gi + 1);
      const int b = gi / G::FN, j = gi % G::FN;
#pragma unroll
      for (int p = 0; p < NP; ++p)
        if (pb[p] == b) {
#pragma unroll
          for (int i = 0; i < G::FM; ++i) acc[p][i][j] = mma(fb, fa[pa[p]][i], acc[p][i][j]);
        }
      between(gi);
    }
  };
  auto step = [&](int kc, const unsigned char *cur, unsigned char *refill) __attribute__((always_inline)) {
    const int later = nk - 1 - kc;        // chunks after kc already issued: min(later, NST - 2)
    if (G::NST > 3 && later >= 2)
      wait_vmcnt<2 * G::kPPW>();
    else if (G::NST > 2 && later >= 1)
      wait_vmcnt<G::kPPW>();
    else
      wait_vmcnt<0>();
    bare_barrier();
    const bool more = kc + G::NST - 1 < nk;   // wave-uniform
    const int kb = (kc + G::NST - 1) * 64;
    // copies q with q * NG / kPPW == gi go after group gi
    compute(cur, [&](int gi) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < G::kPPW; ++q)
        if (more && q * NG / G::kPPW == gi) copy16_to_lds_untracked(src[q] + kb, refill + (w * G::kPPW + q) * 1024);
    });
  };
  unsigned char *const ring[4] = {st0, st1, st2, st3};
#pragma unroll
  for (int s = 0; s < G::NST - 1; ++s)
    if (s < nk) issue(s, ring[s]);
  for (int kc = 0; kc < nk; kc += G::NST) {
    step(kc, st0, ring[G::NST - 1]);
    if (kc + 1 < nk) step(kc + 1, st1, st0);
    if (G::NST > 2 && kc + 2 < nk) step(kc + 2, st2, st1);
    if (G::NST > 3 && kc + 3 < nk) step(kc + 3, st3, st2);
  }
  __syncthreads();                        // every wave is done with the ring
}

// bf16 output tiles [rows][C] (C = 128 or 256) staged in LDS between the products
// and the 16-byte global stores.  A lane writes four consecutive columns (8 bytes,
// unit u = column / 4) of one row; unit u of row r sits at u ^ 2 (r % 16), so the 16
// rows x 2 units that one write instruction serves together fall on distinct banks,
// and a 16-byte chunk c (units 2c, 2c + 1) stays whole, at c ^ (r % 16).
template <int C> __device__ __forceinline__ int stage_w(int r, int u) { return r * C + 4 * (u ^ ((r & 15) << 1)); }
template <int C> __device__ __forceinline__ int stage_r(int r, int c) { return r * C + 8 * (c ^ (r & 15)); }

// ------------------------------------------------------- gradient, forward
// 8 waves, two per SIMD (a 4-wave layout with 64 x 64 wave tiles and AGPR
// accumulators needs a third fewer fragment reads per MFMA but measured 13% slower:
// one wave per SIMD leaves its read latencies exposed).  192 token rows per tile:
// the copy into LDS, not the matrix cores, bounds this kernel, and 192 x 128 is the
// largest tile whose three 48 KB stages fit in LDS (10% faster than 128 x 128).
using FwdGeo = NtGeo<2, 3, 192, 128, 3>;   // A: K, V tokens; B: W1, W3, W2^T hidden rows

__global__ __launch_bounds__(FwdGeo::kThreads) void big_fwd_kernel(BigFwdParams p) {
  using G = FwdGeo;
  __shared__ __attribute__((aligned(1024))) unsigned char st0[G::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[G::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[G::kStage];
  const int t = threadIdx.x;
  const int tiles_u = p.m / G::TN;
  const int64_t tiles_t = p.n_pad / G::TM;
  const int64_t total = (int64_t)p.heads * tiles_t * tiles_u;
  // Work order.  A tile reads 192 K/V token rows and 3 x 128 weight rows over all of d.
  // When the hidden tiles split evenly over the 8 XCDs, XCD x keeps hidden tiles
  // x * tiles_u / 8 .. for every token tile (their weights, 1.5 MB at d = 1024 and
  // m = 2048, stay in its L2) and runs them token tile by token tile, so the tiles in
  // flight together share K/V rows too.  Otherwise each XCD cycles through all hidden
  // tiles of a token tile, and the weights stream from beyond L2.
  int tu;
  int64_t tt;
  int h;
  if (tiles_u % 8 == 0) {
    const int per_x = tiles_u / 8;
    const int64_t j = blockIdx.x >> 3;   // launch-order position within XCD blockIdx.x % 8
    if (j >= total / 8) return;
    tu = (int)(blockIdx.x & 7) * per_x + (int)(j % per_x);
    const int64_t ht = j / per_x;
    tt = ht % tiles_t;
    h = (int)(ht / tiles_t);
  } else {
    const int64_t item = xcd_work_item(total);
    if (item >= total) return;
    tu = (int)(item % tiles_u);
    const int64_t ht = item / tiles_u;
    tt = ht % tiles_t;
    h = (int)(ht / tiles_t);
  }
  const int64_t tok0 = tt * G::TM;
  const int u0 = tu * G::TN;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, g = l >> 4, li = l & 15;
  const int wr = w % G::WR, wc = w / G::WR;
  const int d = p.d, m = p.m;
  const int64_t mat = (int64_t)m * d;

  const char *src[G::kPPW];
#pragma unroll
  for (int q = 0; q < G::kPPW; ++q) {
    const int row = nt_piece_row(w * G::kPPW + q, l);
    const int op = row < 2 * G::TM ? row / G::TM : 2 + (row - 2 * G::TM) / G::TN;   // K, V, W1, W3, W2^T
    const int r = row < 2 * G::TM ? row % G::TM : (row - 2 * G::TM) % G::TN;
    const __bf16 *base;
    if (op < 2) {
      int64_t tok = tok0 + r;
      if (tok >= p.n) tok = p.n - 1;
      base = static_cast<const __bf16 *>(op == 0 ? p.k : p.v) + tok * p.ld + (int64_t)h * d;
    } else {
      const __bf16 *wsrc = static_cast<const __bf16 *>(op == 2 ? p.w1 : (op == 3 ? p.w3 : p.w2t));
      base = wsrc + (int64_t)h * mat + (int64_t)(u0 + r) * d;
    }
    src[q] = reinterpret_cast<const char *>(base) + nt_piece_off(row, l);
  }
  f32x4 acc[3][G::FM][G::FN];
  constexpr int pa[3] = {0, 0, 1}, pb[3] = {0, 1, 2};   // K W1^T, K W3^T, V (W2^T)^T
  nt_mainloop<G, 3>(acc, src, pa, pb, d / 32, st0, st1, st2, st0, w, g, li, wr, wc);

  // SwiGLU backward.  Tile (i, j) holds the products transposed: lane (g, li) has
  // hidden units 64 wc + 16 j + 4 g + r (r = 0..3) of token row WM wr + 16 i + li.
  __bf16 *o1 = reinterpret_cast<__bf16 *>(st0), *o3 = reinterpret_cast<__bf16 *>(st1),
         *oh = reinterpret_cast<__bf16 *>(st2);
  // this lane's rates, fetched together (rows past n read row n - 1 and are zeroed:
  // they contribute nothing)
  const float *eta = p.eta + (int64_t)h * p.eta_hs;
  float nes[G::FM];
#pragma unroll
  for (int i = 0; i < G::FM; ++i) {
    const int64_t tok = tok0 + wr * G::WM + 16 * i + li;
    nes[i] = eta[tok < p.n ? tok : p.n - 1];
  }
#pragma unroll
  for (int i = 0; i < G::FM; ++i) {
    const int tr = wr * G::WM + 16 * i + li;
    const float ne = tok0 + tr < p.n ? -nes[i] : 0.0f;
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      bf16x4 v1, v3, vh;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float z = acc[0][i][j][r], y = acc[1][i][j][r];
        const float sg = sigmoid_fast(z);
        const float act = z * sg;
        const float dh = ne * acc[2][i][j][r];
        v1[r] = (__bf16)(dh * y * (sg + act - act * sg));
        v3[r] = (__bf16)(dh * act);
        vh[r] = (__bf16)(ne * (act * y));
      }
      const int u = (wc * G::WN + 16 * j) / 4 + g;
      *reinterpret_cast<bf16x4 *>(o1 + stage_w<G::TN>(tr, u)) = v1;
      *reinterpret_cast<bf16x4 *>(o3 + stage_w<G::TN>(tr, u)) = v3;
      *reinterpret_cast<bf16x4 *>(oh + stage_w<G::TN>(tr, u)) = vh;
    }
  }
  __syncthreads();
  // 3 outputs x 128 rows x 16 vectors of 8 hidden units
  constexpr int VPO = G::TM * 16 / G::kThreads;            // vectors per thread and output
  const int64_t plane = (int64_t)p.heads * p.n_pad * m;   // elements per output
  __bf16 *dst = static_cast<__bf16 *>(p.out) + ((int64_t)h * p.n_pad + tok0) * m + u0;
#pragma unroll
  for (int it = 0; it < 3 * VPO; ++it) {
    const int k = it / VPO;
    const int rem = t + G::kThreads * (it % VPO);
    const int tr = rem >> 4, cu = rem & 15;
    const __bf16 *srcs = k == 0 ? o1 : (k == 1 ? o3 : oh);
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(srcs + stage_r<G::TN>(tr, cu));
    // the intermediates are read by the next kernel, far beyond what the caches hold:
    // streaming (non-temporal) stores
    __builtin_nontemporal_store(v, reinterpret_cast<bf16x8 *>(dst + k * plane + (int64_t)tr * m + 8 * cu));
  }
}

// --------------------------------------------------- gradient, contractions
// Both operands are token-major tiles of one 32-token block: row = token, the
// features (hidden units or d) contiguous.  The MFMA reduction runs over the
// block's tokens, so every fragment comes from a transposing read
// (ds_read_b64_tr_b16): lane (g, li) supplies row 8g + 4q + li/4, columns
// 16 c + 4 (li % 4) and receives tokens 8g + 4q .. +3 of feature 16 c + li.
// Mode 0: A = dZ1, dZ3 (256 hidden units each), B = K (128 of d): G1, G3.
// Mode 1: A = V (256 of d), B = H' (256 hidden units): G2.
template <int MODE> struct CtrGeo;
template <> struct CtrGeo<0> {
  static constexpr int NA = 2, TM = 256, TN = 128;
};
template <> struct CtrGeo<1> {
  static constexpr int NA = 1, TM = 256, TN = 256;
};
template <int MODE> struct CtrLayout {
  using C = CtrGeo<MODE>;
  static constexpr int NA = C::NA, TM = C::TM, TN = C::TN;
  static constexpr int kATile = 32 * TM * 2, kBTile = 32 * TN * 2;
  static constexpr int kStage = NA * kATile + kBTile;
  static constexpr int kPieces = kStage / 1024, kPPW = kPieces / 8;
  static constexpr int FM = TM / 4 / 16, FN = TN / 2 / 16;
  static_assert(kPieces % 8 == 0, "stage must split evenly over 8 waves");
};

// transposing-read base of a row-major bf16 tile with RB-byte rows (16-byte chunks
// swizzled by swz_rows); column block cb adds XOR 32 cb
template <int RB> __device__ __forceinline__ int tr_base(int g, int li, int q) {
  const int row = 8 * g + 4 * q + (li >> 2);
  const int e = (li & 3) >> 1;
  return row * RB + 16 * (e ^ (swz_rows(row) & (RB / 16 - 1))) + 8 * (li & 1);
}
template <int RB> __device__ __forceinline__ bf16x8 tr_frag(const unsigned char *tile, int b0, int b1, int cb) {
  return cat8(lds_read_tr16(tile + (b0 ^ (32 * cb))), lds_read_tr16(tile + (b1 ^ (32 * cb))));
}

template <int MODE>
__global__ __launch_bounds__(512) void big_contract_kernel(BigCtrParams p) {
  using L = CtrLayout<MODE>;
  constexpr int RBA = L::TM * 2, RBB = L::TN * 2;        // row bytes of the A and B tiles
  __shared__ __attribute__((aligned(1024))) unsigned char st0[L::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[L::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[L::kStage];
  const int t = threadIdx.x;
  const int d = p.d, m = p.m;
  const int rows_out = MODE == 0 ? m : d, cols_out = MODE == 0 ? d : m;
  const int tiles_c = cols_out / L::TN;
  const int tiles = (rows_out / L::TM) * tiles_c;
  const int64_t total = (int64_t)p.heads * p.splits * tiles;
  const int64_t item = xcd_work_item(total);
  if (item >= total) return;
  const int tile = (int)(item % tiles);
  const int64_t hs = item / tiles;
  const int split = (int)(hs % p.splits), h = (int)(hs / p.splits);
  const int r0 = (tile / tiles_c) * L::TM, c0 = (tile % tiles_c) * L::TN;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, g = l >> 4, li = l & 15;
  const int wr = w & 3, wc = w >> 2;
  // this split's 32-token blocks
  const int64_t nblk = p.n_pad / 32;
  const int64_t per = (nblk + p.splits - 1) / p.splits;
  const int64_t b0 = (int64_t)split * per;
  const int64_t b1 = b0 + per < nblk ? b0 + per : nblk;
  const int nb = b0 < b1 ? (int)(b1 - b0) : 0;

  // DMA sources: piece b of a stage is A tile a = b / (kATile / 1024) (rows of RBA
  // bytes) or the B tile; lane l fills row (piece row base) + l / chunks at position
  // l % chunks, the row's chunk (l % chunks) ^ swizzle.
  const int64_t plane = (int64_t)p.heads * p.n_pad * m;
  const __bf16 *ig = static_cast<const __bf16 *>(p.inter);   // dZ1 | dZ3 | H', [H][n_pad][m] each
  const char *src[L::kPPW];
  int64_t sld[L::kPPW];                                        // bytes per token row
#pragma unroll
  for (int q = 0; q < L::kPPW; ++q) {
    const int b = w * L::kPPW + q;
    const bool is_a = b < L::NA * (L::kATile / 1024);
    const int rb = is_a ? RBA : RBB;
    const int pb = is_a ? b % (L::kATile / 1024) : b - L::NA * (L::kATile / 1024);
    const int row = pb * (1024 / rb) + l / (rb / 16);
    const int chunk = (l % (rb / 16)) ^ (swz_rows(row) & (rb / 16 - 1));
    const __bf16 *base;
    int64_t ld;
    if (MODE == 0) {
      if (is_a) {            // dZ1 or dZ3 rows, hidden units r0 ..
        const int a = b / (L::kATile / 1024);
        base = ig + a * plane + (int64_t)h * p.n_pad * m + r0;
        ld = m;
      } else {               // K rows, d columns c0 ..
        base = static_cast<const __bf16 *>(p.k) + (int64_t)h * d + c0;
        ld = p.ld;
      }
    } else {
      if (is_a) {            // V rows, d columns r0 ..
        base = static_cast<const __bf16 *>(p.v) + (int64_t)h * d + r0;
        ld = p.ld;
      } else {               // H' rows, hidden units c0 ..
        base = ig + 2 * plane + (int64_t)h * p.n_pad * m + c0;
        ld = m;
      }
    }
    // token rows past n (K, V) are read from row n - 1; their dZ / H' rows are zero
    src[q] = reinterpret_cast<const char *>(base + (int64_t)row * ld) + 16 * chunk;
    sld[q] = ld * 2;
  }
  auto issue = [&](int blk, unsigned char *dst) __attribute__((always_inline)) {
    const int64_t tok0 = (b0 + blk) * 32;
#pragma unroll
    for (int q = 0; q < L::kPPW; ++q) {
      const int b = w * L::kPPW + q;
      const bool is_a = b < L::NA * (L::kATile / 1024);
      const bool token_rows = MODE == 0 ? !is_a : is_a;    // K / V: clamp to row n - 1
      int64_t t0 = tok0;
      if (token_rows) {
        const int rb = is_a ? RBA : RBB;
        const int pb = is_a ? b % (L::kATile / 1024) : b - L::NA * (L::kATile / 1024);
        const int row = pb * (1024 / rb) + l / (rb / 16);
        if (t0 + row >= p.n) t0 = p.n - 1 - row;
      }
      copy16_to_lds(src[q] + t0 * sld[q], dst + b * 1024);
    }
  };

  f32x4 acc[L::NA][L::FM][L::FN];
#pragma unroll
  for (int a = 0; a < L::NA; ++a)
#pragma unroll
    for (int i = 0; i < L::FM; ++i)
#pragma unroll
      for (int j = 0; j < L::FN; ++j) acc[a][i][j] = f32x4{0, 0, 0, 0};
  const int ba0 = tr_base<RBA>(g, li, 0), ba1 = tr_base<RBA>(g, li, 1);
  const int bb0 = tr_base<RBB>(g, li, 0), bb1 = tr_base<RBB>(g, li, 1);
  auto compute = [&](const unsigned char *stg) __attribute__((always_inline)) {
    bf16x8 fa[L::NA][L::FM];
#pragma unroll
    for (int a = 0; a < L::NA; ++a)
#pragma unroll
      for (int i = 0; i < L::FM; ++i)
        fa[a][i] = tr_frag<RBA>(stg + a * L::kATile, ba0, ba1, wr * L::FM + i);
#pragma unroll
    for (int j = 0; j < L::FN; ++j) {
      const bf16x8 fb = tr_frag<RBB>(stg + L::NA * L::kATile, bb0, bb1, wc * L::FN + j);
#pragma unroll
      for (int a = 0; a < L::NA; ++a)
#pragma unroll
        for (int i = 0; i < L::FM; ++i) acc[a][i][j] = mma(fa[a][i], fb, acc[a][i][j]);
    }
  };
  auto step = [&](int blk, const unsigned char *cur, unsigned char *refill) __attribute__((always_inline)) {
    if (blk + 1 < nb)
      wait_vmcnt<L::kPPW>();
    else
      wait_vmcnt<0>();
    bare_barrier();
    if (blk + 2 < nb) issue(blk + 2, refill);
    compute(cur);
  };
  if (nb > 0) issue(0, st0);
  if (nb > 1) issue(1, st1);
  for (int blk = 0; blk < nb; blk += 3) {
    step(blk, st0, st2);
    if (blk + 1 < nb) step(blk + 1, st1, st0);
    if (blk + 2 < nb) step(blk + 2, st2, st1);
  }

  // partials: rows r0 + 64 wr + 16 i + 4 g + z, columns c0 + (TN / 2) wc + 16 j + li
  const int64_t mat = (int64_t)m * d;
  float *P = p.part + (int64_t)split * 3 * p.heads * mat;
#pragma unroll
  for (int a = 0; a < L::NA; ++a) {
    const int which = MODE == 0 ? a : 2;                 // G1, G3 / G2
    float *Pw = P + ((int64_t)which * p.heads + h) * mat;
#pragma unroll
    for (int i = 0; i < L::FM; ++i)
#pragma unroll
      for (int j = 0; j < L::FN; ++j)
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          const int row = r0 + 64 * wr + 16 * i + 4 * g + z;
          const int col = c0 + (L::TN / 2) * wc + 16 * j + li;
          Pw[(int64_t)row * cols_out + col] = acc[a][i][j][z];
        }
  }
}

// ------------------------------------------------------------------ apply
using HidGeo = NtGeo<1, 2, 256, 128, 4>;   // A: Q tokens; B: W1, W3 hidden rows
using OutGeo = NtGeo<1, 1, 256, 256, 4>;   // A: H tokens; B: W2 rows (d)

__global__ __launch_bounds__(512) void big_hidden_kernel(BigApplyParams p) {
  using G = HidGeo;
  __shared__ __attribute__((aligned(1024))) unsigned char st0[G::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[G::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[G::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char st3[G::kStage];
  const int t = threadIdx.x;
  const int tiles_u = p.m / G::TN;
  const int64_t tiles_t = p.nq_pad / G::TM;
  const int64_t total = (int64_t)p.heads * tiles_t * tiles_u;
  const int64_t item = xcd_work_item(total);
  if (item >= total) return;
  const int tu = (int)(item % tiles_u);
  const int64_t ht = item / tiles_u;
  const int64_t tt = ht % tiles_t;
  const int h = (int)(ht / tiles_t);
  const int64_t tok0 = tt * G::TM;
  const int u0 = tu * G::TN;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, g = l >> 4, li = l & 15;
  const int wr = w & 3, wc = w >> 2;
  const int d = p.d, m = p.m;
  const int64_t mat = (int64_t)m * d;
  const char *src[G::kPPW];
#pragma unroll
  for (int q = 0; q < G::kPPW; ++q) {
    const int row = nt_piece_row(w * G::kPPW + q, l);
    const __bf16 *base;
    if (row < G::TM) {
      int64_t tok = tok0 + row;
      if (tok >= p.nq) tok = p.nq - 1;
      base = static_cast<const __bf16 *>(p.q) + tok * p.ldq + (int64_t)h * d;
    } else {
      const int r = row - G::TM;
      base = static_cast<const __bf16 *>(r < G::TN ? p.w1 : p.w3) + (int64_t)h * mat + (int64_t)(u0 + r % G::TN) * d;
    }
    src[q] = reinterpret_cast<const char *>(base) + nt_piece_off(row, l);
  }
  f32x4 acc[2][G::FM][G::FN];
  constexpr int pa[2] = {0, 0}, pb[2] = {0, 1};
  nt_mainloop<G, 2>(acc, src, pa, pb, d / 32, st0, st1, st2, st3, w, g, li, wr, wc);

  // H = SiLU(z1) o z3, staged as [256 tokens][128 hidden] bf16 in st0 (rows 0..127), st1;
  // tile (i, j) holds the products transposed: lane (g, li) has hidden units
  // 64 wc + 16 j + 4 g + r of token row 64 wr + 16 i + li
  __bf16 *hs0 = reinterpret_cast<__bf16 *>(st0), *hs1 = reinterpret_cast<__bf16 *>(st1);
  __bf16 *hs = wr < 2 ? hs0 : hs1;
#pragma unroll
  for (int i = 0; i < G::FM; ++i) {
    const int tr = wr * G::WM + 16 * i + li;
#pragma unroll
    for (int j = 0; j < G::FN; ++j) {
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float z = acc[0][i][j][r];
        v[r] = (__bf16)(z * sigmoid_fast(z) * acc[1][i][j][r]);
      }
      *reinterpret_cast<bf16x4 *>(hs + stage_w<G::TN>(tr & 127, (wc * G::WN + 16 * j) / 4 + g)) = v;
    }
  }
  __syncthreads();
  __bf16 *dst = static_cast<__bf16 *>(p.hbuf) + ((int64_t)h * p.nq_pad + tok0) * m + u0;
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int v = t + 512 * it;
    const int tr = v >> 4, cu = v & 15;
    const __bf16 *hs = it < 4 ? hs0 : hs1;
    const bf16x8 x = *reinterpret_cast<const bf16x8 *>(hs + stage_r<G::TN>(tr & 127, cu));
    __builtin_nontemporal_store(x, reinterpret_cast<bf16x8 *>(dst + (int64_t)tr * m + 8 * cu));
  }
}

__global__ __launch_bounds__(512) void big_out_kernel(BigApplyParams p) {
  using G = OutGeo;
  __shared__ __attribute__((aligned(1024))) unsigned char st0[G::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[G::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[G::kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char st3[G::kStage];
  const int t = threadIdx.x;
  const int d = p.d, m = p.m;
  const int tiles_d = d / G::TN;
  const int64_t tiles_t = p.nq_pad / G::TM;
  const int64_t total = (int64_t)p.heads * tiles_t * tiles_d;
  const int64_t item = xcd_work_item(total);
  if (item >= total) return;
  const int td = (int)(item % tiles_d);
  const int64_t ht = item / tiles_d;
  const int64_t tt = ht % tiles_t;
  const int h = (int)(ht / tiles_t);
  const int64_t tok0 = tt * G::TM;
  const int d0 = td * G::TN;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63, g = l >> 4, li = l & 15;
  const int wr = w & 3, wc = w >> 2;
  const int64_t mat = (int64_t)m * d;
  const char *src[G::kPPW];
#pragma unroll
  for (int q = 0; q < G::kPPW; ++q) {
    const int row = nt_piece_row(w * G::kPPW + q, l);
    const __bf16 *base;
    if (row < G::TM)   // H rows (every row of the padded tile exists)
      base = static_cast<const __bf16 *>(p.hbuf) + ((int64_t)h * p.nq_pad + tok0 + row) * m;
    else               // W2 row d0 + r: [d][m]
      base = static_cast<const __bf16 *>(p.w2) + (int64_t)h * mat + (int64_t)(d0 + row - G::TM) * m;
    src[q] = reinterpret_cast<const char *>(base) + nt_piece_off(row, l);
  }
  f32x4 acc[1][G::FM][G::FN];
  constexpr int pa[1] = {0}, pb[1] = {0};
  nt_mainloop<G, 1>(acc, src, pa, pb, m / 32, st0, st1, st2, st3, w, g, li, wr, wc);

  // O tile [256 tokens][256 of d] as bf16: tokens 64 b .. in stage b
  auto orow = [&](int blk) __attribute__((always_inline)) -> __bf16 * {
    return reinterpret_cast<__bf16 *>(blk == 0 ? st0 : blk == 1 ? st1 : blk == 2 ? st2 : st3);
  };
  // tile (i, j) holds the products transposed: lane (g, li) has columns
  // 128 wc + 16 j + 4 g + r of token row 16 i + li of the wave's 64-token block
  {
    __bf16 *os = orow(wr);
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
      for (int j = 0; j < G::FN; ++j) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (__bf16)acc[0][i][j][r];
        *reinterpret_cast<bf16x4 *>(os + stage_w<G::TN>(16 * i + li, (wc * G::WN + 16 * j) / 4 + g)) = v;
      }
  }
  __syncthreads();
  __bf16 *out = static_cast<__bf16 *>(p.o) + (int64_t)h * d + d0;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int v = t + 512 * it;
    const int tr = v >> 5, cu = v & 31;           // 256 rows x 32 vectors
    const int64_t tok = tok0 + tr;
    const bf16x8 x = *reinterpret_cast<const bf16x8 *>(orow(it >> 2) + stage_r<G::TN>(tr & 63, cu));
    if (tok < p.nq) __builtin_nontemporal_store(x, reinterpret_cast<bf16x8 *>(out + tok * p.ldo + 8 * cu));
  }
}

}  // namespace

// the tiles span 256 columns of d (contraction mode 1, output kernel) and 256 hidden units
bool big_supported(int d, int m, bool bf16) {
  return bf16 && d >= 512 && d <= 1024 && d % 256 == 0 && m % 256 == 0;
}
int64_t big_pad_tokens(int64_t n) { return (n + 767) / 768 * 768; }

hipError_t launch_big_fwd(const BigFwdParams &p, hipStream_t s) {
  const int64_t total = (int64_t)p.heads * (p.n_pad / FwdGeo::TM) * (p.m / FwdGeo::TN);
  hipLaunchKernelGGL(big_fwd_kernel, dim3((unsigned)((total + 7) / 8 * 8)), dim3(FwdGeo::kThreads), 0, s, p);
  return hipGetLastError();
}

int big_contract_tiles(int d, int m, int mode) {
  return mode == 0 ? (m / CtrGeo<0>::TM) * (d / CtrGeo<0>::TN) : (d / CtrGeo<1>::TM) * (m / CtrGeo<1>::TN);
}

hipError_t launch_big_contract(const BigCtrParams &p, hipStream_t s) {
  for (int mode = 0; mode < 2; ++mode) {
    const int64_t total = (int64_t)p.heads * p.splits * big_contract_tiles(p.d, p.m, mode);
    const dim3 grid((unsigned)((total + 7) / 8 * 8));
    if (mode == 0)
      hipLaunchKernelGGL(big_contract_kernel<0>, grid, dim3(512), 0, s, p);
    else
      hipLaunchKernelGGL(big_contract_kernel<1>, grid, dim3(512), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_big_apply(const BigApplyParams &p, hipStream_t s) {
  const int64_t th = (int64_t)p.heads * (p.nq_pad / HidGeo::TM) * (p.m / HidGeo::TN);
  hipLaunchKernelGGL(big_hidden_kernel, dim3((unsigned)((th + 7) / 8 * 8)), dim3(512), 0, s, p);
  const int64_t to = (int64_t)p.heads * (p.nq_pad / OutGeo::TM) * (p.d / OutGeo::TN);
  hipLaunchKernelGGL(big_out_kernel, dim3((unsigned)((to + 7) / 8 * 8)), dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace ttt
