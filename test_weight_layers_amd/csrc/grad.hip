// Fast-weight gradient of the eta-weighted dot-product loss, split-K over tokens.
//
// ZipMap (关键设计 1) takes one gradient over every token,
//   G = grad_W sum_i eta_i * (-f_W(k_i)^T v_i),  f_W(x) = W2 (SiLU(W1 x) o (W3 x)),
// with the loss of Scal3R eq. (9).  Because dL/df_i = -eta_i v_i does not depend
// on f, the gradient needs, per token and hidden unit j,
//   z1 = w1_j . k,  z3 = w3_j . k,  p = w2t_j . v   (forward on keys, back-projection of v)
//   s = sigmoid(z1), a = z1 s,  dH = -eta p,
//   dZ3 = dH a,  dZ1 = dH z3 (s + a - a s),  H' = -eta a z3
// and the three contractions over tokens
//   G1 = dZ1^T K,  G3 = dZ3^T K,  G2 = V^T H'.
//
// A workgroup owns one head, 64 hidden units (16 per wave), one output d-chunk
// and one contiguous token range (its split); it writes fp32 partial gradients
// that a second kernel sums in fixed split order (deterministic).
//
// Per 32-token block a wave computes z1, z3, p for its 16 hidden units x 32
// tokens (MFMA, tokens as rows), applies the SwiGLU backward in registers, and
// feeds dZ1, dZ3, H' straight back into the MFMA as operands: the tokens'
// row order is permuted (perm_row) so that the accumulator layout of the first
// product is the operand layout of the second, with no LDS round trip.
#include "common.h"
#include "kernels.h"

namespace ttt {
namespace {

// ---------------------------------------------------------------- fast path
// bf16 tokens, D <= 256.  Each 32-token block of K and V is DMA'd into LDS once,
// row-major and swizzled, into one of three stages.  The d-reductions read it as
// MFMA fragments with ds_read_b128; the token reductions read the same tile
// transposed with ds_read_b64_tr_b16.  Each wave keeps its 16 rows of W1, W3 and
// W2^T in registers.
//
// Software pipeline over blocks: iteration i runs the d-reductions of block i,
// then the SwiGLU backward of block i (VALU) interleaved with the token
// contractions of block i-1 (MFMA), while block i+1 streams into the third stage.
template <int D>
struct FastLayout {
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per token row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTile = kTokBlock * kRowBytes;     // one K or V block
  static constexpr int kStage = 2 * kTile;
  static constexpr int kStages = 3;
};

template <int D>
__global__ __launch_bounds__(256, 1) void grad_fast_kernel(GradParams p) {
  using L = FastLayout<D>;
  constexpr int KC = D / 32;   // reduction chunks over d
  constexpr int DT = D / 16;   // 16-wide d tiles of the outputs
  // three separate arrays (not one indexed array) so that the compiler can tell the
  // stage being DMA'd from the two being read and need not wait for the DMA
  __shared__ __attribute__((aligned(16))) unsigned char st0[L::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char st1[L::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char st2[L::kStage];

  const int total = gridDim.x;
  const int b = blockIdx.x;
  const int lin = p.xcd_map ? ((b & 7) * (total >> 3) + (b >> 3)) : b;
  const int mtiles = p.m / kHidTile;
  const int jt = lin % mtiles;
  int grp = lin / mtiles;
  const int h = grp % p.heads;
  const int split = grp / p.heads;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
  const int hid0 = jt * kHidTile + 16 * w;

  // weights of this wave's 16 hidden units, B-operand fragments over d
  bf16x8 w1f[KC], w3f[KC], w2f[KC];
  {
    const int64_t row = ((int64_t)h * p.m + hid0 + li) * D + 8 * g;
    const __bf16 *W1 = static_cast<const __bf16 *>(p.w1) + row;
    const __bf16 *W3 = static_cast<const __bf16 *>(p.w3) + row;
    const __bf16 *W2 = static_cast<const __bf16 *>(p.w2t) + row;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      w1f[kc] = ld8(W1 + 32 * kc);
      w3f[kc] = ld8(W3 + 32 * kc);
      w2f[kc] = ld8(W2 + 32 * kc);
    }
  }

  f32x4 a1[DT], a3[DT], a2[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) a1[i] = a3[i] = a2[i] = f32x4{0, 0, 0, 0};

  const int64_t blk0 = (int64_t)split * p.nblk / p.splits;
  const int64_t blk1 = (int64_t)(split + 1) * p.nblk / p.splits;

  // Staging: each wave instruction DMAs 1 KB (64 lanes x 16 bytes) of a block
  // straight into LDS.  1 KB piece b of a stage holds matrix b / (NPIECE / 2) and
  // rows kRowsPer * (b % (NPIECE / 2)) ..; lane l fills row r = first + l / kChunks at
  // physical chunk p = l % kChunks, i.e. the logical chunk p ^ swizzle(r) of token
  // row r.  Rows past n are fetched from row n-1; their rate eta is set to 0, which
  // zeroes dH, dZ1, dZ3 and H' and so their whole contribution.
  constexpr int kRowsPer = 1024 / L::kRowBytes;           // token rows per 1 KB piece
  constexpr int NPIECE = L::kStage / 1024;                // pieces per stage
  constexpr int PPW = NPIECE / 4;                         // pieces per wave
  const __bf16 *Kh = static_cast<const __bf16 *>(p.k) + (int64_t)h * D;
  const __bf16 *Vh = static_cast<const __bf16 *>(p.v) + (int64_t)h * D;
  // per-lane byte offset of each piece inside a block (row r, logical chunk) and its row
  int srow[PPW], soff[PPW];
#pragma unroll
  for (int q = 0; q < PPW; ++q) {
    const int piece = w * PPW + q;
    const int r = kRowsPer * (piece % (NPIECE / 2)) + l / L::kChunks;
    srow[q] = r;
    soff[q] = (int)(((int64_t)r * p.ld + 8 * ((l % L::kChunks) ^ (swz_rows(r) & (L::kChunks - 1)))) * 2);
  }
  auto stage_block = [&](int64_t blk, unsigned char *dst) {
    const int64_t t0 = blk * kTokBlock;
    // wave-uniform block bases; per-lane 32-bit offsets (a block spans 32 rows)
    const char *kb = reinterpret_cast<const char *>(Kh + t0 * p.ld);
    const char *vb = reinterpret_cast<const char *>(Vh + t0 * p.ld);
    if (t0 + kTokBlock <= p.n) {                                  // wave-uniform: full block
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        const int piece = w * PPW + q;
        copy16_to_lds((piece >= NPIECE / 2 ? vb : kb) + soff[q], dst + piece * 1024);
      }
    } else {                                                      // last block: clamp rows to n-1
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        const int piece = w * PPW + q;
        const int r = srow[q];
        const int64_t shift = (t0 + r < p.n) ? 0 : (p.n - 1 - t0 - r) * p.ld * 2;
        copy16_to_lds((piece >= NPIECE / 2 ? vb : kb) + soff[q] + shift, dst + piece * 1024);
      }
    }
  };

  // eta of this lane's 8 tokens 8g .. 8g+7 of a block (0 past n), loaded one block ahead
  const float *eta = p.eta + (int64_t)h * p.eta_hs;
  float en[8];
  auto load_eta = [&](int64_t blk) {
    const int64_t t0 = blk * kTokBlock + 8 * g;
    if (blk * kTokBlock + kTokBlock <= p.n) {                   // wave-uniform: block is full
      const f32x4 a = *reinterpret_cast<const f32x4 *>(eta + t0);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(eta + t0 + 4);
#pragma unroll
      for (int v = 0; v < 4; ++v) en[v] = a[v], en[4 + v] = b[v];
    } else {
#pragma unroll
      for (int v = 0; v < 8; ++v) en[v] = (t0 + v < p.n) ? eta[t0 + v] : 0.0f;
    }
  };

  // LDS addresses.  Chunk indices 4kc + g (d-reductions) and 2dt + e (token
  // reductions) share no bits with the loop counter's XOR partner, so with the
  // swizzle s of a row:  ((4kc + g) ^ s) * 16 = (16 (g ^ s)) ^ 64 kc  and
  // ((2dt + e) ^ s) * 16 = (16 (e ^ s)) ^ 32 dt: one XOR per read.
  // d-reductions: row perm_row(u, li), chunk 4kc + g.
  int base_a[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int rt = perm_row(u, li);
    base_a[u] = rt * L::kRowBytes + 16 * (g ^ (swz_rows(rt) & (L::kChunks - 1)));
  }
  // token reductions (transposed reads): lane (g, li) supplies row 8g + 4q + li/4,
  // column 16 dt + 4 (li % 4) and receives rows 8g + 4q .. +3 of column 16 dt + li.
  int base_b[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 8 * g + 4 * q + (li >> 2);
    const int e = (li & 3) >> 1;
    base_b[q] = row * L::kRowBytes + 16 * (e ^ (swz_rows(row) & (L::kChunks - 1))) + 8 * (li & 1);
  }

  // d-reductions of one block: z1 = K W1^T, z3 = K W3^T, p = V W2 for this wave's
  // 16 hidden units; rows = tokens perm_row(u, li); fragments one chunk ahead
  f32x4 z1[2], z3[2], pp[2];
  auto forward = [&](const unsigned char *base) {
    constexpr int NA = 2 * KC;
    bf16x8 kf[2], vf[2];
    auto lda = [&](int i, int slot) {
      const int u = i / KC, kc = i % KC;
      const unsigned char *pk = base + (base_a[u] ^ (64 * kc));
      kf[slot] = *reinterpret_cast<const bf16x8 *>(pk);
      vf[slot] = *reinterpret_cast<const bf16x8 *>(pk + L::kTile);
    };
    lda(0, 0);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int u = i / KC, kc = i % KC;
      if (kc == 0) z1[u] = z3[u] = pp[u] = f32x4{0, 0, 0, 0};
      if (i + 1 < NA) lda(i + 1, (i + 1) & 1);
      z1[u] = mma(kf[i & 1], w1f[kc], z1[u]);
      z3[u] = mma(kf[i & 1], w3f[kc], z3[u]);
      pp[u] = mma(vf[i & 1], w2f[kc], pp[u]);
    }
  };
  // SwiGLU backward of element v = 4u + r (token 8g + v, hidden hid0 + li)
  float dz1v[8], dz3v[8], hv[8];
  auto backward_elem = [&](int v, const float *e) {
    const int u = v >> 2, r = v & 3;
    const float z = z1[u][r], y = z3[u][r], ne = e[v];
    const float sg = sigmoid_fast(z);
    const float act = z * sg;
    const float dh = ne * pp[u][r];
    dz3v[v] = dh * act;
    dz1v[v] = dh * y * (sg + act - act * sg);
    hv[v] = ne * (act * y);
  };
  // token contractions of a block: G1 += dZ1^T K, G3 += dZ3^T K, G2 += V^T H', with
  // the SwiGLU backward of the next block (if any) interleaved between the MFMAs
  bf16x8 dz1f, dz3f, hf;
  auto contract = [&](const unsigned char *base, bool with_backward, const float *e) {
    bf16x8 ktf[2], vtf[2];
    auto ldb = [&](int dt, int slot) {
      const unsigned char *p0 = base + (base_b[0] ^ (32 * dt));
      const unsigned char *p1 = base + (base_b[1] ^ (32 * dt));
      ktf[slot] = cat8(lds_read_tr16(p0), lds_read_tr16(p1));
      vtf[slot] = cat8(lds_read_tr16(p0 + L::kTile), lds_read_tr16(p1 + L::kTile));
    };
    ldb(0, 0);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      if (dt + 1 < DT) ldb(dt + 1, (dt + 1) & 1);
      a1[dt] = mma(dz1f, ktf[dt & 1], a1[dt]);
      a3[dt] = mma(dz3f, ktf[dt & 1], a3[dt]);
      a2[dt] = mma(vtf[dt & 1], hf, a2[dt]);
      if (with_backward)   // the 8 backward elements spread evenly over the DT steps
#pragma unroll
        for (int v = dt * 8 / DT; v < (dt + 1) * 8 / DT; ++v) backward_elem(v, e);
    }
  };
  auto pack = [&]() {
    dz1f = pack8<__bf16>(dz1v);
    dz3f = pack8<__bf16>(dz3v);
    hf = pack8<__bf16>(hv);
  };

  if (blk0 < blk1) {
    load_eta(blk0);
    stage_block(blk0, st0);
    if (blk0 + 1 < blk1) stage_block(blk0 + 1, st1);
    wait_all_memory();
    __syncthreads();
    // prologue: forward and backward of the first block
    float e[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) e[v] = -en[v];
    if (blk0 + 1 < blk1) load_eta(blk0 + 1);
    forward(st0);
#pragma unroll
    for (int v = 0; v < 8; ++v) backward_elem(v, e);
    pack();
    // block blk lives in stage (blk - blk0) % 3
    auto iteration = [&](int64_t blk, const unsigned char *cur, const unsigned char *prev, unsigned char *next) {
      // consume the prefetched rates before issuing new memory operations, so that
      // no wait for them can also wait for the DMA issued below
#pragma unroll
      for (int v = 0; v < 8; ++v) e[v] = -en[v];
      if (blk + 1 < blk1) {
        load_eta(blk + 1);
        stage_block(blk + 1, next);     // into the stage freed by block blk-2
      }
      forward(cur);
      contract(prev, true, e);          // block blk-1's contractions + block blk's backward
      pack();
      wait_all_memory();
      __syncthreads();
    };
    for (int64_t blk = blk0 + 1; blk < blk1; blk += 3) {
      iteration(blk, st1, st0, st2);
      if (blk + 1 < blk1) iteration(blk + 1, st2, st1, st0);
      if (blk + 2 < blk1) iteration(blk + 2, st0, st2, st1);
    }
    const int last = (int)((blk1 - 1 - blk0) % 3);
    contract(last == 0 ? st0 : (last == 1 ? st1 : st2), false, e);
  }

  // partials: G1/G3 rows hid0 + 4g + r, cols 16 dt + li;  G2 rows 16 dt + 4g + r, cols hid0 + li
  const int64_t mat = (int64_t)p.m * D;
  float *P1 = p.part + ((int64_t)split * 3 * p.heads + h) * mat;
  float *P3 = P1 + p.heads * mat;
  float *P2 = P3 + p.heads * mat;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      P1[(int64_t)(hid0 + 4 * g + r) * D + 16 * dt + li] = a1[dt][r];
      P3[(int64_t)(hid0 + 4 * g + r) * D + 16 * dt + li] = a3[dt][r];
      P2[(int64_t)(16 * dt + 4 * g + r) * p.m + hid0 + li] = a2[dt][r];
    }
}

// ------------------------------------------------------------- general path
// Any supported d, fp32 or bf16.  The d-reductions read K, V and the weights
// straight from global memory (L1/L2 resident); only the transposed K, V
// columns of this workgroup's output d-chunk go through LDS.  The forward is
// recomputed for every d-chunk.
template <typename T, int D, int DC>
__global__ __launch_bounds__(256) void grad_general_kernel(GradParams p) {
  using F = typename FragOf<T>::type;
  constexpr int KC = D / 32;
  constexpr int DT = DC / 16;
  constexpr int PAD = 16 / sizeof(T);         // keeps 16-byte aligned rows
  constexpr int RS = kTokBlock + PAD;         // LDS row stride (elements)
  __shared__ __attribute__((aligned(16))) T kt[DC * RS];
  __shared__ __attribute__((aligned(16))) T vt[DC * RS];

  const int b = blockIdx.x;
  const int mtiles = p.m / kHidTile;
  const int jt = b % mtiles;
  int grp = b / mtiles;
  const int dc = grp % p.dchunks;
  grp /= p.dchunks;
  const int h = grp % p.heads;
  const int split = grp / p.heads;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
  const int hid0 = jt * kHidTile + 16 * w;
  const int d0 = dc * DC;

  const T *K = static_cast<const T *>(p.k) + (int64_t)h * D;
  const T *V = static_cast<const T *>(p.v) + (int64_t)h * D;
  const int64_t wrow = ((int64_t)h * p.m + hid0 + li) * D + 8 * g;
  const T *W1 = static_cast<const T *>(p.w1) + wrow;
  const T *W3 = static_cast<const T *>(p.w3) + wrow;
  const T *W2 = static_cast<const T *>(p.w2t) + wrow;
  const float *eta = p.eta + (int64_t)h * p.eta_hs;

  f32x4 a1[DT], a3[DT], a2[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) a1[i] = a3[i] = a2[i] = f32x4{0, 0, 0, 0};

  const int64_t blk0 = (int64_t)split * p.nblk / p.splits;
  const int64_t blk1 = (int64_t)(split + 1) * p.nblk / p.splits;
  for (int64_t blk = blk0; blk < blk1; ++blk) {
    const int64_t tb = blk * kTokBlock;
    // stage K, V columns [d0, d0 + DC) of the block, transposed
    for (int e = tid; e < kTokBlock * DC; e += 256) {
      const int i = e / DC, c = e % DC;
      const int64_t tok = tb + i;
      const bool ok = tok < p.n;
      kt[c * RS + i] = ok ? K[tok * p.ld + d0 + c] : from_f32<T>(0.0f);
      vt[c * RS + i] = ok ? V[tok * p.ld + d0 + c] : from_f32<T>(0.0f);
    }
    float e8[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) e8[v] = (tb + 8 * g + v < p.n) ? eta[tb + 8 * g + v] : 0.0f;
    __syncthreads();

    f32x4 z1[2], z3[2], pp[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      z1[u] = z3[u] = pp[u] = f32x4{0, 0, 0, 0};
      const int64_t tok = tb + perm_row(u, li);
      const bool ok = tok < p.n;
#pragma unroll 2
      for (int kc = 0; kc < KC; ++kc) {
        const F kf = ok ? ld8(K + tok * p.ld + 32 * kc + 8 * g) : zero8<T>();
        const F vf = ok ? ld8(V + tok * p.ld + 32 * kc + 8 * g) : zero8<T>();
        z1[u] = mma(kf, ld8(W1 + 32 * kc), z1[u]);
        z3[u] = mma(kf, ld8(W3 + 32 * kc), z3[u]);
        pp[u] = mma(vf, ld8(W2 + 32 * kc), pp[u]);
      }
    }
    float dz1v[8], dz3v[8], hv[8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = 4 * u + r;
        const float z = z1[u][r], y = z3[u][r], ne = -e8[v];
        const float sg = sigmoid_fast(z);
        const float act = z * sg;
        const float dh = ne * pp[u][r];
        dz3v[v] = dh * act;
        dz1v[v] = dh * y * (sg + act - act * sg);
        hv[v] = ne * (act * y);
      }
    const F dz1f = pack8<T>(dz1v), dz3f = pack8<T>(dz3v), hf = pack8<T>(hv);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const F ktf = ld8(&kt[(16 * dt + li) * RS + 8 * g]);
      const F vtf = ld8(&vt[(16 * dt + li) * RS + 8 * g]);
      a1[dt] = mma(dz1f, ktf, a1[dt]);
      a3[dt] = mma(dz3f, ktf, a3[dt]);
      a2[dt] = mma(vtf, hf, a2[dt]);
    }
    __syncthreads();
  }

  const int64_t mat = (int64_t)p.m * D;
  float *P1 = p.part + ((int64_t)split * 3 * p.heads + h) * mat;
  float *P3 = P1 + p.heads * mat;
  float *P2 = P3 + p.heads * mat;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      P1[(int64_t)(hid0 + 4 * g + r) * D + d0 + 16 * dt + li] = a1[dt][r];
      P3[(int64_t)(hid0 + 4 * g + r) * D + d0 + 16 * dt + li] = a3[dt][r];
      P2[(int64_t)(d0 + 16 * dt + 4 * g + r) * p.m + hid0 + li] = a2[dt][r];
    }
}

template <typename T, int D>
hipError_t launch_general(const GradParams &p, int grid, hipStream_t s) {
  constexpr int DC = (sizeof(T) == 2) ? (D < 128 ? D : 128) : (D < 64 ? D : 64);
  hipLaunchKernelGGL((grad_general_kernel<T, D, DC>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_general_d(const GradParams &p, int d, int grid, hipStream_t s) {
  switch (d) {
    case 64: return launch_general<T, 64>(p, grid, s);
    case 128: return launch_general<T, 128>(p, grid, s);
    case 256: return launch_general<T, 256>(p, grid, s);
    case 512: return launch_general<T, 512>(p, grid, s);
    case 768: return launch_general<T, 768>(p, grid, s);
    case 1024: return launch_general<T, 1024>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool grad_fast_supported(int d, bool bf16) { return bf16 && (d == 64 || d == 128 || d == 256); }

int grad_general_dc(int d, bool bf16) {
  if (bf16) return d < 128 ? d : 128;
  return d < 64 ? d : 64;
}

hipError_t launch_grad(const GradParams &p, int d, bool bf16, bool fast, int grid, hipStream_t s) {
  if (fast) {
    switch (d) {
      case 64: hipLaunchKernelGGL(grad_fast_kernel<64>, dim3(grid), dim3(256), 0, s, p); break;
      case 128: hipLaunchKernelGGL(grad_fast_kernel<128>, dim3(grid), dim3(256), 0, s, p); break;
      case 256: hipLaunchKernelGGL(grad_fast_kernel<256>, dim3(grid), dim3(256), 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  return bf16 ? launch_general_d<__bf16>(p, d, grid, s) : launch_general_d<float>(p, d, grid, s);
}

}  // namespace ttt
