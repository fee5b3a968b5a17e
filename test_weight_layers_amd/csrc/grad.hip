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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace ttt {
namespace {

// ---------------------------------------------------------------- fast path
// bf16 tokens, D <= 256.  A workgroup has 8 waves in two roles that share the SIMDs
// (wave w and wave w + 4 run on one SIMD), so the hardware interleaves them:
//   waves 0-3 ("forward"): z1, z3, p of a block for 16 hidden units each (MFMA,
//     weights in registers, K/V fragments from LDS), then the SwiGLU backward (VALU);
//     the packed bf16 operands dZ1, dZ3, H' go to LDS;
//   waves 4-7 ("contraction"): the token contractions of the previous block for
//     the same hidden units, fp32 accumulators G1, G3, G2 in registers.
// K and V of a block are DMA'd into LDS once (row-major, swizzled) into one of three
// stages, with the block's rates; the forward waves read d-fragments as two 8-byte
// halves, the contraction waves read the tile transposed (ds_read_b64_tr_b16).
// Iteration i: forward of block i, contractions of block i-1, DMA of block i+1.
template <int D>
struct FastLayout {
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per token row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTile = kTokBlock * kRowBytes;     // one K or V block
  static constexpr int kEta = 2 * kTile;                  // the block's 32 rates (fp32), 256 bytes reserved
  static constexpr int kPk = kEta + 256;                  // packed dZ1, dZ3, H': [wave][3][lane] x 16 bytes
  static constexpr int kStage = kPk + 4 * 3 * 64 * 16;
};

typedef unsigned long long u64;
typedef u64 u64x2 __attribute__((ext_vector_type(2)));

template <int D>
__global__ __launch_bounds__(512, 1) void grad_fast_kernel(GradParams p) {
  using L = FastLayout<D>;
  constexpr int KC = D / 32;   // reduction chunks over d
  constexpr int DT = D / 16;   // 16-wide d tiles of the outputs
  // three separate arrays (not one indexed array), each named statically, so that
  // the compiler can tell the stage being DMA'd from the ones being read
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
  // wave index, role and hidden group are wave-uniform: keep them scalar
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool forward_role = wv < 4;
  const int w = wv & 3;
  const int l = tid & 63, g = l >> 4, li = l & 15;
  const int hid0 = jt * kHidTile + 16 * w;

  // token and block indices fit 32 bits (the host limits n): the loop control and
  // the ragged-block tests stay on the scalar unit
  const int n = (int)p.n;
  const int blk0 = (int)((int64_t)split * p.nblk / p.splits);
  const int blk1 = (int)((int64_t)(split + 1) * p.nblk / p.splits);
  const int nb = blk1 - blk0;

  // Staging: each wave instruction DMAs 1 KB (64 lanes x 16 bytes) of a block
  // straight into LDS.  1 KB piece b of a stage holds matrix b / (NPIECE / 2) and
  // rows kRowsPer * (b % (NPIECE / 2)) ..; lane l fills row r = first + l / kChunks at
  // physical chunk p = l % kChunks, i.e. the logical chunk p ^ swizzle(r) of token
  // row r.  Rows past n are fetched from row n-1; their rate is 0, which zeroes
  // dH, dZ1, dZ3 and H' and so their whole contribution.
  constexpr int kRowsPer = 1024 / L::kRowBytes;           // token rows per 1 KB piece
  constexpr int NPIECE = 2 * L::kTile / 1024;             // K and V pieces per stage
  constexpr int PPW = NPIECE / 8;                         // pieces per wave
  const __bf16 *Kh = static_cast<const __bf16 *>(p.k) + (int64_t)h * D;
  const __bf16 *Vh = static_cast<const __bf16 *>(p.v) + (int64_t)h * D;
  auto piece_row = [&](int q) { return kRowsPer * ((wv * PPW + q) % (NPIECE / 2)) + l / L::kChunks; };
  unsigned soff[PPW];          // per-lane byte offset of each piece inside a block
  const unsigned row_bytes = (unsigned)(p.ld * 2);
#pragma unroll
  for (int q = 0; q < PPW; ++q) {
    const int r = piece_row(q);
    soff[q] = (unsigned)r * row_bytes + 16u * (unsigned)((l % L::kChunks) ^ (swz_rows(r) & (L::kChunks - 1)));
  }
  // The rates of a block come with it (wave 0, one dword per lane) through a
  // range-checked buffer view that ends at token n: rates past n arrive as 0.
  const float *eta = p.eta + (int64_t)h * p.eta_hs;
  auto stage_block = [&](int blk, unsigned char *dst) {
    const int t0 = blk * kTokBlock;
    if (wv == 0) {
      const int valid = n - t0 < kTokBlock ? n - t0 : kTokBlock;
      const __amdgpu_buffer_rsrc_t er =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(eta + t0), (short)0, valid * 4, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(er, (__attribute__((address_space(3))) void *)(dst + L::kEta), 4,
                                               4u * (unsigned)l, 0, 0, 0);
    }
    // wave-uniform block bases; unsigned per-lane 32-bit offsets (a block spans 32 rows)
    const char *kb = reinterpret_cast<const char *>(Kh + (int64_t)t0 * p.ld);
    const char *vb = reinterpret_cast<const char *>(Vh + (int64_t)t0 * p.ld);
    if (t0 + kTokBlock <= n) {                                    // wave-uniform: full block
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        const int piece = wv * PPW + q;
        copy16_to_lds((piece >= NPIECE / 2 ? vb : kb) + soff[q], dst + piece * 1024);
      }
    } else {                                                      // last block: clamp rows to n-1
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        const int piece = wv * PPW + q;
        const int r = piece_row(q), keep = n - 1 - t0;
        const unsigned off = r <= keep ? soff[q] : soff[q] - (unsigned)(r - keep) * row_bytes;
        copy16_to_lds((piece >= NPIECE / 2 ? vb : kb) + off, dst + piece * 1024);
      }
    }
  };
  auto sync = [&]() {
    wait_all_memory();
    __syncthreads();
  };
  // Pace keeping.  The m / 64 workgroups of one token range (one per hidden tile)
  // run on one XCD and read the same K/V blocks, which its L2 serves once while they
  // stay close; left alone they drift apart over thousands of blocks until the L2
  // no longer holds a block between its readers.  Every kPace blocks, wave 0 counts
  // the workgroup in at its group's counter and waits (bounded: the wait is only a
  // hint, nothing depends on it) until every workgroup of the group has passed the
  // previous checkpoint, so they stay within 2 kPace blocks of each other.
  constexpr int kPace = 32;
  unsigned *const pace = p.group_sync ? p.group_sync + split * p.heads + h : nullptr;
  auto keep_pace = [&](int i) {
    if (pace == nullptr || (i + 1) % kPace != 0 || wv != 0) return;
    if (l == 0) {
      const unsigned c = (unsigned)((i + 1) / kPace);
      __hip_atomic_fetch_add(pace, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned target = (unsigned)mtiles * (c - 1);
      for (int spin = 0; spin < 256; ++spin) {
        if (__hip_atomic_load(pace, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
        __builtin_amdgcn_s_sleep(8);
      }
    }
  };
  // this lane's 16-byte slot of operand op in the packed-operand area of a stage
  const int pk_slot = L::kPk + ((w * 3) * 64 + l) * 16;

  if (nb > 0) {
    stage_block(blk0, st0);
    sync();
  }
  // Both roles run iterations i = 0 .. nb with one barrier each: the forward waves
  // idle in the last, the contraction waves in the first.  Block blk0 + i lives in
  // stage i % 3; the loop is unrolled by 3 so that every stage is named statically.
  if (forward_role) {
    // d-reduction fragments are read as two 8-byte halves; odd lane groups take the
    // upper half first, which spreads one read over all 64 banks.  The MFMA only
    // needs A and B to agree on the k order, so the weights use the same order.
    const int hs = (g & 1) * 8;
    bf16x8 w1f[KC], w3f[KC], w2f[KC];   // B-operand fragments over d, this wave's 16 hidden units
    {
      const int64_t row = ((int64_t)h * p.m + hid0 + li) * D + 8 * g;
      const char *W1 = reinterpret_cast<const char *>(static_cast<const __bf16 *>(p.w1) + row);
      const char *W3 = reinterpret_cast<const char *>(static_cast<const __bf16 *>(p.w3) + row);
      const char *W2 = reinterpret_cast<const char *>(static_cast<const __bf16 *>(p.w2t) + row);
      auto frag = [&](const char *src) {
        const u64 lo = *reinterpret_cast<const u64 *>(src + hs), hi = *reinterpret_cast<const u64 *>(src + 8 - hs);
        return __builtin_bit_cast(bf16x8, u64x2{lo, hi});
      };
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        w1f[kc] = frag(W1 + 64 * kc);
        w3f[kc] = frag(W3 + 64 * kc);
        w2f[kc] = frag(W2 + 64 * kc);
      }
    }
    // LDS addresses.  Chunk 4kc + g of row rt with swizzle s: ((4kc + g) ^ s) * 16 =
    // (16 (g ^ s)) ^ 64 kc, one XOR per read; rows perm_row(u, li).
    int base_a[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int rt = perm_row(u, li);
      const int a = rt * L::kRowBytes + 16 * (g ^ (swz_rows(rt) & (L::kChunks - 1)));
      base_a[u][0] = a + hs;
      base_a[u][1] = a + 8 - hs;
    }
    // forward + backward of the block in stage `cur`; packed operands into `cur`
    auto forward_block = [&](unsigned char *cur) {
      f32x4 z1[2], z3[2], pp[2];
      bf16x8 kf[2], vf[2];
      auto lda = [&](int i, int slot) {
        const int u = i / KC, kc = i % KC;
        // V's addresses pass through an empty asm: otherwise the K and V halves
        // (16 KB apart) merge into paired reads whose results need register moves
        int v0 = base_a[u][0] ^ (64 * kc), v1 = base_a[u][1] ^ (64 * kc);
        const unsigned char *p0 = cur + v0, *p1 = cur + v1;
        asm volatile("" : "+v"(v0), "+v"(v1));
        const unsigned char *q0 = cur + L::kTile + v0, *q1 = cur + L::kTile + v1;
        kf[slot] = __builtin_bit_cast(bf16x8, u64x2{*reinterpret_cast<const u64 *>(p0),
                                                    *reinterpret_cast<const u64 *>(p1)});
        vf[slot] = __builtin_bit_cast(bf16x8, u64x2{*reinterpret_cast<const u64 *>(q0),
                                                    *reinterpret_cast<const u64 *>(q1)});
      };
      constexpr int NA = 2 * KC;
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
      // rates of this lane's tokens 8g .. 8g+7
      const f32x4 ea = *reinterpret_cast<const f32x4 *>(cur + L::kEta + 32 * g);
      const f32x4 eb = *reinterpret_cast<const f32x4 *>(cur + L::kEta + 32 * g + 16);
      // SwiGLU backward of element v = 4u + r (token 8g + v, hidden hid0 + li), with
      // dL/df = -eta v:  dH = -eta p
      bf16x8 pk1, pk3, pkh;
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int u = v >> 2, r = v & 3;
        const float ne = -(v < 4 ? ea[v] : eb[v - 4]);
        const float z = z1[u][r], y = z3[u][r];
        const float sg = sigmoid_fast(z);
        const float act = z * sg;
        const float dh = ne * pp[u][r];
        pk3[v] = (__bf16)(dh * act);
        pk1[v] = (__bf16)(dh * y * (sg + act - act * sg));
        pkh[v] = (__bf16)(ne * (act * y));
      }
      *reinterpret_cast<bf16x8 *>(cur + pk_slot) = pk1;
      *reinterpret_cast<bf16x8 *>(cur + pk_slot + 1024) = pk3;
      *reinterpret_cast<bf16x8 *>(cur + pk_slot + 2048) = pkh;
    };
    auto step = [&](int i, unsigned char *cur, unsigned char *next) {
      if (i + 1 < nb) stage_block(blk0 + i + 1, next);
      forward_block(cur);
      keep_pace(i);
      sync();
    };
    int i = 0;
    for (; i + 3 <= nb; i += 3) {
      step(i, st0, st1);
      step(i + 1, st1, st2);
      step(i + 2, st2, st0);
    }
    if (i < nb) step(i, st0, st1);
    if (i + 1 < nb) step(i + 1, st1, st2);
    if (nb > 0) sync();                // iteration nb: the contraction of the last block
  } else {
    f32x4 a1[DT], a3[DT], a2[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) a1[t] = a3[t] = a2[t] = f32x4{0, 0, 0, 0};
    // transposed reads: lane (g, li) supplies row 8g + 4q + li/4, column 16 dt + 4 (li % 4)
    // and receives rows 8g + 4q .. +3 of column 16 dt + li; chunk 2dt + e of row r with
    // swizzle s: ((2dt + e) ^ s) * 16 = (16 (e ^ s)) ^ 32 dt
    int base_b[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = 8 * g + 4 * q + (li >> 2);
      const int e = (li & 3) >> 1;
      base_b[q] = row * L::kRowBytes + 16 * (e ^ (swz_rows(row) & (L::kChunks - 1))) + 8 * (li & 1);
    }
    // G1 += dZ1^T K, G3 += dZ3^T K, G2 += V^T H' for the block in stage `prev`
    auto contract_block = [&](const unsigned char *prev) {
      const bf16x8 pk1 = *reinterpret_cast<const bf16x8 *>(prev + pk_slot);
      const bf16x8 pk3 = *reinterpret_cast<const bf16x8 *>(prev + pk_slot + 1024);
      const bf16x8 pkh = *reinterpret_cast<const bf16x8 *>(prev + pk_slot + 2048);
      bf16x8 ktf[2], vtf[2];
      auto ldb = [&](int dt, int slot) {
        // the bases pass through an empty asm so that each address is formed (one
        // XOR) right before its read instead of 32 of them being held in registers
        int b0 = base_b[0], b1 = base_b[1];
        asm volatile("" : "+v"(b0), "+v"(b1));
        const unsigned char *p0 = prev + (b0 ^ (32 * dt));
        const unsigned char *p1 = prev + (b1 ^ (32 * dt));
        ktf[slot] = cat8(lds_read_tr16(p0), lds_read_tr16(p1));
        vtf[slot] = cat8(lds_read_tr16(p0 + L::kTile), lds_read_tr16(p1 + L::kTile));
      };
      ldb(0, 0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        if (dt + 1 < DT) ldb(dt + 1, (dt + 1) & 1);
        a1[dt] = mma(pk1, ktf[dt & 1], a1[dt]);
        a3[dt] = mma(pk3, ktf[dt & 1], a3[dt]);
        a2[dt] = mma(vtf[dt & 1], pkh, a2[dt]);
      }
    };
    auto step = [&](int i, const unsigned char *prev, unsigned char *next) {
      if (i + 1 < nb) stage_block(blk0 + i + 1, next);
      if (i > 0) contract_block(prev);
      sync();
    };
    // iteration i: contraction of block i - 1 (stage (i - 1) % 3), DMA of block i + 1
    int i = 0;
    for (; i + 3 <= nb; i += 3) {
      step(i, st2, st1);
      step(i + 1, st0, st2);
      step(i + 2, st1, st0);
    }
    if (i < nb) step(i, st2, st1);
    if (i + 1 < nb) step(i + 1, st0, st2);
    if (nb > 0) {                      // iteration nb: the last block, stage (nb - 1) % 3
      const int last = (nb - 1) % 3;
      contract_block(last == 0 ? st0 : (last == 1 ? st1 : st2));
      sync();
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

__global__ __launch_bounds__(256) void zero_u32_kernel(unsigned *p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_u32(unsigned *p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

bool grad_fast_supported(int d, bool bf16) { return bf16 && (d == 64 || d == 128 || d == 256); }

int grad_general_dc(int d, bool bf16) {
  if (bf16) return d < 128 ? d : 128;
  return d < 64 ? d : 64;
}

hipError_t launch_grad(const GradParams &p, int d, bool bf16, bool fast, int grid, hipStream_t s) {
  if (fast) {
    switch (d) {
      // 8 waves: 4 forward + 4 contraction (see grad_fast_kernel)
      case 64: hipLaunchKernelGGL(grad_fast_kernel<64>, dim3(grid), dim3(512), 0, s, p); break;
      case 128: hipLaunchKernelGGL(grad_fast_kernel<128>, dim3(grid), dim3(512), 0, s, p); break;
      case 256: hipLaunchKernelGGL(grad_fast_kernel<256>, dim3(grid), dim3(512), 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  return bf16 ? launch_general_d<__bf16>(p, d, grid, s) : launch_general_d<float>(p, d, grid, s);
}

}  // namespace ttt
