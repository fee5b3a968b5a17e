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
// tokens (MFMA, tokens as rows) and applies the SwiGLU backward in registers.
// The tokens' row order is permuted (perm_row) so that the accumulator layout of
// the first product is the operand layout of the contractions: dZ1, dZ3, H' are
// packed to bf16 operands as they are.  In the general kernel the same wave then
// runs the contractions from registers; in the fast kernel the packed operands
// pass through a small LDS buffer to the waves that hold the accumulators.
#include "common.h"
#include "kernels.h"

namespace ttt {
namespace {

// ---------------------------------------------------------------- fast path
// bf16 tokens, D <= 256.  A workgroup has 4 + 4 CS waves in two roles that share the
// SIMDs (waves w, w + 4, w + 8 run on one SIMD), so the hardware interleaves them:
//   waves 0-3 ("forward"): z1, z3, p of a block for 16 hidden units each (MFMA,
//     weights in registers, K/V fragments from LDS), then the SwiGLU backward (VALU);
//     the packed bf16 operands dZ1, dZ3, H' go to one of two LDS buffers;
//   waves 4 .. 3 + 4 CS ("contraction"): the token contractions of the previous block,
//     each wave for two hidden groups (32 units) and D / (2 CS) of the output columns,
//     with their fp32 accumulators G1, G3, G2 in registers: every transposed K / V
//     fragment it reads from LDS feeds six products (with one hidden group per wave,
//     three, and the LDS reads per block were 26% higher); four of these waves, one
//     per SIMD, also issue all of the staging DMA.
// K and V of a block are DMA'd into LDS once (row-major, swizzled) into one of four
// stages, with the block's rates; the forward waves read 16-byte d-fragments, the
// contraction waves read the tile transposed (ds_read_b64_tr_b16).
// Iteration i: DMA of block i+2, forward of block i, contractions of block i-1.  The
// DMA has two iterations to land: the barrier that ends an iteration waits only for
// the block needed next (s_waitcnt vmcnt(N) with the N copies just issued still in
// flight), not for the one issued in it.
template <int D>
struct FastLayout {
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per token row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTile = kTokBlock * kRowBytes;     // one K or V block
  static constexpr int kEta = 2 * kTile;                  // the block's 32 rates (fp32), 256 bytes reserved
  static constexpr int kStage = kEta + 256;
};
// packed dZ1, dZ3, H' of one block: [wave][3][lane] x 16 bytes
constexpr int kPkBytes = 4 * 3 * 64 * 16;

typedef unsigned long long u64;
typedef u64 u64x2 __attribute__((ext_vector_type(2)));

// Buffer-view copies into LDS issued through inline asm, so that the compiler does
// not count them (its waits cannot tell a copy in flight across the loop's back
// edge from the stage being read, and it would wait for every copy).  The copying
// waves wait for them with the explicit s_waitcnt in sync().  The leading s_nop 4
// covers an SGPR operand written by a VALU instruction just before.
__device__ __forceinline__ void copy16_untracked(__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned char *dst) {
  const unsigned m0v = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)dst;
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(m0v) : "memory");
}
__device__ __forceinline__ void copy4_untracked(__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned char *dst) {
  const unsigned m0v = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)dst;
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(m0v) : "memory");
}

// 4 kGradCS contraction waves: each takes two of the four hidden groups and
// D / (2 kGradCS) of the output columns
constexpr int kGradCS = 2;

template <int D, int CS>
__global__ __launch_bounds__((4 + 4 * CS) * 64, 1) void grad_fast_kernel(GradParams p) {
  using L = FastLayout<D>;
  constexpr int KC = D / 32;   // reduction chunks over d
  constexpr int DT = D / 16;   // 16-wide d tiles of the outputs
  constexpr int FR = CS == 1 ? 3 : 2;   // forward read ring (registers are scarcer at 3 waves per SIMD)
  // separate arrays (not one indexed array), each named statically, so that the
  // compiler can tell the stages apart
  __shared__ __attribute__((aligned(16))) unsigned char st0[L::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char st1[L::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char st2[L::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char st3[L::kStage];
  __shared__ __attribute__((aligned(16))) unsigned char pkb0[kPkBytes];
  __shared__ __attribute__((aligned(16))) unsigned char pkb1[kPkBytes];

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
  const int w = wv & 3;                 // hidden group (both roles)
  const int c = wv - 4;                 // contraction wave index 0 .. 4 CS - 1
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
  // row r.  Contraction wave 4 + c (c < NDMA) copies K pieces c * PPW .. and the V
  // pieces of the same rows.  Rows past n are fetched from row n-1; their rate is 0,
  // which zeroes dH, dZ1, dZ3 and H' and so their whole contribution.
  // Only the contraction waves DMA (measured fastest: copies on the forward waves,
  // which are the longer chain, slow the block down).  The copies are issued through
  // inline asm that the compiler does not count (copy16_untracked), and sync() waits
  // for them explicitly.
  constexpr int kRowsPer = 1024 / L::kRowBytes;           // token rows per 1 KB piece
  constexpr int NPIECE = 2 * L::kTile / 1024;             // K and V pieces per stage
  // four DMA waves, one per SIMD, so that the other contraction wave of each SIMD
  // starts its products while the copies issue (all eight copying: 1% slower)
  constexpr int PPW = NPIECE / 2 >= 4 ? NPIECE / 2 / 4 : 1;   // K pieces per DMA wave
  constexpr int NDMA = NPIECE / 2 / PPW;                  // contraction waves that DMA
  const __bf16 *Kh = static_cast<const __bf16 *>(p.k) + (int64_t)h * D;
  const __bf16 *Vh = static_cast<const __bf16 *>(p.v) + (int64_t)h * D;
  const unsigned row_bytes = (unsigned)(p.ld * 2);
  // The rates of a block come with it (wave 4, one dword per lane) through a
  // range-checked buffer view that ends at token n: rates past n arrive as 0.
  const float *eta = p.eta + (int64_t)h * p.eta_hs;
  // Per-lane byte offset of each piece's rows inside a block: the same for every block,
  // so it is formed once and held (rebuilding it per block costs the copying waves
  // about 30 VALU instructions per block, measurably more than the two registers).
  unsigned soff[PPW];
#pragma unroll
  for (int q = 0; q < PPW; ++q) {
    const int r = kRowsPer * (c * PPW + q) + l / L::kChunks;
    soff[q] = (unsigned)r * row_bytes + 16u * (unsigned)((l % L::kChunks) ^ (swz_kv(r) & (L::kChunks - 1)));
  }
  auto stage_block = [&](int blk, unsigned char *dst) {
    if (forward_role || c >= NDMA) return;
    const int t0 = blk * kTokBlock;
    if (wv == 4) {
      const int valid = n - t0 < kTokBlock ? n - t0 : kTokBlock;
      const __amdgpu_buffer_rsrc_t er = buffer_view(eta + t0, 4u * (unsigned)valid);
      copy4_untracked(er, 4u * (unsigned)l, dst + L::kEta);
    }
    auto piece_row = [&](int q) { return kRowsPer * (c * PPW + q) + l / L::kChunks; };
    // wave-uniform buffer views of the block's 32 rows; unsigned per-lane offsets
    const __amdgpu_buffer_rsrc_t kr = buffer_view(Kh + (int64_t)t0 * p.ld, kTokBlock * row_bytes);
    const __amdgpu_buffer_rsrc_t vr = buffer_view(Vh + (int64_t)t0 * p.ld, kTokBlock * row_bytes);
    if (t0 + kTokBlock <= n) {                                    // wave-uniform: full block
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        const int piece = c * PPW + q;
        copy16_untracked(kr, soff[q], dst + piece * 1024);
        copy16_untracked(vr, soff[q], dst + (piece + NPIECE / 2) * 1024);
      }
    } else {                                                      // last block: clamp rows to n-1
#pragma unroll
      for (int q = 0; q < PPW; ++q) {
        const int piece = c * PPW + q;
        const int r = piece_row(q), keep = n - 1 - t0;
        const unsigned off = r <= keep ? soff[q] : soff[q] - (unsigned)(r - keep) * row_bytes;
        copy16_untracked(kr, off, dst + piece * 1024);
        copy16_untracked(vr, off, dst + (piece + NPIECE / 2) * 1024);
      }
    }
  };
  // End of an iteration: this wave's LDS writes and every DMA but the `inflight`
  // copies it issued last are complete, then the workgroup barrier.
  auto sync = [&](bool inflight) {
    if (!inflight || forward_role || c >= NDMA) wait_vmcnt_lds<0>();
    else if (wv == 4) wait_vmcnt_lds<2 * PPW + 1>();
    else wait_vmcnt_lds<2 * PPW>();
    bare_barrier();
  };
  // Pace keeping.  The m / 64 workgroups of one token range (one per hidden tile)
  // run on one XCD and read the same K/V blocks, which its L2 serves once while they
  // stay close; left alone they drift apart over thousands of blocks until the L2
  // no longer holds a block between its readers.  Every kPace iterations, wave 0
  // counts the workgroup in at its group's counter and waits (bounded: the wait is
  // only a hint, nothing depends on it) until every workgroup of the group has passed
  // the previous checkpoint, so they stay within 2 kPace blocks of each other.
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
  // this lane's 16-byte slot of operand op in a packed-operand buffer
  const int pk_slot = ((w * 3) * 64 + l) * 16;

  if (nb > 0) {
    stage_block(blk0, st0);
    if (nb > 1) stage_block(blk0 + 1, st1);
    sync(nb > 1);
  }
  // Both roles run iterations i = 0 .. nb with one barrier each.  Block blk0 + i
  // lives in stage i % 4 and its packed operands in buffer i % 2; the loops are
  // unrolled by 4 so that every stage is named statically.
  const int iters = nb > 0 ? nb + 1 : 0;
  if (forward_role) {
    bf16x8 w1f[KC], w3f[KC], w2f[KC];   // B-operand fragments over d, this wave's 16 hidden units
    {
      const int64_t row = ((int64_t)h * p.m + hid0 + li) * D + 8 * g;
      const char *W1 = reinterpret_cast<const char *>(static_cast<const __bf16 *>(p.w1) + row);
      const char *W3 = reinterpret_cast<const char *>(static_cast<const __bf16 *>(p.w3) + row);
      const char *W2 = reinterpret_cast<const char *>(static_cast<const __bf16 *>(p.w2t) + row);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        w1f[kc] = *reinterpret_cast<const bf16x8 *>(W1 + 64 * kc);
        w3f[kc] = *reinterpret_cast<const bf16x8 *>(W3 + 64 * kc);
        w2f[kc] = *reinterpret_cast<const bf16x8 *>(W2 + 64 * kc);
      }
    }
    // LDS addresses.  Chunk 4kc + g of row rt with swizzle s: ((4kc + g) ^ s) * 16 =
    // (16 (g ^ s)) ^ 64 kc, one XOR per read; rows perm_row(u, li).  A d-fragment is one
    // 16-byte read, conflict-free under swz_kv (as are the contraction waves' reads).
    int base_a[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int rt = perm_row(u, li);
      base_a[u] = rt * L::kRowBytes + 16 * (g ^ (swz_kv(rt) & (L::kChunks - 1)));
    }
    // Products of the block in `cur`, its SwiGLU backward, and the packed operands
    // into `pkw`.  Each reduction chunk ends in a scheduling barrier, so that the
    // reads for chunk kc + FR - 1 issue before the products of chunk kc.
    auto forward_block = [&](const unsigned char *cur, unsigned char *pkw) {
      f32x4 z1[2], z3[2], pp[2];
      bf16x8 kf[FR][2], vf[FR][2];
      // the u = 1 rows are the u = 0 rows + 4 (perm_row), which swz_kv ignores (it uses
      // row bits 0, 1 and 3): one address per reduction chunk, the rest immediate offsets
      auto lda = [&](int kc, int slot) {
        const unsigned char *pa = cur + xor_here(base_a[0], 64 * kc);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          kf[slot][u] = *reinterpret_cast<const bf16x8 *>(pa + u * 4 * L::kRowBytes);
          vf[slot][u] = *reinterpret_cast<const bf16x8 *>(pa + L::kTile + u * 4 * L::kRowBytes);
        }
      };
#pragma unroll
      for (int u = 0; u < 2; ++u) z1[u] = z3[u] = pp[u] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < FR - 1 && j < KC; ++j) lda(j, j);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        if (kc + FR - 1 < KC) lda(kc + FR - 1, (kc + FR - 1) % FR);
        const int s = kc % FR;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          z1[u] = mma(kf[s][u], w1f[kc], z1[u]);
          z3[u] = mma(kf[s][u], w3f[kc], z3[u]);
          pp[u] = mma(vf[s][u], w2f[kc], pp[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
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
      *reinterpret_cast<bf16x8 *>(pkw + pk_slot) = pk1;
      *reinterpret_cast<bf16x8 *>(pkw + pk_slot + 1024) = pk3;
      *reinterpret_cast<bf16x8 *>(pkw + pk_slot + 2048) = pkh;
    };
    // iteration i: forward of block i (stage i % 4, packed operands to buffer i % 2)
    auto step = [&](int i, const unsigned char *cur, unsigned char *pkw) {
      if (i < nb) forward_block(cur, pkw);
      keep_pace(i);
      sync(false);
    };
    int i = 0;
    for (; i + 4 <= iters; i += 4) {
      step(i, st0, pkb0);
      step(i + 1, st1, pkb1);
      step(i + 2, st2, pkb0);
      step(i + 3, st3, pkb1);
    }
    if (i < iters) step(i, st0, pkb0);
    if (i + 1 < iters) step(i + 1, st1, pkb1);
    if (i + 2 < iters) step(i + 2, st2, pkb0);
  } else {
    // contraction wave c: hidden groups 2 pr and 2 pr + 1, d tiles DTQ dq .. DTQ dq + DTQ - 1,
    // so that every transposed K / V fragment feeds six products
    constexpr int DTQ = DT / (2 * CS);
    const int pr = c & 1, dq = c >> 1;
    f32x4 a1[2][DTQ], a3[2][DTQ], a2[2][DTQ];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int t = 0; t < DTQ; ++t) a1[e][t] = a3[e][t] = a2[e][t] = f32x4{0, 0, 0, 0};
    // transposed reads: lane (g, li) supplies row 8g + 4q + li/4, column 16 dt + 4 (li % 4)
    // and receives rows 8g + 4q .. +3 of column 16 dt + li; chunk 2dt + e of row r with
    // swizzle s: ((2dt + e) ^ s) * 16 = (16 (e ^ s)) ^ 32 dt
    int base_b[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = 8 * g + 4 * q + (li >> 2);
      const int e = (li & 3) >> 1;
      // tile dt0 + j of this wave: 32 (dt0 + j) = 32 dt0 ^ 32 j (dt0 is a multiple of DTQ > j)
      base_b[q] = (row * L::kRowBytes + 16 * (e ^ (swz_kv(row) & (L::kChunks - 1))) + 8 * (li & 1)) ^ (32 * DTQ * dq);
    }
    // G1 += dZ1^T K, G3 += dZ3^T K, G2 += V^T H' for the block in stage `blk` with its
    // packed operands pk1, pk3, pkh; the transposed reads run one 16-column tile ahead
    // (scheduling barrier per tile)
    auto contract_block = [&](const unsigned char *blk, const bf16x8 (&pk1)[2], const bf16x8 (&pk3)[2],
                              const bf16x8 (&pkh)[2]) {
      bf16x8 ktf[2], vtf[2];
      auto ldb = [&](int dt, int slot) {
        // each address is formed (one XOR) right before its read instead of 32 of them
        // being held in registers
        // the q = 1 rows are the q = 0 rows + 4, which swz_kv ignores
        const unsigned char *p0 = blk + xor_here(base_b[0], 32 * dt);
        const unsigned char *p1 = p0 + 4 * L::kRowBytes;
        ktf[slot] = cat8(lds_read_tr16(p0), lds_read_tr16(p1));
        vtf[slot] = cat8(lds_read_tr16(p0 + L::kTile), lds_read_tr16(p1 + L::kTile));
      };
      ldb(0, 0);
#pragma unroll
      for (int dt = 0; dt < DTQ; ++dt) {
        if (dt + 1 < DTQ) ldb(dt + 1, (dt + 1) & 1);
        const int s = dt & 1;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          a1[e][dt] = mma(pk1[e], ktf[s], a1[e][dt]);
          a3[e][dt] = mma(pk3[e], ktf[s], a3[e][dt]);
          a2[e][dt] = mma(vtf[s], pkh[e], a2[e][dt]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // iteration i: DMA of block i + 2 (stage (i + 2) % 4), contraction of block i - 1
    // (stage (i - 1) % 4, packed operands in buffer (i - 1) % 2).  Iteration 0 has no
    // contraction and runs before the loop, which then starts at i = 1.
    // The packed operands are read before the DMA is issued.
    auto step = [&](int i, const unsigned char *ctr, unsigned char *dma, const unsigned char *pkr) {
      const bool issue = i + 2 < nb;
      bf16x8 pk1[2], pk3[2], pkh[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const unsigned char *ps = pkr + (((2 * pr + e) * 3) * 64 + l) * 16;
        pk1[e] = *reinterpret_cast<const bf16x8 *>(ps);
        pk3[e] = *reinterpret_cast<const bf16x8 *>(ps + 1024);
        pkh[e] = *reinterpret_cast<const bf16x8 *>(ps + 2048);
      }
      if (issue) stage_block(blk0 + i + 2, dma);
      // always true here; written as a test because the unconditional form makes
      // the register allocator spill accumulators at d = 256
      if (i <= nb) contract_block(ctr, pk1, pk3, pkh);
      sync(issue);
    };
    if (iters > 0) {
      const bool issue = nb > 2;
      if (issue) stage_block(blk0 + 2, st2);
      sync(issue);
    }
    int i = 1;
    for (; i + 4 <= iters; i += 4) {
      step(i, st0, st3, pkb0);
      step(i + 1, st1, st0, pkb1);
      step(i + 2, st2, st1, pkb0);
      step(i + 3, st3, st2, pkb1);
    }
    if (i < iters) step(i, st0, st3, pkb0);
    if (i + 1 < iters) step(i + 1, st1, st0, pkb1);
    if (i + 2 < iters) step(i + 2, st2, st1, pkb0);

    // partials: G1/G3 rows hid0 + 4g + r, cols 16 dt + li;  G2 rows 16 dt + 4g + r, cols hid0 + li
    const int64_t mat = (int64_t)p.m * D;
    float *P1 = p.part + ((int64_t)split * 3 * p.heads + h) * mat;
    float *P3 = P1 + p.heads * mat;
    float *P2 = P3 + p.heads * mat;
    const int dt0 = DTQ * dq;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int hid = jt * kHidTile + 16 * (2 * pr + e);
#pragma unroll
      for (int j = 0; j < DTQ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int dt = dt0 + j;
          P1[(int64_t)(hid + 4 * g + r) * D + 16 * dt + li] = a1[e][j][r];
          P3[(int64_t)(hid + 4 * g + r) * D + 16 * dt + li] = a3[e][j][r];
          P2[(int64_t)(16 * dt + 4 * g + r) * p.m + hid + li] = a2[e][j][r];
        }
    }
  }
}

// ------------------------------------------------------------- general path
// Any supported d (a multiple of 64 up to 1024, taken at run time), fp32 or bf16.  The d-reductions read K, V and the weights
// straight from global memory (L1/L2 resident); only the transposed K, V
// columns of this workgroup's output d-chunk go through LDS.  The forward is
// recomputed for every d-chunk.
template <typename T, int DC>
__global__ __launch_bounds__(256) void grad_general_kernel(GradParams p) {
  using F = typename FragOf<T>::type;
  const int D = p.d;
  const int KC = D / 32;
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

template <typename T>
hipError_t launch_general_d(const GradParams &p, int d, int grid, hipStream_t s) {
  if (d < 64 || d > 1024 || d % 64 != 0 || p.d != d) return hipErrorInvalidValue;
  if (grad_general_dc(d, sizeof(T) == 2) == 128)
    hipLaunchKernelGGL((grad_general_kernel<T, 128>), dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((grad_general_kernel<T, 64>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
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

// output d-chunk of the general kernel: 128 columns for bf16 where d allows, else 64
int grad_general_dc(int d, bool bf16) { return bf16 && d % 128 == 0 ? 128 : 64; }

hipError_t launch_grad(const GradParams &p, int d, bool bf16, bool fast, int grid, hipStream_t s) {
  if (fast) {
    switch (d) {
      // 4 forward + 4 kGradCS contraction waves (see grad_fast_kernel)
      case 64: hipLaunchKernelGGL((grad_fast_kernel<64, kGradCS>), dim3(grid), dim3((4 + 4 * kGradCS) * 64), 0, s, p); break;
      case 128: hipLaunchKernelGGL((grad_fast_kernel<128, kGradCS>), dim3(grid), dim3((4 + 4 * kGradCS) * 64), 0, s, p); break;
      case 256: hipLaunchKernelGGL((grad_fast_kernel<256, kGradCS>), dim3(grid), dim3((4 + 4 * kGradCS) * 64), 0, s, p); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  return bf16 ? launch_general_d<__bf16>(p, d, grid, s) : launch_general_d<float>(p, d, grid, s);
}

}  // namespace ttt
