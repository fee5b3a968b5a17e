// Shared device helpers for the gfx950 LaCT kernels: MFMA operand fragments,
// LDS swizzles and small conversions.
//
// MFMA convention used everywhere (16x16 output tiles, wave64):
//   lane l, g = l / 16, li = l % 16.
//   A operand: lane holds A[row = li][k = 8 consecutive values owned by group g]
//   B operand: lane holds B[k = same 8 values of group g][col = li]
//   D (4 floats): D[row = 4*g + r][col = li], r = 0..3
// The k-to-(g, element) assignment only has to agree between A and B, so every
// fragment is "8 consecutive reduction elements per lane group": one
// v_mfma_f32_16x16x32_bf16 for bf16, eight v_mfma_f32_16x16x4_f32 for fp32
// (sub-step s uses element s of every lane).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct FragOf;
template <> struct FragOf<__bf16> { typedef bf16x8 type; };
template <> struct FragOf<float> { typedef f32x8 type; };

__device__ __forceinline__ f32x4 mma(const bf16x8 a, const bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8 a, const f32x8 b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}

// 8 consecutive elements from a 16-byte aligned address (global or LDS).
__device__ __forceinline__ bf16x8 ld8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ f32x8 ld8(const float *p) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <typename T> __device__ __forceinline__ typename FragOf<T>::type zero8();
template <> __device__ __forceinline__ bf16x8 zero8<__bf16>() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}
template <> __device__ __forceinline__ f32x8 zero8<float>() { return f32x8{0, 0, 0, 0, 0, 0, 0, 0}; }

template <typename T> __device__ __forceinline__ typename FragOf<T>::type pack8(const float *v);
template <> __device__ __forceinline__ bf16x8 pack8<__bf16>(const float *v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)v[i];
  return r;
}
template <> __device__ __forceinline__ f32x8 pack8<float>(const float *v) {
  return f32x8{v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
}

__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// sigma(z) = 1 / (1 + e^-z) with the hardware exp2 and reciprocal (~1 ulp each).
__device__ __forceinline__ float sigmoid_fast(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

// Row position of the i-th row (i = 0..15) of the u-th 16-row MFMA tile inside a
// 32-row block, chosen so that the D layout of a "rows x 16" product gives lane
// group g the 8 consecutive rows 8g .. 8g+7 across the two tiles (u = 0, 1):
// D row 4g + r of tile u is block row 8g + 4u + r.
__device__ __forceinline__ int perm_row(int u, int i) { return 8 * (i >> 2) + 4 * u + (i & 3); }

// LDS swizzles (16-byte chunk granularity).  gfx950's LDS serves 256 bytes per
// cycle (64 banks x 4 bytes): a ds_read_b128 is served 16 lanes at a time, a
// ds_read_b64 (also the transposing one) 32 lanes at a time, and a phase is
// conflict-free when its lanes hit distinct bank words.
//
// Row-major tile with rows of >= 256 bytes: chunk c of row r lives at c ^ swz_rows(r).
// swz_rows maps row bits (0, 1, 3, 4) one-to-one onto position bits (1, 2, 3, 0), so
//  * 32 lanes of ds_read_b64_tr_b16 reading rows 8a + 4q + (0..3), a in {0,1} or
//    {2,3}, at chunks 2t and 2t+1 hit 32 distinct 8-byte slots (measured
//    conflict-free on gfx950);
//  * 16 lanes writing 16 consecutive chunks of one row hit 16 positions.
// ds_read_b128 of rows perm_row(u, 0..15) does conflict under it (2-way, measured):
// tiles read both ways use swz_kv below.  For narrower rows the value is masked to
// the row's chunk count (correct, not conflict-optimised).
__device__ __forceinline__ int swz_rows(int r) {
  return ((r >> 4) & 1) | ((r & 3) << 1) | (((r >> 3) & 1) << 3);
}
// Row-major tile with 512-byte rows read with ds_read_b128 only, 16 lanes on rows
// perm_row(u, 0..15) at one chunk: row bits (0, 1, 3, 4) onto position bits
// (0, 1, 2, 3) measured conflict-free on gfx950 (swz_rows is not for this pattern).
__device__ __forceinline__ int swz_rows_b128(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }
// Row-major tile with 512-byte rows read both ways: ds_read_b128 by 16 lanes on rows
// perm_row(u, 0..15) at one chunk, and ds_read_b64_tr_b16 as described for swz_rows.
// The first pattern is conflict-free only when position bit 0 follows row bit 0 or 1,
// the second only when it follows row bit 4, for every one-to-one map; measured on
// gfx950, both are conflict-free when row bit 4 is left out and position bits
// (0, 1, 2, 3) follow row bits (0, 0, 1, 3).
__device__ __forceinline__ int swz_kv(int r) { return 3 * (r & 1) | (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 3); }
// Tile with 64-byte rows (4 chunks, 4 rows per 256 bytes): chunk a of row r lives at
// a ^ swz_64(r).  A ds_read_b128 of rows R + (0..15) (R % 16 == 0), lane group g at
// chunk g, is served 8 rows of two lane groups at a time (the rule the measurements of
// swz_kv show); flipping both chunk bits with row bit 2 spreads each such half over all
// 64 banks.  Measured conflict-free on gfx950 (the former map of row bits 1 and 3
// spent 15% of the wide kernels' cycles in conflicts).
__device__ __forceinline__ int swz_64(int r) { return 3 * ((r >> 2) & 1); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element (i % 4) of
// the 8-byte pieces addressed by lanes 4k + i/4, k = 0..3.  If lane s of the group
// addresses row t0 + s/4, columns c0 + 4(s%4) .. +3 of a row-major 16-bit tile,
// lane i receives rows t0 .. t0+3 of column c0 + i: a transposed 4 x 16 block.
__device__ __forceinline__ bf16x4 lds_read_tr16(const unsigned char *p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
  return __builtin_bit_cast(bf16x4, v);
}
// global_load_lds_dwordx4: every lane fetches 16 bytes from its own global address;
// the wave's 64 pieces land contiguously at lds_wave_base + 16 * lane.
__device__ __forceinline__ void copy16_to_lds(const void *gsrc, unsigned char *lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(gsrc),
                                   (__attribute__((address_space(3))) void *)(lds_wave_base), 16, 0, 0);
}
// buffer_load_dwordx4 ... lds: the same copy through a buffer view (wave-uniform base
// and byte range in `rsrc`), each lane giving a 32-bit byte offset; fetches past the
// range return zeros.  Keeps the per-lane address at one register instead of two.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rsrc, unsigned voffset,
                                              unsigned char *lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)(lds_wave_base), 16,
                                           voffset, 0, 0, 0);
}
// The same copy with a wave-uniform byte offset `soffset` added to every lane's.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rsrc, unsigned voffset, unsigned soffset,
                                              unsigned char *lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)(lds_wave_base), 16,
                                           voffset, soffset, 0, 0);
}
// base ^ k for a wave-uniform k, formed by one VALU instruction at this point.
__device__ __forceinline__ unsigned xor_scalar_here(unsigned base, unsigned k) {
  unsigned r;
  asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "s"(k), "v"(base));
  return r;
}
// Raw buffer view of `bytes` bytes at `base` (32-bit dword format word of gfx9).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void *base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// Wait for this wave's outstanding global/LDS operations (vmcnt = lgkmcnt = 0).
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }
// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// s_waitcnt vmcnt(N) lgkmcnt(0).
template <int N> __device__ __forceinline__ void wait_vmcnt_lds() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}
// Workgroup barrier without the vmcnt(0) that __syncthreads adds (which would
// also wait for the DMAs just issued for later stages).
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// base ^ k formed by one VALU instruction at this point of the program: the compiler
// can neither hoist it out of a loop (holding one register per k) nor needs to copy
// the base first (as an empty asm that modifies a copy of the base would).
__device__ __forceinline__ int xor_here(int base, int k) {
  if (k == 0) return base;
  int r;
  asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "s"(k), "v"(base));
  return r;
}

__device__ __forceinline__ bf16x8 cat8(const bf16x4 a, const bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

}  // namespace ttt
