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

// LDS swizzles (16-byte chunk granularity, 32 banks x 4 bytes assumed).
// Row-major tile whose rows are >= 128 bytes: chunk c of row r lives at
// c ^ swz_rows(r).  Conflict-free for 8 lanes reading perm_row(u, 0..7) at one chunk
// and for 8 lanes writing 8 consecutive chunks of one row.
__device__ __forceinline__ int swz_rows(int r) { return (r & 3) | ((r >> 1) & 4); }
// Tile with 64-byte rows (4 chunks): chunk a of row r lives at a ^ swz_64(r).
// Conflict-free for 8 lanes reading rows R..R+7 (R % 8 == 0) at one chunk.
__device__ __forceinline__ int swz_64(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// Transpose an 8x8 block of 16-bit values held as 8 rows of 16 bytes.
__device__ __forceinline__ void transpose8x8_b16(const u32x4 in[8], u32x4 out[8]) {
  // Row i word w holds elements (i, 2w) in bits 0..15 and (i, 2w+1) in 16..31.
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int w = j >> 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = in[2 * q][w], b = in[2 * q + 1][w];
      out[j][q] = (j & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
  }
}

}  // namespace ttt
