// ShortConv2D on V (VGG-T3 关键设计 2): each frame's patch tokens form a
// grid_h x grid_w image whose channels are the columns of V; every channel is
// cross-correlated with its own 3x3 taps (zero padding, stride 1, no bias).
// The frame's leading n_special tokens pass through unchanged.
//
// HBM-bound: one read and one write of V per element.  A thread owns 8
// channels of one grid column and walks down the rows with a ring of loaded rows,
// so each input vector is loaded by at most three threads (its column and the two
// neighbours, mostly L1/L2 hits) and every output is written once with a 16-byte
// store.  Taps for the thread's 8 channels stay in registers.
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace ttt {
namespace {

template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
  static __device__ __forceinline__ void load(const __bf16 *p, float *v) {
    const bf16x8 x = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)x[i];
  }
  static __device__ __forceinline__ void store(__bf16 *p, const float *v) {
    // V' is not read again by this kernel: a streaming (non-temporal) store
    __builtin_nontemporal_store(pack8<__bf16>(v), reinterpret_cast<bf16x8 *>(p));
  }
};
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float *p, float *v) {
    const f32x8 x = ld8(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = x[i];
  }
  static __device__ __forceinline__ void store(float *p, const float *v) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(p));
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4 *>(p + 4));
  }
};

// Raw 8-channel vectors as loaded (bf16x8 or fp32 pairs), widened to fp32 at use.
template <typename T> struct Raw8;
template <> struct Raw8<__bf16> {
  typedef bf16x8 type;
  static __device__ __forceinline__ type load(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
  static __device__ __forceinline__ type zero() { return zero8<__bf16>(); }
  static __device__ __forceinline__ float at(const type &x, int i) { return (float)x[i]; }
};
template <> struct Raw8<float> {
  typedef f32x8 type;
  static __device__ __forceinline__ type load(const float *p) { return ld8(p); }
  static __device__ __forceinline__ type zero() { return zero8<float>(); }
  static __device__ __forceinline__ float at(const type &x, int i) { return x[i]; }
};

// grid: parts x frames workgroups (1-D, padded to a multiple of 8), where a part is
// 256 of the frame's (C/8) x (grid columns + 1) items.  A thread owns 8
// channels of one grid column and walks down the rows.  The loads are the memory
// traffic, so they run ahead: a ring of 5 rows (columns col-1, col, col+1) holds
// the 3-row window of the output row and the next two rows in flight; the loop is
// unrolled by 5 so that every ring slot is a fixed set of registers.
// f(integral_constant<int, J>) for J in the sequence, in order
template <int... J, class F>
__device__ __forceinline__ void for_each_index(std::integer_sequence<int, J...>, F &&f) {
  (f(std::integral_constant<int, J>{}), ...);
}

template <typename T>
__global__ __launch_bounds__(256) void conv_kernel(const T *__restrict__ v, T *__restrict__ out, int64_t ld,
                                                   const float *__restrict__ wconv, int tpf, int nsp, int gh, int gw,
                                                   int C, int parts, int frames) {
  using R = Raw8<T>;
  typedef typename R::type RawT;
  // Workgroups are dealt round-robin to the 8 XCDs; consecutive `lin` (the parts
  // of one frame, which read each other's edge columns) land on one XCD's L2.
  const int total = gridDim.x, b = blockIdx.x;
  const int lin = (b & 7) * (total >> 3) + (b >> 3);
  if (lin >= parts * frames) return;
  const int64_t f = lin / parts;
  const int groups = C / 8;
  const int item = (lin % parts) * 256 + threadIdx.x;
  if (item >= groups * (gw + 1)) return;
  const int cg = item % groups;
  const int col = item / groups;            // 0..gw-1 grid columns; gw: the special tokens
  const int c0 = 8 * cg;
  const T *V = v + f * tpf * ld + c0;
  T *O = out + f * tpf * ld + c0;

  if (col == gw) {                           // pass the special tokens through
    for (int t = 0; t < nsp; ++t) {
      float x[8];
      Vec8<T>::load(V + (int64_t)t * ld, x);
      Vec8<T>::store(O + (int64_t)t * ld, x);
    }
    return;
  }
  float w[9][8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int k = 0; k < 9; ++k) w[k][c] = wconv[(c0 + c) * 9 + k];

  // rows y-1 .. y+RING-2 of columns col-1, col, col+1 (a deeper ring for the
  // half-size bf16 rows; both keep 2 waves per SIMD)
  constexpr int RING = sizeof(T) == 2 ? 9 : 5;
  RawT ring[RING][3];
  auto load_row = [&](int y, RawT *dst) {
#pragma unroll
    for (int dx = 0; dx < 3; ++dx) {
      const int x = col + dx - 1;
      dst[dx] = (y >= 0 && y < gh && x >= 0 && x < gw) ? R::load(V + (int64_t)(nsp + y * gw + x) * ld) : R::zero();
    }
  };
  // output row y from ring slots a (y-1), b (y), c (y+1)
  auto emit = [&](int y, const RawT *ra, const RawT *rb, const RawT *rc) {
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float s = 0.0f;                       // taps in row-major order
#pragma unroll
      for (int dx = 0; dx < 3; ++dx) s = fmaf(w[dx][c], R::at(ra[dx], c), s);
#pragma unroll
      for (int dx = 0; dx < 3; ++dx) s = fmaf(w[3 + dx][c], R::at(rb[dx], c), s);
#pragma unroll
      for (int dx = 0; dx < 3; ++dx) s = fmaf(w[6 + dx][c], R::at(rc[dx], c), s);
      acc[c] = s;
    }
    Vec8<T>::store(O + (int64_t)(nsp + y * gw + col) * ld, acc);
  };
  // row y lives in slot (y + 1) % RING; iteration y loads row y + RING - 2
#pragma unroll
  for (int k = 0; k < RING - 1; ++k) load_row(k - 1, ring[k]);
  auto step = [&](int y, auto K) {
    constexpr int k = decltype(K)::value;   // (y + 1) % RING
    load_row(y + RING - 2, ring[(k + RING - 2) % RING]);
    emit(y, ring[(k + RING - 1) % RING], ring[k], ring[(k + 1) % RING]);
  };
  for (int y = 0; y < gh; y += RING)        // steps y .. y + RING - 1, with (y + 1) % RING == 1
    for_each_index(std::make_integer_sequence<int, RING>{}, [&](auto J) {
      constexpr int j = decltype(J)::value;
      if (y + j < gh) step(y + j, std::integral_constant<int, (j + 1) % RING>{});
    });
}

}  // namespace

hipError_t launch_conv(const void *v, void *out, int64_t ld, const float *w, int frames, int tpf, int nsp, int gh,
                       int gw, int channels, bool bf16, hipStream_t s) {
  const int items = channels / 8 * (gw + 1);
  const int parts = (items + 255) / 256;
  const size_t esz = bf16 ? 2 : 4;
  const int kMaxFrames = (1 << 28) / parts;               // keeps the 1-D grid far below 2^31
  for (int f0 = 0; f0 < frames; f0 += kMaxFrames) {
    const int fn = frames - f0 < kMaxFrames ? frames - f0 : kMaxFrames;
    const int64_t off = (int64_t)f0 * tpf * ld * esz;
    const void *vin = static_cast<const char *>(v) + off;
    void *vout = static_cast<char *>(out) + off;
    const int64_t blocks = ((int64_t)parts * fn + 7) / 8 * 8;
    if (bf16)
      hipLaunchKernelGGL(conv_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const __bf16 *>(vin),
                         static_cast<__bf16 *>(vout), ld, w, tpf, nsp, gh, gw, channels, parts, fn);
    else
      hipLaunchKernelGGL(conv_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const float *>(vin),
                         static_cast<float *>(vout), ld, w, tpf, nsp, gh, gw, channels, parts, fn);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ttt
