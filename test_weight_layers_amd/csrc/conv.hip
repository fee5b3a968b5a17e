// ShortConv2D on V (VGG-T3 关键设计 2): each frame's patch tokens form a
// grid_h x grid_w image whose channels are the columns of V; every channel is
// cross-correlated with its own 3x3 taps (zero padding, stride 1, no bias).
// The frame's leading n_special tokens pass through unchanged.
//
// HBM-bound: one read and one write of V per element.  A thread owns 8
// channels of one grid column and walks down the rows with a 3-row register
// window, so each input vector is loaded by at most three threads (its column
// and the two neighbours, mostly L1/L2 hits) and every output is written once
// with a 16-byte store.  Taps for the thread's 8 channels stay in registers.
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
    *reinterpret_cast<bf16x8 *>(p) = pack8<__bf16>(v);
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
    *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
};

// grid: x = channel groups of 8 (C/8) x grid columns, y = frames.
template <typename T>
__global__ __launch_bounds__(256) void conv_kernel(const T *__restrict__ v, T *__restrict__ out, int64_t ld,
                                                   const float *__restrict__ wconv, int tpf, int nsp, int gh, int gw,
                                                   int C) {
  const int groups = C / 8;
  const int item = blockIdx.x * 256 + threadIdx.x;
  const int64_t f = blockIdx.y;
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

  // rows y-1, y, y+1 of columns col-1, col, col+1 (zeros outside the grid)
  float win[3][3][8];
  auto load_row = [&](int y, float dst[3][8]) {
#pragma unroll
    for (int dx = 0; dx < 3; ++dx) {
      const int x = col + dx - 1;
      if (y >= 0 && y < gh && x >= 0 && x < gw) {
        Vec8<T>::load(V + (int64_t)(nsp + y * gw + x) * ld, dst[dx]);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) dst[dx][c] = 0.0f;
      }
    }
  };
  load_row(-1, win[0]);
  load_row(0, win[1]);
  for (int y = 0; y < gh; ++y) {
    load_row(y + 1, win[2]);
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float s = 0.0f;
#pragma unroll
      for (int dy = 0; dy < 3; ++dy)
#pragma unroll
        for (int dx = 0; dx < 3; ++dx) s = fmaf(w[dy * 3 + dx][c], win[dy][dx][c], s);
      acc[c] = s;
    }
    Vec8<T>::store(O + (int64_t)(nsp + y * gw + col) * ld, acc);
#pragma unroll
    for (int dx = 0; dx < 3; ++dx)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        win[0][dx][c] = win[1][dx][c];
        win[1][dx][c] = win[2][dx][c];
      }
  }
}

}  // namespace

hipError_t launch_conv(const void *v, void *out, int64_t ld, const float *w, int frames, int tpf, int nsp, int gh,
                       int gw, int channels, bool bf16, hipStream_t s) {
  const int items = channels / 8 * (gw + 1);
  const size_t esz = bf16 ? 2 : 4;
  for (int f0 = 0; f0 < frames; f0 += 65535) {          // grid.y limit
    const int fn = frames - f0 < 65535 ? frames - f0 : 65535;
    const int64_t off = (int64_t)f0 * tpf * ld * esz;
    const void *vin = static_cast<const char *>(v) + off;
    void *vout = static_cast<char *>(out) + off;
    const dim3 grid((items + 255) / 256, fn);
    if (bf16)
      hipLaunchKernelGGL(conv_kernel<__bf16>, grid, dim3(256), 0, s, static_cast<const __bf16 *>(vin),
                         static_cast<__bf16 *>(vout), ld, w, tpf, nsp, gh, gw, channels);
    else
      hipLaunchKernelGGL(conv_kernel<float>, grid, dim3(256), 0, s, static_cast<const float *>(vin),
                         static_cast<float *>(vout), ld, w, tpf, nsp, gh, gw, channels);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ttt
