// Dense bf16 MFMA rate probe: a measurement aid beside the layer's kernels, not a
// step of the layer.  Every wave runs kProbeChains independent accumulation chains
// of 16x16x32 bf16 MFMAs on register operands, with no memory traffic in the loop
// (three or more chains keep the pipe full), two waves per SIMD on every compute
// unit.  The rate it reaches is the matrix cores' sustained dense bf16 rate at the
// clock the chip holds under that load, the practical ceiling of the contraction
// kernels next to the published 2.5 PFLOP/s (which assumes a 2.4 GHz clock).
#include "common.h"
#include "kernels.h"

namespace ttt {
namespace {

constexpr int kProbeChains = 8;
constexpr int kProbeWaves = 8;                      // two per SIMD

}  // namespace

// external linkage: a store to it cannot be dropped as unobservable
__device__ float ttt_probe_sink[64 * kProbeWaves];

namespace {

__global__ __launch_bounds__(64 * kProbeWaves) void mfma_probe_kernel(int iters) {
  const int t = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.125f * (float)((t + i) & 7));
    b[i] = (__bf16)(0.0625f * (float)((t * 3 + i) & 15));
  }
  f32x4 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x4{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = mma(a, b, acc[c]);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  // the operands are non-negative, so this store never happens; it keeps the chains live
  if (s < 0.0f) ttt_probe_sink[t] = s;
}

}  // namespace

hipError_t launch_mfma_probe(int iters, hipStream_t s, double *flop) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(cus), dim3(64 * kProbeWaves), 0, s, iters);
  *flop = (double)cus * kProbeWaves * kProbeChains * 16.0 * 16.0 * 32.0 * 2.0 * (double)iters;
  return hipGetLastError();
}

}  // namespace ttt
