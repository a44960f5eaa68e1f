// Plain contiguous read of a device buffer: the yardstick that the streaming
// pass's bandwidth is compared with at the same byte count.  Built into the
// benchmark's own library (libdspark_bench.so), not into libdspark.so:
// nothing on the verification path calls it.
//
// One workgroup of 512 threads per compute unit, as the streaming pass.  Wave
// w of the grid reads 8 KB tiles w, w + W, w + 2W, ... (W waves), each as
// eight coalesced 16-byte loads per lane, all eight in flight at once, and
// folds the words into a checksum; the bytes past the last whole tile are
// read 16 at a time.  The checksum is stored only when it equals a fixed
// constant, which keeps the loads without writing anything in practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dspark_bench.h"

namespace {

constexpr int kProbeBlock = 512;
constexpr int kProbeWave = 64;
constexpr uint32_t kProbeMagic = 0x9e3779b9u;

__global__ void __launch_bounds__(kProbeBlock) k_read_probe(const uint4* __restrict__ x,
                                                             size_t nvec, uint32_t* sink) {
  const int lane = (int)(threadIdx.x % kProbeWave);
  const size_t waves = (size_t)gridDim.x * (kProbeBlock / kProbeWave);
  const size_t wave = (size_t)blockIdx.x * (kProbeBlock / kProbeWave) + threadIdx.x / kProbeWave;
  const size_t tiles = nvec / 512;  // 512 vectors = 8 KB
  uint32_t acc = 0;
  for (size_t t = wave; t < tiles; t += waves) {
    const uint4* p = x + t * 512;
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[i * kProbeWave + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= (v[i].x + v[i].y) ^ (v[i].z + v[i].w);
  }
  // the ragged end: vectors [tiles * 512, nvec), one per thread of the grid
  const size_t rest = tiles * 512 + wave * kProbeWave + lane;
  if (rest < nvec) {
    const uint4 q = x[rest];
    acc ^= (q.x + q.y) ^ (q.z + q.w);
  }
  if (acc == kProbeMagic) sink[0] = acc;
}

int compute_units_now() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return 256;
  return cus;
}

}  // namespace

extern "C" int dspark_bench_read_probe(const void* x, size_t bytes, uint32_t* sink, void* stream) {
  if (!x || !sink) return 1;
  if (bytes == 0 || bytes % 16 != 0 || (uintptr_t)x % 16 != 0) return 7;
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)compute_units_now()), dim3(kProbeBlock), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(x), bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
