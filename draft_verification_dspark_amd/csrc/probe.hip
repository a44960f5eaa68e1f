// Plain contiguous read of a device buffer: the reference that the streaming
// pass's bandwidth is compared with at the same byte count (measurement aid;
// nothing on the verification path calls it).
//
// One workgroup of 768 threads per compute unit, as the streaming pass.  Wave
// w of the grid reads 8 KB tiles w, w + W, w + 2W, ... (W waves), each as
// eight coalesced 16-byte loads per lane, all eight in flight at once, and
// folds the words into a checksum; the bytes past the last whole tile are
// read 16 at a time.  The checksum is stored only when it equals a fixed
// constant, which keeps the loads without writing anything in practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace dspark {
int compute_units();
}

namespace dspark {

constexpr int kProbeBlock = 768;
constexpr uint32_t kProbeMagic = 0x9e3779b9u;

__global__ void __launch_bounds__(kProbeBlock) k_read_probe(const uint4* __restrict__ x,
                                                             size_t nvec, uint32_t* sink) {
  const int lane = lane_id();
  const size_t waves = (size_t)gridDim.x * (kProbeBlock / kWave);
  const size_t wave = (size_t)blockIdx.x * (kProbeBlock / kWave) + threadIdx.x / kWave;
  const size_t tiles = nvec / 512;  // 512 vectors = 8 KB
  uint32_t acc = 0;
  for (size_t t = wave; t < tiles; t += waves) {
    const uint4* p = x + t * 512;
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[i * kWave + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= (v[i].x + v[i].y) ^ (v[i].z + v[i].w);
  }
  // the ragged end: vectors [tiles * 512, nvec), one per thread of the grid
  const size_t rest = tiles * 512 + wave * kWave + lane;
  if (rest < nvec) {
    const uint4 q = x[rest];
    acc ^= (q.x + q.y) ^ (q.z + q.w);
  }
  if (acc == kProbeMagic) sink[0] = acc;
}

int launch_read_probe(const void* x, size_t bytes, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)compute_units()), dim3(kProbeBlock), 0, st,
                     static_cast<const uint4*>(x), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_LAUNCH;
}

}  // namespace dspark
