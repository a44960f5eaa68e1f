// Device-side building blocks shared by the gfx950 kernels: wave64
// reductions, 16-byte vector loads of logits rows, workspace records.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

constexpr int kWave = 64;
constexpr int kUnroll = 8;        // 16-byte vectors per lane per work item
constexpr int kBlock = 256;       // 4 waves per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr float kLog2e = 1.4426950408889634f;
// a lane whose normalised mass reaches 2^-12 is recomputed in fp64 in the
// residual pass (p - q cancels there)
constexpr float kHeavy = 1.0f / 4096.0f;

// Elements per 16-byte vector and per work item for each storage type.
template <int DT> struct Elem;
template <> struct Elem<DSPARK_BF16> {
  static constexpr int kPerVec = 8;
  static constexpr int kBytes = 2;
};
template <> struct Elem<DSPARK_F32> {
  static constexpr int kPerVec = 4;
  static constexpr int kBytes = 4;
};
template <int DT> constexpr int item_elems() { return kWave * kUnroll * Elem<DT>::kPerVec; }

// smallest item (fp32) sizes the workspace for either dtype
__host__ __device__ inline int chunks_per_row_max(int V) {
  return (V + item_elems<DSPARK_F32>() - 1) / item_elems<DSPARK_F32>();
}
template <int DT> __host__ __device__ inline int chunks_per_row(int V) {
  return (V + item_elems<DT>() - 1) / item_elems<DT>();
}

// ---------------------------------------------------------------- records

// Per-chunk summary of one logits row.  Softmax rows: k = integer shift
// ceil(max * c) used for the chunk, s = sum over the chunk of
// 2^(x*c - k).  Greedy rows: k = chunk maximum, idx = its lowest index.
struct alignas(16) Partial {
  float k;
  int idx;
  double s;
};

// Per-request state handed between the kernels of one verify call.
enum : int { kModeNone = 0, kModeResidual = 1, kModeDrawP = 2, kModeDone = 3 };
enum : int { kKindSoftmax = 0, kKindGreedy = 1, kKindSkip = 2 };

struct alignas(16) ReqState {
  int L;        // clamped verify length
  int kind;     // kKind*
  float c;      // log2(e) / T as fp32 (softmax rows)
  int a;        // accepted count
  int mode;     // final draw: kMode*
  int row;      // target row of the final draw
  float kt;     // shift of the target row used by the final draw
  float kd;     // shift of the draft row (residual mode)
  double st;    // sum of 2^(x*c - kt) over that target row
  double sd;    // same for the draft row
};

// ---------------------------------------------------------------- wave ops

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o);
  return v;
}

// (value desc, index asc) argmax merge
__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o);
    int oi = __shfl_xor(i, o);
    argmax_merge(v, i, ov, oi);
  }
}

// inclusive prefix sum over the wave (lane order)
__device__ __forceinline__ double wave_incl_scan(double v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    double t = __shfl_up(v, o);
    if (l >= o) v += t;
  }
  return v;
}

// ---------------------------------------------------------------- loads

// One work item: kUnroll 16-byte vectors per lane.  Lane l, vector v covers
// elements [(v*64 + l) * kPerVec, +kPerVec) of the chunk, so a wave reads
// 64 consecutive 16-byte segments per vector step (fully coalesced) and a
// lane's elements are in increasing index order.  Elements past `n` are
// filled with -inf.
template <int DT> struct Tile {
  uint32_t w[kUnroll][4];

  __device__ __forceinline__ void load(const void* chunk_base, int n, bool vec_ok) {
    const int l = lane_id();
    constexpr int P = Elem<DT>::kPerVec;
#pragma unroll
    for (int v = 0; v < kUnroll; ++v) {
      const int e0 = (v * kWave + l) * P;
      if (vec_ok && e0 + P <= n) {
        const uint4 q = *reinterpret_cast<const uint4*>(
            static_cast<const char*>(chunk_base) + (size_t)e0 * Elem<DT>::kBytes);
        w[v][0] = q.x; w[v][1] = q.y; w[v][2] = q.z; w[v][3] = q.w;
      } else {
        // scalar path: unaligned rows or the ragged end of a row
#pragma unroll
        for (int e = 0; e < P; ++e) set_neg_inf(v, e);
        for (int e = 0; e < P; ++e) {
          if (e0 + e < n) set_raw(v, e, chunk_base, e0 + e);
        }
      }
    }
  }

  __device__ __forceinline__ void set_neg_inf(int v, int e) {
    if constexpr (DT == DSPARK_BF16) {
      uint32_t& x = w[v][e >> 1];
      if (e & 1) x = (x & 0x0000ffffu) | 0xff800000u;
      else x = (x & 0xffff0000u) | 0x0000ff80u;
    } else {
      w[v][e] = 0xff800000u;
    }
  }

  __device__ __forceinline__ void set_raw(int v, int e, const void* base, int idx) {
    if constexpr (DT == DSPARK_BF16) {
      const uint32_t h = static_cast<const uint16_t*>(base)[idx];
      uint32_t& x = w[v][e >> 1];
      if (e & 1) x = (x & 0x0000ffffu) | (h << 16);
      else x = (x & 0xffff0000u) | h;
    } else {
      w[v][e] = static_cast<const uint32_t*>(base)[idx];
    }
  }

  // element e (0..kPerVec-1) of vector v as fp32 (exact widening)
  __device__ __forceinline__ float at(int v, int e) const {
    if constexpr (DT == DSPARK_BF16) {
      const uint32_t x = w[v][e >> 1];
      return (e & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
    } else {
      return __uint_as_float(w[v][e]);
    }
  }
};

// scalar element fetch (exact widening)
template <int DT> __device__ __forceinline__ float load_elem(const void* row, int idx) {
  if constexpr (DT == DSPARK_BF16) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(row)[idx]) << 16);
  } else {
    return static_cast<const float*>(row)[idx];
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void flag(int32_t* st, int bits) {
  if (bits) atomicOr(st, bits);
}

}  // namespace dspark
