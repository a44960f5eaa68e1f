// Device-side building blocks shared by the gfx950 kernels: wave64
// reductions, 16-byte vector loads of logits rows, workspace records.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <climits>

#include "dspark.h"

namespace dspark {

constexpr int kWave = 64;
#ifndef DSPARK_UNROLL
#define DSPARK_UNROLL 8
#endif
constexpr int kUnroll = DSPARK_UNROLL;  // 16-byte vectors per lane per work item
constexpr int kBlock = 256;       // 4 waves per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr float kLog2e = 1.4426950408889634f;

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

// Per-chunk summary of one logits row (16 bytes, written by one store).
// Softmax rows: k = integer shift ceil(max * c) used for the chunk, s = sum
// over the chunk of 2^(x*c - k), idx = device-status bits found in the
// chunk.  Greedy rows: k = chunk maximum, idx = its lowest index, s = the
// status bits as a double.
struct alignas(16) Partial {
  float k;
  int idx;
  double s;
};

// One merged row: softmax rows carry the shift K* and S = sum 2^(x*c - K*);
// greedy rows the maximum (k) and its lowest index; both the status bits.
struct alignas(8) RowSum {
  double s;
  float k;
  int idx;
  int bad;
  int pad;
};

// Per-quarter-chunk sums of the rejected row pair (residual tasks to the
// draw): with d(v) the difference of the target and the rescaled draft term
// of token v and e2(v) that draft term, z = sum max(0, d), d = sum d, q = sum
// of e2 where d > 0 (e2 unused, padding).
struct alignas(16) ResidualChunk {
  double z, d, q, e2;
};

// Per-request draw state of a rejected request, published by its decision
// for the residual tasks and the draw (8-byte words).
enum : int { kModeNone = 0, kModeResidual = 1 };
enum : int { kKindSoftmax = 0, kKindGreedy = 1, kKindSkip = 2 };

struct alignas(8) ReqState {
  int mode;     // kModeResidual
  int row;      // the rejected position's row (target and draft)
  int a;        // accepted count (column of the drawn token)
  float c;      // log2(e) / T as fp32
  float clo;    // log2(e) / T - c
  float kt;     // shift of the target row
  float kd;     // shift of the draft row
  int pad;
  double st;    // sum of 2^(x*c - kt) over the target row
  double sd;    // same for the draft row
};

// ---------------------------------------------------------------- wave ops

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// a wave-uniform value moved to a scalar register
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
__device__ __forceinline__ size_t uniform(size_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return ((size_t)hi << 32) | lo;
}

// Wave64 reductions with DPP: four in-row steps (xor 1, xor 2 within quads,
// then half-row and row mirrors) leave every lane of each 16-lane row with
// the row's result; the four row results are read as scalars.  DPP moves cost
// a few cycles, against ~100 for a cross-lane LDS permute.
template <int CTRL> __device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}
template <int CTRL> __device__ __forceinline__ double dpp(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp<CTRL>((int)b), hi = dpp<CTRL>((int)(b >> 32));
  return __longlong_as_double(((long long)(unsigned)hi << 32) | (unsigned)lo);
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

template <typename T> __device__ __forceinline__ T readlane(T v, int lane);
template <> __device__ __forceinline__ int readlane<int>(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}
template <> __device__ __forceinline__ float readlane<float>(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
template <> __device__ __forceinline__ double readlane<double>(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __longlong_as_double(((long long)(unsigned)hi << 32) | (unsigned)lo);
}

template <typename T, typename Op> __device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp<kQuadXor1>(v));
  v = op(v, dpp<kQuadXor2>(v));
  v = op(v, dpp<kRowHalfMirror>(v));
  v = op(v, dpp<kRowMirror>(v));
  return op(op(readlane(v, 0), readlane(v, 16)), op(readlane(v, 32), readlane(v, 48)));
}

// The same four DPP steps alone: every lane of each 16-lane row ends with
// its row's result (used where a wave works on four rows at once).
template <typename T, typename Op> __device__ __forceinline__ T row16_reduce(T v, Op op) {
  v = op(v, dpp<kQuadXor1>(v));
  v = op(v, dpp<kQuadXor2>(v));
  v = op(v, dpp<kRowHalfMirror>(v));
  v = op(v, dpp<kRowMirror>(v));
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ double wave_sum(double v) {
  return wave_reduce(v, [](double x, double y) { return x + y; });
}
__device__ __forceinline__ int wave_or(int v) {
  return wave_reduce(v, [](int x, int y) { return x | y; });
}
__device__ __forceinline__ int wave_max_i(int v) {
  return wave_reduce(v, [](int x, int y) { return x > y ? x : y; });
}
__device__ __forceinline__ int wave_min_i(int v) {
  return wave_reduce(v, [](int x, int y) { return x < y ? x : y; });
}

// (value desc, index asc) argmax merge
__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

template <int CTRL> __device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = dpp<CTRL>(v);
  const int oi = dpp<CTRL>(i);
  argmax_merge(v, i, ov, oi);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<kQuadXor1>(v, i);
  argmax_step<kQuadXor2>(v, i);
  argmax_step<kRowHalfMirror>(v, i);
  argmax_step<kRowMirror>(v, i);
  float bv = readlane(v, 0);
  int bi = readlane(i, 0);
#pragma unroll
  for (int r = 16; r < kWave; r += 16) argmax_merge(bv, bi, readlane(v, r), readlane(i, r));
  v = bv;
  i = bi;
}

__device__ __forceinline__ void row16_argmax(float& v, int& i) {
  argmax_step<kQuadXor1>(v, i);
  argmax_step<kQuadXor2>(v, i);
  argmax_step<kRowHalfMirror>(v, i);
  argmax_step<kRowMirror>(v, i);
}

// inclusive prefix sum over the wave in lane order: Hillis-Steele within each
// 16-lane row (row_shr 1, 2, 4, 8; lanes without a source add 0), then each
// row adds the totals of the rows before it
template <int CTRL> __device__ __forceinline__ double dpp_shr(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xF, 0xF, true);
  return __longlong_as_double(((long long)(unsigned)hi << 32) | (unsigned)lo);
}
__device__ __forceinline__ double wave_incl_scan(double v) {
  v += dpp_shr<0x111>(v);  // row_shr:1
  v += dpp_shr<0x112>(v);  // row_shr:2
  v += dpp_shr<0x114>(v);  // row_shr:4
  v += dpp_shr<0x118>(v);  // row_shr:8
  const double t0 = readlane(v, 15), t1 = readlane(v, 31), t2 = readlane(v, 47);
  const int row = lane_id() >> 4;
  const double add = row == 0 ? 0.0 : (row == 1 ? t0 : (row == 2 ? t0 + t1 : (t0 + t1) + t2));
  return v + add;
}

// Exact power-of-two rescaling between integer shifts (a difference below
// -2000, -inf included, scales to 0).
__device__ __forceinline__ int shift_amount(float d) { return d < -2000.f ? -2000 : (int)d; }


// ---------------------------------------------------------------- loads

// One work item: kUnroll 16-byte vectors per lane.  Lane l, vector v covers
// elements [(v*64 + l) * kPerVec, +kPerVec) of the chunk, so a wave reads
// 64 consecutive 16-byte segments per vector step (fully coalesced) and a
// lane's elements are in increasing index order.  Elements past `n` are
// filled with -inf.
// TileN<DT, U> holds U of those vectors, starting at vector v0 of the chunk.
template <int DT, int U> struct TileN {
  static constexpr uint32_t kNegInfWord = DT == DSPARK_BF16 ? 0xff80ff80u : 0xff800000u;
  uint32_t w[U][4];
  int n_, v0_;

  // this lane's vector v lies inside the row
  __device__ __forceinline__ bool valid(int v) const {
    return ((v0_ + v) * kWave + lane_id()) * Elem<DT>::kPerVec < n_;
  }

  // VEC: rows start on 16-byte boundaries and V is a multiple of the vector
  // width, so each 16-byte vector is wholly inside or wholly past the row.
  template <bool VEC>
  __device__ __forceinline__ void load(const void* chunk_base, int n, int v0 = 0) {
    const int l = lane_id();
    constexpr int P = Elem<DT>::kPerVec;
    n_ = n;
    v0_ = v0;
    if constexpr (VEC) {
      // Straight-line loads and no later writes to these registers, so the
      // compiler waits for exactly these loads and not for ones issued after
      // them.  Vectors past the end of the row re-read the chunk's first
      // vector: duplicates of real elements cannot change a maximum, and sums
      // drop them with valid(v).
      const char* cb = static_cast<const char*>(__builtin_assume_aligned(chunk_base, 16));
      if (n >= (v0 + U) * kWave * P) {  // wave-uniform: the whole tile is in the row
#pragma unroll
        for (int v = 0; v < U; ++v) {
          const uint4 q = *reinterpret_cast<const uint4*>(cb + (size_t)((v0 + v) * kWave + l) * 16);
          w[v][0] = q.x; w[v][1] = q.y; w[v][2] = q.z; w[v][3] = q.w;
        }
      } else {
#pragma unroll
        for (int v = 0; v < U; ++v) {
          const int e0 = ((v0 + v) * kWave + l) * P;
          const int ea = e0 < n ? e0 : 0;
          const uint4 q = *reinterpret_cast<const uint4*>(cb + (size_t)ea * Elem<DT>::kBytes);
          w[v][0] = q.x; w[v][1] = q.y; w[v][2] = q.z; w[v][3] = q.w;
        }
      }
      return;
    }
#pragma unroll
    for (int v = 0; v < U; ++v) {
      const int e0 = ((v0 + v) * kWave + l) * P;
      {
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

  // The tile's largest element (exact), found on the raw bit patterns with
  // integer max / min so that no NaN handling is needed: read as signed
  // integers, non-negative floats order like their values and negative ones
  // in reverse, so the largest non-negative pattern is the maximum when there
  // is one, and otherwise the smallest (most negative) pattern is.  bf16
  // pairs use packed 16-bit max / min.  NaN patterns can win; a NaN shift
  // makes the exponent sum NaN, which is reported there.
  // The largest key is the largest element unless every element is
  // negative (sign bit set); only then, wave-uniformly, a second pass takes
  // the smallest key, which is the largest negative element.
  __device__ __forceinline__ float shift_max() const {
    if constexpr (DT == DSPARK_BF16) {
      typedef short s16x2 __attribute__((ext_vector_type(2)));
      s16x2 mx = {(short)-32768, (short)-32768};
#pragma unroll
      for (int v = 0; v < U; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          mx = __builtin_elementwise_max(mx, __builtin_bit_cast(s16x2, w[v][i]));
      const int hi = wave_max_i(mx.x > mx.y ? mx.x : mx.y);
      if (hi >= 0) return __uint_as_float((uint32_t)hi << 16);
      s16x2 mn = {(short)32767, (short)32767};
#pragma unroll
      for (int v = 0; v < U; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          mn = __builtin_elementwise_min(mn, __builtin_bit_cast(s16x2, w[v][i]));
      const int lo = wave_min_i(mn.x < mn.y ? mn.x : mn.y);
      return __uint_as_float((uint32_t)(lo & 0xffff) << 16);
    } else {
      int mx = INT_MIN;
#pragma unroll
      for (int v = 0; v < U; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = max(mx, (int)w[v][i]);
      mx = wave_max_i(mx);
      if (mx >= 0) return __int_as_float(mx);
      int mn = INT_MAX;
#pragma unroll
      for (int v = 0; v < U; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) mn = min(mn, (int)w[v][i]);
      return __int_as_float(wave_min_i(mn));
    }
  }

  // Hide the words' values from the compiler (no instruction is emitted), so
  // conversions made before this point are recomputed after it instead of
  // being kept live in registers.
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int v = 0; v < U; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(w[v][i]));
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

template <int DT> using Tile = TileN<DT, kUnroll>;

// LaneRun<DT, NV>: a chunk laid out so that thread `owner` holds NV
// consecutive 16-byte vectors, i.e. elements [owner*NV*P, (owner+1)*NV*P) in
// token order.  Used by the draws, which scan one chunk: a block scan over
// the per-thread totals finds the crossing thread.  Elements past `n` are
// -inf.
template <int DT, int NV> struct LaneRun {
  static constexpr int P = Elem<DT>::kPerVec;
  static constexpr int kElems = NV * P;
  uint32_t w[NV][4];

  template <bool VEC>
  __device__ __forceinline__ void load(const void* chunk_base, int n, int owner) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e0 = (owner * NV + v) * P;
      if (VEC && e0 + P <= n) {
        const uint4 q = *reinterpret_cast<const uint4*>(
            static_cast<const char*>(chunk_base) + (size_t)e0 * Elem<DT>::kBytes);
        w[v][0] = q.x; w[v][1] = q.y; w[v][2] = q.z; w[v][3] = q.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[v][i] = DT == DSPARK_BF16 ? 0xff80ff80u : 0xff800000u;
        for (int e = 0; e < P; ++e) {
          if (e0 + e < n) {
            if constexpr (DT == DSPARK_BF16) {
              const uint32_t h = static_cast<const uint16_t*>(chunk_base)[e0 + e];
              uint32_t& x = w[v][e >> 1];
              x = (e & 1) ? ((x & 0x0000ffffu) | (h << 16)) : ((x & 0xffff0000u) | h);
            } else {
              w[v][e] = static_cast<const uint32_t*>(chunk_base)[e0 + e];
            }
          }
        }
      }
    }
  }
  // element i (0..kElems-1) of this thread's run, exact widening; i compile-time
  __device__ __forceinline__ float at(int i) const {
    const int v = i / P, e = i % P;
    if constexpr (DT == DSPARK_BF16) {
      const uint32_t x = w[v][e >> 1];
      return (e & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
    } else {
      return __uint_as_float(w[v][e]);
    }
  }
};

// scalar element fetch as stored bits, and their exact widening
template <int DT> __device__ __forceinline__ uint32_t load_raw(const void* row, int idx) {
  if constexpr (DT == DSPARK_BF16)
    return static_cast<uint32_t>(static_cast<const uint16_t*>(row)[idx]);
  else
    return static_cast<const uint32_t*>(row)[idx];
}
template <int DT> __device__ __forceinline__ float raw_to_float(uint32_t x) {
  return DT == DSPARK_BF16 ? __uint_as_float(x << 16) : __uint_as_float(x);
}

// scalar element fetch (exact widening)
template <int DT> __device__ __forceinline__ float load_elem(const void* row, int idx) {
  if constexpr (DT == DSPARK_BF16) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(row)[idx]) << 16);
  } else {
    return static_cast<const float*>(row)[idx];
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^a in fp64 for the few elements that need it: range reduction a = n + f,
// |f| <= 1/2, then the Taylor series of e^t, t = f ln 2, to degree 9 by
// Horner's rule (truncation below t^10/10! < 1e-11 relative) and an exact
// scaling by 2^n.  Arguments below -2000 (and NaN) give 0.  Branch-free, so
// that independent calls interleave.
__device__ __forceinline__ double exp2_f64(double a) {
  const double aa = fmax(a, -2000.0);  // NaN gives -2000 here and 0 below
  const double n = rint(aa);
  const double t = (aa - n) * 0.69314718055994530942;
  double p = 1.0 / 362880.0;
  p = fma(p, t, 1.0 / 40320.0);
  p = fma(p, t, 1.0 / 5040.0);
  p = fma(p, t, 1.0 / 720.0);
  p = fma(p, t, 1.0 / 120.0);
  p = fma(p, t, 1.0 / 24.0);
  p = fma(p, t, 1.0 / 6.0);
  p = fma(p, t, 0.5);
  p = fma(p, t, 1.0);
  p = fma(p, t, 1.0);
  const double r = ldexp(p, (int)n);
  return a > -2000.0 ? r : 0.0;
}

// p(x) = 2^(x*c - kmax) / S in fp64, for a row summarised as (kmax, S).
__device__ __forceinline__ double row_prob(float x, float c, float kmax, double S) {
  if (!(S > 0.0)) return 0.0;
  return exp2_f64((double)x * (double)c - (double)kmax) / S;
}

__device__ __forceinline__ void flag(int32_t* st, int bits) {
  if (bits) atomicOr(st, bits);
}

}  // namespace dspark
