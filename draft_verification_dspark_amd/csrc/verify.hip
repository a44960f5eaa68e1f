// Batched block verification on gfx950.
//
// What is computed (DSpark Deep Dive, "Speculative Decoding From First
// Principles" and "The Verification Phase"; DSpark Guide, "1. The Mathematics
// of Suffix Decay"): for each request, temperature softmaxes of the scheduled
// target and draft rows, the accept test u < min(1, p(y)/q(y)) at every
// scheduled position, the first rejection, and one more token drawn either
// from the normalised residual max(0, p - q) at the rejected position or,
// when everything was accepted, from the target row after the last draft.
// Requests with temperature 0 use the greedy rule (accept while the draft
// equals the target argmax).  Rows past the scheduled length are never read
// (DSpark Deep Dive, "GPU-Resident Scheduling": maximum-length buffers,
// variable lengths by masking).
//
// Three launches on the caller's stream, shapes fixed by (B, K, V); kernel
// boundaries are the only cross-workgroup synchronisation:
//   k_stream_rows  the streaming pass.  Every workgroup first lays out the
//                  scheduled rows of all requests (target rows 0..L, draft
//                  rows 0..L-1, or target rows only for greedy requests) as a
//                  dense list of 4096-token tiles in LDS; waves then walk the
//                  list with a stride, double-buffering the 16-byte loads of
//                  the next tile while summarising the current one: an integer
//                  exponent shift k = ceil(max * c) and the sum of 2^(x*c - k)
//                  (fp32 terms, fp64 accumulation), or (max, lowest index).
//   k_decide       `groups` workgroups per request: each merges the request's
//                  row summaries (shifts align by exact powers of two), forms
//                  p(y), q(y), alpha, the accept ballot and the first
//                  rejection; workgroup 0 writes the outputs; on a
//                  rejection every workgroup sums the
//                  residual mass of its 2048-token pieces of the rejected row
//                  pair (fp32, elements with normalised mass >= 2^-12 in fp64).
//   k_draw         one wave per request: the bonus token (from the pass-1
//                  chunk summaries of target row L) or the correction token
//                  (from the residual pieces); locates the chunk or piece
//                  holding the draw, re-reads it with each lane holding a
//                  contiguous run of tokens, and finds the token with one wave
//                  scan plus a sequential scan inside the crossing lane.
#include <hip/hip_runtime.h>

#include "args.hpp"

namespace dspark {

__device__ __forceinline__ const char* target_row(const VerifyArgs& a, int b, int j, int s) {
  return static_cast<const char*>(a.target) + ((size_t)b * (a.K + 1) + j) * (size_t)a.V * s;
}
__device__ __forceinline__ const char* draft_row(const VerifyArgs& a, int b, int j, int s) {
  return static_cast<const char*>(a.draft) + ((size_t)b * a.K + j) * (size_t)a.V * s;
}
// first chunk summary of row j of request b (side 0 target, 1 draft)
__device__ __forceinline__ Partial* row_parts(const VerifyArgs& a, int b, int j, int side) {
  return a.part1 + (((size_t)b * (a.K + 1) + j) * 2 + side) * a.G;
}

// The request's rule, derived the same way by every kernel from the caller's
// arrays: clamped length, greedy / softmax / skipped, c = log2(e) / T.
struct ReqInfo {
  int L, kind, bad;
  float c;
};

__device__ __forceinline__ ReqInfo req_info(const VerifyArgs& a, int b) {
  ReqInfo r;
  r.bad = 0;
  r.c = 0.f;
  int L = a.lengths ? a.lengths[b] : a.K;
  if (L < 0 || L > a.K) {
    r.bad |= DSPARK_DEV_BAD_LENGTH;
    L = L < 0 ? 0 : a.K;
  }
  r.L = L;
  if (a.greedy_only) {
    r.kind = kKindGreedy;
  } else {
    const float T = a.temperature[b];
    if (!(T >= 0.f)) {
      r.bad |= DSPARK_DEV_BAD_TEMP;
      r.kind = kKindSkip;
    } else if (T == 0.f) {
      r.kind = kKindGreedy;
    } else {
      r.kind = kKindSoftmax;
      r.c = (float)(1.4426950408889634 / (double)T);
    }
  }
  return r;
}

// ------------------------------------------------------------------ pass 1

// Softmax summary of one tile (wave-uniform results).  Branch-free, so the
// streaming loop has the same memory operations on every path.
template <int DT>
__device__ __forceinline__ void softmax_summary(const Tile<DT>& t0, float c, float& k, double& s,
                                                int& bad) {
  constexpr int P = Elem<DT>::kPerVec;
  const float m = t0.shift_max();  // wave-uniform
  Tile<DT> t = t0;
  t.opaque();
  // integer shift: the chunk maximum maps to about 0, nothing overflows, and
  // chunks of a row merge by exact powers of two.  A chunk of -inf only gets
  // shift 0 and sums to 0 (NaN elements still make the sum NaN).
  const bool none = m == -INFINITY;
  const float kk = ceilf(m * c);
  const float nk = none ? 0.f : -kk;
  double acc = 0.0;
#pragma unroll
  for (int v = 0; v < kUnroll; ++v) {
    float p[P];
#pragma unroll
    for (int e = 0; e < P; ++e) p[e] = fast_exp2(fmaf(t.at(v, e), c, nk));
    float s4 = (p[0] + p[1]) + (p[2] + p[3]);
    if constexpr (P == 8) s4 += (p[4] + p[5]) + (p[6] + p[7]);
    acc += (double)(t0.valid(v) ? s4 : 0.f);
  }
  s = wave_sum(acc);
  k = none ? -INFINITY : kk;
  if (!(s < INFINITY) || m == INFINITY) bad |= DSPARK_DEV_NONFINITE;  // NaN or +inf
}

// Greedy summary of one tile: (max, lowest index), compared as floats.
// The maximum comes from the integer-key max / min; the lowest index holding
// it from a reverse-order pass in which the last match wins.
template <int DT>
__device__ __forceinline__ void argmax_summary(const Tile<DT>& t0, int first, float& best,
                                               int& bi, int& bad) {
  constexpr int P = Elem<DT>::kPerVec;
  const int l = lane_id();
  const float m = t0.shift_max();  // wave-uniform exact maximum (or a NaN pattern)
  Tile<DT> t = t0;
  t.opaque();
  int ord = -1;
#pragma unroll
  for (int i = kUnroll * P - 1; i >= 0; --i)
    if (t.at(i / P, i % P) == m) ord = i;
  bi = ord < 0 ? 0x7fffffff : first + ((ord / P) * kWave + l) * P + (ord % P);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) bi = min(bi, __shfl_xor(bi, o));
  best = m;
  // NaN anywhere: magnitude bits above those of infinity
  uint32_t nanw = 0;
#pragma unroll
  for (int v = 0; v < kUnroll; ++v)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (DT == DSPARK_BF16) {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        const u16x2 a = __builtin_bit_cast(u16x2, t.w[v][q] & 0x7fff7fffu);
        const u16x2 c = __builtin_bit_cast(u16x2, nanw);
        nanw = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, c));
      } else {
        nanw = max(nanw, t.w[v][q] & 0x7fffffffu);
      }
    }
  uint32_t top;
  if constexpr (DT == DSPARK_BF16)
    top = max(nanw & 0xffffu, nanw >> 16) << 16;
  else
    top = nanw;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) top = max(top, (uint32_t)__shfl_xor((int)top, o));
  if (top > 0x7f800000u || m == INFINITY) bad |= DSPARK_DEV_NONFINITE;
}

// One tile of the streaming pass, decoded from its index in the plan.
struct TileRef {
  const char* base;   // first element of the tile
  Partial* out;       // its summary slot
  int n;              // elements in the tile
  int e0;             // index of the first element in the row
  int b;              // request
};

// Per-workgroup plan in LDS: start[b] = index of request b's first tile,
// start[B] = total; info[b] = L | kind << 8; cval[b] = log2(e) / T.  Request
// b's tiles are its rows (target 0..L, then draft 0..L-1) times G chunks,
// row-major.
__device__ void build_plan(const VerifyArgs& a, int* start, int* info, float* cval) {
  __shared__ int wsum[kWavesPerBlock];
  const int tid = threadIdx.x;
  const int per = (a.B + kBlock - 1) / kBlock;
  const int b0 = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < a.B) {
      const ReqInfo r = req_info(a, b);
      const int rows = r.kind == kKindSoftmax ? 2 * r.L + 1 : (r.kind == kKindGreedy ? r.L + 1 : 0);
      info[b] = r.L | (r.kind << 8);
      cval[b] = r.c;
      start[b] = rows * a.G;  // count for now
      local += rows * a.G;
    }
  }
  // exclusive scan of the per-thread totals across the workgroup
  int incl = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane_id() >= o) incl += t;
  }
  if (lane_id() == kWave - 1) wsum[tid / kWave] = incl;
  __syncthreads();
  int off = incl - local;
  for (int w = 0; w < tid / kWave; ++w) off += wsum[w];
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < a.B) {
      const int cnt = start[b];
      start[b] = off;
      off += cnt;
    }
  }
  if (tid == kBlock - 1) start[a.B] = off;
  __syncthreads();
}

template <int DT>
__device__ __forceinline__ TileRef decode_tile(const VerifyArgs& a, const int* start,
                                               const int* info, int t) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int E = item_elems<DT>();
  // request: last b with start[b] <= t (binary search; rows with no tiles
  // have start[b] == start[b+1] and are never chosen)
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  const int b = uniform(lo);
  const int q = t - uniform(start[b]);
  const int row = q / a.G;
  const int c = q - row * a.G;
  const int L = uniform(info[b]) & 0xff;
  const int side = row <= L ? 0 : 1;
  const int j = side ? row - L - 1 : row;
  TileRef ref;
  ref.e0 = c * E;
  ref.n = min(E, a.V - ref.e0);
  // the byte offset is made wave-uniform; the base stays a kernel argument so
  // the loads remain global (not flat) accesses
  const size_t row_off = side ? ((size_t)b * a.K + j) : ((size_t)b * (a.K + 1) + j);
  const size_t off = uniform((row_off * (size_t)a.V + (size_t)ref.e0) * S);
  ref.base = (side ? static_cast<const char*>(a.draft) : static_cast<const char*>(a.target)) + off;
  ref.out = row_parts(a, b, j, side) + c;
  ref.b = b;
  return ref;
}

// Summary of one tile into its slot.  Every lane stores the same 16 bytes
// (no lane-0 branch), keeping the memory operations of the loop identical on
// all paths; status bits travel in the record and are reported by k_decide.
template <int DT>
__device__ __forceinline__ void summarise_tile(const Tile<DT>& t, const TileRef& ref, int kind,
                                               float c) {
  int bad = 0;
  Partial out;
  if (kind == kKindSoftmax) {
    softmax_summary<DT>(t, c, out.k, out.s, bad);
    out.idx = bad;
  } else {
    argmax_summary<DT>(t, ref.e0, out.k, out.idx, bad);
    out.s = (double)bad;
  }
  *ref.out = out;
}

#ifndef DSPARK_STREAM_MIN_WAVES
#define DSPARK_STREAM_MIN_WAVES 1
#endif

template <int DT, bool VEC>
__global__ void __launch_bounds__(kBlock, DSPARK_STREAM_MIN_WAVES) k_stream_rows(VerifyArgs a) {
  extern __shared__ int plan[];
  int* start = plan;                                        // [B + 1]
  int* info = plan + a.B + 1;                               // [B]
  float* cval = reinterpret_cast<float*>(plan + 2 * a.B + 1);  // [B]
  build_plan(a, start, info, cval);
  const int total = uniform(start[a.B]);
  const int W = gridDim.x * kWavesPerBlock;
  int t0 = uniform((int)(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave));
  // Two tile buffers: the next tile's loads are in flight while the current
  // one is summarised.  The prefetch is issued unconditionally (past the end
  // of the list a wave re-reads its current tile, a cache hit, and drops
  // it), so every path has the same loads outstanding and the compiler can
  // wait for the older tile only.
  Tile<DT> A, Bt;
  TileRef ra, rb;
  if (t0 >= total) return;
  ra = decode_tile<DT>(a, start, info, t0);
  A.template load<VEC>(ra.base, ra.n);
  while (true) {
    const int t1 = t0 + W;
    rb = decode_tile<DT>(a, start, info, t1 < total ? t1 : t0);
    Bt.template load<VEC>(rb.base, rb.n);
    summarise_tile<DT>(A, ra, uniform(info[ra.b]) >> 8, uniform(cval[ra.b]));
    if (t1 >= total) break;
    t0 = t1 + W;
    ra = decode_tile<DT>(a, start, info, t0 < total ? t0 : t1);
    A.template load<VEC>(ra.base, ra.n);
    summarise_tile<DT>(Bt, rb, uniform(info[rb.b]) >> 8, uniform(cval[rb.b]));
    if (t0 >= total) break;
  }
}

// ------------------------------------------------------------------ merges

// Softmax row from its chunk summaries: shift K* = max k_c over chunks with
// mass, S = sum_c s_c * 2^(k_c - K*) (exact scaling).  Wave-cooperative.
__device__ RowSum merge_softmax_row(const Partial* p, int G) {
  const int l = lane_id();
  float km = -INFINITY;
  double s = 0.0;
  int fl = 0;
  for (int c0 = 0; c0 < G; c0 += kWave) {
    const int c = c0 + l;
    if (c < G) {
      fl |= p[c].idx;
      if (p[c].s > 0.0) km = fmaxf(km, p[c].k);
    }
  }
  km = wave_max(km);
  if (km > -INFINITY) {
    for (int c0 = 0; c0 < G; c0 += kWave) {
      const int c = c0 + l;
      if (c < G) {
        const double sc = p[c].s;
        if (sc > 0.0) {
          const float d = p[c].k - km;  // integer valued, <= 0
          s += ldexp(sc, d < -2000.f ? -2000 : (int)d);
        }
      }
    }
  }
  RowSum r;
  r.k = km;
  r.s = wave_sum(s);
  r.idx = 0;
  r.bad = wave_or(fl);
  r.pad = 0;
  return r;
}

// Greedy row: (max, lowest index) over its chunk summaries.
__device__ RowSum merge_argmax_row(const Partial* p, int G) {
  const int l = lane_id();
  float best = -INFINITY;
  int bi = 0x7fffffff, fl = 0;
  for (int c = l; c < G; c += kWave) {
    argmax_merge(best, bi, p[c].k, p[c].idx);
    fl |= (int)p[c].s;
  }
  wave_argmax(best, bi);
  RowSum r;
  r.k = best;
  r.idx = bi == 0x7fffffff ? 0 : bi;  // no element above -inf: lowest index
  r.s = 0.0;
  r.bad = wave_or(fl);
  r.pad = 0;
  return r;
}

// probability of logit x under a merged row: 2^(x*c - K*) / S, in fp64
__device__ __forceinline__ double row_prob(float x, float c, float kmax, double S) {
  if (!(S > 0.0)) return 0.0;
  return exp2_f64((double)x * (double)c - (double)kmax) / S;
}

// k_merge: one wave per row slot (request, row j, side), merging the chunk
// summaries of every scheduled row once.
__global__ void __launch_bounds__(kBlock) k_merge(VerifyArgs a) {
  const int slot = uniform((int)(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave));
  const int per_req = 2 * (a.K + 1);
  if (slot >= a.B * per_req) return;
  const int b = slot / per_req;
  const int j = (slot - b * per_req) >> 1;
  const int side = slot & 1;
  const ReqInfo r = req_info(a, b);
  if (r.kind == kKindSkip || j > r.L) return;
  if (side == 1 && (r.kind != kKindSoftmax || j >= r.L)) return;
  const Partial* pr = row_parts(a, b, j, side);
  const RowSum m = r.kind == kKindSoftmax ? merge_softmax_row(pr, a.G) : merge_argmax_row(pr, a.G);
  if (lane_id() == 0) a.rows[slot] = m;
}

__device__ __forceinline__ const RowSum& row_sum(const VerifyArgs& a, int b, int j, int side) {
  return a.rows[((size_t)b * (a.K + 1) + j) * 2 + side];
}

// ------------------------------------------------------------------ draws

// Chunk masses of one draw, held in registers (up to kMaxGroups*64 chunks;
// more are re-read): total, then the chunk whose inclusive prefix first
// exceeds u * total (if rounding leaves none, the last chunk with mass and
// `past_end`), and `base`, the mass before it.
constexpr int kMaxGroups = 4;
template <typename ChunkFn>
__device__ int locate_chunk(ChunkFn chunk_mass, int G, double u, double& total, double& base,
                            bool& past_end) {
  const int l = lane_id();
  double w[kMaxGroups];
  double sum = 0.0;
#pragma unroll
  for (int i = 0; i < kMaxGroups; ++i) {
    const int c = i * kWave + l;
    w[i] = c < G ? chunk_mass(c) : 0.0;
    sum += w[i];
  }
  for (int c = kMaxGroups * kWave + l; c < G; c += kWave) sum += chunk_mass(c);
  total = wave_sum(sum);
  const double target = u * total;
  int cstar = -1, clast = -1;
  base = 0.0;
  for (int c0 = 0; c0 < G && cstar < 0; c0 += kWave) {
    const int g = c0 / kWave;
    double x = 0.0;
#pragma unroll
    for (int i = 0; i < kMaxGroups; ++i)
      if (i == g) x = w[i];
    if (g >= kMaxGroups) x = c0 + l < G ? chunk_mass(c0 + l) : 0.0;
    const double incl = wave_incl_scan(x);
    const uint64_t hit = __ballot(base + incl > target && x > 0.0);
    const uint64_t pos = __ballot(x > 0.0);
    if (pos) clast = c0 + 63 - __builtin_clzll(pos);
    if (hit) {
      const int hl = __builtin_ctzll(hit);
      cstar = c0 + hl;
      base += readlane(incl - x, hl);
    } else {
      base += readlane(incl, kWave - 1);
    }
  }
  past_end = cstar < 0;
  return past_end ? clast : cstar;
}

// Inside one chunk held as LaneRuns (lane l owns a contiguous run of N
// tokens), the first token whose running mass exceeds `target`, else the last
// token with mass (-1 if none).  mass(i) is this lane's element i.
template <int N, typename MassFn>
__device__ int scan_runs(MassFn mass, double target) {
  const int l = lane_id();
  double ls = 0.0;
  int lp = -1;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const double m = mass(i);
    ls += m;
    if (m > 0.0) lp = l * N + i;
  }
  const double incl = wave_incl_scan(ls);
  const uint64_t hit = __ballot(incl > target && ls > 0.0);
  int found = -1;
  if (hit) {
    const int x = __builtin_ctzll(hit);
    if (l == x) {
      double run = incl - ls;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const double m = mass(i);
        run += m;
        if (found < 0 && run > target && m > 0.0) found = l * N + i;
      }
      if (found < 0) found = lp;
    }
    found = readlane(found, x);
  } else {
    found = wave_max_i(lp);
  }
  return found;
}

// Draw from the softmax of target row `row` (bonus token, or the fallback of
// an all-zero residual): chunk masses come from the row's pass-1 summaries
// scaled to the merged shift; the chosen chunk is recomputed with the same
// fp32 arithmetic.  One wave.
template <int DT, bool VEC>
__device__ int draw_from_p(const VerifyArgs& a, int b, int row, float c, double u) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int E = item_elems<DT>();
  const Partial* pr = row_parts(a, b, row, 0);
  const float kp = row_sum(a, b, row, 0).k;
  auto chunk_mass = [&](int ci) -> double {
    const Partial p = pr[ci];
    if (!(p.s > 0.0)) return 0.0;
    const float d = p.k - kp;
    return ldexp(p.s, d < -2000.f ? -2000 : (int)d);
  };
  double total, base;
  bool past_end;
  const int cstar = locate_chunk(chunk_mass, a.G, u, total, base, past_end);
  if (cstar < 0) return 0;
  const int e0 = cstar * E;
  const int n = min(E, a.V - e0);
  LaneRun<DT, kUnroll> run;
  run.template load<VEC>(target_row(a, b, row, S) + (size_t)e0 * S, n);
  const float kc = pr[cstar].k;
  const float d = kc - kp;
  const int sh = d < -2000.f ? -2000 : (int)d;
  const int f = scan_runs<LaneRun<DT, kUnroll>::kElems>(
      [&](int i) -> double { return ldexp((double)fast_exp2(fmaf(run.at(i), c, -kc)), sh); },
      past_end ? INFINITY : u * total - base);
  return e0 + (f >= 0 ? f : 0);
}

// Residual p - q of one row pair at fp32 speed, with the elements whose
// normalised p or q reaches 2^-12 redone in fp64 (their fp32 rounding would
// show after dividing by a small residual mass).
struct ResidualRows {
  float c, nbt, nbd, kt, kd;
  double st, sd;
  __device__ ResidualRows(float c_, float kt_, double st_, float kd_, double sd_)
      : c(c_), kt(kt_), kd(kd_), st(st_), sd(sd_) {
    nbt = (float)(-(double)kt - log2(st));
    nbd = (float)(-(double)kd - log2(sd));
  }
  __device__ __forceinline__ float fast(float xt, float xd, float& big) const {
    const float p = fast_exp2(fmaf(xt, c, nbt));
    const float q = fast_exp2(fmaf(xd, c, nbd));
    big = fmaxf(p, q);
    return fmaxf(p - q, 0.f);
  }
  __device__ __forceinline__ double exact(float xt, float xd) const {
    const double p = exp2_f64((double)xt * (double)c - (double)kt) / st;
    const double q = exp2_f64((double)xd * (double)c - (double)kd) / sd;
    return fmax(p - q, 0.0);
  }
  // the value every kernel uses for one element
  __device__ __forceinline__ double mass(float xt, float xd) const {
    float big;
    const float r = fast(xt, xd, big);
    return big >= kHeavy ? exact(xt, xd) : (double)r;
  }
};

// Residual pieces: 2048 tokens (bf16) or 1024 (fp32), i.e. 4 vectors a lane.
constexpr int kPieceVecs = 4;
template <int DT> constexpr int piece_elems() { return kWave * kPieceVecs * Elem<DT>::kPerVec; }
template <int DT> __host__ __device__ inline int pieces_per_row(int V) {
  return (V + piece_elems<DT>() - 1) / piece_elems<DT>();
}

// Residual mass of one piece (wave total).
template <int DT, bool VEC>
__device__ double residual_piece_mass(const ResidualRows& rr, const char* tpiece,
                                      const char* dpiece, int n) {
  constexpr int P = Elem<DT>::kPerVec;
  constexpr int H = kPieceVecs;
  TileN<DT, H> tt, td;
  tt.template load<VEC>(tpiece, n);
  td.template load<VEC>(dpiece, n);
  float light = 0.f;
  float vbig[H];
#pragma unroll
  for (int v = 0; v < H; ++v) {
    float r[P];
    float hv = 0.f;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      float big;
      const float x = rr.fast(tt.at(v, e), td.at(v, e), big);
      hv = fmaxf(hv, big);
      r[e] = big >= kHeavy ? 0.f : x;
    }
    const bool ok = tt.valid(v);
    vbig[v] = ok ? hv : 0.f;
    float s4 = (r[0] + r[1]) + (r[2] + r[3]);
    if constexpr (P == 8) s4 += (r[4] + r[5]) + (r[6] + r[7]);
    light += ok ? s4 : 0.f;
  }
  // heavy elements in fp64; a vector without any is skipped by the wave
  double heavy = 0.0;
#pragma unroll
  for (int v = 0; v < H; ++v) {
    if (vbig[v] >= kHeavy) {
#pragma unroll
      for (int e = 0; e < P; ++e) {
        float big;
        rr.fast(tt.at(v, e), td.at(v, e), big);
        if (big >= kHeavy) heavy += rr.exact(tt.at(v, e), td.at(v, e));
      }
    }
  }
  return wave_sum((double)light + heavy);
}

// ------------------------------------------------------------------ decide

template <int DT, bool VEC>
__global__ void __launch_bounds__(kBlock) k_decide(VerifyArgs a) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int PE = piece_elems<DT>();
  __shared__ int s_a, s_bad;
  __shared__ RowSum s_rt, s_rd;
  const int b = blockIdx.x / a.groups;
  const int g = blockIdx.x - b * a.groups;
  const int w = uniform((int)(threadIdx.x / kWave));
  const int l = lane_id();
  const int K = a.K;
  const ReqInfo r = req_info(a, b);
  const int L = r.L;
  int32_t* tok = a.tokens + (size_t)b * (K + 1);
  const bool lead = g == 0;

  if (r.kind == kKindSkip) {
    if (lead && w == 0) {
      for (int i = l; i <= K; i += kWave) tok[i] = -1;
      if (l < K) {
        if (a.p_tok) a.p_tok[(size_t)b * K + l] = 0.f;
        if (a.q_tok) a.q_tok[(size_t)b * K + l] = 0.f;
      }
      if (l == 0) {
        a.accepted[b] = 0;
        a.req[b].mode = kModeNone;
        flag(a.dev_status, r.bad);
      }
    }
    return;
  }

  if (w == 0) {
    // lane l: position l+1 (drafted id, its logits, merged rows 0..L)
    int bad = r.bad;
    int y = 0;
    bool yok = true;
    float xt = 0.f, xd = 0.f, u = 0.f;
    if (l < L) {
      y = a.drafted[(size_t)b * K + l];
      yok = y >= 0 && y < a.V;
      if (yok) {
        xt = load_elem<DT>(target_row(a, b, l, S), y);
        if (r.kind == kKindSoftmax) xd = load_elem<DT>(draft_row(a, b, l, S), y);
      }
      if (r.kind == kKindSoftmax) u = a.uniforms[(size_t)b * (K + 1) + l];
    }
    RowSum rt{}, rd{};
    if (l <= L) rt = row_sum(a, b, l, 0);
    if (l < L && r.kind == kKindSoftmax) rd = row_sum(a, b, l, 1);
    RowSum r64{};
    if (L == 64) r64 = row_sum(a, b, 64, 0);  // the row past lane 63
    if (!yok) bad |= DSPARK_DEV_BAD_TOKEN;
    if (l <= L) bad |= rt.bad;
    if (l < L) bad |= rd.bad;
    if (L == 64 && l == 0) bad |= r64.bad;
    bool acc = false;
    float pf = 0.f, qf = 0.f;
    if (r.kind == kKindSoftmax) {
      if (l <= L && !(rt.s > 0.0)) bad |= DSPARK_DEV_NONFINITE;  // no finite logit
      if (l < L) {
        if (!(rd.s > 0.0)) bad |= DSPARK_DEV_NONFINITE;
        if (!(u >= 0.f && u < 1.f)) bad |= DSPARK_DEV_BAD_UNIFORM;
        if (yok) {
          const double p = row_prob(xt, r.c, rt.k, rt.s);
          const double q = row_prob(xd, r.c, rd.k, rd.s);
          const double alpha = p == 0.0 ? 0.0 : (q == 0.0 ? 1.0 : fmin(1.0, p / q));
          acc = (double)u < alpha;
          pf = (float)p;
          qf = (float)q;
        }
      }
      if (l == 0) {
        if (L == 64 && !(r64.s > 0.0)) bad |= DSPARK_DEV_NONFINITE;
        const float uf = a.uniforms[(size_t)b * (K + 1) + K];
        if (!(uf >= 0.f && uf < 1.f)) bad |= DSPARK_DEV_BAD_UNIFORM;
      }
    } else {
      if (l <= L && rt.k == -INFINITY) bad |= DSPARK_DEV_NONFINITE;  // no finite logit
      if (l == 0 && L == 64 && r64.k == -INFINITY) bad |= DSPARK_DEV_NONFINITE;
      acc = l < L && yok && y == rt.idx;
    }
    const uint64_t m = __ballot(acc);
    const uint64_t want = L >= 64 ? ~0ull : ((1ull << L) - 1ull);
    const uint64_t rej = ~m & want;
    const int an = rej ? __builtin_ctzll(rej) : L;
    bad = wave_or(bad);
    int gtok = 0;
    if (r.kind == kKindGreedy) gtok = an < 64 ? readlane(rt.idx, an) : readlane(r64.idx, 0);
    if (lead) {
      if (l < K) {
        if (a.p_tok) a.p_tok[(size_t)b * K + l] = pf;
        if (a.q_tok) a.q_tok[(size_t)b * K + l] = qf;
      }
      for (int i = l; i <= K; i += kWave) {
        if (i < an) tok[i] = a.drafted[(size_t)b * K + i];
        else if (i > an || r.kind == kKindGreedy) tok[i] = i == an ? gtok : -1;
      }
      if (l == 0) {
        a.accepted[b] = an;
        if (bad) flag(a.dev_status, bad);
      }
    }
    if (an < L && an == l) {
      s_rt = rt;
      s_rd = rd;
    }
    if (l == 0) {
      s_a = an;
      s_bad = bad;
    }
  }
  __syncthreads();
  const int an = s_a;
  const int bad = s_bad;
  if (r.kind == kKindGreedy || (bad & (DSPARK_DEV_BAD_TOKEN | DSPARK_DEV_NONFINITE))) {
    // greedy requests are complete; faulty ones have unspecified outputs
    if (lead && threadIdx.x == 0) a.req[b].mode = kModeNone;
    return;
  }
  if (an == L) {
    // everything accepted: k_draw draws the bonus token from target row L
    if (lead && threadIdx.x == 0) {
      ReqState& st = a.req[b];
      st.mode = kModeBonus;
      st.row = L;
      st.a = an;
      st.c = r.c;
    }
    return;
  }
  // rejection at position an+1: residual mass of this workgroup's pieces
  const RowSum rt = s_rt, rd = s_rd;
  const ResidualRows rr(r.c, rt.k, rt.s, rd.k, rd.s);
  if (lead && threadIdx.x == 0) {
    ReqState& st = a.req[b];
    st.mode = kModeResidual;
    st.row = an;
    st.a = an;
    st.c = r.c;
    st.kt = rr.kt;
    st.kd = rr.kd;
    st.st = rr.st;
    st.sd = rr.sd;
  }
  const int G2 = pieces_per_row<DT>(a.V);
  const int pi = g * kWavesPerBlock + w;
  if (pi < G2) {
    const int e0 = pi * PE;
    const int n = min(PE, a.V - e0);
    const double z = residual_piece_mass<DT, VEC>(rr, target_row(a, b, an, S) + (size_t)e0 * S,
                                                  draft_row(a, b, an, S) + (size_t)e0 * S, n);
    if (l == 0) a.part2[(size_t)b * G2 + pi] = z;
  }
}

// ------------------------------------------------------------------ draw

template <int DT, bool VEC>
__global__ void __launch_bounds__(kBlock) k_draw(VerifyArgs a) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int PE = piece_elems<DT>();
  const int b = uniform((int)(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave));
  if (b >= a.B) return;
  const ReqState st = a.req[b];
  if (st.mode != kModeResidual && st.mode != kModeBonus) return;
  const int K = a.K;
  const int G2 = pieces_per_row<DT>(a.V);
  const double u = (double)a.uniforms[(size_t)b * (K + 1) + K];
  int t = 0;
  bool from_p = st.mode == kModeBonus;
  if (!from_p) {
    const double* z = a.part2 + (size_t)b * G2;
    double Z, base;
    bool past_end;
    const int pstar = locate_chunk([&](int ci) -> double { return z[ci]; }, G2, u, Z, base, past_end);
    if (!(Z > 0.0)) {
      from_p = true;  // no residual mass: draw from p at the rejected position
    } else if (pstar >= 0) {
      const ResidualRows rr(st.c, st.kt, st.st, st.kd, st.sd);
      const int e0 = pstar * PE;
      const int n = min(PE, a.V - e0);
      LaneRun<DT, kPieceVecs> rt, rd;
      rt.template load<VEC>(target_row(a, b, st.row, S) + (size_t)e0 * S, n);
      rd.template load<VEC>(draft_row(a, b, st.row, S) + (size_t)e0 * S, n);
      const int f = scan_runs<LaneRun<DT, kPieceVecs>::kElems>(
          [&](int i) -> double { return rr.mass(rt.at(i), rd.at(i)); },
          past_end ? INFINITY : u * Z - base);
      t = e0 + (f >= 0 ? f : 0);
    }
  }
  if (from_p) t = draw_from_p<DT, VEC>(a, b, st.row, st.c, u);
  if (lane_id() == 0) a.tokens[(size_t)b * (K + 1) + st.a] = t;
}

// ------------------------------------------------------------------ launch

template <int DT, bool VEC>
static int launch_verify_t(VerifyArgs& a, hipStream_t st) {
  const size_t lds = sizeof(int) * (3 * (size_t)a.B + 1);
  const long tiles = (long)a.B * a.G * (2 * a.K + 1);
  long grid = (tiles + kWavesPerBlock - 1) / kWavesPerBlock;
  const int resident =
      resident_blocks(reinterpret_cast<const void*>(&k_stream_rows<DT, VEC>), kBlock, lds);
  if (grid > resident) grid = resident;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((k_stream_rows<DT, VEC>), dim3((unsigned)grid), dim3(kBlock), lds, st, a);
  const long slots = (long)a.B * 2 * (a.K + 1);
  hipLaunchKernelGGL(k_merge, dim3((unsigned)((slots + kWavesPerBlock - 1) / kWavesPerBlock)),
                     dim3(kBlock), 0, st, a);
  a.groups = (pieces_per_row<DT>(a.V) + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL((k_decide<DT, VEC>), dim3((unsigned)((long)a.B * a.groups)), dim3(kBlock), 0,
                     st, a);
  if (!a.greedy_only) {
    const int gb = (a.B + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL((k_draw<DT, VEC>), dim3(gb), dim3(kBlock), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_LAUNCH;
}

int launch_verify(VerifyArgs& a, int dtype, hipStream_t st) {
  if (dtype == DSPARK_BF16)
    return a.vec_ok ? launch_verify_t<DSPARK_BF16, true>(a, st)
                    : launch_verify_t<DSPARK_BF16, false>(a, st);
  return a.vec_ok ? launch_verify_t<DSPARK_F32, true>(a, st)
                  : launch_verify_t<DSPARK_F32, false>(a, st);
}

}  // namespace dspark
