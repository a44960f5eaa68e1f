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
//   k_stream_rows  the streaming pass, one workgroup per compute unit.  Each
//                  workgroup lays out the scheduled rows of all requests
//                  (target rows 0..L, draft rows 0..L-1, or target rows only
//                  for greedy requests) as a dense list of 4096-token tiles in
//                  LDS and takes every n-th tile of it (n workgroups); its
//                  waves take those tiles through an LDS counter,
//                  double-buffering the 16-byte loads of the next tile while
//                  summarising the current one: an integer exponent shift
//                  k = ceil(max * c) and the sum of 2^(x*c - k) (fp32 terms,
//                  fp64 accumulation), or (max, lowest index).  For the
//                  schedule + verify call it first works out the schedule
//                  itself (every workgroup, from the confidences, while its
//                  first tile loads are in flight).
//   k_decide       `groups` workgroups per request: each merges the request's
//                  row summaries (shifts align by exact powers of two), and
//                  wave 0 forms p(y), q(y), alpha, the accept ballot and the
//                  first rejection; workgroup 0 writes the outputs and the
//                  draw state (after its other work); on a rejection every
//                  wave sums the residual mass of one 4096-token chunk of the
//                  rejected row pair (fp32, elements with normalised mass
//                  >= 2^-12 in fp64).
//   k_draw         one workgroup per request with a pending draw: the bonus
//                  token (from the pass-1 chunk sums of target row L) or the
//                  correction token (from the residual chunk masses); a block
//                  scan locates the chunk holding the draw, the chunk is
//                  re-read with each thread owning a contiguous run of
//                  tokens, and a second block scan finds the token.
#include <hip/hip_runtime.h>

#include "args.hpp"
#include "schedule_core.hpp"

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
  float c;    // log2(e) / T rounded to fp32 (the streaming pass's factor)
  float clo;  // log2(e) / T - c, so that c + clo carries it to ~2^-48
};

// L: the request's length as given (checked and clamped here); T: its
// temperature (unused on a greedy-only call)
__device__ __forceinline__ ReqInfo req_info_lt(const VerifyArgs& a, int L, float T) {
  ReqInfo r;
  r.bad = 0;
  r.c = 0.f;
  r.clo = 0.f;
  if (L < 0 || L > a.K) {
    r.bad |= DSPARK_DEV_BAD_LENGTH;
    L = L < 0 ? 0 : a.K;
  }
  r.L = L;
  if (a.greedy_only) {
    r.kind = kKindGreedy;
  } else {
    if (!(T >= 0.f)) {
      r.bad |= DSPARK_DEV_BAD_TEMP;
      r.kind = kKindSkip;
    } else if (T == 0.f) {
      r.kind = kKindGreedy;
    } else {
      r.kind = kKindSoftmax;
      const double c64 = 1.4426950408889634 / (double)T;
      r.c = (float)c64;
      r.clo = (float)(c64 - (double)r.c);
    }
  }
  return r;
}

__device__ __forceinline__ ReqInfo req_info(const VerifyArgs& a, int b) {
  return req_info_lt(a, a.lengths ? a.lengths[b] : a.K, a.greedy_only ? 0.f : a.temperature[b]);
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

// Threads of a streaming workgroup: one workgroup per compute unit, 12 waves
// (three per SIMD), which is what the kernel's register use allows.
#ifndef DSPARK_STREAM_BLOCK
#define DSPARK_STREAM_BLOCK 768
#endif
constexpr int kStreamBlock = DSPARK_STREAM_BLOCK;
constexpr int kStreamWaves = kStreamBlock / kWave;
static_assert(kFusedMaxB == kStreamBlock && kFusedMaxPositions == kSchedLds,
              "fused schedule limits: one request per streaming thread, keys in LDS");

// The tile list.  Tiles [0, B*G) are target row 0 of every request (chunk c of
// request b is tile b*G + c): that row is read whatever the length, so these
// tiles are known before the plan exists.  The rest follow request by
// request: target rows 1..L and draft rows 0..L-1 of a sampled request,
// target rows 1..L of a greedy one, nothing for a skipped one, each row as G
// chunks in order.
//
// Per-workgroup plan in LDS: start[b] = index of request b's first tile after
// row 0, start[B] = total; info[b] = L | kind << 8; cval[b] = log2(e) / T.
// With `has_pre`, `pre` is this thread's request (one request per thread).
__device__ __forceinline__ void build_plan(const VerifyArgs& a, int* start, int* info,
                                           float* cval, bool has_pre, ReqInfo pre) {
  __shared__ int wsum[kStreamWaves];
  const int tid = threadIdx.x;
  const int per = (a.B + kStreamBlock - 1) / kStreamBlock;
  const int b0 = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < a.B) {
      const ReqInfo r = has_pre ? pre : req_info(a, b);
      const int rows = r.kind == kKindSoftmax ? 2 * r.L : (r.kind == kKindGreedy ? r.L : 0);
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
  int off = a.B * a.G + incl - local;
  for (int w = 0; w < tid / kWave; ++w) off += wsum[w];
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    if (b < a.B) {
      const int cnt = start[b];
      start[b] = off;
      off += cnt;
    }
  }
  if (tid == kStreamBlock - 1) start[a.B] = off;
  __syncthreads();
}

// Tile t of the list.  Tiles of target row 0 need no plan.
template <int DT>
__device__ __forceinline__ TileRef decode_tile(const VerifyArgs& a, const int* start,
                                               const int* info, int t) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int E = item_elems<DT>();
  const int P0 = a.B * a.G;
  int b, c, side, j;
  if (t < P0) {
    b = t / a.G;
    c = t - b * a.G;
    side = 0;
    j = 0;
  } else {
    // request: last b with start[b] <= t (binary search; requests with no
    // tiles have start[b] == start[b+1] and are never chosen)
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (start[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    b = uniform(lo);
    const int q = t - uniform(start[b]);
    const int row = q / a.G;
    c = q - row * a.G;
    const int L = uniform(info[b]) & 0xff;
    side = row < L ? 0 : 1;
    j = side ? row - L : row + 1;
  }
  b = uniform(b);
  c = uniform(c);
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

// k_stream_rows: one workgroup per compute unit.  Workgroup g takes tiles
// g, g + n, g + 2n, ... of the list (n workgroups), spreading every
// workgroup's reads over the whole list; its waves take these tiles in turn
// through an LDS counter, so that waves which the compute unit's arbitration
// serves more slowly simply take fewer tiles.  A wave's first tile, when it
// is a row-0 tile, is requested before the plan is built.
//
// FUSED (the schedule + verify call, at most kStreamBlock requests and
// kSchedLds positions): every workgroup first works out the whole schedule
// from the confidences `s` itself, while its row-0 loads are in flight, and
// takes the lengths from it; the schedule is deterministic, so all agree.
// Workgroup g writes the schedule's outputs (lengths, mask, survival,
// status) of the requests b with b % n == g, which the later launches read;
// one workgroup writing them all would start streaming last.
template <int DT, bool VEC, bool FUSED>
__global__ void __launch_bounds__(kStreamBlock) k_stream_rows(VerifyArgs a, ScheduleArgs s) {
  extern __shared__ int plan[];
  __shared__ int s_next;
  int* start = plan;                                        // [B + 1]
  int* info = plan + a.B + 1;                               // [B]
  float* cval = reinterpret_cast<float*>(plan + 2 * a.B + 1);  // [B]
  const int n = gridDim.x, g = blockIdx.x;
  const int w = uniform((int)(threadIdx.x / kWave));
  auto tile_of = [&](int k) { return g + n * k; };
  // Two tile buffers: the next tile's loads are in flight while the current
  // one is summarised.  The prefetch is issued unconditionally (past the end
  // of the range a wave re-reads its current tile, a cache hit, and drops
  // it), so every path has the same loads outstanding and the compiler can
  // wait for the older tile only.
  Tile<DT> A, Bt;
  TileRef ra, rb;
  int t0 = w;
  // With one request per thread, the thread's request data (length and
  // temperature, or for FUSED its confidences, at most 16) is requested
  // first and, on the vector path, a wave whose first tile is a row-0 tile
  // requests it right after: the plan then waits for the request data only,
  // with the tile still in flight.
  const bool one_each = a.B <= kStreamBlock;
  const bool mine_req = one_each && (int)threadIdx.x < a.B;
  int l_raw = a.K;
  float t_raw = 0.f;
  float cpre[16];
  if (mine_req) {
    if (!a.greedy_only) t_raw = a.temperature[threadIdx.x];
    if constexpr (FUSED) {
      // one path of plain loads (two would meet in a copy that waits)
      const float* cr = s.conf + (size_t)threadIdx.x * s.K;
#pragma unroll
      for (int i = 0; i < 16; ++i) cpre[i] = cr[min(i, s.K - 1)];
    } else {
      if (a.lengths) l_raw = a.lengths[threadIdx.x];
    }
  }
  // Every wave issues the same eight loads here, so that waiting for the
  // request data above never waits for them: its first tile when that is a
  // row-0 tile (needs no plan), else another wave's row-0 tile (a tile of a
  // workgroup on the same XCD, usually served from L2), dropped.
  const int P0 = a.B * a.G;
  const bool early = VEC && tile_of(t0) < P0;
  if constexpr (VEC) {
    ra = decode_tile<DT>(a, start, info, early ? tile_of(t0) : tile_of(t0) % P0);
    A.template load<VEC>(ra.base, ra.n);
  }
  ReqInfo mine{0, kKindSkip, 0, 0.f};
  if constexpr (FUSED) {
    const int len = schedule_body<kStreamBlock, 16, true>(s, s.tau, s.budget, g, n, cpre);
    if (mine_req) mine = req_info_lt(a, len, t_raw);
  } else {
    if (mine_req) mine = req_info_lt(a, l_raw, t_raw);
  }
  build_plan(a, start, info, cval, one_each, mine);
  const int total = uniform(start[a.B]);
  const int end = uniform((total - g + n - 1) / n);  // tiles of this workgroup
  if (threadIdx.x == 0) s_next = kStreamWaves;
  __syncthreads();
  // next tile index for this wave (one LDS atomic by lane 0)
  auto grab = [&]() -> int {
    int x = 0;
    if (lane_id() == 0) x = atomicAdd(&s_next, 1);
    return uniform(readlane(x, 0));
  };
  if (t0 >= end) return;
  if (!early) {
    ra = decode_tile<DT>(a, start, info, tile_of(t0));
    A.template load<VEC>(ra.base, ra.n);
  }
  while (true) {
    const int t1 = grab();
    rb = decode_tile<DT>(a, start, info, tile_of(t1 < end ? t1 : t0));
    Bt.template load<VEC>(rb.base, rb.n);
    summarise_tile<DT>(A, ra, uniform(info[ra.b]) >> 8, uniform(cval[ra.b]));
    if (t1 >= end) break;
    t0 = grab();
    ra = decode_tile<DT>(a, start, info, tile_of(t0 < end ? t0 : t1));
    A.template load<VEC>(ra.base, ra.n);
    summarise_tile<DT>(Bt, rb, uniform(info[rb.b]) >> 8, uniform(cval[rb.b]));
    if (t0 >= end) break;
  }
}

// ------------------------------------------------------------------ merges


// Chunk summaries of one row folded into a merged row, wave-cooperatively.
// Each lane folds the chunks c = lane, lane + 64, ... (the first one passed
// in, already loaded) with exact power-of-two rescaling, then the wave takes
// K* = max shift and S = sum of the lane sums scaled to K*.
__device__ RowSum merge_softmax(Partial first, const Partial* p, int G) {
  const int l = lane_id();
  float km = -INFINITY;
  double s = 0.0;
  int fl = 0;
  Partial q = first;
  for (int c = l; c < G; c += kWave) {
    if (c != l) q = p[c];
    fl |= q.idx;
    if (q.s > 0.0) {
      if (q.k > km) {
        s = ldexp(s, shift_amount(km - q.k));
        km = q.k;
      }
      s += ldexp(q.s, shift_amount(q.k - km));
    }
  }
  RowSum r;
  r.k = wave_max(km);
  r.s = wave_sum(km > -INFINITY ? ldexp(s, shift_amount(km - r.k)) : 0.0);
  r.idx = 0;
  r.bad = wave_or(fl);
  r.pad = 0;
  return r;
}

// Greedy row: (max, lowest index) over its chunk summaries.
__device__ RowSum merge_argmax(Partial first, const Partial* p, int G) {
  const int l = lane_id();
  float best = -INFINITY;
  int bi = 0x7fffffff, fl = 0;
  Partial q = first;
  for (int c = l; c < G; c += kWave) {
    if (c != l) q = p[c];
    argmax_merge(best, bi, q.k, q.idx);
    fl |= (int)q.s;
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

// The same merges by one 16-lane group from summaries staged in LDS: lane
// `sub` folds chunks sub, sub + 16, ...; the group then combines its lanes.
__device__ RowSum merge_softmax16(const Partial* p, int G, int sub) {
  float km = -INFINITY;
  double s = 0.0;
  int fl = 0;
  for (int c = sub; c < G; c += 16) {
    const Partial q = p[c];
    fl |= q.idx;
    if (q.s > 0.0) {
      if (q.k > km) {
        s = ldexp(s, shift_amount(km - q.k));
        km = q.k;
      }
      s += ldexp(q.s, shift_amount(q.k - km));
    }
  }
  RowSum r;
  r.k = row16_reduce(km, [](float x, float y) { return fmaxf(x, y); });
  r.s = row16_reduce(km > -INFINITY ? ldexp(s, shift_amount(km - r.k)) : 0.0,
                     [](double x, double y) { return x + y; });
  r.idx = 0;
  r.bad = row16_reduce(fl, [](int x, int y) { return x | y; });
  r.pad = 0;
  return r;
}

__device__ RowSum merge_argmax16(const Partial* p, int G, int sub) {
  float best = -INFINITY;
  int bi = 0x7fffffff, fl = 0;
  for (int c = sub; c < G; c += 16) {
    const Partial q = p[c];
    argmax_merge(best, bi, q.k, q.idx);
    fl |= (int)q.s;
  }
  row16_argmax(best, bi);
  RowSum r;
  r.k = best;
  r.idx = bi == 0x7fffffff ? 0 : bi;
  r.s = 0.0;
  r.bad = row16_reduce(fl, [](int x, int y) { return x | y; });
  r.pad = 0;
  return r;
}

// The residual of a rejected row pair, element by element, in a form whose
// rounding error is relative to the difference itself rather than to p or
// q.  With x1 = xt*c - kt, x2 = xd*c - kd + log2(St'/Sd') and g = x1 - x2,
//   e1 = 2^x1,  e2 = 2^x2,  d = e1 - e2 = 2^x1 (1 - 2^-g)  (g >= 0; the
//   mirror image for g < 0),
// where St', Sd' are the merged rows' sums from the streaming pass.  In units
// of the target row's sum, e1 is p(v) and e2 is q(v) rescaled by St'/Sd'.
// g = (xt - xd)*c - D0, D0 = kt - kd + log2(St'/Sd'), is formed from the
// exact difference of the two logits (bf16 values differ exactly in fp32;
// fp32 values close enough to cancel differ exactly too), with c and D0 each
// carried as an fp32 pair (hi + lo), so g keeps its relative precision
// however small it is; 1 - 2^-|g| comes from its Taylor series below 1 and
// from the exponentials above.  Elements whose p or q reaches 2^-12 are
// redone in fp64 with the same formula.  c is log2(e)/T to fp64 precision.
//
// The streaming pass's St'/Sd' is accurate to about 1e-7, and its error
// would move every d by a multiple of e2; divided by a small residual mass
// that would show in the draw.  The pass over the rejected pair therefore
// also sums, per chunk, D = sum d, E2 = sum e2 and Q = sum of e2 over the
// elements with d > 0: the exact ratio of the two rows' sums is
// rho * St'/Sd' with rho - 1 = (sum D)/(sum E2), formed from accurately
// computed differences, and the residual at the exact ratio is
// max(0, d - (rho - 1) e2), whose chunk mass is Z - (rho - 1) Q to first
// order (elements that change sign contribute at second order).
struct ResidualRows {
  float chi, clo, nkt, nd0hi, nd0lo, theta;
  double c64, kt64, d0;
  __device__ ResidualRows(float c_, float clo_, float kt_, double st, float kd_, double sd)
      : chi(c_), clo(clo_) {
    c64 = (double)c_ + (double)clo_;
    kt64 = (double)kt_;
    d0 = (double)kt_ - (double)kd_ + (log2(st) - log2(sd));
    nkt = -kt_;
    nd0hi = (float)(-d0);
    nd0lo = (float)(-d0 - (double)nd0hi);
    theta = (float)(log2(st) - 12.0);  // p or q >= 2^-12  <=>  x1 or x2 >= theta
  }
  // fp32 path: d and e2 of one element; `heavy` reports an element to redo
  // with exact()
  __device__ __forceinline__ float fast(float xt, float xd, float& e2, bool& heavy) const {
    const float dx = xt - xd;
    const float g = fmaf(dx, chi, nd0hi) + fmaf(dx, clo, nd0lo);
    const float x1 = fmaf(xt, clo, fmaf(xt, chi, nkt));
    const float x2 = x1 - g;
    heavy = fmaxf(x1, x2) >= theta;
    const float e1 = fast_exp2(x1);
    e2 = fast_exp2(x2);
    // 1 - 2^-|g| = 1 - e^-z, z = |g| ln 2 < 0.7: Taylor series to z^10 (the
    // truncation is below 2e-8 relative)
    const float ag = fabsf(g);
    const float z = ag * 0.69314718f;
    float t = -1.f / 3628800.f;
    t = fmaf(t, z, 1.f / 362880.f);
    t = fmaf(t, z, -1.f / 40320.f);
    t = fmaf(t, z, 1.f / 5040.f);
    t = fmaf(t, z, -1.f / 720.f);
    t = fmaf(t, z, 1.f / 120.f);
    t = fmaf(t, z, -1.f / 24.f);
    t = fmaf(t, z, 1.f / 6.f);
    t = fmaf(t, z, -0.5f);
    t = fmaf(t, z, 1.f);
    const float big = g >= 0.f ? e1 : e2;
    const float ad = ag >= 1.f ? fabsf(e1 - e2) : big * (t * z);
    const float d = g >= 0.f ? ad : -ad;
    return g == g ? d : 0.f;  // both logits -inf: nothing on either side
  }
  // fp64 path, same formula (1 - 2^-|g| from expm1, so that a small |g|
  // keeps its relative precision against the exponentials' own error)
  __device__ __forceinline__ double exact(float xt, float xd, double& e2) const {
    const double x1 = (double)xt * c64 - kt64;
    const double g = ((double)xt - (double)xd) * c64 - d0;
    const double e1 = exp2_f64(x1);
    e2 = exp2_f64(x1 - g);
    const double ag = fabs(g);
    const double ad = ag >= 1.0 ? fabs(e1 - e2) : (g >= 0.0 ? e1 : e2) * -expm1(-ag * 0.69314718055994530942);
    const double d = g >= 0.0 ? ad : -ad;
    return g == g ? d : 0.0;
  }
};

// element i of a register-held run, i only known at run time (select chain)
template <int DT, int NV>
__device__ __forceinline__ float run_elem(const uint32_t (&w)[NV][4], int i) {
  constexpr int P = Elem<DT>::kPerVec;
  constexpr int WPV = 4;
  const int word = DT == DSPARK_BF16 ? (i >> 1) : i;  // word index within the run
  uint32_t x = 0;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int q = 0; q < WPV; ++q)
      if (word == v * WPV + q) x = w[v][q];
  (void)P;
  if constexpr (DT == DSPARK_BF16)
    return (i & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
  else
    return __uint_as_float(x);
}

// element e of one 16-byte vector, e only known at run time
template <int DT>
__device__ __forceinline__ float vec_elem(const uint32_t (&w)[4], int e) {
  const int word = DT == DSPARK_BF16 ? (e >> 1) : e;
  const uint32_t x = word == 0 ? w[0] : word == 1 ? w[1] : word == 2 ? w[2] : w[3];
  if constexpr (DT == DSPARK_BF16)
    return (e & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
  else
    return __uint_as_float(x);
}

// The residual sums of U of a chunk's kUnroll vectors per lane, starting at
// vector v0, of the rejected row pair (wave totals).  Vector by vector: the
// fp32 terms, then, for a vector holding an element with p or q >= 2^-12,
// those elements again in fp64 (a rolled loop).  The empty asm statements
// keep each vector's work in place, so that the compiler does not spread all
// vectors' conversions over the whole pass.
template <int DT, bool VEC, int U>
__device__ ResidualChunk residual_piece(const ResidualRows& rr, const char* tchunk,
                                        const char* dchunk, int n, int v0) {
  constexpr int P = Elem<DT>::kPerVec;
  TileN<DT, U> tt, td;
  tt.template load<VEC>(tchunk, n, v0);
  td.template load<VEC>(dchunk, n, v0);
  float lz = 0.f, ld = 0.f, lq = 0.f, le = 0.f;
  double hz = 0.0, hd = 0.0, hq = 0.0, he = 0.0;
#pragma unroll
  for (int v = 0; v < U; ++v) {
    uint32_t hm = 0;  // this lane's heavy elements of vector v
    float sz = 0.f, sd = 0.f, sq = 0.f, se = 0.f;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      bool h;
      float e2;
      const float d = rr.fast(tt.at(v, e), td.at(v, e), e2, h);
      hm |= h ? 1u << e : 0u;
      const float dl = h ? 0.f : d, el = h ? 0.f : e2;
      sz += fmaxf(dl, 0.f);
      sd += dl;
      sq += dl > 0.f ? el : 0.f;
      se += el;
    }
    const bool ok = tt.valid(v);
    lz += ok ? sz : 0.f;
    ld += ok ? sd : 0.f;
    lq += ok ? sq : 0.f;
    le += ok ? se : 0.f;
    if (!ok) hm = 0;
    if (hm) {
      // each lane walks its own heavy elements (usually one)
      const uint32_t wt[4] = {tt.w[v][0], tt.w[v][1], tt.w[v][2], tt.w[v][3]};
      const uint32_t wd[4] = {td.w[v][0], td.w[v][1], td.w[v][2], td.w[v][3]};
      while (hm) {
        const int e = __builtin_ctz(hm);
        hm &= hm - 1;
        double e2;
        const double d = rr.exact(vec_elem<DT>(wt, e), vec_elem<DT>(wd, e), e2);
        hz += fmax(d, 0.0);
        hd += d;
        hq += d > 0.0 ? e2 : 0.0;
        he += e2;
      }
    }
    asm volatile("" : "+v"(lz), "+v"(ld), "+v"(lq), "+v"(le));
  }
  ResidualChunk c;
  c.z = wave_sum((double)lz + hz);
  c.d = wave_sum((double)ld + hd);
  c.q = wave_sum((double)lq + hq);
  c.e2 = wave_sum((double)le + he);
  return c;
}

// Inverse CDF over at most 64 non-negative weights, one per lane (lanes past
// the count hold 0), in lane order: the first lane whose running sum exceeds
// u * total (and has weight), else the last lane with weight (`past_end`),
// else -1.  `base` = the sum before it.  Wave-uniform results, no barrier.
struct Located {
  int idx;
  int past_end;
  double base;
  double total;
};
__device__ __forceinline__ Located wave_locate(double x, double u) {
  const double incl = wave_incl_scan(x);
  Located r;
  r.total = readlane(incl, kWave - 1);
  const double target = u * r.total;
  const uint64_t hit = __ballot(incl > target && x > 0.0);
  const uint64_t pos = __ballot(x > 0.0);
  if (hit) {
    r.idx = __builtin_ctzll(hit);
    r.past_end = 0;
    r.base = readlane(incl - x, r.idx);
  } else {
    r.idx = pos ? 63 - __builtin_clzll(pos) : -1;
    r.past_end = 1;
    r.base = r.total;
  }
  return r;
}

// ------------------------------------------------------------------ decide

// k_decide: `groups` workgroups of kDecideBlock threads per request.  Each
// stages the request's chunk summaries in LDS and merges its rows (16-lane
// groups, one row each), then wave 0 decides: p(y), q(y), alpha, the accept
// ballot, the first rejection.  On a rejection the workgroup then sums the
// residual mass of kChunksPerGroup chunks of the rejected row pair,
// kWavesPerChunk waves per chunk.  Workgroup 0 finally writes the outputs and
// the draw state.
#ifndef DSPARK_DECIDE_BLOCK
#define DSPARK_DECIDE_BLOCK 640
#endif
#ifndef DSPARK_WAVES_PER_CHUNK
#define DSPARK_WAVES_PER_CHUNK 1
#endif
constexpr int kDecideBlock = DSPARK_DECIDE_BLOCK;
constexpr int kDecideWaves = kDecideBlock / kWave;
// waves per residual chunk (each takes an equal share of its vectors).  Ten
// waves with one wave per chunk: a request at 151,936 tokens (38 chunks)
// needs 4 workgroups, so a batch of 64 requests is one workgroup per compute
// unit, all resident at once (two waves per chunk measured slower at full
// length and no faster as scheduled)
constexpr int kWavesPerChunk = DSPARK_WAVES_PER_CHUNK;
constexpr int kChunksPerGroup = kDecideWaves / kWavesPerChunk;
constexpr int kMaxRows = 2 * 64 + 1;
// chunk summaries staged in LDS per round of the merges (30 KB)
constexpr int kStage = 3 * kDecideBlock;

template <int DT, bool VEC>
__global__ void __launch_bounds__(kDecideBlock) k_decide(VerifyArgs a) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int E = item_elems<DT>();
  __shared__ RowSum s_rows[kMaxRows + 2];  // merged rows, then the rejected pair
  __shared__ Partial s_part[kStage];       // chunk summaries of the rows being merged
  __shared__ int s_a, s_bad;
  __shared__ ResidualChunk s_half[kDecideWaves];
  const int b = blockIdx.x / a.groups;
  const int g = blockIdx.x - b * a.groups;
  const int w = uniform((int)(threadIdx.x / kWave));
  const int l = lane_id();
  const int K = a.K;
  // Requested together, before anything waits: the request's length and
  // temperature, the final uniform and, for wave 0 lane l, the drafted id
  // and accept uniform of position l+1.  Loads whose value is used later are
  // kept out of lane-dependent branches (lanes past K re-read column K-1),
  // so that the compiler does not wait for them on the spot.
  const int lcol = min(l, K - 1);
  // (a greedy-only call has no uniforms: the drafted ids stand in, unused)
  const float* ub = a.uniforms ? a.uniforms + (size_t)b * (K + 1)
                               : reinterpret_cast<const float*>(a.drafted);
  const int y = a.drafted[(size_t)b * K + lcol];
  const float u = ub[a.uniforms ? lcol : 0];
  const float u_draw = a.uniforms ? ub[K] : 0.f;
  const ReqInfo r = req_info(a, b);
  const int L = r.L;
  int32_t* tok = a.tokens + (size_t)b * (K + 1);
  const bool lead = g == 0;  // writes the request's outputs

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
  const bool soft = r.kind == kKindSoftmax;

  // The drafted tokens' logits, gathered with the first staged summaries so
  // that one round trip covers both.  Lanes past L (and bad ids) read a
  // scheduled row at id 0 and ignore it: only target rows 0..L and draft
  // rows 0..L-1 are touched.
  const bool in_range = y >= 0 && y < a.V;
  const int yc = in_range ? y : 0;
  const bool yok = l >= L || in_range;
  const char* trow = target_row(a, b, min(l, L), S);
  const char* drow = soft && L > 0 ? draft_row(a, b, min(l, L - 1), S) : trow;  // unused then
  uint32_t xt_raw = 0, xd_raw = 0;

  // Merges.  Row order q: soft requests take target rows 0..L-1 (q = j),
  // draft rows 0..L-1 (q = L + j), then target row L (q = 2L); greedy
  // requests target rows 0..L (q = j).  Target row L comes last so that its
  // summaries are still staged when the bonus chunk is located.
  const int G = a.G;
  const int nrows = soft ? 2 * L + 1 : L + 1;
  const int qL = nrows - 1;
  auto row_of = [&](int q, int& side) -> int {
    side = (soft && q >= L && q < 2 * L) ? 1 : 0;
    return side ? q - L : (q == qL ? L : q);
  };
  int q_last = 0;  // first row of the last staged round
  if (G <= kStage) {
    // all threads stage up to kStage summaries at once, then 16-lane groups
    // merge one row each
    const int per_round = kStage / G;
    const int grp = threadIdx.x >> 4, sub = threadIdx.x & 15;
    for (int q0 = 0; q0 < nrows; q0 += per_round) {
      const int nr = min(per_round, nrows - q0);
      const int cnt = nr * G;
      q_last = q0;
      if (q0 > 0) __syncthreads();  // the previous round's merges are done
      // every load first (slots past the count re-read the first summary),
      // then every LDS store, so the loads share one round trip
      constexpr int kPer = kStage / kDecideBlock;
      Partial tmp[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = k * kDecideBlock + (int)threadIdx.x;
        const int ii = i < cnt ? i : 0;
        const int rr = ii / G;
        int side;
        const int j = row_of(q0 + rr, side);
        tmp[k] = row_parts(a, b, j, side)[ii - rr * G];
      }
      xt_raw = load_raw<DT>(trow, yc);  // (re-gathered in later rounds)
      xd_raw = load_raw<DT>(drow, yc);
#pragma unroll
      for (int k = 0; k < kPer; ++k) asm volatile("" : "+v"(tmp[k].k), "+v"(tmp[k].idx), "+v"(tmp[k].s));
      asm volatile("" : "+v"(xt_raw), "+v"(xd_raw));
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = k * kDecideBlock + (int)threadIdx.x;
        if (i < cnt) s_part[i] = tmp[k];
      }
      __syncthreads();
      for (int rr = grp; rr < nr; rr += kDecideBlock / 16) {
        const RowSum m = soft ? merge_softmax16(s_part + rr * G, G, sub)
                              : merge_argmax16(s_part + rr * G, G, sub);
        if (sub == 0) s_rows[q0 + rr] = m;
      }
    }
  } else {
    // very long rows: waves merge whole rows straight from global memory
    xt_raw = load_raw<DT>(trow, yc);
    xd_raw = load_raw<DT>(drow, yc);
    for (int q = w; q < nrows; q += kDecideWaves) {
      int side;
      const int j = row_of(q, side);
      const Partial* base = row_parts(a, b, j, side);
      const Partial first = l < G ? base[l] : Partial{-INFINITY, 0x7fffffff, 0.0};
      const RowSum m = soft ? merge_softmax(first, base, G) : merge_argmax(first, base, G);
      if (l == 0) s_rows[q] = m;
    }
  }
  __syncthreads();
  const float xt = raw_to_float<DT>(xt_raw), xd = raw_to_float<DT>(xd_raw);

  // outputs of this request (wave 0), written at the end of the kernel
  int an = 0, bad = 0, gtok = 0;
  float pf = 0.f, qf = 0.f;
  ReqState st{};
  if (w == 0) {
    const RowSum rL = s_rows[qL];  // target row L: the bonus row
    RowSum rt{}, rd{};
    if (l < L) {
      rt = s_rows[l];
      if (soft) rd = s_rows[L + l];
    }
    bad = r.bad;
    if (!yok) bad |= DSPARK_DEV_BAD_TOKEN;
    if (l < L) bad |= rt.bad | rd.bad;
    if (l == 0) bad |= rL.bad;
    bool acc = false;
    if (soft) {
      if (l < L) {
        if (!(rt.s > 0.0) || !(rd.s > 0.0)) bad |= DSPARK_DEV_NONFINITE;  // no finite logit
        if (!(u >= 0.f && u < 1.f)) bad |= DSPARK_DEV_BAD_UNIFORM;
        if (yok) {
          const double p = row_prob(xt, r.c, rt.k, rt.s);
          const double qv = row_prob(xd, r.c, rd.k, rd.s);
          const double alpha = p == 0.0 ? 0.0 : (qv == 0.0 ? 1.0 : fmin(1.0, p / qv));
          acc = (double)u < alpha;
          pf = (float)p;
          qf = (float)qv;
        }
      }
      if (l == 0) {
        if (!(rL.s > 0.0)) bad |= DSPARK_DEV_NONFINITE;
        if (!(u_draw >= 0.f && u_draw < 1.f)) bad |= DSPARK_DEV_BAD_UNIFORM;
      }
    } else {
      if (l < L && rt.k == -INFINITY) bad |= DSPARK_DEV_NONFINITE;  // no finite logit
      if (l == 0 && rL.k == -INFINITY) bad |= DSPARK_DEV_NONFINITE;
      acc = l < L && yok && y == rt.idx;
    }
    const uint64_t m = __ballot(acc);
    const uint64_t want = L >= 64 ? ~0ull : ((1ull << L) - 1ull);
    const uint64_t rej = ~m & want;
    an = rej ? __builtin_ctzll(rej) : L;
    bad = wave_or(bad);
    if (lead) {
      if (!soft) gtok = an < L ? readlane(rt.idx, an) : rL.idx;
      // draw state: the target row of the draw and, on a rejection, the
      // draft row's shift and sum as well
      const RowSum dt = an < L ? RowSum{readlane(rt.s, an), readlane(rt.k, an), 0, 0, 0} : rL;
      const RowSum dd = an < L ? RowSum{readlane(rd.s, an), readlane(rd.k, an), 0, 0, 0} : RowSum{};
      // the bonus draw's chunk, located now from the staged summaries of
      // target row L (the last row staged)
      Located bonus{-1, 0, 0.0, 0.0};
      const bool located = soft && an == L && G <= kWave && G <= kStage;
      if (located) {
        const Partial pc = l < G ? s_part[(qL - q_last) * G + l] : Partial{-INFINITY, 0, 0.0};
        const double mass = l < G && pc.s > 0.0 ? ldexp(pc.s, shift_amount(pc.k - rL.k)) : 0.0;
        bonus = wave_locate(mass, (double)u_draw);
      }
      st.mode = (!soft || (bad & (DSPARK_DEV_BAD_TOKEN | DSPARK_DEV_NONFINITE)))
                    ? kModeNone
                    : (an == L ? kModeBonus : kModeResidual);
      st.row = an;
      st.a = an;
      st.c = r.c;
      st.clo = r.clo;
      st.kt = dt.k;
      st.st = dt.s;
      st.kd = dd.k;
      st.sd = dd.s;
      st.cstar = bonus.idx;
      st.past_end = bonus.past_end;
      st.base = bonus.base;
      st.total = bonus.total;
    }
    if (an < L && an == l) {
      s_rows[kMaxRows] = rt;  // the rejected target row
      s_rows[kMaxRows + 1] = rd;  // and its draft row
    }
    if (l == 0) {
      s_a = an;
      s_bad = bad;
    }
  }
  __syncthreads();
  // on a rejection (sampled, no fault) every workgroup of the request sums
  // the residual of its chunks; greedy requests are complete, faulty ones
  // have unspecified outputs, and after a full acceptance k_draw draws the
  // bonus token from the pass-1 sums
  const int an_all = s_a;
  const int bad_all = s_bad;
  if (soft && !(bad_all & (DSPARK_DEV_BAD_TOKEN | DSPARK_DEV_NONFINITE)) && an_all < L) {
    const int an = an_all;
    const RowSum rt = s_rows[kMaxRows], rd = s_rows[kMaxRows + 1];
    const ResidualRows rr(r.c, r.clo, rt.k, rt.s, rd.k, rd.s);
    constexpr int kPart = kUnroll / kWavesPerChunk;  // vectors per wave
    const int cl = w % kChunksPerGroup, part = w / kChunksPerGroup;
    const int pi = g * kChunksPerGroup + cl;
    ResidualChunk z{0.0, 0.0, 0.0, 0.0};
    if (pi < a.G) {
      const int e0 = pi * E;
      const int n = min(E, a.V - e0);
      z = residual_piece<DT, VEC, kPart>(rr, target_row(a, b, an, S) + (size_t)e0 * S,
                                         draft_row(a, b, an, S) + (size_t)e0 * S, n,
                                         part * kPart);
    }
    if (kWavesPerChunk == 1) {
      if (pi < a.G && l == 0) a.part2[(size_t)b * a.G + pi] = z;
    } else {
      if (l == 0) s_half[w] = z;
      __syncthreads();
      if (part == 0 && pi < a.G && l == 0) {
        ResidualChunk t{0.0, 0.0, 0.0, 0.0};
        for (int h = 0; h < kWavesPerChunk; ++h) {
          const ResidualChunk& o = s_half[w + h * kChunksPerGroup];
          t.z += o.z;
          t.d += o.d;
          t.q += o.q;
          t.e2 += o.e2;
        }
        a.part2[(size_t)b * a.G + pi] = t;
      }
    }
  }
  // the lead workgroup writes the request's outputs last, so that none of its
  // stores holds up the residual work above
  if (lead && w == 0) {
    if (l < K) {
      if (a.p_tok) a.p_tok[(size_t)b * K + l] = pf;
      if (a.q_tok) a.q_tok[(size_t)b * K + l] = qf;
    }
    for (int i = l; i <= K; i += kWave) {
      if (i < an) tok[i] = y;  // lane i holds the drafted id of position i+1
      else if (i > an || !soft) tok[i] = i == an ? gtok : -1;
    }
    if (l == 0) {
      a.accepted[b] = an;
      if (bad) flag(a.dev_status, bad);
      a.req[b] = st;
    }
  }
}

// ------------------------------------------------------------------ draw

struct DrawShared {
  double w[kWavesPerBlock];
  int i[kWavesPerBlock];
  double base, total;
  int idx, past_end, found;
};

// Inverse CDF over n > 64 weights f(0..n-1) for the whole block, in index
// order (same rule as wave_locate), in rounds of kBlock weights.  Every
// thread must call it.
template <typename F>
__device__ Located block_locate(F f, int n, double u, DrawShared& sh) {
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  double part = 0.0;
  for (int i = tid; i < n; i += kBlock) part += f(i);
  const double pw = wave_sum(part);
  if (l == 0) sh.w[w] = pw;
  __syncthreads();
  double total = 0.0;
#pragma unroll
  for (int k = 0; k < kWavesPerBlock; ++k) total += sh.w[k];
  __syncthreads();
  const double target = u * total;
  double run = 0.0;
  int last = -1;
  for (int r0 = 0; r0 < n; r0 += kBlock) {
    const int i = r0 + tid;
    const double x = i < n ? f(i) : 0.0;
    const double incl_w = wave_incl_scan(x);
    const int lpw = wave_max_i(x > 0.0 ? i : -1);
    if (l == kWave - 1) {
      sh.w[w] = incl_w;
      sh.i[w] = lpw;
    }
    __syncthreads();
    double pre = run, cum = run;
    int ws = -1;
#pragma unroll
    for (int k = 0; k < kWavesPerBlock; ++k) {
      const double t = sh.w[k];
      if (k < w) pre += t;
      cum += t;
      if (ws < 0 && cum > target && t > 0.0) ws = k;
      last = max(last, sh.i[k]);
    }
    if (w == ws) {
      const double incl = pre + incl_w;
      const uint64_t hit = __ballot(incl > target && x > 0.0);
      const int hl = hit ? __builtin_ctzll(hit) : 0;
      const double before = readlane(incl - x, hl);
      if (l == 0) {
        sh.idx = hit ? r0 + w * kWave + hl : lpw;
        sh.base = hit ? before : cum;
      }
    }
    __syncthreads();
    if (ws >= 0) {
      Located r;
      r.idx = sh.idx;
      r.past_end = 0;
      r.base = sh.base;
      r.total = total;
      return r;
    }
    run = cum;
  }
  Located r;
  r.idx = last;
  r.past_end = 1;
  r.base = total;
  r.total = total;
  return r;
}

// Inside one chunk whose elements are split into contiguous runs of R per
// thread (masses m), the first element whose running mass exceeds `target`,
// else the last element with mass, else 0.  Two barriers: wave totals, then
// the crossing thread's answer.
template <int R>
__device__ int block_scan_run(const double (&m)[R], double target, DrawShared& sh) {
  const int tid = threadIdx.x, w = tid / kWave, l = lane_id();
  double ls = 0.0;
  int lp = -1;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    ls += m[i];
    if (m[i] > 0.0) lp = tid * R + i;
  }
  const double incl_w = wave_incl_scan(ls);
  const int lpw = wave_max_i(lp);
  if (l == kWave - 1) {
    sh.w[w] = incl_w;
    sh.i[w] = lpw;
  }
  __syncthreads();
  double pre = 0.0, cum = 0.0;
  int ws = -1, last = -1;
#pragma unroll
  for (int i = 0; i < kWavesPerBlock; ++i) {
    const double t = sh.w[i];
    if (i < w) pre += t;
    cum += t;
    if (ws < 0 && cum > target && t > 0.0) ws = i;
    last = max(last, sh.i[i]);
  }
  if (w == ws) {
    const double incl = pre + incl_w;
    const uint64_t hit = __ballot(incl > target && ls > 0.0);
    if (!hit) {
      if (l == 0) sh.found = lpw;  // rounding left no crossing lane
    } else if (l == __builtin_ctzll(hit)) {
      double run = incl - ls;
      int f = -1;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        run += m[i];
        if (f < 0 && run > target && m[i] > 0.0) f = tid * R + i;
      }
      sh.found = f >= 0 ? f : lp;
    }
  }
  __syncthreads();
  const int f = ws >= 0 ? sh.found : last;
  return f >= 0 ? f : 0;
}

// Draw from the softmax of target row `row` (bonus token, or the fallback of
// an all-zero residual): chunk masses come from the row's pass-1 summaries
// scaled to the merged shift kp (the chunk may already be located); the
// chosen chunk is recomputed with the same fp32 arithmetic as pass 1.
template <int DT, bool VEC>
__device__ int draw_from_p(const VerifyArgs& a, int b, int row, float c, float kp, double u,
                           Located loc, DrawShared& sh) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int E = item_elems<DT>();
  constexpr int R = E / kBlock;
  constexpr int NV = R / Elem<DT>::kPerVec;
  const Partial* pr = row_parts(a, b, row, 0);
  auto chunk_mass = [&](int ci) -> double {
    const Partial p = pr[ci];
    return p.s > 0.0 ? ldexp(p.s, shift_amount(p.k - kp)) : 0.0;
  };
  if (loc.idx < 0) {
    if (a.G <= kWave)
      loc = wave_locate(lane_id() < a.G ? chunk_mass(lane_id()) : 0.0, u);
    else
      loc = block_locate(chunk_mass, a.G, u, sh);
  }
  if (loc.idx < 0) return 0;
  const int e0 = loc.idx * E;
  const int n = min(E, a.V - e0);
  LaneRun<DT, NV> run;
  run.template load<VEC>(target_row(a, b, row, S) + (size_t)e0 * S, n, threadIdx.x);
  const float kc = pr[loc.idx].k;
  const int sh_c = shift_amount(kc - kp);
  double m[R];
#pragma unroll
  for (int i = 0; i < R; ++i) m[i] = ldexp((double)fast_exp2(fmaf(run.at(i), c, -kc)), sh_c);
  const int f = block_scan_run<R>(m, loc.past_end ? INFINITY : u * loc.total - loc.base, sh);
  return e0 + f;
}

// k_draw: one workgroup per request with a pending draw.
template <int DT, bool VEC>
__global__ void __launch_bounds__(kBlock) k_draw(VerifyArgs a) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int E = item_elems<DT>();
  constexpr int R = E / kBlock;
  constexpr int NV = R / Elem<DT>::kPerVec;
  __shared__ DrawShared sh;
  const int b = blockIdx.x;
  const int K = a.K;
  const int l = lane_id();
  // requested together: the draw state, the final uniform and this
  // request's residual chunk sums (used only after a rejection)
  const ReqState st = a.req[b];
  const double u = (double)a.uniforms[(size_t)b * (K + 1) + K];
  const ResidualChunk* zc = a.part2 + (size_t)b * a.G;
  ResidualChunk zl = l < a.G ? zc[l] : ResidualChunk{0.0, 0.0, 0.0, 0.0};
  asm volatile("" : "+v"(zl.z), "+v"(zl.d), "+v"(zl.q), "+v"(zl.e2));
  if (st.mode != kModeResidual && st.mode != kModeBonus) return;
  int t = 0;
  bool from_p = st.mode == kModeBonus;
  if (!from_p) {
    // rho - 1: the correction of the streaming pass's ratio of the two rows'
    // sums (see ResidualRows), from the signed differences of every chunk
    double sd_ = 0.0, se_ = 0.0;
    if (a.G <= kWave) {
      sd_ = wave_sum(zl.d);
      se_ = wave_sum(zl.e2);
    } else {
      double pd = 0.0, pe = 0.0;
      for (int ci = threadIdx.x; ci < a.G; ci += kBlock) {
        pd += zc[ci].d;
        pe += zc[ci].e2;
      }
      pd = wave_sum(pd);
      pe = wave_sum(pe);
      if (l == 0) {
        sh.w[threadIdx.x / kWave] = pd;
        sh.i[threadIdx.x / kWave] = 0;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kWavesPerBlock; ++k) sd_ += sh.w[k];
      __syncthreads();
      if (l == 0) sh.w[threadIdx.x / kWave] = pe;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kWavesPerBlock; ++k) se_ += sh.w[k];
      __syncthreads();
    }
    const double rm1 = se_ > 0.0 ? sd_ / se_ : 0.0;
    auto corrected = [&](const ResidualChunk& c) -> double {
      return fmax(c.z - rm1 * c.q, 0.0);
    };
    const Located loc = a.G <= kWave ? wave_locate(l < a.G ? corrected(zl) : 0.0, u)
                                     : block_locate([&](int ci) -> double {
                                         return corrected(zc[ci]);
                                       }, a.G, u, sh);
    if (!(loc.total > 0.0) || loc.idx < 0) {
      from_p = true;  // no residual mass: draw from p at the rejected position
    } else {
      const ResidualRows rr(st.c, st.clo, st.kt, st.st, st.kd, st.sd);
      const int e0 = loc.idx * E;
      const int n = min(E, a.V - e0);
      LaneRun<DT, NV> rt, rd;
      rt.template load<VEC>(target_row(a, b, st.row, S) + (size_t)e0 * S, n, threadIdx.x);
      rd.template load<VEC>(draft_row(a, b, st.row, S) + (size_t)e0 * S, n, threadIdx.x);
      // the residual at the corrected ratio, max(0, d - (rho - 1) e2): fp32
      // terms, then the heavy elements redone in fp64 by a rolled loop
      double m[R];
      uint32_t heavy = 0;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        bool h;
        float e2;
        const float d = rr.fast(rt.at(i), rd.at(i), e2, h);
        m[i] = fmax((double)d - rm1 * (double)e2, 0.0);
        if (h) heavy |= 1u << i;
      }
      while (heavy) {
        const int i = __builtin_ctz(heavy);
        heavy &= heavy - 1;
        double e2;
        const double d = rr.exact(run_elem<DT, NV>(rt.w, i), run_elem<DT, NV>(rd.w, i), e2);
        const double ex = fmax(d - rm1 * e2, 0.0);
#pragma unroll
        for (int j = 0; j < R; ++j)
          if (j == i) m[j] = ex;
      }
      const int f = block_scan_run<R>(m, loc.past_end ? INFINITY : u * loc.total - loc.base, sh);
      t = e0 + f;
    }
  }
  if (from_p) {
    Located loc{-1, 0, 0.0, 0.0};
    if (st.mode == kModeBonus && st.cstar >= 0) {
      loc.idx = st.cstar;
      loc.past_end = st.past_end;
      loc.base = st.base;
      loc.total = st.total;
    }
    t = draw_from_p<DT, VEC>(a, b, st.row, st.c, st.kt, u, loc, sh);
  }
  if (threadIdx.x == 0) a.tokens[(size_t)b * (K + 1) + st.a] = t;
}

// ------------------------------------------------------------------ launch

template <int DT, bool VEC>
static int launch_verify_t(VerifyArgs& a, hipStream_t st, int phases, const ScheduleArgs* fused) {
  const size_t lds = sizeof(int) * (3 * (size_t)a.B + 1);
  const int grid = compute_units();
  if (phases & kPhaseStream) {
    if (fused)
      hipLaunchKernelGGL((k_stream_rows<DT, VEC, true>), dim3((unsigned)grid), dim3(kStreamBlock),
                         lds, st, a, *fused);
    else
      hipLaunchKernelGGL((k_stream_rows<DT, VEC, false>), dim3((unsigned)grid),
                         dim3(kStreamBlock), lds, st, a, ScheduleArgs{});
  }
  if (phases & kPhaseFinish) {
    a.groups = (a.G + kChunksPerGroup - 1) / kChunksPerGroup;
    hipLaunchKernelGGL((k_decide<DT, VEC>), dim3((unsigned)((long)a.B * a.groups)),
                       dim3(kDecideBlock), 0, st, a);
    if (!a.greedy_only)
      hipLaunchKernelGGL((k_draw<DT, VEC>), dim3((unsigned)a.B), dim3(kBlock), 0, st, a);
  }
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_LAUNCH;
}

int launch_verify(VerifyArgs& a, int dtype, hipStream_t st, int phases,
                  const ScheduleArgs* fused) {
  if (fused && (a.B > kStreamBlock || a.K > kFusedMaxK || a.B * a.K > kSchedLds))
    return DSPARK_ERR_SHAPE;
  if (dtype == DSPARK_BF16)
    return a.vec_ok ? launch_verify_t<DSPARK_BF16, true>(a, st, phases, fused)
                    : launch_verify_t<DSPARK_BF16, false>(a, st, phases, fused);
  return a.vec_ok ? launch_verify_t<DSPARK_F32, true>(a, st, phases, fused)
                  : launch_verify_t<DSPARK_F32, false>(a, st, phases, fused);
}

}  // namespace dspark
