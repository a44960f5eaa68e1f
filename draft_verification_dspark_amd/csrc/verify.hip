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
// Two launches on the caller's stream, shapes fixed by (B, K, V):
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
//                  first tile loads are in flight).  It also clears the
//                  requests' tags in the sync block for the next launch.
//   k_finish       persistent, one workgroup per compute unit.  Phase 1: a
//                  workgroup per request merges the row summaries (shifts
//                  align by exact powers of two), and wave 0 forms p(y),
//                  q(y), alpha, the accept ballot and the first rejection,
//                  writes the outputs and publishes the draw state.  Phase 2:
//                  the residual max(0, p - q) of every rejected row pair,
//                  split into quarter chunks over all waves of the grid (fp32
//                  with the difference carried exactly, elements with
//                  normalised mass >= 2^-12 in fp64); the wave that completes
//                  a request draws its correction token.  Bonus tokens (full
//                  acceptance) are drawn by the deciding workgroup's wave 0.
//                  Draws locate the chunk (or quarter) holding the target
//                  mass, re-read it with each lane owning a contiguous run of
//                  tokens, and scan the crossing lane's run a token per lane.
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

// Threads of a streaming workgroup: one workgroup per compute unit, 8 waves
// (two per SIMD; measured faster than 12 waves: 21.8 against 23.9 us as
// configured, each wave taking more tiles behind its first).
#ifndef DSPARK_STREAM_BLOCK
#define DSPARK_STREAM_BLOCK 512
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

// The plan when the fused schedule has already taken the prefix of the
// requests' tile counts at its own barrier (one request per thread): the
// same layout as build_plan, with one barrier fewer.
__device__ __forceinline__ void build_plan_known(const VerifyArgs& a, int* start, int* info,
                                                 float* cval, ReqInfo pre, const PlanPrefix& pp) {
  const int b = threadIdx.x;
  if (b < a.B) {
    info[b] = pre.L | (pre.kind << 8);
    cval[b] = pre.c;
    start[b] = a.B * a.G + pp.off;
  }
  if (b == kStreamBlock - 1) start[a.B] = a.B * a.G + pp.total;
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
// all paths; status bits travel in the record and are reported by k_finish.
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
// status) of the requests b with b % n == g, which the later launches read,
// after its streaming loop; one workgroup writing them all would start
// streaming last.
// Sync block of the workspace, per request b: line 2b holds the tag (8 bytes)
// and the ReqState (at byte 16), line 2b + 1 the done counter.  The
// streaming pass (of a call with sampled requests; a greedy-only call's
// finish kernel uses none of this) clears every tag and done counter and
// fills every ReqState and quarter record (z, d, q) with kUnset, after its
// streaming loop; the finish kernel then writes a
// request's ReqState and tag, and each quarter's record, without waiting for
// those stores to land: a tag seen set during a finish launch was set by
// that launch, and a reader that finds a kUnset word in a state or record
// that must be there reads it again until the store arrives.  Tag bits: 0
// set, 1 a residual to draw, 8 and up the rejected row (which row pair the
// residual tasks read).
// kUnset: a signalling-NaN pattern that no arithmetic produces and that, as
// a ReqState word, holds a negative mode or count or a NaN shift or sum.
constexpr uint64_t kUnset = 0x7ff4a5a5a5a5a5a5ull;
__device__ __forceinline__ uint64_t make_tag(int mode, int row) {
  return 1ull | ((uint64_t)(mode == kModeResidual) << 1) | ((uint64_t)(uint32_t)row << 8);
}
__device__ __forceinline__ uint64_t* sync_tag(const VerifyArgs& a, int b) {
  return reinterpret_cast<uint64_t*>(a.sync + (size_t)(2 * b) * kSyncLine);
}
__device__ __forceinline__ ReqState* sync_state(const VerifyArgs& a, int b) {
  return reinterpret_cast<ReqState*>(a.sync + (size_t)(2 * b) * kSyncLine + 16);
}
__device__ __forceinline__ uint64_t* sync_done(const VerifyArgs& a, int b) {
  return reinterpret_cast<uint64_t*>(a.sync + (size_t)(2 * b + 1) * kSyncLine);
}

// FUSED: 0 lengths given, 1 schedule inside, 2 schedule inside with each
// request's confidences read as 16-byte pieces (K a multiple of 4, rows
// 16-byte aligned).
template <int DT, bool VEC, int FUSED>
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
      if constexpr (FUSED == 2) {
        const float4* cr = reinterpret_cast<const float4*>(s.conf + (size_t)threadIdx.x * s.K);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = cr[min(q, s.K / 4 - 1)];
          cpre[4 * q] = v.x;
          cpre[4 * q + 1] = v.y;
          cpre[4 * q + 2] = v.z;
          cpre[4 * q + 3] = v.w;
        }
      } else {
        const float* cr = s.conf + (size_t)threadIdx.x * s.K;
#pragma unroll
        for (int i = 0; i < 16; ++i) cpre[i] = cr[min(i, s.K - 1)];
      }
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
  int len = 0;  // FUSED: this thread's request's length, stored after the loop
  PlanPrefix pp;
  if constexpr (FUSED) {
    // the request's tiles after row 0 at length L, as build_plan counts them
    auto tiles_at = [&](int L) -> int {
      if (!mine_req) return 0;
      const ReqInfo r = req_info_lt(a, L, t_raw);
      return (r.kind == kKindSoftmax ? 2 * r.L : (r.kind == kKindGreedy ? r.L : 0)) * a.G;
    };
    // (cpre returns the survival products)
    len = schedule_body<kStreamBlock, 16, true>(s, s.tau, s.budget, g, n, cpre, tiles_at, &pp);
    if (mine_req) mine = req_info_lt(a, len, t_raw);
  } else {
    if (mine_req) mine = req_info_lt(a, l_raw, t_raw);
  }
  // the tile counter, published by the plan's closing barrier
  if (threadIdx.x == 0) s_next = kStreamWaves;
  // (pp.off is the same sign in every thread: whether the budget binds)
  if (FUSED && pp.off >= 0)
    build_plan_known(a, start, info, cval, mine, pp);
  else
    build_plan(a, start, info, cval, one_each, mine);
  const int total = uniform(start[a.B]);
  const int end = uniform((total - g + n - 1) / n);  // tiles of this workgroup
  // next tile index for this wave (one LDS atomic by lane 0)
  auto grab = [&]() -> int {
    int x = 0;
    if (lane_id() == 0) x = atomicAdd(&s_next, 1);
    return uniform(readlane(x, 0));
  };
  if (t0 < end) {
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
  // Stores once nothing more is loaded (stores and loads share one in-order
  // counter): the schedule's outputs of this workgroup's requests, and the
  // finish kernel's sync block and records reset for its launch (a greedy-only
  // call's finish kernel uses neither).
  if constexpr (FUSED) schedule_store_own(s, g, n, len, cpre);
  if (a.greedy_only) return;
  for (int b = g * kStreamBlock + (int)threadIdx.x; b < a.B; b += n * kStreamBlock) {
    *sync_tag(a, b) = 0;
    *sync_done(a, b) = 0;
    uint64_t* st = reinterpret_cast<uint64_t*>(sync_state(a, b));
#pragma unroll
    for (int i = 0; i < (int)(sizeof(ReqState) / 8); ++i) st[i] = kUnset;
  }
  for (long long i = (long long)g * kStreamBlock + threadIdx.x; i < (long long)a.B * a.QT;
       i += (long long)n * kStreamBlock) {
    uint64_t* r = reinterpret_cast<uint64_t*>(a.part2 + i);
    r[0] = kUnset;
    r[1] = kUnset;
    r[2] = kUnset;
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
// from the exponentials above.  Elements whose p or q reaches 2^-12, and
// elements with a -inf logit on either side, are redone in fp64 with the
// same formula.  c is log2(e)/T to fp64 precision.
//
// The streaming pass's St'/Sd' is accurate to about 1e-7, and its error
// would move every d by a multiple of e2; divided by a small residual mass
// that would show in the draw.  The pass over the rejected pair therefore
// also sums, per chunk, D = sum d and Q = sum of e2 over the elements with
// d > 0: the exact ratio of the two rows' sums is rho * St'/Sd' with
// rho - 1 = (sum D)/(sum e2), formed from accurately computed differences
// (sum e2 is St' to within the ~1e-7 of the ratio itself, which changes
// rho - 1 only at second order), and the residual at the exact ratio is
// max(0, d - (rho - 1) e2), whose chunk mass is Z - (rho - 1) Q to first
// order (elements that change sign contribute at second order).
struct ResidualRows {
  float chi, clo, nkt, nd0hi, nd0lo;
  uint32_t hbits;  // bits of St' 2^-12: p or q >= 2^-12  <=>  e1 or e2 >= it
  double c64, kt64, d0;
  __device__ ResidualRows(float c_, float clo_, float kt_, double st, float kd_, double sd)
      : chi(c_), clo(clo_) {
    c64 = (double)c_ + (double)clo_;
    kt64 = (double)kt_;
    d0 = (double)kt_ - (double)kd_ + (log2(st) - log2(sd));
    nkt = -kt_;
    nd0hi = (float)(-d0);
    nd0lo = (float)(-d0 - (double)nd0hi);
    hbits = __float_as_uint((float)(st * 0x1p-12));
  }
  // fp32 path: d and e2 of one element; `heavy` reports an element to redo
  // with exact(): p or q at least 2^-12, or an undefined exponential (a
  // logit of -inf on either side makes x*chi + x*clo or x1 - g an inf - inf;
  // the one such case left defined, a -inf draft logit with clo > 0, gives
  // e2 = 0 and the right d = e1).  d and e2 of a heavy element are not used.
  __device__ __forceinline__ float fast(float xt, float xd, float& e2, bool& heavy) const {
    const float dx = xt - xd;
    const float g = fmaf(dx, chi, nd0hi) + fmaf(dx, clo, nd0lo);
    const float x1 = fmaf(xt, clo, fmaf(xt, chi, nkt));
    const float x2 = x1 - g;
    const float e1 = fast_exp2(x1);
    e2 = fast_exp2(x2);
    // e1, e2 are >= 0 or NaN: as unsigned bit patterns they order as numbers,
    // with every NaN (of either sign) above +inf, so one unsigned max and min
    // give the larger and smaller value and the heavy test together
    const uint32_t b1 = __float_as_uint(e1), b2 = __float_as_uint(e2);
    const uint32_t bb = b1 > b2 ? b1 : b2, bs = b1 > b2 ? b2 : b1;
    heavy = bb >= hbits;
    const float big = __uint_as_float(bb), small = __uint_as_float(bs);
    // 1 - 2^-|g| = z f(z), z = |g| ln 2 < 0.7, f(z) = (1 - e^-z)/z, with f a
    // degree-5 polynomial fitted to it on [0, ln 2] for least maximum
    // relative error (1.1e-8); its k-th coefficient times (ln 2)^(k+1),
    // rounded to fp32, gives P with 1 - 2^-a = a P(a) (1.4e-8 relative, below
    // fp32 rounding), one multiplication fewer per element
    const float ag = fabsf(g);
    float t = -0.000115207164f;
    t = fmaf(t, ag, 0.00129251310f);
    t = fmaf(t, ag, -0.00959801860f);
    t = fmaf(t, ag, 0.0554997176f);
    t = fmaf(t, ag, -0.240226194f);
    t = fmaf(t, ag, 0.693147182f);
    float series = big * (ag * t);
    // both sides computed: a select, not a branch (the lanes of a wave take
    // both sides anyway)
    asm volatile("" : "+v"(series));
    const float ad = ag >= 1.f ? big - small : series;
    return copysignf(ad, g);
  }
  // fp64 path, same formula (1 - 2^-|g| from expm1, so that a small |g|
  // keeps its relative precision against the exponentials' own error).
  // x2 = xd c - kt + d0 is formed from the draft logit itself, so that a
  // -inf logit on either side gives a zero exponential and d = e1 - e2
  // (an infinite or undefined g takes that branch).
  __device__ __forceinline__ double exact(float xt, float xd, double& e2) const {
    const double x1 = (double)xt * c64 - kt64;
    const double x2 = (double)xd * c64 - (kt64 - d0);
    const double g = ((double)xt - (double)xd) * c64 - d0;
    const double e1 = exp2_f64(x1);
    e2 = exp2_f64(x2);
    const double ag = fabs(g);
    if (!(ag < 1.0)) return e1 - e2;
    const double ad = (g >= 0.0 ? e1 : e2) * -expm1(-ag * 0.69314718055994530942);
    return g >= 0.0 ? ad : -ad;
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

// Token i = lane of lane h's run (the raw words broadcast from lane h, h
// wave-uniform), for the first NV * kPerVec lanes; -inf on the others.  Lets
// the whole wave take one lane's run a token per lane.
template <int DT, int NV>
__device__ __forceinline__ float lane_run_elem(const LaneRun<DT, NV>& run, int h) {
  constexpr int R = NV * Elem<DT>::kPerVec;
  const int i = lane_id();
  const int word = DT == DSPARK_BF16 ? (i >> 1) : i;
  uint32_t x = 0;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t sw = (uint32_t)__builtin_amdgcn_readlane((int)run.w[v][q], h);
      if (word == v * 4 + q) x = sw;
    }
  float f;
  if constexpr (DT == DSPARK_BF16)
    f = (i & 1) ? __uint_as_float(x & 0xffff0000u) : __uint_as_float(x << 16);
  else
    f = __uint_as_float(x);
  return i < R ? f : -INFINITY;
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
template <int DT, int U>
__device__ ResidualChunk residual_sums(const ResidualRows& rr, const TileN<DT, U>& tt,
                                       const TileN<DT, U>& td) {
  constexpr int P = Elem<DT>::kPerVec;
  float lz = 0.f, ld = 0.f, lq = 0.f;
  double hz = 0.0, hd = 0.0, hq = 0.0;
#pragma unroll
  for (int v = 0; v < U; ++v) {
    uint32_t hm = 0;  // this lane's heavy elements of vector v
    float sz = 0.f, sd = 0.f, sq = 0.f;
#pragma unroll
    for (int e = 0; e < P; ++e) {
      bool h;
      float e2;
      const float d = rr.fast(tt.at(v, e), td.at(v, e), e2, h);
      hm |= h ? 1u << e : 0u;
      // heavy elements stay out of the fp32 sums (their value would dominate
      // the partial sum's rounding, or is not defined) and are added in fp64
      // below
      const bool pos = !h && d > 0.f;
      sz += pos ? d : 0.f;
      sd += h ? 0.f : d;
      sq += pos ? e2 : 0.f;
    }
    const bool ok = tt.valid(v);
    lz += ok ? sz : 0.f;
    ld += ok ? sd : 0.f;
    lq += ok ? sq : 0.f;
    if (!ok) hm = 0;
    if (hm) {
      // each lane walks its own heavy elements (usually one) in fp64
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
      }
    }
    asm volatile("" : "+v"(lz), "+v"(ld), "+v"(lq));
  }
  ResidualChunk c;
  c.z = wave_sum((double)lz + hz);
  c.d = wave_sum((double)ld + hd);
  c.q = wave_sum((double)lq + hq);
  c.e2 = 0.0;
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

// ------------------------------------------------------------------ finish

// k_finish: the decision, the residual and the draw of every request, in one
// persistent launch of one workgroup per compute unit (kFinishBlock threads,
// 8 waves), after the streaming pass.
//   Phase 1  workgroup g decides requests g, g + n, ... (n workgroups): it
//            stages the request's chunk summaries in LDS, merges its rows
//            (16-lane groups, one row each), and wave 0 forms p(y), q(y),
//            alpha, the accept ballot and the first rejection and writes the
//            outputs.  Greedy requests are then complete; after a full
//            acceptance wave 0 draws the bonus token itself; after a
//            rejection it publishes the draw state (ReqState) and sets the
//            request's tag.
//   Phase 2  the residual of every rejected request is split into quarter
//            chunks (a quarter of a chunk each, QT per request, none past
//            the row's end); the grid's W waves take runs of consecutive
//            tasks.  A task sums its quarter (d, D, Q; see ResidualRows) and
//            counts itself done on the request's counter.  The wave that
//            completes the request draws the correction token.
// Cross-workgroup hand-over goes through the sync block of the workspace:
// per request a tag line (tag, ReqState) and a counter line, each on its own
// 128-byte line (atomics on a shared line serialise).  Stores that another
// workgroup reads are agent-scope atomic stores, completed (waitcnt) before
// the store or atomic that publishes them; readers use agent-scope atomic
// loads issued after they saw the publication.  Waits poll with
// s_sleep and give up after kSpinLimit ticks of the 100 MHz real-time
// counter (DSPARK_DEV_INCOMPLETE), so every wave ends.
// The waits need every workgroup of the launch resident at once (one per
// compute unit, which the register and LDS use allow): a workgroup that
// cannot start until a waiting one ends leaves its requests undecided, and
// the waits on them end by time-out.
constexpr int kFinishBlock = 512;
constexpr int kFinishWaves = kFinishBlock / kWave;
constexpr int kMaxRows = 2 * 64 + 1;
// chunk summaries staged in LDS per round of the merges (24 KB)
constexpr int kStage = 3 * kFinishBlock;
constexpr uint64_t kSpinLimit = 100000000ull;  // 1 s at 100 MHz
constexpr int kTaskBatch = 3;  // most quarter tasks a wave has in flight at once

// A full acceptance's bonus draw, deferred by wave 0 (at most kMaxPending
// per workgroup; more are drawn at once)
struct PendingBonus {
  int b, L;
  float c, kp;
  double u;
  Located loc;
};
constexpr int kMaxPending = 16;


__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// a record of 8-byte words moved with agent-scope atomic stores / loads
template <typename T> __device__ __forceinline__ void st_rec(T* dst, const T& v) {
  static_assert(sizeof(T) % 8 == 0, "8-byte words");
  const uint64_t* s = reinterpret_cast<const uint64_t*>(&v);
  uint64_t* d = reinterpret_cast<uint64_t*>(dst);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 8); ++i) st_agent(d + i, s[i]);
}
template <typename T> __device__ __forceinline__ T ld_rec(const T* src) {
  T v;
  uint64_t* d = reinterpret_cast<uint64_t*>(&v);
  const uint64_t* s = reinterpret_cast<const uint64_t*>(src);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 8); ++i) d[i] = ld_agent(s + i);
  return v;
}

constexpr int kStateWords = sizeof(ReqState) / 8;
constexpr int kRecWords = 3;  // z, d, q of a ResidualChunk
// whether every one of the first `words` 8-byte words of v has arrived (none
// is kUnset)
template <typename T> __device__ __forceinline__ bool rec_set(const T& v, int words) {
  const uint64_t* w = reinterpret_cast<const uint64_t*>(&v);
  bool ok = true;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 8); ++i)
    if (i < words) ok = ok && w[i] != kUnset;
  return ok;
}
// Read a record that another wave has written (or is writing) until every
// one of its first `words` words has arrived; false (and the last read) on
// time-out.
template <typename T> __device__ bool ld_rec_set(const T* src, T& v, int words) {
  v = ld_rec(src);
  if (rec_set(v, words)) return true;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  do {
    __builtin_amdgcn_s_sleep(2);
    v = ld_rec(src);
    if (rec_set(v, words)) return true;
  } while (__builtin_amdgcn_s_memrealtime() - t0 <= kSpinLimit);
  return false;
}

// Inverse CDF over n weights f(0..n-1) by one wave, in index order, in
// rounds of 64 (same rule as wave_locate): the index and the mass before it.
template <typename F>
__device__ Located wave_locate_rounds(F f, int n, double u) {
  const int l = lane_id();
  double part = 0.0;
  for (int i = l; i < n; i += kWave) part += f(i);
  const double total = wave_sum(part);
  const double target = u * total;
  double run = 0.0;
  int last = -1;
  for (int r0 = 0; r0 < n; r0 += kWave) {
    const int i = r0 + l;
    const double x = i < n ? f(i) : 0.0;
    const double incl = run + wave_incl_scan(x);
    const uint64_t hit = __ballot(incl > target && x > 0.0);
    const uint64_t pos = __ballot(x > 0.0);
    if (pos) last = r0 + 63 - __builtin_clzll(pos);
    if (hit) {
      const int h = __builtin_ctzll(hit);
      Located r;
      r.idx = r0 + h;
      r.past_end = 0;
      r.base = readlane(incl - x, h);
      r.total = total;
      return r;
    }
    run = readlane(incl, kWave - 1);
  }
  Located r;
  r.idx = last;
  r.past_end = 1;
  r.base = total;
  r.total = total;
  return r;
}

// Inside runs of tokens laid out R per lane in token order (LaneRun), the
// first token whose running mass exceeds `target`, else the last with mass,
// else 0.  One wave: each lane sums its run, a wave scan finds the lane h
// holding the crossing, then lane h's run is taken a token per lane and
// scanned again.  mass(x) is the mass of a token of value x (0 for -inf).
template <int DT, int NV, typename M>
__device__ int wave_scan_runs(const LaneRun<DT, NV>& run, M mass, double target) {
  constexpr int R = NV * Elem<DT>::kPerVec;
  const int l = lane_id();
  double ls = 0.0;
  int lp = -1;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const double x = mass(run.at(i));
    ls += x;
    if (x > 0.0) lp = l * R + i;
    // keep each group of 8 masses in place (no hoisting of every
    // exponential ahead of the sum, which would not fit in registers)
    if ((i & 7) == 7) asm volatile("" : "+v"(ls), "+v"(lp));
  }
  const double incl = wave_incl_scan(ls);
  const int last = wave_max_i(lp);
  const uint64_t hit = __ballot(incl > target && ls > 0.0);
  if (!hit) return last >= 0 ? last : 0;
  const int h = __builtin_ctzll(hit);
  const double x = mass(lane_run_elem<DT, NV>(run, h));  // 0 past the run
  const double sc = wave_incl_scan(x);
  const double base = readlane(incl - ls, h);
  const uint64_t hit2 = __ballot(base + sc > target && x > 0.0);
  // rounding can leave no crossing inside lane h's run: its last token with mass
  return hit2 ? h * R + __builtin_ctzll(hit2) : readlane(lp, h);
}

// Draw from the softmax of target row `row` (the bonus token, or the
// fallback of an all-zero residual), by one wave: chunk masses from the
// row's pass-1 summaries scaled to the merged shift kp, then the chosen
// chunk re-read as four quarters (each lane a run of consecutive tokens of
// each) with the pass's own fp32 arithmetic: the quarter holding the target,
// then the token inside it.  `loc` may hold the chunk already located from
// staged summaries.
template <int DT, bool VEC>
__device__ int draw_from_row(const VerifyArgs& a, int b, int row, float c, float kp, double u,
                             Located loc) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int E = item_elems<DT>();
  constexpr int EQ = E / 4;
  constexpr int R = EQ / kWave;
  constexpr int NV = R / Elem<DT>::kPerVec;
  const Partial* pr = row_parts(a, b, row, 0);
  auto chunk_mass = [&](int ci) -> double {
    const Partial p = pr[ci];
    return p.s > 0.0 ? ldexp(p.s, shift_amount(p.k - kp)) : 0.0;
  };
  if (loc.idx < 0) loc = wave_locate_rounds(chunk_mass, a.G, u);
  if (loc.idx < 0) return 0;
  const int e0 = loc.idx * E;
  const int n = min(E, a.V - e0);
  const char* base = target_row(a, b, row, S) + (size_t)e0 * S;
  LaneRun<DT, NV> qr[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    qr[k].template load<VEC>(base + (size_t)k * EQ * S, max(0, min(EQ, n - k * EQ)), lane_id());
  const float kc = pr[loc.idx].k;
  const int sh_c = shift_amount(kc - kp);
  double qs[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    double ls = 0.0;
#pragma unroll
    for (int i = 0; i < R; ++i) ls += ldexp((double)fast_exp2(fmaf(qr[k].at(i), c, -kc)), sh_c);
    qs[k] = wave_sum(ls);
  }
  // the quarter holding the target (else the last with mass)
  const double target = loc.past_end ? INFINITY : u * loc.total - loc.base;
  double before = 0.0;
  int kq = -1, klast = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (qs[k] > 0.0) klast = k;
    if (kq < 0 && before + qs[k] > target && qs[k] > 0.0) kq = k;
    if (kq < 0) before += qs[k];
  }
  const bool past = kq < 0;
  if (past) kq = klast;
  LaneRun<DT, NV> run = qr[0];
#pragma unroll
  for (int k = 1; k < 4; ++k)
    if (kq == k) run = qr[k];
  return e0 + kq * EQ +
         wave_scan_runs<DT, NV>(
             run,
             [&](float x) -> double { return ldexp((double)fast_exp2(fmaf(x, c, -kc)), sh_c); },
             past ? INFINITY : target - before);
}

// Quarter records of a request held in registers, kRecLanes per lane (quarter
// q = lane + 64 k): read in one batch of loads, so that the sums and the
// locate below cost one memory round trip.  Requests with more quarters
// (V above 64 k * kRecLanes / 4 * 4096 tokens) read them in rounds instead.
constexpr int kRecLanes = 4;

// The correction token of a rejected request, by one wave: quarter masses
// corrected to the exact ratio of the row sums, the quarter holding u * Z,
// then its 4096/4 tokens recomputed (each lane a run of consecutive tokens).
template <int DT, bool VEC>
__device__ int draw_residual(const VerifyArgs& a, int b, double u, int& tok_pos) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int E = item_elems<DT>();
  constexpr int EQ = E / 4;          // tokens per quarter
  constexpr int R = EQ / kWave;      // per lane
  constexpr int NV = R / Elem<DT>::kPerVec;
  const ResidualChunk* zq = a.part2 + (size_t)b * a.QT;
  const int l = lane_id();
  Located loc;
  double rm1;
  // the draw state, loaded with the quarter records below
  const ReqState st = ld_rec(sync_state(a, b));
  tok_pos = st.a;
  if (a.QT <= kWave * kRecLanes) {
    double z[kRecLanes], d[kRecLanes], q[kRecLanes];
    auto load = [&]() -> bool {
      bool ok = true;
#pragma unroll
      for (int k = 0; k < kRecLanes; ++k) {
        const int i = l + kWave * k;
        const uint64_t* p = reinterpret_cast<const uint64_t*>(zq + (i < a.QT ? i : 0));
        const uint64_t wz = ld_agent(p + 0), wd = ld_agent(p + 1), wq = ld_agent(p + 2);
        ok = ok && wz != kUnset && wd != kUnset && wq != kUnset;
        z[k] = __longlong_as_double((long long)wz);
        d[k] = __longlong_as_double((long long)wd);
        q[k] = __longlong_as_double((long long)wq);
      }
      return ok;
    };
    // records counted before their stores landed are read again
    if (__ballot(!load())) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      bool ok;
      do {
        __builtin_amdgcn_s_sleep(2);
        ok = !__ballot(!load());
      } while (!ok && __builtin_amdgcn_s_memrealtime() - t0 <= kSpinLimit);
      if (!ok && l == 0) flag(a.dev_status, DSPARK_DEV_INCOMPLETE);
    }
    // rho - 1 from the signed differences over sum e2 = St' (see ResidualRows)
    double pd = 0.0;
#pragma unroll
    for (int k = 0; k < kRecLanes; ++k) pd += l + kWave * k < a.QT ? d[k] : 0.0;
    const double sd = wave_sum(pd);
    rm1 = st.st > 0.0 ? sd / st.st : 0.0;
    double m[kRecLanes], part = 0.0;
#pragma unroll
    for (int k = 0; k < kRecLanes; ++k) {
      m[k] = l + kWave * k < a.QT ? fmax(z[k] - rm1 * q[k], 0.0) : 0.0;
      part += m[k];
    }
    // inverse CDF in quarter order, as wave_locate_rounds does
    const double total = wave_sum(part);
    const double target = u * total;
    double run = 0.0;
    int last = -1;
    loc = Located{-1, 1, total, total};
#pragma unroll
    for (int k = 0; k < kRecLanes; ++k) {
      const double incl = run + wave_incl_scan(m[k]);
      const uint64_t hit = __ballot(incl > target && m[k] > 0.0);
      const uint64_t pos = __ballot(m[k] > 0.0);
      if (pos) last = kWave * k + 63 - __builtin_clzll(pos);
      if (hit && loc.past_end) {
        const int h = __builtin_ctzll(hit);
        loc = Located{kWave * k + h, 0, readlane(incl - m[k], h), total};
      }
      run = readlane(incl, kWave - 1);
    }
    if (loc.past_end) loc.idx = last;
  } else {
    // every record arrived (read until it has) before the two passes below
    bool ok = true;
    for (int i = l; i < a.QT; i += kWave) {
      ResidualChunk c;
      ok = ld_rec_set(zq + i, c, kRecWords) && ok;
    }
    if (!ok) flag(a.dev_status, DSPARK_DEV_INCOMPLETE);
    auto rd = [&](int i) -> ResidualChunk { return ld_rec(zq + i); };
    double pd = 0.0;
    for (int i = l; i < a.QT; i += kWave) pd += rd(i).d;
    const double sd = wave_sum(pd);
    rm1 = st.st > 0.0 ? sd / st.st : 0.0;
    loc = wave_locate_rounds(
        [&](int i) -> double {
          const ResidualChunk c = rd(i);
          return fmax(c.z - rm1 * c.q, 0.0);
        },
        a.QT, u);
  }
  if (!(loc.total > 0.0) || loc.idx < 0)
    return draw_from_row<DT, VEC>(a, b, st.row, st.c, st.kt, u, Located{-1, 0, 0.0, 0.0});
  const ResidualRows rr(st.c, st.clo, st.kt, st.st, st.kd, st.sd);
  const int e0 = loc.idx * EQ;
  const int n = min(EQ, a.V - e0);
  LaneRun<DT, NV> rt, rdr;
  rt.template load<VEC>(target_row(a, b, st.row, S) + (size_t)e0 * S, n, lane_id());
  rdr.template load<VEC>(draft_row(a, b, st.row, S) + (size_t)e0 * S, n, lane_id());
  // the residual at the corrected ratio, max(0, d - (rho - 1) e2): the fp32
  // form, and for an element whose p or q reaches 2^-12 the fp64 one, taken
  // in a rolled loop over those few elements (one copy of the fp64 code)
  auto mass = [&](float xt, float xd, bool& h) -> double {
    float e2f;
    const float d = rr.fast(xt, xd, e2f, h);
    return fmax((double)d - rm1 * (double)e2f, 0.0);
  };
  auto exact_mass = [&](float xt, float xd) -> double {
    double e2;
    const double dx = rr.exact(xt, xd, e2);
    return fmax(dx - rm1 * e2, 0.0);
  };
  double ls = 0.0;
  int lp = -1;
  uint32_t heavy = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    bool h;
    const double x = mass(rt.at(i), rdr.at(i), h);
    heavy |= h ? 1u << i : 0u;
    ls += h ? 0.0 : x;
    if (!h && x > 0.0) lp = l * R + i;
  }
  for (uint32_t hm = heavy; hm; hm &= hm - 1) {
    const int i = __builtin_ctz(hm);
    const double x = exact_mass(run_elem<DT, NV>(rt.w, i), run_elem<DT, NV>(rdr.w, i));
    ls += x;
    if (x > 0.0) lp = max(lp, l * R + i);
  }
  const double target = loc.past_end ? INFINITY : u * loc.total - loc.base;
  const double incl = wave_incl_scan(ls);
  const int last = wave_max_i(lp);
  const uint64_t hit = __ballot(incl > target && ls > 0.0);
  int f = last;
  if (hit) {
    // lane h holds the crossing: its run a token per lane, scanned again with
    // the same per-token arithmetic (fp64 for the heavy ones)
    const int h = __builtin_ctzll(hit);
    const float xt = lane_run_elem<DT, NV>(rt, h), xd = lane_run_elem<DT, NV>(rdr, h);
    double x = 0.0;
    if (l < R) {
      bool hh;
      x = mass(xt, xd, hh);
      if (hh) x = exact_mass(xt, xd);
    }
    const double sc = wave_incl_scan(x);
    const double base = readlane(incl - ls, h);
    const uint64_t hit2 = __ballot(base + sc > target && x > 0.0);
    // rounding can leave no crossing inside lane h's run: its last token with mass
    f = hit2 ? h * R + __builtin_ctzll(hit2) : readlane(lp, h);
  }
  return e0 + (f >= 0 ? f : 0);
}

// Phase 1 for request b by the whole workgroup (every thread must call it).
template <int DT, bool VEC>
__device__ void decide_request(const VerifyArgs& a, int b, RowSum* s_rows, Partial* s_part,
                               PendingBonus* s_pend, int& npend) {
  constexpr int S = Elem<DT>::kBytes;
  const int w = uniform((int)(threadIdx.x / kWave));
  const int l = lane_id();
  const int K = a.K;
  // Requested together, before anything waits: the request's length and
  // temperature, the final uniform and, for wave 0 lane l, the drafted id
  // and accept uniform of position l+1 (lanes past K re-read column K-1).
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

  if (r.kind == kKindSkip) {
    if (w == 0) {
      for (int i = l; i <= K; i += kWave) tok[i] = -1;
      if (l < K) {
        if (a.p_tok) a.p_tok[(size_t)b * K + l] = 0.f;
        if (a.q_tok) a.q_tok[(size_t)b * K + l] = 0.f;
      }
      if (l == 0) {
        a.accepted[b] = 0;
        flag(a.dev_status, r.bad);
      }
    }
    return;
  }
  const bool soft = r.kind == kKindSoftmax;

  // The drafted tokens' logits, gathered with the first staged summaries so
  // that one round trip covers both.  Lanes past L (and bad ids) read a
  // scheduled row at id 0 and ignore it.
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
    const int per_round = kStage / G;
    const int grp = threadIdx.x >> 4, sub = threadIdx.x & 15;
    for (int q0 = 0; q0 < nrows; q0 += per_round) {
      const int nr = min(per_round, nrows - q0);
      const int cnt = nr * G;
      q_last = q0;
      if (q0 > 0) __syncthreads();  // the previous round's merges are done
      constexpr int kPer = kStage / kFinishBlock;
      Partial tmp[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = k * kFinishBlock + (int)threadIdx.x;
        const int ii = i < cnt ? i : 0;
        const int rr = ii / G;
        int side;
        const int j = row_of(q0 + rr, side);
        tmp[k] = row_parts(a, b, j, side)[ii - rr * G];
      }
      xt_raw = load_raw<DT>(trow, yc);  // (re-gathered in later rounds)
      xd_raw = load_raw<DT>(drow, yc);
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        asm volatile("" : "+v"(tmp[k].k), "+v"(tmp[k].idx), "+v"(tmp[k].s));
      asm volatile("" : "+v"(xt_raw), "+v"(xd_raw));
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = k * kFinishBlock + (int)threadIdx.x;
        if (i < cnt) s_part[i] = tmp[k];
      }
      __syncthreads();
      for (int rr = grp; rr < nr; rr += kFinishBlock / 16) {
        const RowSum m = soft ? merge_softmax16(s_part + rr * G, G, sub)
                              : merge_argmax16(s_part + rr * G, G, sub);
        if (sub == 0) s_rows[q0 + rr] = m;
      }
    }
  } else {
    // very long rows: waves merge whole rows straight from global memory
    xt_raw = load_raw<DT>(trow, yc);
    xd_raw = load_raw<DT>(drow, yc);
    for (int q = w; q < nrows; q += kFinishWaves) {
      int side;
      const int j = row_of(q, side);
      const Partial* base = row_parts(a, b, j, side);
      const Partial first = l < G ? base[l] : Partial{-INFINITY, 0x7fffffff, 0.0};
      const RowSum m = soft ? merge_softmax(first, base, G) : merge_argmax(first, base, G);
      if (l == 0) s_rows[q] = m;
    }
  }
  __syncthreads();
  if (w != 0) return;  // wave 0 decides; the others move on
  const float xt = raw_to_float<DT>(xt_raw), xd = raw_to_float<DT>(xd_raw);
  const RowSum rL = s_rows[qL];  // target row L: the bonus row
  RowSum rt{}, rd{};
  if (l < L) {
    rt = s_rows[l];
    if (soft) rd = s_rows[L + l];
  }
  int bad = r.bad;
  if (!yok) bad |= DSPARK_DEV_BAD_TOKEN;
  if (l < L) bad |= rt.bad | rd.bad;
  if (l == 0) bad |= rL.bad;
  bool acc = false;
  float pf = 0.f, qf = 0.f;
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
  const int an = rej ? __builtin_ctzll(rej) : L;
  bad = wave_or(bad);
  const bool fault = (bad & (DSPARK_DEV_BAD_TOKEN | DSPARK_DEV_NONFINITE)) != 0;
  int gtok = 0;
  if (!soft) gtok = an < L ? readlane(rt.idx, an) : rL.idx;
  // outputs: the accepted prefix, p(y) and q(y), and (greedy) the last token
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
  }
  if (!soft) return;  // greedy done
  // the draw state for the residual tasks, which wait for every sampled
  // request with L > 0: kModeNone releases them when there is no residual
  // (a full acceptance, or a faulty request, whose tokens are unspecified)
  ReqState st{};
  st.mode = kModeNone;
  if (!fault && an < L) {
    st.mode = kModeResidual;
    st.row = an;
    st.a = an;
    st.c = r.c;
    st.clo = r.clo;
    st.kt = readlane(rt.k, an);
    st.st = readlane(rt.s, an);
    st.kd = readlane(rd.k, an);
    st.sd = readlane(rd.s, an);
  }
  if (l == 0) {
    // the tag may land before the state: the tasks read the state until
    // it has arrived (no kUnset word)
    st_rec(sync_state(a, b), st);
    st_agent(sync_tag(a, b), make_tag(st.mode, st.row));
  }
  if (fault) return;
  if (an == L) {
    // full acceptance: the bonus token from target row L, its chunk located
    // from the staged summaries when they are all there
    Located bonus{-1, 0, 0.0, 0.0};
    if (G <= kWave && G <= kStage) {
      const Partial pc = l < G ? s_part[(qL - q_last) * G + l] : Partial{-INFINITY, 0, 0.0};
      const double mass = l < G && pc.s > 0.0 ? ldexp(pc.s, shift_amount(pc.k - rL.k)) : 0.0;
      bonus = wave_locate(mass, (double)u_draw);
    }
    if (npend < kMaxPending) {
      // drawn after this wave's residual tasks (the draw's memory round trips
      // would otherwise hold the whole workgroup back from them)
      if (l == 0) s_pend[npend] = PendingBonus{b, L, r.c, rL.k, (double)u_draw, bonus};
      ++npend;
      return;
    }
    const int t = draw_from_row<DT, VEC>(a, b, L, r.c, rL.k, (double)u_draw, bonus);
    if (l == 0) tok[L] = t;
  }
}

// The requests with a residual to draw, by one wave: every sampled request
// with L > 0 has its tag set in phase 1 (lane l polls request b0 + l, 64 at
// a time, bounded by kSpinLimit); those whose tag says residual go to s_live
// in request order as (request | row << 16).  A tag not set in time flags
// DSPARK_DEV_INCOMPLETE in `bad` and leaves the request out.
__device__ int live_requests(const VerifyArgs& a, int* s_live, int& bad) {
  int nlive = 0;
  for (int b0 = 0; b0 < a.B; b0 += kWave) {
    const int b = b0 + lane_id();
    bool want = false;
    if (b < a.B) {
      const ReqInfo r = req_info(a, b);
      want = r.kind == kKindSoftmax && r.L > 0;
    }
    uint64_t tag = 0;
    int ok = 1;
    if (want) {
      const uint64_t* p = sync_tag(a, b);
      const uint64_t ts = __builtin_amdgcn_s_memrealtime();
      while (!((tag = ld_agent(p)) & 1ull)) {
        __builtin_amdgcn_s_sleep(2);
        if (__builtin_amdgcn_s_memrealtime() - ts > kSpinLimit) {
          ok = 0;
          break;
        }
      }
    }
    if (!ok) bad |= DSPARK_DEV_INCOMPLETE;
    const bool live = want && ok && ((tag >> 1) & 1ull);
    const uint64_t m = __ballot(live);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    if (live) s_live[nlive + below] = b | ((int)(tag >> 8) << 16);
    nlive += __builtin_popcountll(m);
  }
  return nlive;
}

template <int DT, bool VEC>
__global__ void __launch_bounds__(kFinishBlock) k_finish(VerifyArgs a) {
  constexpr int S = Elem<DT>::kBytes;
  constexpr int E = item_elems<DT>();
  constexpr int EQ = E / 4;
  constexpr int UQ = kUnroll / 4;  // vectors per lane in a quarter task
  __shared__ RowSum s_rows[kMaxRows];
  __shared__ Partial s_part[kStage];
  __shared__ int s_nlive;
  __shared__ PendingBonus s_pend[kMaxPending];
  const int n = gridDim.x, g = blockIdx.x;
  const int w = uniform((int)(threadIdx.x / kWave));
  const int l = lane_id();
  // Phase 1: this workgroup's decisions
  int npend = 0;  // wave 0's deferred bonus draws
  for (int b = g; b < a.B; b += n) {
    decide_request<DT, VEC>(a, b, s_rows, s_part, s_pend, npend);
    __syncthreads();  // LDS reused by the next request
  }
  if (a.greedy_only) return;  // (no bonus draws: greedy requests take the argmax)
  // Phase 2.  Wave 0 lists the requests that have a residual (from their
  // tags) in LDS; their quarter tasks, t = live * QT + quarter, are split
  // over the grid's W waves in W runs of consecutive tasks whose lengths
  // differ by at most one (wave k: tasks k T / W to (k + 1) T / W), so that
  // the sums' arithmetic is spread over every wave and no wave holds back
  // its draws with a second round.  A wave takes its run kTaskBatch tasks
  // at a time: the batch's row tiles and draw states all in flight before
  // the sums; it stores its records and counts itself done without waiting
  // for them to land.
  int* s_live = reinterpret_cast<int*>(s_part);  // free after phase 1
  if (w == 0) {
    int badl = 0;
    const int nl = live_requests(a, s_live, badl);
    if (badl) flag(a.dev_status, badl);
    if (l == 0) s_nlive = nl;
  }
  __syncthreads();
  const int W = n * kFinishWaves;
  const int gw = w * n + g;  // neighbouring tasks on different compute units
  const long long ntask = (long long)s_nlive * a.QT;
  const long long t_end = ntask * (gw + 1) / W;
  for (long long t0 = ntask * gw / W; t0 < t_end; t0 += kTaskBatch) {
    int tb[kTaskBatch], tq[kTaskBatch], trow[kTaskBatch];
    bool live[kTaskBatch];
#pragma unroll
    for (int j = 0; j < kTaskBatch; ++j) {
      const long long t = t0 + j;
      live[j] = t < t_end;
      const int li = live[j] ? (int)(t / a.QT) : 0;
      tq[j] = live[j] ? (int)(t - (long long)li * a.QT) : 0;
      const int e = s_live[li];
      tb[j] = e & 0xffff;
      trow[j] = e >> 16;
    }
    TileN<DT, UQ> tt[kTaskBatch], td[kTaskBatch];
    ReqState sj[kTaskBatch];
#pragma unroll
    for (int j = 0; j < kTaskBatch; ++j) {
      if (!live[j]) continue;
      const int e0 = (tq[j] >> 2) * E;
      const int nn = min(E, a.V - e0);
      const int v0 = (tq[j] & 3) * UQ;
      tt[j].template load<VEC>(target_row(a, tb[j], trow[j], S) + (size_t)e0 * S, nn, v0);
      td[j].template load<VEC>(draft_row(a, tb[j], trow[j], S) + (size_t)e0 * S, nn, v0);
      sj[j] = ld_rec(sync_state(a, tb[j]));
    }
    ResidualChunk zj[kTaskBatch];
#pragma unroll
    for (int j = 0; j < kTaskBatch; ++j) {
      if (!live[j]) continue;
      // a state read before its stores landed is read again (checked task by
      // task, so that task j waits only for its own loads)
      if (!rec_set(sj[j], kStateWords) &&
          !ld_rec_set(sync_state(a, tb[j]), sj[j], kStateWords))
        flag(a.dev_status, DSPARK_DEV_INCOMPLETE);
      const ResidualRows rr(sj[j].c, sj[j].clo, sj[j].kt, sj[j].st, sj[j].kd, sj[j].sd);
      zj[j] = residual_sums<DT, UQ>(rr, tt[j], td[j]);
    }
    int last[kTaskBatch];
#pragma unroll
    for (int j = 0; j < kTaskBatch; ++j) last[j] = 0;
    if (l == 0) {
#pragma unroll
      for (int j = 0; j < kTaskBatch; ++j)
        if (live[j]) st_rec(a.part2 + (size_t)tb[j] * a.QT + tq[j], zj[j]);
      // counted without waiting for the records to land: the drawing wave
      // reads a record until it has arrived
#pragma unroll
      for (int j = 0; j < kTaskBatch; ++j)
        if (live[j]) {
          const uint64_t old = __hip_atomic_fetch_add(sync_done(a, tb[j]), 1ull,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          last[j] = old + 1 == (uint64_t)a.QT;
        }
    }
    // the requests this wave completed: their correction tokens
    int done_mask = 0;
#pragma unroll
    for (int j = 0; j < kTaskBatch; ++j)
      if (live[j] && readlane(last[j], 0)) done_mask |= 1 << j;
    for (int j = 0; j < kTaskBatch; ++j) {
      if (!((done_mask >> j) & 1)) continue;
      const int b = readlane(tb[j], 0);
      const double u = (double)a.uniforms[(size_t)b * (a.K + 1) + a.K];
      int pos;
      const int tk = draw_residual<DT, VEC>(a, b, u, pos);
      if (l == 0) a.tokens[(size_t)b * (a.K + 1) + pos] = tk;
    }
  }
  // wave 0's deferred bonus draws, after its residual tasks
  if (w == 0)
    for (int i = 0; i < npend; ++i) {
      const PendingBonus pb = s_pend[i];
      const int t = draw_from_row<DT, VEC>(a, pb.b, pb.L, pb.c, pb.kp, pb.u, pb.loc);
      if (l == 0) a.tokens[(size_t)pb.b * (a.K + 1) + pb.L] = t;
    }
  (void)EQ;
}

// ------------------------------------------------------------------ launch

template <int DT, bool VEC>
static int launch_verify_t(VerifyArgs& a, hipStream_t st, int phases, const ScheduleArgs* fused) {
  const size_t lds = sizeof(int) * (3 * (size_t)a.B + 1);
  const int grid = compute_units();
  if (phases & kPhaseStream) {
    if (fused && fused->vec4)
      hipLaunchKernelGGL((k_stream_rows<DT, VEC, 2>), dim3((unsigned)grid), dim3(kStreamBlock),
                         lds, st, a, *fused);
    else if (fused)
      hipLaunchKernelGGL((k_stream_rows<DT, VEC, 1>), dim3((unsigned)grid), dim3(kStreamBlock),
                         lds, st, a, *fused);
    else
      hipLaunchKernelGGL((k_stream_rows<DT, VEC, 0>), dim3((unsigned)grid),
                         dim3(kStreamBlock), lds, st, a, ScheduleArgs{});
  }
  if (phases & kPhaseFinish)
    hipLaunchKernelGGL((k_finish<DT, VEC>), dim3((unsigned)grid), dim3(kFinishBlock), 0, st, a);
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
