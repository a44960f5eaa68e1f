// The schedule's core, shared by the schedule kernel and the streaming pass
// of the fused schedule + verify call: survival products, threshold lengths
// and the budget cut by radix select, for one workgroup of kSchedThreads
// threads (DSpark Guide, "2. Confidence-Scheduled Dynamic Verification";
// DSpark Deep Dive, "Variable-Length Drafts" and "The Optimization Logic").
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>

#include "schedule_args.hpp"

namespace dspark {

constexpr int kSchedMaxThreads = 1024;
constexpr int kSchedLds = 12288;  // positions whose keys fit in LDS (48 KB)
constexpr int kSchedRegs = 8;     // requests per thread kept in registers
#ifndef DSPARK_CONF_STAGE
#define DSPARK_CONF_STAGE 8
#endif
constexpr int kConfStage = DSPARK_CONF_STAGE;  // confidences per thread loaded at once

__device__ __forceinline__ uint32_t surv_key(float C) {
  return C == 0.f ? 0u : __float_as_uint(C);  // -0 and +0 are one key
}

// Sums over each 16-lane row of 16 per-lane counters c[0..15], by a
// transposing butterfly of DPP moves: at each exchange a lane keeps half of
// the counters it still holds and adds its partner's copy of that half.  The
// partners (row mirror, half-row mirror, quad xor 2, quad xor 1) differ from
// the lane in bit 3, 2, 1, 0 of its row position, so lane l ends with the
// row's sum for digit l & 15.
__device__ __forceinline__ uint32_t row_sum16(const uint32_t (&c)[16]) {
  const int l = lane_id();
  uint32_t c8[8], c4[4], c2[2];
  bool hi = (l >> 3) & 1;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    c8[j] = (hi ? c[j + 8] : c[j]) + (uint32_t)dpp<kRowMirror>((int)(hi ? c[j] : c[j + 8]));
  hi = (l >> 2) & 1;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    c4[j] = (hi ? c8[j + 4] : c8[j]) + (uint32_t)dpp<kRowHalfMirror>((int)(hi ? c8[j] : c8[j + 4]));
  hi = (l >> 1) & 1;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    c2[j] = (hi ? c4[j + 2] : c4[j]) + (uint32_t)dpp<kQuadXor2>((int)(hi ? c4[j] : c4[j + 2]));
  hi = l & 1;
  return (hi ? c2[1] : c2[0]) + (uint32_t)dpp<kQuadXor1>((int)(hi ? c2[0] : c2[1]));
}

// inclusive prefix sum within each 16-lane row (row_shr 1, 2, 4, 8; lanes
// without a source add 0)
__device__ __forceinline__ int row_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
  return v;
}

// Key sources of the radix passes.  Key of position i = b*K + (k-1):
// survival bits + 1 for a candidate, else 0.  LdsKeys reads the keys stored
// in LDS; MemKeys recomputes them from the stored survival and threshold
// length.  Both read unconditionally (the caller passes a valid index), so a
// loop over several keys has all its loads in flight at once.
struct LdsKeys {
  const uint32_t* s;
  __device__ __forceinline__ uint32_t operator()(int i) const { return s[i]; }
};
struct MemKeys {
  const float* surv;
  const int32_t* lthr;
  int K, ml;
  __device__ __forceinline__ uint32_t operator()(int i) const {
    const int b = i / K, k = i - b * K + 1;
    const int lt = lthr[b];
    const uint32_t key = surv_key(surv[i]) + 1u;
    return (k > ml && k <= lt) ? key : 0u;
  }
};

// One radix pass over the n positions whose pass key has the bits under
// `pmask` equal to `prefix`.  The pass key is the position's key (kIndex
// false) or, for positions whose key equals `kmatch`, the flat index (kIndex
// true; other positions do not take part).  Finds the digit at `shift` that
// holds the rank-th pass key counted from the top (desc) or from the bottom
// (asc), the rank within that digit and the number of pass keys with that
// digit, in every thread.  Each lane counts in 4-bit fields of one 64-bit
// word (field d counts digit d; at most kFlush keys between flushes into
// 32-bit counters), each 16-lane row sums its lanes, and every wave reads the
// per-row sums from `cnt` (this pass's buffer: consecutive passes alternate
// two buffers, so one barrier per pass suffices).
template <int kSchedThreads, bool kIndex, typename Src>
__device__ void radix_pass(int n, const Src& src, uint32_t kmatch, int shift, bool desc,
                           uint32_t prefix, uint32_t pmask, long long& rank, long long& bucket,
                           uint32_t& digit, int (*cnt)[16][4]) {
  constexpr int kSchedWaves = kSchedThreads / kWave;
  constexpr int kGroup = 4;             // keys per lane in flight
  constexpr int kFlush = 3 * kGroup;    // keys per lane between flushes (<= 15)
  const int tid = threadIdx.x;
  const int l = lane_id();
  uint32_t c[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) c[d] = 0;
  for (int b0 = 0; b0 < n; b0 += kFlush * kSchedThreads) {
    const int lim = min(n, b0 + kFlush * kSchedThreads);
    uint64_t nib = 0;
    for (int base = b0; base < lim; base += kGroup * kSchedThreads) {
      uint32_t kv[kGroup];
#pragma unroll
      for (int r = 0; r < kGroup; ++r) kv[r] = src(min(base + r * kSchedThreads + tid, n - 1));
#pragma unroll
      for (int r = 0; r < kGroup; ++r) {
        const int i = base + r * kSchedThreads + tid;
        bool ok = i < lim;
        uint32_t key = kv[r];
        if (kIndex) {
          ok = ok && key == kmatch;
          key = (uint32_t)i;
        }
        ok = ok && ((key & pmask) == prefix);
        const uint32_t d = (key >> shift) & 15u;
        nib += (uint64_t)(ok ? 1u : 0u) << (4 * d);
      }
    }
#pragma unroll
    for (int d = 0; d < 16; ++d) c[d] += (uint32_t)(nib >> (4 * d)) & 15u;
  }
  // lane l holds its row's count of digit l & 15
  cnt[tid / kWave][l & 15][l >> 4] = (int)row_sum16(c);
  __syncthreads();
  // lane s (= l & 15, in every row) holds digit dd = 15 - s (desc) or s
  // (asc), counted over the waves and rows; an inclusive scan over the 16
  // lanes of a row finds the digit whose running count first reaches the
  // rank
  const int s = l & 15;
  const int dd = desc ? 15 - s : s;
  int tot = 0;
#pragma unroll
  for (int ww = 0; ww < kSchedWaves; ++ww) {
    const int4 v = *reinterpret_cast<const int4*>(cnt[ww][dd]);
    tot += (v.x + v.y) + (v.z + v.w);
  }
  const int incl = row_incl_scan(tot);
  const uint64_t reach = __ballot(l < 16 && (long long)incl >= rank);
  const int first = reach ? __builtin_ctzll(reach) : 15;  // rank never exceeds the total
  const int before = __builtin_amdgcn_readlane(incl - tot, first);
  bucket = __builtin_amdgcn_readlane(tot, first);
  digit = (uint32_t)(desc ? 15 - first : first);
  rank -= before;
}

// The budget cut: the m-th largest key kstar (m < number of candidates, so
// it is a candidate's; all candidates' keys exceed every other key) and,
// when the cut splits the positions with key kstar, the largest flat index
// istar among those taken (else istar = 0xffffffff).  ncand: the number of
// candidates.  The candidates share the bits above the highest bit where the
// OR and the AND of their keys differ, so the passes start at the digit
// holding that bit.  red_or / red_and: per-wave scratch in LDS.
template <int kSchedThreads, typename Src>
__device__ void budget_cut(int n, const Src& src, long long m, long long ncand, uint32_t* red_or,
                           uint32_t* red_and, int (*cnt)[kSchedThreads / kWave][16][4],
                           uint32_t& kstar, uint32_t& istar) {
  constexpr int kSchedWaves = kSchedThreads / kWave;
  uint32_t kor = 0u, kand = 0xffffffffu;  // candidates' keys are the non-zero ones
  for (int i = threadIdx.x; i < n; i += kSchedThreads) {
    const uint32_t key = src(i);
    kor |= key;
    kand &= key ? key : 0xffffffffu;
  }
  kor = (uint32_t)wave_reduce((int)kor, [](int x, int y) { return x | y; });
  kand = (uint32_t)wave_reduce((int)kand, [](int x, int y) { return x & y; });
  if (lane_id() == 0) {
    red_or[threadIdx.x / kWave] = kor;
    red_and[threadIdx.x / kWave] = kand;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kSchedWaves; ++w) {
    kor |= red_or[w];
    kand &= red_and[w];
  }
  int pass = 0;  // selects the count buffer
  long long rank = m, bucket = ncand;
  const uint32_t diff = kor ^ kand;
  if (diff != 0u) {
    const int s0 = (31 - __builtin_clz(diff)) & ~3;
    uint32_t pmask = s0 + 4 < 32 ? 0xffffffffu << (s0 + 4) : 0u;
    uint32_t prefix = kand & pmask;
    for (int shift = s0; shift >= 0; shift -= 4) {
      uint32_t dg;
      radix_pass<kSchedThreads, false>(n, src, 0u, shift, true, prefix, pmask, rank, bucket, dg,
                                       cnt[pass++ & 1]);
      prefix |= dg << shift;
      pmask |= 15u << shift;
    }
    kstar = prefix;
  } else {
    kstar = kand;  // one key for every candidate
  }
  // `bucket` positions share key kstar; take the `rank` of them with the
  // smallest flat index
  istar = 0xffffffffu;
  if (rank < bucket) {
    uint32_t ip = 0, im = 0;
    long long b2 = 0;
    // the flat index has fewer than 32 bits: higher digits are all 0
    int top = 0;
    while (top < 28 && (((uint32_t)(n - 1)) >> (top + 4)) != 0u) top += 4;
    for (int shift = top; shift >= 0; shift -= 4) {
      uint32_t dg;
      radix_pass<kSchedThreads, true>(n, src, kstar, shift, false, ip, im, rank, b2, dg,
                                      cnt[pass++ & 1]);
      ip |= dg << shift;
      im |= 15u << shift;
    }
    istar = ip;
  }
}

// Length and mask of request b.
__device__ __forceinline__ void store_len_mask(const ScheduleArgs& a, int b, int len) {
  const int K = a.K;
  a.lengths[b] = len;
  if (a.mask) {
    uint8_t* mr = a.mask + (size_t)b * K;
    if ((K & 3) == 0 && ((uintptr_t)a.mask & 3) == 0) {
      // four mask bytes per store
      uint32_t* mw = reinterpret_cast<uint32_t*>(mr);
      for (int k = 0; k < K; k += 4) {
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) word |= (uint32_t)(k + q < len ? 1u : 0u) << (8 * q);
        mw[k >> 2] = word;
      }
    } else {
      for (int k = 0; k < K; ++k) mr[k] = (uint8_t)(k < len ? 1 : 0);
    }
  }
}

// Tile-count prefix of a caller's plan over the requests in thread order,
// worked out at the schedule's own barrier when the budget does not bind
// (off stays negative otherwise: the lengths change after the barrier).
struct PlanPrefix {
  int off = -1;   // the counts of the requests before this thread's
  int total = 0;  // the counts of all requests
};
struct NoPlanCount {
  __device__ int operator()(int) const { return 0; }
};

// The schedule of the whole batch by one workgroup of kSchedThreads threads
// (every thread calls it; thread t owns requests t, t + T, ...).  The
// outputs of request b (survival products, length, mask, status bits) go to
// memory when b % nwg == wg: with nwg = 1 this workgroup writes them all
// (and the threshold lengths that the budget cut may read back); with
// several workgroups working out the same schedule, each writes its share,
// and the caller guarantees that nothing has to be read back (B * K <=
// kSchedLds and B <= kSchedThreads * kSchedRegs).  Returns the length of
// request threadIdx.x (0 for threads without a request).
// kStage: confidences per thread loaded at once (one round trip per kStage
// positions).  kPre: the caller has loaded them already, into `pre`, for its
// own request (one request per thread, K <= kStage); `pre` then returns the
// survival products, and the request's outputs (survival products, length,
// mask) are left to the caller, who writes them with schedule_store_own once
// it has nothing more to wait for: on this target stores and loads share one
// in-order counter, and a store inside a branch makes the compiler wait for
// younger loads as well.  With `plan` (kPre only), plan_count(L) is the
// caller's count for its request at length L, and `plan` receives the
// prefix of those counts at the threshold lengths when the budget does not
// bind, so that the caller's plan needs no barrier of its own for it.
template <int kSchedThreads, int kStage = kConfStage, bool kPre = false,
          typename PlanCount = NoPlanCount>
__device__ int schedule_body(const ScheduleArgs& a, float tau, int budget, int wg, int nwg,
                             float* pre = nullptr, PlanCount plan_count = PlanCount{},
                             PlanPrefix* plan = nullptr) {
  constexpr int kSchedWaves = kSchedThreads / kWave;
  __shared__ long long red[kSchedWaves];
  __shared__ int red_plan[kSchedWaves];
  __shared__ uint32_t red_or[kSchedWaves], red_and[kSchedWaves];
  __shared__ __align__(16) int cnt[2][kSchedWaves][16][4];  // [pass & 1][wave][digit][row]
  __shared__ uint32_t s_key[kSchedLds];
  const int tid = threadIdx.x;
  const int B = a.B, K = a.K;
  const int n = B * K;
  const int ml = a.min_len;
  const bool keys_in_lds = n <= kSchedLds;
  int my_len = 0;

  // survival product and threshold length, one thread per request; the
  // candidates' keys go to LDS on the way
  int lt_reg[kSchedRegs];
  long long local = 0;
  int bad = 0;
  int pc = 0;  // kPre: the caller's plan count at the threshold length
  if constexpr (kPre) {
    // One request per thread, its K <= kStage confidences in registers: the
    // same steps straight-line, with no branch per position.  A position
    // past K leaves the product and the run as they are and stores again
    // the last position's key into that position's slot.
    const int b = tid;
    if (b < B) {
      const bool write = nwg == 1 || b % nwg == wg;
      float C = 1.f;
      int run = 0;
      bool go = true;
      uint32_t key = 0u;
#pragma unroll
      for (int k = 0; k < kStage; ++k) {
        const bool in = k < K;  // the same in every thread
        const float c = pre[k];
        if (in && !(c >= 0.f && c <= 1.f)) bad |= DSPARK_DEV_BAD_CONF;
        const float Cn = k == 0 ? c : C * c;
        C = in ? Cn : C;
        const bool gn = go && C >= tau;
        go = in ? gn : go;
        run += (in && go) ? 1 : 0;
        key = in ? ((go && k + 1 > ml) ? surv_key(C) + 1u : 0u) : key;
        const int slot = k < K ? k : K - 1;
        if (keys_in_lds) s_key[(size_t)b * K + slot] = key;
        pre[k] = C;
      }
      const int lt = max(ml, run);
      lt_reg[0] = lt;
      pc = plan_count(lt);
      if (nwg == 1 && !keys_in_lds) a.lthr[b] = lt;  // read back by the budget cut
      local = lt;
      if (write && bad) flag(a.dev_status, bad);
    }
  } else {
  for (int j = 0, b = tid; b < B; ++j, b += kSchedThreads) {
    const bool write = nwg == 1 || b % nwg == wg;  // this request's outputs
    const float* __restrict__ cr = a.conf + (size_t)b * K;
    float* __restrict__ sr = a.surv + (size_t)b * K;
    float C = 1.f;
    int run = 0;  // leading positions with C >= tau
    bool go = true;
    // up to kStage confidences are loaded at once (16-byte loads when
    // rows are 16-byte aligned), ahead of the dependent products; the
    // survival values overwrite them and are stored the same way
    for (int k0 = 0; k0 < K; k0 += kStage) {
      float ck[kStage];
      if (a.vec4) {
#pragma unroll
        for (int q = 0; q < kStage / 4; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(cr + min(k0 + 4 * q, K - 4));
          ck[4 * q] = v.x;
          ck[4 * q + 1] = v.y;
          ck[4 * q + 2] = v.z;
          ck[4 * q + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < kStage; ++i) ck[i] = cr[min(k0 + i, K - 1)];
      }
#pragma unroll
      for (int i = 0; i < kStage; ++i) {
        const int k = k0 + i;  // 0-based position
        if (k < K) {
          if (!(ck[i] >= 0.f && ck[i] <= 1.f)) bad |= DSPARK_DEV_BAD_CONF;
          C = k == 0 ? ck[i] : C * ck[i];
          ck[i] = C;
          go = go && C >= tau;
          if (go) ++run;
          // candidate: past the floor and inside the leading run
          if (keys_in_lds) s_key[(size_t)b * K + k] = (go && k + 1 > ml) ? surv_key(C) + 1u : 0u;
        }
      }
      if (!write) {
      } else if (a.vec4) {
#pragma unroll
        for (int q = 0; q < kStage / 4; ++q)
          if (k0 + 4 * q < K)
            *reinterpret_cast<float4*>(sr + k0 + 4 * q) =
                make_float4(ck[4 * q], ck[4 * q + 1], ck[4 * q + 2], ck[4 * q + 3]);
      } else {
#pragma unroll
        for (int i = 0; i < kStage; ++i)
          if (k0 + i < K) sr[k0 + i] = ck[i];
      }
    }
    const int lt = max(ml, run);
    if (j < kSchedRegs) lt_reg[j] = lt;
    // in memory: rows past the registers, and every row when the keys are
    // recomputed from memory below
    if (nwg == 1 && (j >= kSchedRegs || !keys_in_lds)) a.lthr[b] = lt;
    local += lt;
    if (write && bad) flag(a.dev_status, bad);
    bad = 0;
  }
  }
  auto lthr_of = [&](int j, int b) -> int {
    int v = 0;
#pragma unroll
    for (int jj = 0; jj < kSchedRegs; ++jj)
      if (jj == j) v = lt_reg[jj];
    return j < kSchedRegs ? v : a.lthr[b];
  };
  // block sum of Lthr (the barrier also publishes the LDS keys and the
  // stored survival and threshold lengths to the other threads; a wave's sum
  // is at most B*K <= 2^30: int)
  int pc_excl = 0;
  if constexpr (kPre) {
    // the plan counts scanned across the wave, published at the same barrier
    int incl = pc;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane_id() >= o) incl += t;
    }
    if (lane_id() == kWave - 1) red_plan[tid / kWave] = incl;
    pc_excl = incl - pc;
  }
  const int wsum = wave_reduce((int)local, [](int x, int y) { return x + y; });
  if (lane_id() == 0) red[tid / kWave] = wsum;
  __syncthreads();
  long long total = 0;
  for (int w = 0; w < kSchedWaves; ++w) total += red[w];

  const long long floor_all = (long long)B * ml;
  const bool binds = budget >= 0 && total > budget;
  if constexpr (kPre) {
    if (plan && !binds) {
      int off = pc_excl, all = 0;
      for (int w = 0; w < kSchedWaves; ++w) {
        const int x = red_plan[w];
        if (w < tid / kWave) off += x;
        all += x;
      }
      plan->off = off;
      plan->total = all;
    }
  }
  const long long m = binds ? (long long)budget - floor_all : 0;  // free slots, >= 0
  uint32_t kstar = 0xffffffffu, istar = 0u;  // no candidate is taken by default
  if (binds && m > 0) {
    if (keys_in_lds)
      budget_cut<kSchedThreads>(n, LdsKeys{s_key}, m, total - floor_all, red_or, red_and, cnt,
                                kstar, istar);
    else
      budget_cut<kSchedThreads>(n, MemKeys{a.surv, a.lthr, K, ml}, m, total - floor_all, red_or,
                                red_and, cnt, kstar, istar);
  }
  // lengths and mask, each request by its owner thread
  for (int j = 0, b = tid; b < B; ++j, b += kSchedThreads) {
    const int lt = lthr_of(j, b);
    int len = lt;
    if (binds) {
      int take = 0;
      if (m > 0) {
        for (int k = ml + 1; k <= lt; ++k) {
          const int i = b * K + k - 1;
          const uint32_t key = keys_in_lds ? s_key[i] : surv_key(a.surv[i]) + 1u;
          take += (key > kstar || (key == kstar && (uint32_t)i <= istar)) ? 1 : 0;
        }
      }
      len = ml + take;
    }
    if (b == tid) my_len = len;
    if (kPre || !(nwg == 1 || b % nwg == wg)) continue;
    store_len_mask(a, b, len);
  }
  return my_len;
}

// The outputs of request threadIdx.x that schedule_body<..., kPre = true>
// left to its caller: `surv` (its survival products) and `len` go to memory
// when this workgroup owns the request.
template <int kN>
__device__ __forceinline__ void schedule_store_own(const ScheduleArgs& a, int wg, int nwg,
                                                   int len, const float (&surv)[kN]) {
  const int b = threadIdx.x;
  if (b >= a.B || !(nwg == 1 || b % nwg == wg)) return;
  float* __restrict__ sr = a.surv + (size_t)b * a.K;
  if (a.vec4) {
#pragma unroll
    for (int q = 0; q < kN / 4; ++q)
      if (4 * q < a.K)
        *reinterpret_cast<float4*>(sr + 4 * q) =
            make_float4(surv[4 * q], surv[4 * q + 1], surv[4 * q + 2], surv[4 * q + 3]);
  } else {
#pragma unroll
    for (int k = 0; k < kN; ++k)
      if (k < a.K) sr[k] = surv[k];
  }
  store_len_mask(a, b, len);
}

}  // namespace dspark
