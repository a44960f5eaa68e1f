// Confidence-scheduled truncation with a global verify-token budget, on the
// GPU (DSpark Deep Dive, "GPU-Resident Scheduling": the scheduler reads the
// confidences and writes one verify length per request without leaving the
// device).
//
// What is computed (DSpark Guide, "2. Confidence-Scheduled Dynamic
// Verification"; DSpark Deep Dive, "Variable-Length Drafts" and "The
// Optimization Logic"):
//   C[b,k]   = prod_{i<=k} conf[b,i], one fp32 multiply per step, left to right
//   Lthr[b]  = max(min_len, number of leading k with C[b,k] >= tau)
//   budget:  if sum Lthr > budget, every request keeps min_len positions and
//            the free slots go to the candidates (b,k), min_len < k <= Lthr[b],
//            in order (C desc, b asc, k asc).
//
// One workgroup (1024 threads, 256 for at most 256 requests); thread t owns
// requests t, t + T, t + 2T, ... for T threads.
// The budget cut is a radix select over one 32-bit key per position: a
// candidate's key is its survival bit pattern plus one (non-negative floats
// order like their bits), every other position's key is 0, so that the m-th
// largest key (m = free slots, fewer than the candidates) is a candidate's.
// Eight 4-bit passes count digit histograms with wave ballots (no LDS
// atomics, so equal digits do not serialise); ties at the cut are resolved by
// a second select on the flat index b*K + (k-1), smallest first.  The keys
// live in LDS when there are at most kSchedLds positions (else they are
// recomputed from the stored survival), and each thread keeps the threshold
// lengths of its first kSchedRegs requests in registers.
#include <hip/hip_runtime.h>

#include "args.hpp"

namespace dspark {

constexpr int kSchedMaxThreads = 1024;
constexpr int kSchedLds = 12288;  // positions whose keys fit in LDS (48 KB)
constexpr int kSchedRegs = 8;     // requests per thread kept in registers

__device__ __forceinline__ uint32_t surv_key(float C) {
  return C == 0.f ? 0u : __float_as_uint(C);  // -0 and +0 are one key
}

// One radix pass over the n keys key_of(i) whose bits under `pmask` equal
// `prefix`: the digit at `shift` that holds the rank-th key counted from the
// top (desc) or from the bottom (asc), and the rank within that digit, in
// shared memory for every thread.
template <int kSchedThreads, typename KeyFn>
__device__ void radix_pass(int n, KeyFn key_of, int shift, bool desc, uint32_t prefix,
                           uint32_t pmask, long long& rank, int (*cnt)[16], uint32_t* s_digit,
                           long long* s_rank, long long* s_bucket) {
  constexpr int kSchedWaves = kSchedThreads / kWave;
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  int c[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) c[d] = 0;
  for (int base = 0; base < n; base += kSchedThreads) {
    const int i = base + tid;
    uint32_t key = 0;
    bool ok = false;
    if (i < n) ok = key_of(i, key);
    ok = ok && ((key & pmask) == prefix);
    const uint32_t d = (key >> shift) & 15u;
#pragma unroll
    for (int dd = 0; dd < 16; ++dd) c[dd] += __popcll(__ballot(ok && d == (uint32_t)dd));
  }
  if (lane_id() == 0) {
#pragma unroll
    for (int dd = 0; dd < 16; ++dd) cnt[w][dd] = c[dd];
  }
  __syncthreads();
  if (tid < kWave) {
    // lane s (< 16) holds digit dd = 15 - s (desc) or s (asc), counted over
    // the waves; an inclusive scan over those 16 lanes finds the digit whose
    // running count first reaches the rank
    const int s = tid & 15;
    const int dd = desc ? 15 - s : s;
    int tot = 0;
#pragma unroll
    for (int ww = 0; ww < kSchedWaves; ++ww) tot += cnt[ww][dd];
    if (tid >= 16) tot = 0;
    int incl = tot;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int t = __shfl_up(incl, o, 16);
      if (s >= o) incl += t;
    }
    const uint64_t reach = __ballot(tid < 16 && (long long)incl >= rank);
    const int first = reach ? __builtin_ctzll(reach) : 15;  // rank never exceeds the total
    const int before = __shfl(incl - tot, first);
    const int bucket = __shfl(tot, first);
    if (tid == 0) {
      *s_digit = (uint32_t)(desc ? 15 - first : first);
      *s_rank = rank - before;
      *s_bucket = bucket;
    }
  }
  __syncthreads();
  rank = *s_rank;
}

// kSchedThreads threads: 1024, or 256 for small batches (a smaller
// workgroup starts sooner; one thread per request still covers them)
template <int kSchedThreads>
__global__ void __launch_bounds__(kSchedThreads) k_schedule(ScheduleArgs a) {
  constexpr int kSchedWaves = kSchedThreads / kWave;
  __shared__ long long red[kSchedWaves];
  __shared__ int cnt[kSchedMaxThreads / kWave][16];
  __shared__ uint32_t s_digit;
  __shared__ long long s_rank, s_bucket;
  __shared__ uint32_t s_key[kSchedLds];
  const int tid = threadIdx.x;
  const int B = a.B, K = a.K;
  const int n = B * K;
  const int ml = a.min_len;
  const bool keys_in_lds = n <= kSchedLds;

  // survival product and threshold length, one thread per request; the
  // candidates' keys go to LDS on the way
  int lt_reg[kSchedRegs];
  long long local = 0;
  int bad = 0;
  for (int j = 0, b = tid; b < B; ++j, b += kSchedThreads) {
    const float* __restrict__ cr = a.conf + (size_t)b * K;
    float* __restrict__ sr = a.surv + (size_t)b * K;
    float C = 1.f;
    int run = 0;  // leading positions with C >= tau
    bool go = true;
    // confidences are loaded 8 at a time ahead of the dependent products
    for (int k0 = 0; k0 < K; k0 += 8) {
      float ck[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ck[i] = cr[min(k0 + i, K - 1)];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = k0 + i;  // 0-based position
        if (k < K) {
          if (!(ck[i] >= 0.f && ck[i] <= 1.f)) bad |= DSPARK_DEV_BAD_CONF;
          C = k == 0 ? ck[i] : C * ck[i];
          sr[k] = C;
          go = go && C >= a.tau;
          if (go) ++run;
          // candidate: past the floor and inside the leading run
          if (keys_in_lds) s_key[(size_t)b * K + k] = (go && k + 1 > ml) ? surv_key(C) + 1u : 0u;
        }
      }
    }
    const int lt = max(ml, run);
    if (j < kSchedRegs) lt_reg[j] = lt;
    // in memory: rows past the registers, and every row when the keys are
    // recomputed from memory below
    if (j >= kSchedRegs || !keys_in_lds) a.lthr[b] = lt;
    local += lt;
  }
  if (bad) flag(a.dev_status, bad);
  auto lthr_of = [&](int j, int b) -> int {
    int v = 0;
#pragma unroll
    for (int jj = 0; jj < kSchedRegs; ++jj)
      if (jj == j) v = lt_reg[jj];
    return j < kSchedRegs ? v : a.lthr[b];
  };
  // block sum of Lthr (the barrier also publishes the LDS keys and the
  // stored survival and threshold lengths to the other threads)
  for (int o = 32; o > 0; o >>= 1) local += __shfl_xor(local, o);
  if (lane_id() == 0) red[tid / kWave] = local;
  __syncthreads();
  long long total = 0;
  for (int w = 0; w < kSchedWaves; ++w) total += red[w];

  const long long floor_all = (long long)B * ml;
  const bool binds = a.budget >= 0 && total > a.budget;
  const long long m = binds ? (long long)a.budget - floor_all : 0;  // free slots, >= 0
  uint32_t kstar = 0xffffffffu, istar = 0u;  // no candidate is taken by default
  if (binds && m > 0) {
    const float* surv = a.surv;
    const int* lthr_mem = a.lthr;
    // key of position i: survival bits + 1 for a candidate, else 0 (from
    // LDS, or recomputed from the stored survival and threshold length)
    auto key_at = [=](int i) -> uint32_t {
      if (keys_in_lds) return s_key[i];
      const int b = i / K, k = i - b * K + 1;
      const int lt = lthr_mem[b];
      return (k > ml && k <= lt) ? surv_key(surv[i]) + 1u : 0u;
    };
    // m-th largest key (all candidates' keys exceed every other key)
    uint32_t prefix = 0, pmask = 0;
    long long rank = m, bucket = 0;
    for (int shift = 28; shift >= 0; shift -= 4) {
      radix_pass<kSchedThreads>(n, [=](int i, uint32_t& key) {
                   key = key_at(i);
                   return true;
                 },
                 shift, true, prefix, pmask, rank, cnt, &s_digit, &s_rank, &s_bucket);
      prefix |= s_digit << shift;
      pmask |= 15u << shift;
      bucket = s_bucket;
    }
    kstar = prefix;
    // `bucket` positions share key kstar; take the `rank` of them with the
    // smallest flat index
    istar = 0xffffffffu;
    if (rank < bucket) {
      uint32_t ip = 0, im = 0;
      long long r2 = rank;
      // the flat index has fewer than 32 bits: higher digits are all 0
      int top = 0;
      while (top < 28 && (((uint32_t)(n - 1)) >> (top + 4)) != 0u) top += 4;
      for (int shift = top; shift >= 0; shift -= 4) {
        radix_pass<kSchedThreads>(n, [=](int i, uint32_t& key) {
                     if (key_at(i) != kstar) return false;
                     key = (uint32_t)i;
                     return true;
                   },
                   shift, false, ip, im, r2, cnt, &s_digit, &s_rank, &s_bucket);
        ip |= s_digit << shift;
        im |= 15u << shift;
      }
      istar = ip;
    }
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
}

int launch_schedule(ScheduleArgs& a, hipStream_t st) {
  if (a.B <= 256)
    hipLaunchKernelGGL(k_schedule<256>, dim3(1), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_schedule<1024>, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_LAUNCH;
}

}  // namespace dspark
