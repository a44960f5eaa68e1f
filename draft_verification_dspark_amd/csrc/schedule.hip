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
// One workgroup of 1024 threads.  The budget cut is a radix select: the key
// of candidate (b,k) is the bit pattern of C (non-negative floats order like
// their bits), the m-th largest key is found in eight 4-bit passes whose
// digit histograms are counted with wave ballots (no LDS atomics, so equal
// digits do not serialise), and ties at the cut are resolved by a second
// select on the flat index b*K + (k-1), smallest first.
#include <hip/hip_runtime.h>

#include "args.hpp"

namespace dspark {

constexpr int kSchedThreads = 1024;
constexpr int kSchedWaves = kSchedThreads / kWave;

__device__ __forceinline__ uint32_t surv_key(float C) {
  return C == 0.f ? 0u : __float_as_uint(C);  // -0 and +0 are one key
}

// One radix pass over the candidates selected by `pred_key`: returns, in
// shared memory, the digit at `shift` that holds the rank-th element counted
// from the top (desc) or from the bottom (asc), and the updated rank.
template <typename KeyFn>
__device__ void radix_pass(int n, KeyFn key_of, int shift, bool desc, uint32_t prefix,
                           uint32_t pmask, long long& rank, int (*cnt)[16], uint32_t* s_digit,
                           long long* s_rank, long long* s_bucket) {
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
  if (tid == 0) {
    long long r = rank;
    int chosen = desc ? 0 : 15;
    long long bucket = 0;
    for (int s = 0; s < 16; ++s) {
      const int dd = desc ? 15 - s : s;
      long long tot = 0;
      for (int ww = 0; ww < kSchedWaves; ++ww) tot += cnt[ww][dd];
      if (r <= tot) {
        chosen = dd;
        bucket = tot;
        break;
      }
      r -= tot;
    }
    *s_digit = (uint32_t)chosen;
    *s_rank = r;
    *s_bucket = bucket;
  }
  __syncthreads();
  rank = *s_rank;
}

__global__ void __launch_bounds__(kSchedThreads) k_schedule(ScheduleArgs a) {
  __shared__ long long red[kSchedWaves];
  __shared__ int cnt[kSchedWaves][16];
  __shared__ uint32_t s_digit;
  __shared__ long long s_rank, s_bucket;
  const int tid = threadIdx.x;
  const int B = a.B, K = a.K;
  const int n = B * K;

  // survival product and threshold length, one thread per request
  long long local = 0;
  int bad = 0;
  for (int b = tid; b < B; b += kSchedThreads) {
    const float* __restrict__ cr = a.conf + (size_t)b * K;
    float* __restrict__ sr = a.surv + (size_t)b * K;
    float C = 1.f;
    int cnt_keep = 0;
    bool go = true;
    // confidences are loaded 8 at a time ahead of the dependent products
    for (int k0 = 0; k0 < K; k0 += 8) {
      float ck[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ck[i] = k0 + i < K ? cr[k0 + i] : 1.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (k0 + i >= K) break;
        if (!(ck[i] >= 0.f && ck[i] <= 1.f)) bad |= DSPARK_DEV_BAD_CONF;
        C = k0 + i == 0 ? ck[i] : C * ck[i];
        sr[k0 + i] = C;
        if (go && C >= a.tau) ++cnt_keep;
        else go = false;
      }
    }
    const int lt = max(a.min_len, cnt_keep);
    a.lthr[b] = lt;
    local += lt;
  }
  if (bad) flag(a.dev_status, bad);
  // block sum of Lthr
  for (int o = 32; o > 0; o >>= 1) local += __shfl_xor(local, o);
  if (lane_id() == 0) red[tid / kWave] = local;
  __syncthreads();
  long long total = 0;
  for (int w = 0; w < kSchedWaves; ++w) total += red[w];

  const long long floor_all = (long long)B * a.min_len;
  if (a.budget < 0 || total <= a.budget) {
    for (int b = tid; b < B; b += kSchedThreads) a.lengths[b] = a.lthr[b];
  } else {
    const long long m = (long long)a.budget - floor_all;  // free slots, >= 0
    if (m <= 0) {
      for (int b = tid; b < B; b += kSchedThreads) a.lengths[b] = a.min_len;
    } else {
      const int* lthr = a.lthr;
      const float* surv = a.surv;
      const int ml = a.min_len;
      auto cand = [=](int i) -> bool {
        const int b = i / K, k = i - b * K + 1;
        return k > ml && k <= lthr[b];
      };
      // m-th largest survival key among the candidates
      uint32_t prefix = 0, pmask = 0;
      long long rank = m, bucket = 0;
      for (int shift = 28; shift >= 0; shift -= 4) {
        radix_pass(n, [=](int i, uint32_t& key) {
                     if (!cand(i)) return false;
                     key = surv_key(surv[i]);
                     return true;
                   },
                   shift, true, prefix, pmask, rank, cnt, &s_digit, &s_rank, &s_bucket);
        prefix |= s_digit << shift;
        pmask |= 15u << shift;
        bucket = s_bucket;
      }
      const uint32_t kstar = prefix;
      // `bucket` candidates share key kstar; take the `rank` of them with the
      // smallest flat index
      uint32_t istar = 0xffffffffu;
      if (rank < bucket) {
        uint32_t ip = 0, im = 0;
        long long r2 = rank;
        for (int shift = 28; shift >= 0; shift -= 4) {
          radix_pass(n, [=](int i, uint32_t& key) {
                       if (!cand(i) || surv_key(surv[i]) != kstar) return false;
                       key = (uint32_t)i;
                       return true;
                     },
                     shift, false, ip, im, r2, cnt, &s_digit, &s_rank, &s_bucket);
          ip |= s_digit << shift;
          im |= 15u << shift;
        }
        istar = ip;
      }
      for (int b = tid; b < B; b += kSchedThreads) {
        const int lt = lthr[b];
        int take = 0;
        for (int k = ml + 1; k <= lt; ++k) {
          const int i = b * K + k - 1;
          const uint32_t key = surv_key(surv[i]);
          take += (key > kstar || (key == kstar && (uint32_t)i <= istar)) ? 1 : 0;
        }
        a.lengths[b] = ml + take;
      }
    }
  }
  if (a.mask) {
    __syncthreads();
    for (int i = tid; i < n; i += kSchedThreads) {
      const int b = i / K;
      a.mask[i] = (uint8_t)((i - b * K) < a.lengths[b] ? 1 : 0);
    }
  }
}

int launch_schedule(ScheduleArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(kSchedThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_LAUNCH;
}

}  // namespace dspark
