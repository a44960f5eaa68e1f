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
// 4-bit passes start at the highest bit where the candidates' keys differ
// (the bits above are common to all of them).  Each lane counts digits in
// 4-bit fields of one 64-bit word (a few instructions per key, no LDS
// atomics, so equal digits do not serialise) and each wave sums its lanes
// with a transposing butterfly.  Ties at the cut are resolved by a second
// select on the flat index b*K + (k-1), smallest first.  The keys live in
// LDS when there are at most kSchedLds positions (else they are recomputed
// from the stored survival), and each thread keeps the threshold lengths of
// its first kSchedRegs requests in registers.
#include <hip/hip_runtime.h>

#include "schedule_core.hpp"

namespace dspark {

// Load-aware threshold and budget (DSpark Guide, "Dynamic Verification
// Scheduling Algorithm", steps 1-2; DSpark Deep Dive, "The Throughput Curve"
// and "The Optimization Logic"), worked out by every wave on its own, so no
// barrier is needed: lane i (1 <= i < n) takes the slope of curve segment i
// and one ballot finds the first segment whose gain is below the slot cost.
struct LoadDecision {
  float tau;
  int budget;
  int bad;
};

__device__ LoadDecision load_decision(const ScheduleArgs& a) {
  LoadDecision d;
  d.bad = 0;
  // load factor in fp32: the two ratios, the products, the sum, then [0, 1];
  // a bad figure reads as full load
  const float q = a.load[0], m = a.load[1];
  float lf = 1.f;
  if (q >= 0.f && m >= 0.f && q <= FLT_MAX && m <= FLT_MAX) {
    lf = 0.6f * (q / a.q_max) + 0.4f * (m / a.m_max);
    lf = fminf(fmaxf(lf, 0.f), 1.f);
  } else {
    d.bad |= DSPARK_DEV_BAD_LOAD;
  }
  d.tau = a.tau_min + (a.tau_max - a.tau_min) * (lf * lf);
  const int n = a.n_curve;
  d.budget = -1;
  if (n == 0) return d;
  // curve point l and the one before it (lanes past the curve read point 0)
  const int l = lane_id();
  const int i = l < n ? l : 0;
  const int ip = i > 0 ? i - 1 : 0;
  const float x = a.curve[2 * i], t = a.curve[2 * i + 1];
  const float xp = a.curve[2 * ip], tp = a.curve[2 * ip + 1];
  const bool ok = (x >= 1.f && x <= 16777216.f && floorf(x) == x && fabsf(t) <= FLT_MAX &&
                   (i == 0 || x > xp));
  if (__ballot(l < n && !ok)) {
    d.bad |= DSPARK_DEV_BAD_CURVE;
    return d;
  }
  const double g = ((double)t - (double)tp) / ((double)x - (double)xp);
  const uint64_t drop = __ballot(l >= 1 && l < n && g < (double)a.slot_cost);
  const int last = drop ? __builtin_ctzll(drop) - 1 : n - 1;  // the last point kept
  const int xstar = (int)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), last));
  d.budget = max(a.B * a.min_len, xstar - a.B);
  return d;
}

// kSchedThreads threads: 1024, or 256 for small batches (a smaller
// workgroup starts sooner; one thread per request still covers them)
template <int kSchedThreads>
__global__ void __launch_bounds__(kSchedThreads) k_schedule(ScheduleArgs a) {
  float tau = a.tau;
  int budget = a.budget;
  if (a.load) {
    const LoadDecision d = load_decision(a);
    tau = d.tau;
    budget = d.budget;
    if (threadIdx.x == 0) {
      if (d.bad) flag(a.dev_status, d.bad);
      if (a.tau_out) *a.tau_out = tau;
      if (a.budget_out) *a.budget_out = budget;
    }
  }
  schedule_body<kSchedThreads>(a, tau, budget, 0, 1);
}

int launch_schedule(ScheduleArgs& a, hipStream_t st) {
  if (a.B <= 256)
    hipLaunchKernelGGL(k_schedule<256>, dim3(1), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_schedule<1024>, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_LAUNCH;
}

}  // namespace dspark
