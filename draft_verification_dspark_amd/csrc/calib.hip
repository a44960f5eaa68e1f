// Online calibration of the per-position confidences, on the GPU (DSpark
// Deep Dive, "Online Calibration"):
//   k_calibrate     calibrated[b,k] = sigmoid(logit(raw[b,k]) / theta[k])
//                   ("Sequential Temperature Scaling": one temperature per
//                   draft position), in fp64, stored as fp32;
//   k_calib_observe one round's outcomes into a window kept in device memory
//                   ("The Calibration Loop in Practice"): per position, the
//                   tokens whose accept test ran (k <= L_b and k <= a_b + 1),
//                   how many were accepted (k <= a_b) and the sum of their
//                   calibrated scores; per equal-width bin of the score, the
//                   same counts.  After `window` rounds: per position
//                   theta += lr * (mean score - acceptance fraction), floored
//                   at theta_min; the window's expected calibration error
//                   sum_bins |accepted - sum of scores| / tokens; a fresh
//                   window.  One workgroup, so the step needs no
//                   cross-workgroup synchronisation.
#include <hip/hip_runtime.h>

#include <cfloat>

#include "calib_args.hpp"

namespace dspark {

__global__ void __launch_bounds__(256) k_calibrate(CalibArgs a) {
  const long long n = (long long)a.B * a.K;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int k = (int)(i % a.K);
  const float x = a.raw[i];
  const float t = a.theta[k];
  float out = x;
  int bad = 0;
  if (!(t > 0.f && t <= FLT_MAX)) {
    bad = DSPARK_DEV_BAD_CONF;  // temperature NaN, infinite or not positive
  } else if (!(x >= 0.f && x <= 1.f)) {
    bad = DSPARK_DEV_BAD_CONF;  // score NaN or outside [0, 1]
  } else if (x > 0.f && x < 1.f) {
    const double xd = (double)x;
    const double z = (log(xd) - log1p(-xd)) / (double)t;
    out = (float)(1.0 / (1.0 + exp(-z)));
  }
  a.calibrated_out[i] = out;
  if (bad) flag(a.dev_status, bad);
}

// State layout (8-byte words): rounds; n[K]; acc[K]; pred[K] (double);
// bn[M]; bacc[M]; bconf[M] (double).
__global__ void __launch_bounds__(kCalibThreads) k_calib_observe(CalibArgs a) {
  __shared__ int s_n[kCalibMax], s_acc[kCalibMax], s_bn[kCalibMax], s_bacc[kCalibMax];
  __shared__ double s_pred[kCalibMax], s_bconf[kCalibMax];
  __shared__ double s_gap[kCalibMax];  // per bin: |accepted - sum of scores| over the window
  __shared__ int s_cnt[kCalibMax];     // per bin: tokens over the window
  __shared__ int s_bad, s_end;
  const int tid = threadIdx.x;
  const int K = a.K, M = a.n_bins;
  if (tid < kCalibMax) {
    s_n[tid] = s_acc[tid] = s_bn[tid] = s_bacc[tid] = 0;
    s_pred[tid] = s_bconf[tid] = 0.0;
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();
  int bad = 0;
  const long long n = (long long)a.B * K;
  for (long long i = tid; i < n; i += kCalibThreads) {
    const int b = (int)(i / K), k = (int)(i - (long long)b * K);
    int L = a.lengths ? a.lengths[b] : K;
    int acc = a.accepted[b];
    if (L < 0 || L > K || acc < 0 || acc > L) bad |= DSPARK_DEV_BAD_LENGTH;
    L = min(max(L, 0), K);
    acc = min(max(acc, 0), L);
    if (k + 1 > L || k + 1 > acc + 1) continue;  // this position's test did not run
    const float c = a.calibrated[i];
    if (!(c >= 0.f && c <= 1.f)) bad |= DSPARK_DEV_BAD_CONF;
    const double cd = c == c ? (double)c : 0.0;
    const int ok = k + 1 <= acc ? 1 : 0;
    // bin of the score: the product is exact in fp64
    int m = (int)floor(cd * (double)M);
    m = min(max(m, 0), M - 1);
    atomicAdd(&s_n[k], 1);
    atomicAdd(&s_acc[k], ok);
    atomicAdd(&s_pred[k], cd);
    atomicAdd(&s_bn[m], 1);
    atomicAdd(&s_bacc[m], ok);
    atomicAdd(&s_bconf[m], cd);
  }
  if (bad) atomicOr(&s_bad, bad);
  __syncthreads();
  long long* st = reinterpret_cast<long long*>(a.state);
  long long* rounds = st;
  long long* wn = st + 1;
  long long* wacc = wn + K;
  double* wpred = reinterpret_cast<double*>(wacc + K);
  long long* wbn = reinterpret_cast<long long*>(wpred + K);
  long long* wbacc = wbn + M;
  double* wbconf = reinterpret_cast<double*>(wbacc + M);
  // this round into the window, one thread per position (threads 0..K-1)
  // or bin (threads 64..64+M-1); whether the window ends is broadcast in LDS
  long long pn = 0, pacc = 0;
  double ppred = 0.0;
  if (tid < K) {
    pn = wn[tid] + s_n[tid];
    pacc = wacc[tid] + s_acc[tid];
    ppred = wpred[tid] + s_pred[tid];
  } else if (tid >= 64 && tid < 64 + M) {
    const int m = tid - 64;
    const long long bn = wbn[m] + s_bn[m];
    const long long bacc = wbacc[m] + s_bacc[m];
    const double bconf = wbconf[m] + s_bconf[m];
    wbn[m] = bn;
    wbacc[m] = bacc;
    wbconf[m] = bconf;
    s_gap[m] = fabs((double)bacc - bconf);
    s_cnt[m] = (int)min(bn, (long long)INT32_MAX);
  }
  __syncthreads();
  if (tid == 0) {
    if (s_bad) flag(a.dev_status, s_bad);
    const long long r = *rounds + 1;
    const int end = r >= a.window;
    *rounds = end ? 0 : r;
    s_end = end;
  }
  __syncthreads();
  const bool end = s_end != 0;
  if (tid < K) {
    if (end && pn > 0) {
      // the temperature step (the same thread holds the position's sums)
      const double err = ppred / (double)pn - (double)pacc / (double)pn;
      const double th = (double)a.theta[tid] + (double)a.lr * err;
      a.theta[tid] = (float)fmax((double)a.theta_min, th);
    }
    wn[tid] = end ? 0 : pn;
    wacc[tid] = end ? 0 : pacc;
    wpred[tid] = end ? 0.0 : ppred;
  }
  if (!end) return;
  if (tid < kWave) {
    // the window's ECE from the bins' gaps and counts (M <= 64: one per lane)
    const double gsum = wave_sum(tid < M ? s_gap[tid] : 0.0);
    const double csum = wave_sum(tid < M ? (double)s_cnt[tid] : 0.0);
    if (tid == 0 && a.ece_out) a.ece_out[0] = csum > 0.0 ? (float)(gsum / csum) : 0.f;
  } else if (tid >= 64 && tid < 64 + M) {
    const int m = tid - 64;
    wbn[m] = 0;
    wbacc[m] = 0;
    wbconf[m] = 0.0;
  }
}

int launch_calibrate(CalibArgs& a, hipStream_t st) {
  const long long n = (long long)a.B * a.K;
  hipLaunchKernelGGL(k_calibrate, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_LAUNCH;
}

int launch_calib_observe(CalibArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_calib_observe, dim3(1), dim3(kCalibThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_LAUNCH;
}

}  // namespace dspark
