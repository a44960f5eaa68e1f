// Argument block of the calibration kernels, passed by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace dspark {

constexpr int kCalibThreads = 1024;
constexpr int kCalibMax = 64;  // positions (K) and bins at most

struct CalibArgs {
  const float* raw;         // [B,K] (k_calibrate)
  const float* calibrated;  // [B,K] (k_calib_observe)
  float* theta;             // [K] per-position temperatures
  int B, K;
  const int32_t* lengths;   // [B] or null (= K)
  const int32_t* accepted;  // [B]
  float lr, theta_min;
  int window, n_bins;
  void* state;              // window state, 8-byte words
  float* ece_out;           // [1] or null
  float* calibrated_out;    // [B,K] (k_calibrate)
  int32_t* dev_status;
};

int launch_calibrate(CalibArgs& a, hipStream_t st);
int launch_calib_observe(CalibArgs& a, hipStream_t st);

}  // namespace dspark
