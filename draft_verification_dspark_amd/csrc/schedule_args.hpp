// Argument block of the schedule kernel, passed by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace dspark {

struct ScheduleArgs {
  const float* conf;   // [B,K]
  int B, K;
  float tau;
  int budget;
  int min_len;
  int32_t* lengths;    // [B]
  uint8_t* mask;       // [B,K] or null
  float* surv;         // [B,K] survival (the caller's output or workspace)
  int32_t* lthr;       // [B] workspace
  int32_t* dev_status;
  int vec4;            // K % 4 == 0 and conf, surv 16-byte aligned
  // load-aware mode (non-null `load`): tau and budget above are replaced by
  // the values derived on the device from these
  const float* load;   // [2] queue depth, memory in use
  float q_max, m_max, tau_min, tau_max;
  const float* curve;  // [n_curve][2] (tokens per forward pass, tokens/s)
  int n_curve;
  float slot_cost;
  float* tau_out;      // [1] or null
  int32_t* budget_out; // [1] or null
};

int launch_schedule(ScheduleArgs& a, hipStream_t st);

}  // namespace dspark
