// Argument blocks passed by value to the kernels of one call.
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

struct VerifyArgs {
  const void* target;  // [B,K+1,V]
  const void* draft;   // [B,K,V]
  const int32_t* drafted;
  const int32_t* lengths;
  const float* temperature;
  const float* uniforms;
  int32_t* accepted;
  int32_t* tokens;
  float* p_tok;
  float* q_tok;
  int32_t* dev_status;
  ReqState* req;       // [B]
  Partial* part1;      // [B*(K+1)*2*G] chunk summaries, (request, row j, side) major
  double* part2;       // [B*G] residual mass per chunk of the rejected row pair
  int B, K, V, G;
  int groups;          // k_decide workgroups per request
  int greedy_only;
  int vec_ok;
};

// ev_before / ev_after: optional events recorded around the streaming pass
int launch_verify(VerifyArgs& a, int dtype, hipStream_t st, hipEvent_t ev_before,
                  hipEvent_t ev_after);
int compute_units();  // of the current device

// Requests per launch sequence of dspark_verify (the streaming kernel keeps
// a per-request plan of this many entries in LDS); larger batches run as
// consecutive sub-batches on the same stream.
constexpr int kLaunchBatch = 2048;
int launch_schedule(ScheduleArgs& a, hipStream_t st);

}  // namespace dspark
