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
  int32_t* n_rows;     // [1]
  int32_t* rows;       // [B*(2K+1)]
  Partial* part1;      // [B*(2K+1)*G]
  double* part2;       // [B*G]
  int B, K, V, G;
  int greedy_only;
  int vec_ok;
};

int launch_verify(VerifyArgs& a, int dtype, hipStream_t st);
int launch_schedule(ScheduleArgs& a, hipStream_t st);

}  // namespace dspark
