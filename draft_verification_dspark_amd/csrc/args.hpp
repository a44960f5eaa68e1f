// Argument block of the verify kernels, passed by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace dspark {

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
  char* sync;          // sync block: start counter, per request a tag line and a counter line
  Partial* part1;      // [B*(K+1)*2*G] chunk summaries, (request, row j, side) major
  ResidualChunk* part2;  // [B*QT] residual sums per quarter chunk of the rejected row pair
  int B, K, V, G;
  int QT;              // quarter tasks per request: one per quarter chunk up to the row's end
  int greedy_only;
  int vec_ok;
};

struct ScheduleArgs;

// phases: kPhaseStream enqueues the streaming pass, kPhaseFinish the launches
// after it (decide, draw), both the whole call.
// fused: the schedule to work out inside the streaming pass (at most
// kFusedMaxB requests and kFusedMaxPositions positions), else NULL.
constexpr int kPhaseStream = DSPARK_PHASE_STREAM;
constexpr int kPhaseFinish = DSPARK_PHASE_FINISH;
int launch_verify(VerifyArgs& a, int dtype, hipStream_t st, int phases,
                  const ScheduleArgs* fused = nullptr);
int compute_units();  // of the current device

// Requests per launch sequence of dspark_verify (the streaming kernel keeps
// a per-request plan of this many entries in LDS); larger batches run as
// consecutive sub-batches on the same stream.
constexpr int kLaunchBatch = 2048;

// The sync block at the start of a verify workspace (k_finish): two 128-byte
// lines per request of a launch (tag and draw state, done counter).  The
// streaming pass clears the tags, so the block needs no initialisation.
constexpr int kSyncLine = 128;
inline size_t sync_bytes(int B) { return (size_t)2 * B * kSyncLine; }

// Largest batch whose schedule the fused schedule + verify call works out
// inside the streaming pass (one request per thread of a streaming
// workgroup, at most 16 positions per request, every position's key in
// LDS); larger batches launch the schedule on its own first.
constexpr int kFusedMaxB = 512;
constexpr int kFusedMaxK = 16;  // a thread's confidences are loaded in one round trip
constexpr int kFusedMaxPositions = 12288;

}  // namespace dspark
