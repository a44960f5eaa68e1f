// Argument block of the Markov drafting kernels, passed by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace dspark {

constexpr int kMarkovRows = 64;      // vocabulary rows per workgroup tile
constexpr int kMarkovBatch = 64;     // requests per workgroup tile
constexpr int kMarkovMaxRank = 256;  // rank r: a multiple of 16, at most this

struct MarkovArgs {
  const void* base;          // [B,K,V] parallel logits (dtype)
  const uint16_t* U;         // [V,r] bf16
  const uint16_t* Vm;        // [V,r] bf16
  int r;
  float scale;
  const int32_t* y0;         // [B] token before the block
  const float* temperature;  // [B]
  const float* uniforms;     // [B,K]
  void* corrected;           // [B,K,V] out (dtype)
  int32_t* drafted;          // [B,K] out
  float* q_tok;              // [B,K] out or null
  int32_t* dev_status;
  Partial* part;             // [B, tiles] workspace: per-tile softmax summaries
  int B, K, V, tiles;
  int step;                  // position k (1-based) of this launch pair
};

int launch_markov(MarkovArgs& a, int dtype, hipStream_t st);
int compute_units();  // of the current device

}  // namespace dspark
