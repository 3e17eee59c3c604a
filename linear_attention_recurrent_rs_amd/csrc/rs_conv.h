// Launch structures of the short causal convolution and its window rollback (rs_conv.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rs_internal.h"

namespace rs {

struct ConvArgs {
  int B, T, C, num_slots;
  int layers;                // commit: layers rolled back by one launch (grid y)
  size_t state_layer_stride; // commit: elements between layers' states
  size_t x_layer_stride;     // commit: elements between layers' window inputs
  int out_bf16;              // y in bf16 (round to nearest even) instead of fp32
  int silu;                  // apply x * sigmoid(x) after the bias
  const void* x;             // [tokens, C] window inputs, act dtype
  const void* weight;        // [C, K] act dtype, tap K-1 on the current input
  const void* bias;          // [C] act dtype or NULL
  const void* state;         // [num_slots, K-1, C] act dtype (verify: read only)
  void* state_rw;            // the same, written by the commit
  const int32_t* slot_idx;   // [B]
  const int32_t* accept;     // [B] (commit)
  void* y;                   // [tokens, C] out dtype (verify)
};

hipError_t launch_conv_verify(bool act_bf16, int width, int tmax, const ConvArgs& a,
                              const RowWindows& w, hipStream_t s);
hipError_t launch_conv_commit(bool act_bf16, int width, const ConvArgs& a,
                              const RowWindows& w, hipStream_t s);

}  // namespace rs
