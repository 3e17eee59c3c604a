// Launch structures of the snapshot-verify baseline (rs_snapshot.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rs {

struct SnapArgs {
  int B, T, hk, hv, dk, dv, G, NV, nblocks, num_slots;
  float scale;              // query scale of the outputs
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  const void* gate;
  const void* state;        // [num_slots, hv, dk, dv], read only
  void* snapshots;          // [B, T, hv, dk, dv], state dtype
  const int32_t* slot_idx;
  float* out;               // [B*T, hv, dv]
};

struct SnapCommitArgs {
  int B, T, hv, dk, dv, num_slots, elem_bytes;
  void* state;
  const void* snapshots;
  const int32_t* slot_idx;
  const int32_t* accept;
};

// LDS bytes of one snapshot-verify workgroup (dk x bv fp32 tile, partial sums, k, q and
// per-channel gates of the current token, one delta per column).
inline int snapshot_lds_bytes(int dk, int bv) {
  const int ng = 256 / bv;
  return 4 * (dk * bv + ng * bv + 3 * dk + bv);
}

hipError_t launch_snapshot_verify(bool kda, int act_bf16, int state_bf16, int bv,
                                  const SnapArgs& a, hipStream_t s);
hipError_t launch_snapshot_commit(const SnapCommitArgs& a, hipStream_t s);

}  // namespace rs
