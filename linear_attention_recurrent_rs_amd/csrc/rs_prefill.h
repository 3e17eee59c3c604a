// Launch structures of the chunked GDN prefill (rs_prefill.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rs {

struct PrefillArgs {
  int B, hk, hv, dv, G, NV, nblocks, num_slots, ntok;
  float scale;
  const int32_t* cu_seqlens;   // [B + 1]: row r's prompt is tokens [cu[r], cu[r + 1])
  const void* q;               // [ntok, hk, 128] bf16
  const void* k;
  const void* v;               // [ntok, hv, dv] bf16
  const void* beta;            // [ntok, hv] bf16
  const void* gate;            // [ntok, hv] bf16
  void* state;                 // [num_slots, hv, 128, dv] fp32 or bf16, read and written
  int32_t* cursor;             // [num_slots], set to 0 for live rows
  const int32_t* slot_idx;     // [B]
  float* out;                  // [ntok, hv, dv] fp32
};

int prefill_lds_bytes();
hipError_t launch_prefill(bool state_bf16, const PrefillArgs& a, hipStream_t s);

}  // namespace rs
