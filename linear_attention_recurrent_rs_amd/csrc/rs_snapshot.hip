// Snapshot verify: the baseline design that ReplaySSM replaces (sglang PR: the snapshot
// verify keeps one full state per draft token, 72.6 GB against 3.04 GB of ring at TP1
// with 128 requests; the commit scatters the accepted snapshot).  Kept for the A/B
// comparison in time and memory, not on the hot path.
//
// One workgroup per (value tile, value head, request).  The [dk x BV] tile sits in LDS in
// fp32; thread (c, g) owns column c of rows [g dk/NG, (g+1) dk/NG), so each token is
//   S <- alpha (.) S;  d = beta (v - S^T k);  S <- S + k d^T;  o = S^T q
// with two cross-thread column sums (one LDS round each), and S after each token is
// written out, rounded to the state dtype.  Tokens run strictly in order, so a value at
// draft t reaches only snapshots and outputs from t on.
#include "rs_device.h"
#include "rs_snapshot.h"

namespace rs {

template <bool KDA, typename AT, typename ST, int BV>
__global__ __launch_bounds__(kThreads) void snapshot_verify_kernel(SnapArgs a) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  constexpr int NG = kThreads / BV;
  const int tid = threadIdx.x, c = tid % BV, g = tid / BV;
  const int lid = xcd_remap(blockIdx.x, a.nblocks);
  const int vt = umod(lid, a.NV);
  const int h = umod(udiv(lid, a.NV), a.hv);
  const int row = udiv(lid, a.NV * a.hv);
  const int slot = a.slot_idx[row];
  if (slot < 0 || slot >= a.num_slots) return;          // null row: no reads, no writes
  const int dk = a.dk, dv = a.dv, hv = a.hv, hk = a.hk, T = a.T;
  const int kh = udiv(h, a.G), col0 = vt * BV, rp = dk / NG, r0 = g * rp;

  float* tile = sm;                  // [dk x BV]
  float* part = tile + dk * BV;      // [NG x BV]
  float* kq = part + NG * BV;        // k_t [dk], q_t [dk]
  float* gv = kq + 2 * dk;           // KDA gates of token t [dk]
  float* dd = gv + dk;               // d_t [BV]

  const AT* qg = static_cast<const AT*>(a.q);
  const AT* kg = static_cast<const AT*>(a.k);
  const AT* vg = static_cast<const AT*>(a.v);
  const AT* bg = static_cast<const AT*>(a.beta);
  const AT* gg = static_cast<const AT*>(a.gate);
  const ST* S = static_cast<const ST*>(a.state) + ((size_t)slot * hv + h) * dk * dv + col0;
  for (int r = r0; r < r0 + rp; ++r) tile[r * BV + c] = to_f32(S[(size_t)r * dv + c]);

  for (int t = 0; t < T; ++t) {
    const size_t tok = (size_t)row * T + t;
    for (int i = tid; i < dk; i += kThreads) {
      kq[i] = to_f32(kg[(tok * hk + kh) * dk + i]);
      kq[dk + i] = to_f32(qg[(tok * hk + kh) * dk + i]);
      if (KDA) gv[i] = to_f32(gg[(tok * hv + h) * dk + i]);
    }
    __syncthreads();
    const float alpha = KDA ? 1.f : to_f32(gg[tok * hv + h]);
    const float beta = to_f32(bg[tok * hv + h]);
    float acc = 0.f;
    for (int r = r0; r < r0 + rp; ++r) {
      const float sv = tile[r * BV + c] * (KDA ? gv[r] : alpha);
      tile[r * BV + c] = sv;
      acc = fmaf(sv, kq[r], acc);
    }
    part[g * BV + c] = acc;
    __syncthreads();
    if (tid < BV) {
      float p = 0.f;
      for (int j = 0; j < NG; ++j) p += part[j * BV + tid];
      dd[tid] = beta * (to_f32(vg[(tok * hv + h) * dv + col0 + tid]) - p);
    }
    __syncthreads();
    const float d = dd[c];
    ST* snap = static_cast<ST*>(a.snapshots) + (tok * hv + h) * dk * dv + col0;
    acc = 0.f;
    for (int r = r0; r < r0 + rp; ++r) {
      const float sv = fmaf(kq[r], d, tile[r * BV + c]);
      tile[r * BV + c] = sv;
      acc = fmaf(sv, kq[dk + r], acc);
      snap[(size_t)r * dv + c] = from_f32<ST>(sv);
    }
    part[g * BV + c] = acc;
    __syncthreads();
    if (tid < BV) {
      float o = 0.f;
      for (int j = 0; j < NG; ++j) o += part[j * BV + tid];
      a.out[(tok * hv + h) * dv + col0 + tid] = o * a.scale;
    }
    __syncthreads();                 // k, q, gates and partials are rewritten next token
  }
}

// state[slot] <- snapshot[row, accept - 1] for live rows with accept > 0 (16-byte copies).
__global__ __launch_bounds__(kThreads) void snapshot_commit_kernel(SnapCommitArgs a) {
  const int row = blockIdx.x / a.hv, h = blockIdx.x % a.hv;
  const int slot = a.slot_idx[row];
  if (slot < 0 || slot >= a.num_slots) return;
  int acc = a.accept[row];
  acc = acc < 0 ? 0 : (acc > a.T ? a.T : acc);
  if (acc == 0) return;
  const size_t bytes = (size_t)a.dk * a.dv * a.elem_bytes;
  const uint4* src = reinterpret_cast<const uint4*>(
      static_cast<const char*>(a.snapshots) + (((size_t)row * a.T + acc - 1) * a.hv + h) * bytes);
  uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(a.state) + ((size_t)slot * a.hv + h) * bytes);
  for (size_t i = threadIdx.x; i < bytes / 16; i += kThreads) dst[i] = src[i];
}

template <bool KDA, typename AT, typename ST, int BV>
static hipError_t run_snapshot(const SnapArgs& a, hipStream_t s) {
  auto k = snapshot_verify_kernel<KDA, AT, ST, BV>;
  const int lds = snapshot_lds_bytes(a.dk, BV);
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  hipLaunchKernelGGL(k, dim3(a.nblocks), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <bool KDA, typename AT, typename ST>
static hipError_t snapshot_bv(int bv, const SnapArgs& a, hipStream_t s) {
  switch (bv) {
    case 16: return run_snapshot<KDA, AT, ST, 16>(a, s);
    case 32: return run_snapshot<KDA, AT, ST, 32>(a, s);
    case 64: return run_snapshot<KDA, AT, ST, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

template <bool KDA>
static hipError_t snapshot_types(int act_bf16, int state_bf16, int bv, const SnapArgs& a,
                                 hipStream_t s) {
  if (act_bf16) return state_bf16 ? snapshot_bv<KDA, bf16, bf16>(bv, a, s)
                                  : snapshot_bv<KDA, bf16, float>(bv, a, s);
  return state_bf16 ? snapshot_bv<KDA, float, bf16>(bv, a, s)
                    : snapshot_bv<KDA, float, float>(bv, a, s);
}

hipError_t launch_snapshot_verify(bool kda, int act_bf16, int state_bf16, int bv,
                                  const SnapArgs& a, hipStream_t s) {
  return kda ? snapshot_types<true>(act_bf16, state_bf16, bv, a, s)
             : snapshot_types<false>(act_bf16, state_bf16, bv, a, s);
}

hipError_t launch_snapshot_commit(const SnapCommitArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(snapshot_commit_kernel, dim3(a.B * a.hv), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace rs
