// C ABI of the ReplaySSM library: host-side validation, tile choice and kernel launch.
// Every entry point enqueues on the caller's stream and returns without synchronising.
#include <cmath>

#include "rs.h"
#include "rs_internal.h"
#include "rs_conv.h"
#include "rs_prefill.h"
#include "rs_snapshot.h"

namespace {

constexpr int kMaxLds = 160 * 1024;   // LDS per workgroup on gfx950

bool dtype_ok(rs_dtype d) { return d == RS_F32 || d == RS_BF16; }
int dbytes(rs_dtype d) { return d == RS_BF16 ? 2 : 4; }

rs_status check_common(const rs_dims* d, bool need_T) {
  if (!d) return RS_E_NULLPTR;
  if (!dtype_ok(d->act_dtype) || !dtype_ok(d->state_dtype)) return RS_E_DTYPE;
  if (d->batch < 0 || d->hk < 1 || d->hv < 1 || d->hv % d->hk != 0) return RS_E_SHAPE;
  if (d->dk < 16 || d->dk > 256 || d->dk % 16 != 0) return RS_E_SHAPE;
  if (d->dv < 16 || d->dv % 16 != 0) return RS_E_SHAPE;
  if (d->num_slots < 1 || d->ring_cap < 1 || d->ring_cap > 256) return RS_E_SHAPE;
  if (need_T && (d->T < 1 || d->T > 16)) return RS_E_SHAPE;
  if (need_T && d->ring_cap < d->T) return RS_E_RING_TOO_SMALL;
  if (d->tile_v != 0) {
    if (d->tile_v != 16 && d->tile_v != 32 && d->tile_v != 64 && d->tile_v != 128) return RS_E_SHAPE;
    if (d->dv % d->tile_v != 0) return RS_E_SHAPE;
  }
  return RS_OK;
}

// The query scale the verifies apply to their outputs: finite and nonzero.
bool scale_ok(const rs_dims* d) { return std::isfinite(d->scale) && d->scale != 0.f; }

int tmax_of(int T) {
  int t = 1;
  while (t < T) t <<= 1;
  return t;
}

// Value columns per workgroup: the caller's tile, else the widest of 64/32/16 dividing dv.
int choose_bv(const rs_dims* d) {
  if (d->tile_v) return d->tile_v;
  if (d->dv % 64 == 0) return 64;
  if (d->dv % 32 == 0) return 32;
  return 16;
}

// The dk = 128 / bf16-input kernels (rs_verify_fast.hip, rs_fold_fast.hip) cover the tile
// widths 32, 64 and 128; every other shape takes the general kernels (rs_kernels.hip).
bool use_fast(const rs_dims* d, int bv) {
  return d->dk == 128 && d->act_dtype == RS_BF16 && (bv == 32 || bv == 64 || bv == 128);
}

struct VerifyPlan {
  int bv = 0, tmax = 0;
  bool fast = false;
  rs::LdsLayout lay{};
  rs::FastLayout flay{};
  int lds() const { return fast ? flay.total : lay.total; }
};

rs_status verify_plan(const rs_dims* d, bool kda, VerifyPlan* p) {
  rs_status st = check_common(d, true);
  if (st != RS_OK) return st;
  if (kda && d->hv != d->hk) return RS_E_SHAPE;
  if (!scale_ok(d)) return RS_E_VALUE;
  p->bv = choose_bv(d);
  // a bf16 state tile of 64 columns is only 16 KB: the fast verify takes whole 128-column
  // rows then, so that a workgroup moves as many bytes as an fp32 tile of 64 columns
  if (d->tile_v == 0 && d->state_dtype == RS_BF16 && d->dv % 128 == 0 && use_fast(d, 128))
    p->bv = 128;
  for (;;) {
    p->fast = use_fast(d, p->bv);
    // the fast verify is compiled for every window up to 4 and for 8 and 16 beyond
    p->tmax = (p->fast && d->T <= 4) ? d->T : tmax_of(d->T);
    if (p->fast) p->flay = rs::fast_layout(kda, d->state_dtype == RS_BF16, p->bv, p->tmax, d->T,
                                           d->ring_cap);
    else p->lay = rs::verify_layout(kda, dbytes(d->state_dtype), p->bv, p->tmax, d->T, d->dk,
                                    d->ring_cap);
    if (p->lds() <= kMaxLds || d->tile_v != 0 || p->bv <= 16) break;
    p->bv /= 2;
  }
  if (p->lds() > kMaxLds) return RS_E_SHAPE;
  return RS_OK;
}

// cu_seqlens == NULL: every row verifies T tokens; else row r verifies tokens
// [cu_seqlens[r], cu_seqlens[r + 1]) of ntok packed tokens.
rs_status verify_impl(bool kda, const rs_dims* d, const int32_t* cu_seqlens, int32_t ntok,
                      const void* q, const void* k, const void* v,
                      const void* beta, const void* gate, void* state, void* ring_k,
                      float* ring_d, float* ring_g, const int32_t* cursor,
                      const int32_t* slot_idx, float* out, int32_t* write_pos_out,
                      int32_t* group_counter, hipStream_t stream) {
  VerifyPlan plan;
  rs_status st = verify_plan(d, kda, &plan);
  if (st != RS_OK) return st;
  if (cu_seqlens && ntok < 0) return RS_E_SHAPE;
  if (d->batch == 0) return RS_OK;
  if (!q || !k || !v || !beta || !gate || !state || !ring_k || !ring_d || !ring_g || !cursor ||
      !slot_idx || !out || !group_counter)
    return RS_E_NULLPTR;
  const int bv = plan.bv;
  rs::VerifyArgs a{};
  a.B = d->batch; a.T = d->T; a.hk = d->hk; a.hv = d->hv; a.dk = d->dk; a.dv = d->dv;
  a.L = d->ring_cap; a.G = d->hv / d->hk; a.NV = d->dv / bv; a.num_slots = d->num_slots;
  a.nblocks = d->batch * d->hv * a.NV; a.scale = d->scale;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.gate = gate;
  a.state = state; a.ring_k = ring_k; a.ring_d = ring_d; a.ring_g = ring_g;
  a.cursor = cursor; a.slot_idx = slot_idx; a.out = out; a.write_pos_out = write_pos_out;
  a.group_counter = group_counter; a.lay = plan.lay;
  const rs::RowWindows w{cu_seqlens, ntok};
  hipError_t e = plan.fast
      ? rs::launch_verify_fast(kda, d->state_dtype == RS_BF16, bv, plan.tmax, a, plan.flay, w,
                               stream)
      : rs::launch_verify(kda, d->act_dtype == RS_BF16, d->state_dtype == RS_BF16, bv, plan.tmax,
                          a, w, stream);
  return e == hipSuccess ? RS_OK : RS_E_LAUNCH;
}

rs_status fold_impl(const rs_dims* d, int is_kda, const void* state_in, void* state_out,
                    const void* ring_k, const float* ring_d, const float* ring_g,
                    const int32_t* nrec, const int32_t* slot_idx, bool materialize,
                    hipStream_t stream) {
  rs_status st = check_common(d, false);
  if (st != RS_OK) return st;
  const bool kda = is_kda != 0;
  if (kda && d->hv != d->hk) return RS_E_SHAPE;
  int bv = choose_bv(d);
  // dk = 128 with bf16 keys and a bf16 state, in whole 128-column rows: the row-coalesced
  // fold (rs_fold_fast.hip fold_bf16_kernel), when its records fit in LDS
  if (d->state_dtype == RS_BF16 && (d->tile_v == 0 || d->tile_v == 128) && d->dv % 128 == 0 &&
      use_fast(d, 128)) {
    const rs::FoldFastLayout flay = rs::fold_fast_layout(kda, 128, d->ring_cap, false);
    if (flay.total <= kMaxLds) {
      if (d->batch == 0) return RS_OK;
      if (!state_in || !state_out || !ring_k || !ring_d || !ring_g || !nrec || !slot_idx)
        return RS_E_NULLPTR;
      rs::FoldArgs a{};
      a.B = d->batch; a.hk = d->hk; a.hv = d->hv; a.dk = d->dk; a.dv = d->dv;
      a.L = d->ring_cap; a.G = d->hv / d->hk; a.NV = d->dv / 128; a.num_slots = d->num_slots;
      a.nblocks = d->batch * d->hv * a.NV;
      a.state_in = state_in; a.state_out = state_out; a.ring_k = ring_k; a.ring_d = ring_d;
      a.ring_g = ring_g; a.nrec = nrec; a.slot_idx = slot_idx;
      return rs::launch_fold_bf16(kda, materialize, a, flay, stream) == hipSuccess ? RS_OK
                                                                                 : RS_E_LAUNCH;
    }
  }
  // dk = 128 with bf16 keys and an fp32 state: the register-tile MFMA fold
  // (rs_fold_fast.hip).  A bf16 state would reach those registers by 8-byte loads, 32-byte
  // row pieces per 16-column block; it takes the fold above or the LDS-staged fold
  // (rs_kernels.hip).
  const bool f32_state = d->state_dtype == RS_F32;
  bool fast = false;
  rs::FoldFastLayout flay{};
  rs::LdsLayout lay{};
  for (;;) {
    fast = f32_state && use_fast(d, bv);
    if (fast) flay = rs::fold_fast_layout(kda, bv, d->ring_cap, true);
    else lay = rs::fold_layout(kda, dbytes(d->state_dtype), bv, d->dk, d->ring_cap, false);
    const int lds = fast ? flay.total : lay.total;
    if (lds <= kMaxLds || d->tile_v != 0 || bv <= 16) break;
    bv /= 2;
  }
  if ((fast ? flay.total : lay.total) > kMaxLds) return RS_E_SHAPE;
  if (d->batch == 0) return RS_OK;
  if (!state_in || !state_out || !ring_k || !ring_d || !ring_g || !nrec || !slot_idx)
    return RS_E_NULLPTR;
  rs::FoldArgs a{};
  a.B = d->batch; a.hk = d->hk; a.hv = d->hv; a.dk = d->dk; a.dv = d->dv; a.L = d->ring_cap;
  a.G = d->hv / d->hk; a.NV = d->dv / bv; a.num_slots = d->num_slots;
  a.nblocks = d->batch * d->hv * a.NV;
  a.state_in = state_in; a.state_out = state_out; a.ring_k = ring_k; a.ring_d = ring_d;
  a.ring_g = ring_g; a.nrec = nrec; a.slot_idx = slot_idx; a.lay = lay;
  hipError_t e = fast
      ? rs::launch_fold_fast(kda, d->state_dtype == RS_BF16, bv, materialize, a, flay, stream)
      : rs::launch_fold(kda, d->act_dtype == RS_BF16, d->state_dtype == RS_BF16, bv,
                        materialize, a, stream);
  return e == hipSuccess ? RS_OK : RS_E_LAUNCH;
}

rs_status conv_check(const rs_conv_dims* d, const int32_t* cu_seqlens, int32_t ntok) {
  if (!d) return RS_E_NULLPTR;
  if (!dtype_ok(d->act_dtype) || !dtype_ok(d->out_dtype)) return RS_E_DTYPE;
  if (d->batch < 0 || d->T < 1 || d->T > 16 || d->num_slots < 1) return RS_E_SHAPE;
  if (d->channels < 8 || d->channels % 8 != 0) return RS_E_SHAPE;
  if (d->width < 2 || d->width > 4) return RS_E_SHAPE;
  if (cu_seqlens && ntok < 0) return RS_E_SHAPE;
  if (d->activation != RS_ACT_NONE && d->activation != RS_ACT_SILU) return RS_E_VALUE;
  return RS_OK;
}

rs::ConvArgs conv_args(const rs_conv_dims* d) {
  rs::ConvArgs a{};
  a.B = d->batch; a.T = d->T; a.C = d->channels; a.num_slots = d->num_slots; a.layers = 1;
  a.out_bf16 = d->out_dtype == RS_BF16; a.silu = d->activation == RS_ACT_SILU;
  return a;
}

}  // namespace

extern "C" {

rs_status rs_gdn_prefill(const rs_dims* dims, const int32_t* cu_seqlens, int32_t total_tokens,
                         const void* q, const void* k, const void* v, const void* beta,
                         const void* gate, void* state, int32_t* cursor,
                         const int32_t* slot_idx, float* out, hipStream_t stream) {
  if (!dims) return RS_E_NULLPTR;
  const rs_dims* d = dims;
  if (!dtype_ok(d->act_dtype) || !dtype_ok(d->state_dtype)) return RS_E_DTYPE;
  if (d->act_dtype != RS_BF16) return RS_E_DTYPE;
  if (d->batch < 0 || d->hk < 1 || d->hv < 1 || d->hv % d->hk != 0 || d->num_slots < 1)
    return RS_E_SHAPE;
  if (d->dk != 128 || d->dv < 64 || d->dv % 64 != 0 || total_tokens < 0) return RS_E_SHAPE;
  if (!scale_ok(d)) return RS_E_VALUE;
  if (d->batch == 0) return RS_OK;
  if (!cu_seqlens || !q || !k || !v || !beta || !gate || !state || !cursor || !slot_idx || !out)
    return RS_E_NULLPTR;
  rs::PrefillArgs a{};
  a.B = d->batch; a.hk = d->hk; a.hv = d->hv; a.dv = d->dv; a.G = d->hv / d->hk;
  a.NV = d->dv / 64; a.nblocks = d->batch * d->hv * a.NV; a.num_slots = d->num_slots;
  a.ntok = total_tokens; a.scale = d->scale; a.cu_seqlens = cu_seqlens;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.gate = gate; a.state = state; a.cursor = cursor;
  a.slot_idx = slot_idx; a.out = out;
  return rs::launch_prefill(d->state_dtype == RS_BF16, a, stream) == hipSuccess ? RS_OK
                                                                               : RS_E_LAUNCH;
}

rs_status rs_conv_verify(const rs_conv_dims* dims, const int32_t* cu_seqlens,
                         int32_t total_tokens, const void* x, const void* weight,
                         const void* bias, const void* conv_state, const int32_t* slot_idx,
                         void* y, hipStream_t stream) {
  const rs_status st = conv_check(dims, cu_seqlens, total_tokens);
  if (st != RS_OK) return st;
  if (dims->batch == 0) return RS_OK;
  if (!x || !weight || !conv_state || !slot_idx || !y) return RS_E_NULLPTR;
  rs::ConvArgs a = conv_args(dims);
  a.x = x; a.weight = weight; a.bias = bias; a.state = conv_state; a.slot_idx = slot_idx;
  a.y = y;
  const rs::RowWindows w{cu_seqlens, total_tokens};
  return rs::launch_conv_verify(dims->act_dtype == RS_BF16, dims->width, tmax_of(dims->T), a, w,
                                stream) == hipSuccess ? RS_OK : RS_E_LAUNCH;
}

rs_status rs_conv_commit(const rs_conv_dims* dims, const int32_t* cu_seqlens,
                         int32_t total_tokens, int32_t layers, void* conv_state, const void* x,
                         const int32_t* slot_idx, const int32_t* accept_len,
                         hipStream_t stream) {
  const rs_status st = conv_check(dims, cu_seqlens, total_tokens);
  if (st != RS_OK) return st;
  if (layers < 1 || layers > 65535) return RS_E_SHAPE;
  if (dims->batch == 0) return RS_OK;
  if (!conv_state || !x || !slot_idx || !accept_len) return RS_E_NULLPTR;
  rs::ConvArgs a = conv_args(dims);
  a.x = x; a.state_rw = conv_state; a.slot_idx = slot_idx; a.accept = accept_len;
  a.layers = layers;
  a.state_layer_stride = (size_t)dims->num_slots * (dims->width - 1) * dims->channels;
  a.x_layer_stride = (size_t)(cu_seqlens ? total_tokens : dims->batch * dims->T) * dims->channels;
  const rs::RowWindows w{cu_seqlens, total_tokens};
  return rs::launch_conv_commit(dims->act_dtype == RS_BF16, dims->width, a, w, stream) ==
                 hipSuccess ? RS_OK : RS_E_LAUNCH;
}


rs_status rs_gdn_verify(const rs_dims* dims, const void* q, const void* k, const void* v,
                        const void* beta, const void* gate, void* state, void* ring_k,
                        float* ring_d, float* ring_g, const int32_t* cursor,
                        const int32_t* slot_idx, float* out, int32_t* write_pos_out,
                        int32_t* group_counter, hipStream_t stream) {
  return verify_impl(false, dims, nullptr, 0, q, k, v, beta, gate, state, ring_k, ring_d, ring_g,
                     cursor, slot_idx, out, write_pos_out, group_counter, stream);
}

rs_status rs_kda_verify(const rs_dims* dims, const void* q, const void* k, const void* v,
                        const void* beta, const void* gate, void* state, void* ring_k,
                        float* ring_d, float* ring_g, const int32_t* cursor,
                        const int32_t* slot_idx, float* out, int32_t* write_pos_out,
                        int32_t* group_counter, hipStream_t stream) {
  return verify_impl(true, dims, nullptr, 0, q, k, v, beta, gate, state, ring_k, ring_d, ring_g,
                     cursor, slot_idx, out, write_pos_out, group_counter, stream);
}

rs_status rs_gdn_verify_varlen(const rs_dims* dims, const int32_t* cu_seqlens,
                               int32_t total_tokens, const void* q, const void* k,
                               const void* v, const void* beta, const void* gate, void* state,
                               void* ring_k, float* ring_d, float* ring_g,
                               const int32_t* cursor, const int32_t* slot_idx, float* out,
                               int32_t* write_pos_out, int32_t* group_counter,
                               hipStream_t stream) {
  if (!cu_seqlens && dims && dims->batch > 0) return RS_E_NULLPTR;
  return verify_impl(false, dims, cu_seqlens, total_tokens, q, k, v, beta, gate, state, ring_k,
                     ring_d, ring_g, cursor, slot_idx, out, write_pos_out, group_counter, stream);
}

rs_status rs_kda_verify_varlen(const rs_dims* dims, const int32_t* cu_seqlens,
                               int32_t total_tokens, const void* q, const void* k,
                               const void* v, const void* beta, const void* gate, void* state,
                               void* ring_k, float* ring_d, float* ring_g,
                               const int32_t* cursor, const int32_t* slot_idx, float* out,
                               int32_t* write_pos_out, int32_t* group_counter,
                               hipStream_t stream) {
  if (!cu_seqlens && dims && dims->batch > 0) return RS_E_NULLPTR;
  return verify_impl(true, dims, cu_seqlens, total_tokens, q, k, v, beta, gate, state, ring_k,
                     ring_d, ring_g, cursor, slot_idx, out, write_pos_out, group_counter, stream);
}

rs_status rs_gdn_verify_noalloc(const rs_dims* dims, const void* q, const void* k,
                                const void* v, const void* beta, const void* gate, void* state,
                                void* ring_k, float* ring_d, float* ring_g,
                                const int32_t* cursor, const int32_t* slot_idx, float* out,
                                int32_t* write_pos_out, hipStream_t stream) {
  VerifyPlan plan;
  rs_status st = verify_plan(dims, false, &plan);
  if (st != RS_OK) return st;
  if ((int64_t)dims->batch * dims->hk > rs::kNoAllocCounters) return RS_E_SCRATCH;
  if (dims->batch == 0) return RS_OK;
  int32_t* counters = nullptr;
  if (rs::noalloc_counters(&counters) != hipSuccess) return RS_E_LAUNCH;
  if (rs::launch_zero_counters(counters, dims->batch * dims->hk, stream) != hipSuccess)
    return RS_E_LAUNCH;
  return verify_impl(false, dims, nullptr, 0, q, k, v, beta, gate, state, ring_k, ring_d, ring_g,
                     cursor, slot_idx, out, write_pos_out, counters, stream);
}

static rs_status advance_impl(const rs_dims* dims, const int32_t* cu_seqlens, int32_t ntok,
                              int32_t* cursor, int32_t* fold_len, const int32_t* slot_idx,
                              const int32_t* accept_len, rs_fold_policy policy, int32_t next_T,
                              const uint8_t* force_mask, hipStream_t stream) {
  if (!dims) return RS_E_NULLPTR;
  if (dims->batch < 0 || dims->T < 1 || dims->T > 16 || dims->num_slots < 1 ||
      dims->ring_cap < 1 || dims->ring_cap > 256)
    return RS_E_SHAPE;
  if (dims->ring_cap < dims->T) return RS_E_RING_TOO_SMALL;
  if (policy < RS_FOLD_NONE || policy > RS_FOLD_FORCE) return RS_E_SHAPE;
  if (policy == RS_FOLD_LAZY && (next_T < 1 || next_T > 16)) return RS_E_SHAPE;
  if (cu_seqlens && ntok < 0) return RS_E_SHAPE;
  if (dims->batch == 0) return RS_OK;
  if (!cursor || !fold_len || !slot_idx || !accept_len) return RS_E_NULLPTR;
  rs::AdvanceArgs a{};
  a.B = dims->batch; a.T = dims->T; a.L = dims->ring_cap; a.num_slots = dims->num_slots;
  a.policy = int(policy); a.next_T = next_T;
  a.cu_seqlens = cu_seqlens; a.ntok = ntok;
  a.cursor = cursor; a.fold_len = fold_len; a.slot_idx = slot_idx; a.accept = accept_len;
  a.force_mask = force_mask;
  return rs::launch_advance(a, stream) == hipSuccess ? RS_OK : RS_E_LAUNCH;
}

rs_status rs_cursor_advance(const rs_dims* dims, int32_t* cursor, int32_t* fold_len,
                            const int32_t* slot_idx, const int32_t* accept_len,
                            rs_fold_policy policy, int32_t next_T, const uint8_t* force_mask,
                            hipStream_t stream) {
  return advance_impl(dims, nullptr, 0, cursor, fold_len, slot_idx, accept_len, policy, next_T,
                      force_mask, stream);
}

rs_status rs_cursor_advance_varlen(const rs_dims* dims, const int32_t* cu_seqlens,
                                   int32_t total_tokens, int32_t* cursor, int32_t* fold_len,
                                   const int32_t* slot_idx, const int32_t* accept_len,
                                   rs_fold_policy policy, int32_t next_T,
                                   const uint8_t* force_mask, hipStream_t stream) {
  if (!cu_seqlens && dims && dims->batch > 0) return RS_E_NULLPTR;
  return advance_impl(dims, cu_seqlens, total_tokens, cursor, fold_len, slot_idx, accept_len,
                      policy, next_T, force_mask, stream);
}

rs_status rs_commit_fold(const rs_dims* dims, int is_kda, void* state, const void* ring_k,
                         const float* ring_d, const float* ring_g, const int32_t* fold_len,
                         const int32_t* slot_idx, hipStream_t stream) {
  return fold_impl(dims, is_kda, state, state, ring_k, ring_d, ring_g, fold_len, slot_idx,
                   false, stream);
}

rs_status rs_materialize(const rs_dims* dims, int is_kda, const void* state, const void* ring_k,
                         const float* ring_d, const float* ring_g, const int32_t* cursor,
                         const int32_t* slot_idx, float* out_state, hipStream_t stream) {
  if (out_state == nullptr && dims && dims->batch > 0) return RS_E_NULLPTR;
  return fold_impl(dims, is_kda, state, out_state, ring_k, ring_d, ring_g, cursor, slot_idx,
                   true, stream);
}

rs_status rs_snapshot_verify(const rs_dims* dims, int is_kda, const void* q, const void* k,
                             const void* v, const void* beta, const void* gate,
                             const void* state, void* snapshots, const int32_t* slot_idx,
                             float* out, hipStream_t stream) {
  rs_status st = check_common(dims, true);
  if (st != RS_OK) return st;
  const bool kda = is_kda != 0;
  if (kda && dims->hv != dims->hk) return RS_E_SHAPE;
  if (!scale_ok(dims)) return RS_E_VALUE;
  int bv = dims->tile_v ? dims->tile_v : (dims->dv % 64 == 0 ? 64 : dims->dv % 32 == 0 ? 32 : 16);
  if (bv > 64) bv = 64;
  if (dims->dv % bv != 0 || rs::snapshot_lds_bytes(dims->dk, bv) > kMaxLds) return RS_E_SHAPE;
  if (dims->batch == 0) return RS_OK;
  if (!q || !k || !v || !beta || !gate || !state || !snapshots || !slot_idx || !out)
    return RS_E_NULLPTR;
  rs::SnapArgs a{};
  a.B = dims->batch; a.T = dims->T; a.hk = dims->hk; a.hv = dims->hv; a.dk = dims->dk;
  a.dv = dims->dv; a.G = dims->hv / dims->hk; a.NV = dims->dv / bv;
  a.nblocks = dims->batch * dims->hv * a.NV; a.num_slots = dims->num_slots;
  a.scale = dims->scale;
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.gate = gate; a.state = state;
  a.snapshots = snapshots; a.slot_idx = slot_idx; a.out = out;
  return rs::launch_snapshot_verify(kda, dims->act_dtype == RS_BF16, dims->state_dtype == RS_BF16,
                                    bv, a, stream) == hipSuccess ? RS_OK : RS_E_LAUNCH;
}

rs_status rs_snapshot_commit(const rs_dims* dims, void* state, const void* snapshots,
                             const int32_t* slot_idx, const int32_t* accept_len,
                             hipStream_t stream) {
  rs_status st = check_common(dims, true);
  if (st != RS_OK) return st;
  if (dims->batch == 0) return RS_OK;
  if (!state || !snapshots || !slot_idx || !accept_len) return RS_E_NULLPTR;
  rs::SnapCommitArgs a{};
  a.B = dims->batch; a.T = dims->T; a.hv = dims->hv; a.dk = dims->dk; a.dv = dims->dv;
  a.num_slots = dims->num_slots; a.elem_bytes = dbytes(dims->state_dtype);
  a.state = state; a.snapshots = snapshots; a.slot_idx = slot_idx; a.accept = accept_len;
  return rs::launch_snapshot_commit(a, stream) == hipSuccess ? RS_OK : RS_E_LAUNCH;
}

const char* rs_status_str(rs_status s) {
  switch (s) {
    case RS_OK: return "RS_OK";
    case RS_E_NULLPTR: return "RS_E_NULLPTR: a required pointer is NULL";
    case RS_E_SHAPE: return "RS_E_SHAPE: unsupported or inconsistent dimensions";
    case RS_E_DTYPE: return "RS_E_DTYPE: unsupported dtype";
    case RS_E_RING_TOO_SMALL: return "RS_E_RING_TOO_SMALL: ring_cap < T";
    case RS_E_LAUNCH: return "RS_E_LAUNCH: kernel launch failed";
    case RS_E_VALUE: return "RS_E_VALUE: a scalar argument is out of range (scale)";
    case RS_E_SCRATCH:
      return "RS_E_SCRATCH: batch * hk exceeds the allocation-free verify's static workspace";
  }
  return "unknown rs_status";
}

rs_status rs_verify_launch_info(const rs_dims* dims, int is_kda, int32_t* tile_v,
                                int32_t* workgroups, int32_t* lds_bytes) {
  VerifyPlan plan;
  rs_status st = verify_plan(dims, is_kda != 0, &plan);
  if (st != RS_OK) return st;
  if (tile_v) *tile_v = plan.bv;
  if (workgroups) *workgroups = dims->batch * dims->hv * (dims->dv / plan.bv);
  if (lds_bytes) *lds_bytes = plan.lds();
  return RS_OK;
}

}  // extern "C"
