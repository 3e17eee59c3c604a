// Host <-> device launch structures shared by the kernels and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rs {

// Byte offsets of the regions of a workgroup's dynamic LDS (all 16-byte aligned).
struct LdsLayout {
  int tile_raw;   // state tile as stored [dk x bv], swizzled
  int tile32;     // fp32 tile after history replay or fold (aliases tile_raw for fp32 S)
  int khat;       // history keys scaled by their suffix decay [L4 x dk] fp32
  int dhist;      // history deltas of this tile's columns [L4 x bv] fp32
  int hg;         // history gates [L] (GDN) or [L x dk] (KDA) fp32
  int xraw;       // window q_t, k_t as fp32 [2*tmax x xs_stride]
  int xs;         // window q_t, k_t scaled by the in-window prefix decay [nvec_pad x xs_stride]
  int gw;         // window gates [tmax] (GDN) or [tmax x dk] (KDA)
  int bw;         // window betas [tmax]
  int gam;        // total history decay per key channel [dk]
  int P;          // readout H^T xs [2*tmax x bv]
  int red;        // cross-wave reduction scratch [4 x vpp x bv]
  int Am;         // beta_t (k_t . dec(u,t) k_u), u < t  [tmax x tmax]
  int Qm;         // q_t . dec(u,t) k_u, u <= t          [tmax x tmax]
  int flags;      // [0]: this workgroup is the last of its key group to arrive
  int total;
  int xs_stride;  // dk + 4 floats
  int nvec_pad;   // 2T rounded up to the readout batch
};

struct VerifyArgs {
  int B, T, hk, hv, dk, dv, L, G, NV, nblocks, num_slots;
  float scale;              // query scale of the outputs (fills the padding before q)
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  const void* gate;
  void* state;
  void* ring_k;
  float* ring_d;
  float* ring_g;
  const int32_t* cursor;
  const int32_t* slot_idx;
  float* out;
  int32_t* write_pos_out;
  int32_t* group_counter;
  LdsLayout lay;
};

// Ragged windows: row r verifies tokens [cu_seqlens[r], cu_seqlens[r + 1]) of ntok packed
// tokens (at most T of them); cu_seqlens NULL = every row T tokens at r * T.  The verify
// kernels take it as their last argument, so that the other arguments keep their offsets.
struct RowWindows {
  const int32_t* cu_seqlens;
  int ntok;
};

struct FoldArgs {
  int B, hk, hv, dk, dv, L, G, NV, nblocks, num_slots;
  const void* state_in;     // S (read)
  void* state_out;          // S (commit fold) or the fp32 materialize output
  const void* ring_k;
  const float* ring_d;
  const float* ring_g;
  const int32_t* nrec;      // fold_len (commit) or cursor (materialize), per slot
  const int32_t* slot_idx;
  LdsLayout lay;
};

struct AdvanceArgs {
  int B, T, L, num_slots, policy, next_T;
  int32_t* cursor;
  int32_t* fold_len;
  const int32_t* slot_idx;
  const int32_t* accept;
  const uint8_t* force_mask;
  const int32_t* cu_seqlens;   // ragged windows as in VerifyArgs, or NULL
  int ntok;
};

// The verify window of a request row: its first token and its width.  Uniform windows
// put row r's T tokens at r * T.  Ragged windows read them from the cumulative lengths,
// clamped to the packed token count and to T, so that out-of-contract lengths stay inside
// the caller's buffers (every kernel of a step clamps them the same way).
__device__ __forceinline__ void row_window(const int32_t* cu, int ntok, int T, int row,
                                           int* width, size_t* first) {
  if (cu == nullptr) {
    *width = T;
    *first = (size_t)row * T;
    return;
  }
  int b = cu[row], e = cu[row + 1];
  b = b < 0 ? 0 : (b > ntok ? ntok : b);
  e = e < b ? b : (e > ntok ? ntok : e);
  *width = (e - b) > T ? T : (e - b);
  *first = (size_t)b;
}

// Readout batch: window vectors (2T of them) processed per pass over the tile.
inline int readout_vpp(int tmax) { return 2 * tmax < 8 ? 2 * tmax : 8; }

inline LdsLayout verify_layout(bool kda, int st_bytes, int bv, int tmax, int T, int dk, int L) {
  auto al = [](int x) { return (x + 15) & ~15; };
  const int vpp = readout_vpp(tmax);
  LdsLayout l{};
  int o = 0;
  l.tile_raw = o; o += al(dk * bv * st_bytes);
  if (st_bytes == 4) { l.tile32 = l.tile_raw; } else { l.tile32 = o; o += al(dk * bv * 4); }
  const int L4 = (L + 3) & ~3;
  l.khat = o; o += al(L4 * dk * 4);
  l.dhist = o; o += al(L4 * bv * 4);
  l.hg = o; o += al(kda ? L * dk * 4 : L * 4);
  l.xs_stride = dk + 4;
  l.nvec_pad = ((2 * T + vpp - 1) / vpp) * vpp;
  l.xraw = o; o += al(2 * tmax * l.xs_stride * 4);
  l.xs = o; o += al(l.nvec_pad * l.xs_stride * 4);
  l.gw = o; o += al(kda ? tmax * dk * 4 : tmax * 4);
  l.bw = o; o += al(tmax * 4);
  l.gam = o; o += al(dk * 4);
  l.P = o; o += al(2 * tmax * bv * 4);
  l.red = o; o += al(4 * vpp * bv * 4);
  l.Am = o; o += al(tmax * tmax * 4);
  l.Qm = o; o += al(tmax * tmax * 4);
  l.flags = o; o += 16;
  l.total = o;
  return l;
}

inline LdsLayout fold_layout(bool kda, int st_bytes, int bv, int dk, int L, bool need_tile32) {
  auto al = [](int x) { return (x + 15) & ~15; };
  LdsLayout l{};
  int o = 0;
  l.tile_raw = o; o += al(dk * bv * st_bytes);
  if (st_bytes == 4 || !need_tile32) { l.tile32 = l.tile_raw; } else { l.tile32 = o; o += al(dk * bv * 4); }
  const int L4 = (L + 3) & ~3;
  l.khat = o; o += al(L4 * dk * 4);
  l.dhist = o; o += al(L4 * bv * 4);
  l.hg = o; o += al(kda ? L * dk * 4 : L * 4);
  l.gam = o; o += al(dk * 4);
  l.total = o;
  return l;
}

// LDS plan of the dk = 128, bf16-input verify (rs_verify_fast.hip).  Byte offsets.
// Rows of 128 bf16 (keys, queries, KDA gates) sit kKeyStride elements apart.
struct FastLayout {
  int xkq;      // window q_t then k_t, bf16 [2T x 128]             (HBM -> LDS copy)
  int xv;       // window v_t of this tile, bf16 [T x bv]           (HBM -> LDS copy)
  int xg;       // KDA window gates, bf16 [T x 128]                 (HBM -> LDS copy)
  int hkeys;    // history keys, bf16 [L x 128]                     (HBM -> LDS copy)
  int hd;       // history deltas of this tile, fp32 [L x bv]       (HBM -> LDS copy)
  int hg;       // history gates, fp32 [L] (GDN) or [L x 128] (KDA) (HBM -> LDS copy)
  int gam_i;    // GDN: suffix decay of each history record, fp32 [L]
  int khat;     // KDA: keys times their suffix decay, fp32 [L x 128], in place of hg
  int Gam;      // KDA: total history decay per key channel, fp32 [128]
  int xs;       // KDA: window vectors times the in-window prefix decay [2*tmax x xs_stride]
  int xr;       // readout vectors, q_t and k_t interleaved [nvec_pad x xs_stride]
  int C;        // history scores [lp x cs] (GDN: undecayed; KDA: of the decayed keys)
  int red;      // per-wave readout partial sums [4 x vpp x bv]; all vectors on the MFMA
                //   readout (bv 64, tmax >= 8): [4 x nvec_pad x bv]
  int hist;     // history part of the readout [nvec_pad x bv] (MFMA readout only)
  int Am, Qm;   // window pair scalars [tmax x tmax]
  int total;
  int xs_stride;
  int nvec_pad;
  int cs;       // row stride of C: 2*tmax rounded up to 16
  int lp;       // rows of C: L rounded up to 16
  int kreg;     // 1: GDN fp32 state, 64-column tiles, windows 5..8, ring of 17..64 records:
                //   the history keys go to registers (each wave the keys of its 16-row
                //   score tile), not to hkeys; a folding workgroup, which forms no history
                //   scores, copies them unpadded to fkeys instead
  int fkeys;    // (kreg) a folding workgroup's history keys, bf16 [L x 128], over C, hist
                //   and the space after them
};

constexpr int kKeyStride = 136;   // 128 bf16 + 16 bytes of padding

// The fast verify's readout on bf16 MFMAs: GDN, a bf16 state, 128-column tiles, windows
// 2..8 (at most 16 readout vectors).
__host__ __device__ constexpr bool fast_bf16_mfma(bool kda, bool bf16_state, int bv, int tmax) {
  return !kda && bf16_state && bv == 128 && tmax >= 2 && tmax <= 8;
}

// The fast verify's readout on bf16 MFMAs over a split fp32 state (high and low bf16
// parts): GDN, an fp32 state, 64-column tiles, windows 3..4 and 5..8 (at most 16 readout
// vectors).  At 5..8 it also needs no fp32 readout vectors in LDS, and its partials reuse
// the history region.
__host__ __device__ constexpr bool fast_f32_split(bool kda, bool bf16_state, int bv, int tmax) {
  return !kda && !bf16_state && bv == 64 && (tmax == 3 || tmax == 4 || tmax == 8);
}

// The same for KDA (fp32 state, 64-column tiles, windows 3..4): the decayed readout vectors
// split into high and mid bf16 parts (kept where the fp32 vectors would be), the state into
// high and low parts, three MFMAs per block.  Its lane mapping also carries the fold on
// fp32 MFMAs.  (At window 3 the FMA readout alone measured faster; with the MFMA fold the
// pair measured 41.5 against 42.0 us.)
__host__ __device__ constexpr bool fast_kda_split(bool kda, bool bf16_state, int bv, int tmax) {
  return kda && !bf16_state && bv == 64 && (tmax == 3 || tmax == 4);
}

inline FastLayout fast_layout(bool kda, bool bf16_state, int bv, int tmax, int T, int L) {
  auto al = [](int x) { return (x + 15) & ~15; };
  const int dk = 128, vpp = readout_vpp(tmax), ks = kKeyStride;
  FastLayout l{};
  int o = 0;
  l.xs_stride = dk + 4;
  l.nvec_pad = ((2 * T + vpp - 1) / vpp) * vpp;
  l.cs = (2 * tmax + 15) & ~15;
  l.lp = (L + 15) & ~15;
  const bool bfm = fast_bf16_mfma(kda, bf16_state, bv, tmax);
  const bool all_vec = (bv == 64 && tmax >= 8) || bfm || fast_f32_split(kda, bf16_state, bv, tmax) ||
                       fast_kda_split(kda, bf16_state, bv, tmax);
  const int red_bytes = al(4 * (all_vec ? l.nvec_pad : vpp) * bv * 4);
  l.xkq = o; o += al(2 * tmax * ks * 2);
  l.xv = o; o += al(tmax * bv * 2);
  bool hist_set = false;
  if (kda) {
    // KDA: the decayed history keys replace the history gates in place (rows of 128).  The
    // window gates, the raw history keys and the decayed window vectors lie together: the
    // keys are dead once decayed, the gates and vectors once the scores are formed, so
    // the readout partials reuse them when they fit.  The split readout (windows 3..4)
    // also puts there the history part of the readout (formed after the scores) and,
    // inside the partials' range but clear of the gates and vectors, the history scores
    // (read before the partials are written): 28.3 -> 25.8 KB at window 3, ring 16, six
    // workgroups per CU instead of five.
    l.hd = o; o += al(L * bv * 4);
    l.hg = o; o += al(L * dk * 4);
    l.khat = l.hg;
    l.gam_i = o;
    l.Gam = o; o += al(dk * 4);
    const int dead = o;
    l.xg = o; o += al(tmax * ks * 2);
    l.hkeys = o; o += al(L * ks * 2);
    const int xs_at = o;
    l.xs = o; o += al(2 * tmax * l.xs_stride * 4);
    const int dead_end = o;
    l.xr = o; o += al(l.nvec_pad * l.xs_stride * 4);
    const int hist_b = al(l.nvec_pad * bv * 4), c_b = al(l.lp * l.cs * 4);
    if (fast_kda_split(kda, bf16_state, bv, tmax) && hist_b >= al(tmax * ks * 2) &&
        dead + hist_b + red_bytes <= dead_end && dead + hist_b + c_b <= xs_at) {
      l.hist = dead;
      l.red = dead + hist_b;
      l.C = l.red;
      hist_set = true;
    } else {
      l.C = o; o += c_b;
      if (dead_end - l.hkeys >= red_bytes) {
        l.red = l.hkeys;
      } else {
        l.red = o; o += red_bytes;
      }
    }
  } else {
    const bool split8 = fast_f32_split(kda, bf16_state, bv, tmax) && tmax == 8;
    l.kreg = split8 && L > 16 && L <= 64;
    l.xg = o;
    l.hkeys = o; o += l.kreg ? 0 : al(L * ks * 2);
    l.hd = o; o += al(L * bv * 4);
    l.hg = o; o += al(L * 4);
    l.gam_i = o; o += al(L * 4);
    l.khat = o;
    l.Gam = o;
    l.xs = o;
    l.xr = o; o += split8 ? 0 : al(l.nvec_pad * l.xs_stride * 4);
    l.C = o; o += al(l.lp * l.cs * 4);
    // per-wave partials: of one pass of vpp vectors, or of all vectors (MFMA readouts).  The
    // bf16 MFMA readouts of a bf16 state and of a split fp32 state at windows 5..8 write
    // them after their last read of the history records, keys and scores (behind a
    // barrier), so they reuse that region when it is large enough.
    if ((bfm || split8) && o - l.hkeys >= red_bytes) {
      l.red = l.hkeys;
    } else {
      l.red = o; o += red_bytes;
    }
  }
  if (!hist_set) { l.hist = o; o += all_vec ? al(l.nvec_pad * bv * 4) : 0; }
  if (l.kreg) {                                          // C and hist are adjacent
    l.fkeys = l.C;
    if (o < l.C + al(L * 128 * 2)) o = l.C + al(L * 128 * 2);
  }
  l.Am = o; o += al(tmax * tmax * 4);
  l.Qm = o; o += al(tmax * tmax * 4);
  l.total = o;
  // GDN, fp32 state, uniform window 1 (the decode): its kernel needs 80 VGPRs, room for six
  // workgroups per CU, and runs faster at five (27.7 against 28.3 us); LDS past 160/6 KB
  // holds it there
  if (!kda && !bf16_state && bv == 64 && tmax == 1 && l.total < 28 * 1024) l.total = 28 * 1024;
  return l;
}

// LDS plan of the dk = 128 commit fold / materialize (rs_fold_fast.hip).  Byte offsets.
struct FoldFastLayout {
  int hkeys;    // history keys, bf16 [L x kKeyStride]               (HBM -> LDS copy)
  int hd;       // history deltas of this tile, fp32 [L x bv]       (HBM -> LDS copy)
  int hg;       // gates, fp32 [L] (GDN) or [L x 128] (KDA; then the decayed keys)
  int gam_i;    // GDN: suffix decay of each record [L]
  int Gam;      // KDA: total decay per key channel [128]
  int stage;    // fp32 fold: per wave 16 rows x (bv + 4) fp32 to write whole row segments,
                // over the records (dead by then)
  int total;
};

inline FoldFastLayout fold_fast_layout(bool kda, int bv, int L, bool stage_rows) {
  auto al = [](int x) { return (x + 15) & ~15; };
  FoldFastLayout l{};
  int o = 0;
  l.hkeys = o; o += al(L * kKeyStride * 2);
  l.hd = o; o += al(L * bv * 4);
  l.hg = o; o += al(kda ? L * 128 * 4 : L * 4);
  l.gam_i = o; o += kda ? 0 : al(L * 4);
  l.Gam = o; o += kda ? al(128 * 4) : 0;
  l.stage = 0;
  const int stage_bytes = stage_rows ? 4 * 16 * (bv + 4) * 4 : 0;   // 4 waves
  l.total = o > stage_bytes ? o : stage_bytes;
  return l;
}

// Launchers (defined in rs_kernels.hip, rs_verify_fast.hip and rs_fold_fast.hip).  Return hipGetLastError() after the launch.
hipError_t launch_verify(bool kda, int act_bf16, int state_bf16, int bv, int tmax,
                         const VerifyArgs& a, const RowWindows& w, hipStream_t s);
hipError_t launch_verify_fast(bool kda, int state_bf16, int bv, int tmax, const VerifyArgs& a,
                              const FastLayout& lay, const RowWindows& w, hipStream_t s);
hipError_t launch_fold(bool kda, int act_bf16, int state_bf16, int bv, bool materialize,
                       const FoldArgs& a, hipStream_t s);
hipError_t launch_fold_fast(bool kda, int state_bf16, int bv, bool materialize,
                            const FoldArgs& a, const FoldFastLayout& lay, hipStream_t s);
hipError_t launch_fold_bf16(bool kda, bool materialize, const FoldArgs& a,
                            const FoldFastLayout& lay, hipStream_t s);
hipError_t launch_advance(const AdvanceArgs& a, hipStream_t s);

// The allocation-free verify's fold counters (rs_noalloc.hip): a file-scope device array of
// kNoAllocCounters int32 (256 KiB per GPU), so batch * hk <= kNoAllocCounters.
constexpr int kNoAllocCounters = 65536;
// Device address of the current device's array (looked up once per device).
hipError_t noalloc_counters(int32_t** out);
// Zero the first n counters on the stream (a fill kernel).
hipError_t launch_zero_counters(int32_t* p, int n, hipStream_t s);

}  // namespace rs
