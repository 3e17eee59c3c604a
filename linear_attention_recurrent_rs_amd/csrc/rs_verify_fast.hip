// Verify for dk = 128 with bf16 inputs (the Qwen3.5-shaped GDN and KDA layers), gfx950.
//
// Same method as verify_kernel in rs_kernels.hip; the difference is how the workgroup
// spends its time.  The [128 x BV] state tile is the only large operand, and it streams
// (non-temporal loads: read once, no reuse) straight into registers (four rows x four columns per thread, 256-byte row segments per
// 16 lanes) as one block of loads, issued after every small operand has been queued by
// direct HBM->LDS copies.  One explicit wait for "all but the tile" then lets everything
// that does not need the state run while the tile is still in flight, and that part is
// kept short: a workgroup holds its slot on the CU until its last instruction, and every
// cycle it spends after its tile has landed is a cycle in which the slot moves no bytes.
//
//  * Window and history scores are small dense contractions over dk: one 16 x 16 MFMA
//    tile covers up to 16 score rows (history records, then window keys) against up to 16
//    window vectors (q_0.., k_0..).  GDN feeds the bf16 inputs to bf16 MFMAs (products
//    are exact in fp32) and applies the scalar decays to the results; KDA's decays are
//    per channel, so its history keys are scaled first and go through fp32 MFMAs, each
//    wave taking a quarter of dk.
//  * The history part of the readout, sum_i d_i (khat_i . x), is summed into registers
//    before the tile is touched.
//
// History is not replayed into the tile.  With H = Gam (.) S + sum_i khat_i d_i^T
// (khat_i = gamma_i (.) k_i), the readout splits into
//   H^T x = S^T (Gam (.) x) + sum_i d_i (khat_i . x),
// a pass over the registers plus nh scores per window vector (the history terms only
// when write_pos is nonzero).  A row whose window would overflow the ring instead folds
// its prefix into the registers, writes the state back once and reads out with no
// history.  Every sum over window positions runs over causal positions only, so values at
// rejected positions never reach accepted outputs.
#include <type_traits>

#include "rs_device.h"
#include "rs_internal.h"

namespace rs {

// The aligned 32-bit word holding the bf16 at p, through the scalar cache (p uniform);
// hi: whether the value is the word's high half.
__device__ __forceinline__ uint32_t load_word_uniform(const bf16* p, int& hi) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  hi = (a & 2) != 0;
  return *(const __attribute__((address_space(4))) uint32_t*)(a & ~uintptr_t(3));
}

// A bf16 value at a workgroup-uniform address, through the scalar data cache.
__device__ __forceinline__ float load_bf16_uniform(const bf16* p) {
  int hi;
  const uint32_t w = load_word_uniform(p, hi);
  return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
}

// The bf16 in the high (odd element) or low half of a word, as fp32.
__device__ __forceinline__ float bf16_half(uint32_t w, int hi) {
  return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
}

// N uniform words, all loaded by this point (an empty asm reads up to eight together).
template <int N>
__device__ __forceinline__ void pin_words(uint32_t* w) {
  if constexpr (N == 1) asm volatile("" : "+s"(w[0]));
  else if constexpr (N == 2) asm volatile("" : "+s"(w[0]), "+s"(w[1]));
  else if constexpr (N == 3) asm volatile("" : "+s"(w[0]), "+s"(w[1]), "+s"(w[2]));
  else if constexpr (N == 4) asm volatile("" : "+s"(w[0]), "+s"(w[1]), "+s"(w[2]), "+s"(w[3]));
  else if constexpr (N == 5)
    asm volatile("" : "+s"(w[0]), "+s"(w[1]), "+s"(w[2]), "+s"(w[3]), "+s"(w[4]));
  else if constexpr (N == 6)
    asm volatile("" : "+s"(w[0]), "+s"(w[1]), "+s"(w[2]), "+s"(w[3]), "+s"(w[4]), "+s"(w[5]));
  else if constexpr (N == 7)
    asm volatile("" : "+s"(w[0]), "+s"(w[1]), "+s"(w[2]), "+s"(w[3]), "+s"(w[4]), "+s"(w[5]),
                 "+s"(w[6]));
  else if constexpr (N == 8)
    asm volatile("" : "+s"(w[0]), "+s"(w[1]), "+s"(w[2]), "+s"(w[3]), "+s"(w[4]), "+s"(w[5]),
                 "+s"(w[6]), "+s"(w[7]));
  else {                                                 // eight at a time
    pin_words<8>(w);
    pin_words<N - 8>(w + 8);
  }
}

// A workgroup-uniform value, computed by this point and held in a scalar register from here
// on (the empty asm takes it there and keeps the compiler from sinking its computation).
__device__ __forceinline__ float pin_uniform(float x) {
  uint32_t u = __builtin_amdgcn_readfirstlane(__float_as_uint(x));
  asm volatile("" : "+s"(u));
  return __uint_as_float(u);
}

__device__ __forceinline__ f4 bf16x4(const bf16* p) { return load4(p); }

// Product of the window gates held in registers over a lane-dependent range of window
// positions, (lo, hi], by selection rather than register-array indexing.
template <int TMAX>
__device__ __forceinline__ float gate_product(const float (&g)[TMAX], int lo, int hi) {
  float p = 1.f;
#pragma unroll
  for (int w = 0; w < TMAX; ++w)
    if (w > lo && w <= hi) p *= g[w];
  return p;
}

// A DPP lane move within 16-lane rows; lanes without a source in their row get 1.
template <int CTRL>
__device__ __forceinline__ float dpp_one(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(v), CTRL,
                                                    0xF, 0xF, false));
}

// Sum over groups of N = 2, 4 or 8 adjacent lanes (every lane of a group gets the sum):
// quad_perm swaps within quads, then the other quad of an 8-lane half row by mirroring.
template <int N>
__device__ __forceinline__ float adjacent_sum(float v) {
  static_assert(N == 2 || N == 4 || N == 8, "groups of 2, 4 or 8 lanes");
  auto mv = [](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value,
                                                      0xF, 0xF, false));
  };
  v += mv(v, std::integral_constant<int, 0xB1>{});       // quad_perm 1,0,3,2
  if constexpr (N >= 4) v += mv(v, std::integral_constant<int, 0x4E>{});   // 2,3,0,1
  if constexpr (N == 8) v += mv(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  return v;
}

template <int TMAX>
__device__ __forceinline__ float pick(const float (&x)[TMAX], int t) {
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < TMAX; ++w)
    if (w == t) r = x[w];
  return r;
}

// One arrival at the fold counter of key group (row, kh); returns the count before it.  A
// per-lane zero the compiler cannot see through keeps the address divergent, so that the
// atomic is not rewritten into a wave reduction that reads its result back at once.
__device__ __forceinline__ int arrive(const VerifyArgs& a, int row, int kh) {
  int zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  return __hip_atomic_fetch_add(a.group_counter + (size_t)row * a.hk + kh + zero, 1,
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A thread's part of a [128 x BV] tile, rows 4 (rg + RG j) + i, columns 4 cc .. 4 cc + 3,
// written to the tile at so (row stride dv) with non-temporal stores.  The addresses are
// a uniform row pointer plus one per-thread byte offset: they take one VGPR, and do not
// keep the 64-bit addresses of the tile loads alive until a fold writes the tile back.
template <int QPT, int RG, typename ST>
__device__ __forceinline__ void store_tile(ST* so, const f4 (&s)[QPT][4], int rg, int cc,
                                           int dv) {
  const uint32_t voff = (uint32_t)(4 * rg * dv + 4 * cc) * (uint32_t)sizeof(ST);
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      char* rowp = reinterpret_cast<char*>(so + (size_t)(4 * RG * j + i) * dv);
      store4_nt(reinterpret_cast<ST*>(rowp + voff), s[j][i]);
    }
  }
}

// Workgroups per CU the register cap is set for.  More resident workgroups keep more tile
// bytes in flight, so the cap is raised where that fits without spills and measures
// faster: six per CU (at most 80 VGPRs) for 64-column tiles at windows 2-3 (KDA at window
// 3: its split readout, whose LDS plan also fits six), five (96 VGPRs) for the other
// 64-column tiles up to window 3 and GDN's at window 4, four (128 VGPRs) for 128-column
// bf16 tiles up to window 3.  (At window 1 six per CU fit too but run slower; KDA at
// window 4 fits five in 81 VGPRs, which measured the same as its four.)
constexpr int fast_min_blocks(bool kda, int bv, int tmax, bool bf16_state) {
  return (bv <= 64 && (tmax == 2 || (tmax == 3 && !kda))) ? 6
         : fast_kda_split(kda, bf16_state, bv, tmax) && tmax == 3 ? 6
         : (bv <= 64 && (tmax <= 3 || (tmax == 4 && !kda))) ? 5
         : fast_bf16_mfma(kda, bf16_state, bv, tmax)       ? 5
         : (bv == 128 && bf16_state && tmax <= 3)          ? 4
                                                           : 1;
}

__device__ __forceinline__ s4 column_of(const u4 (&r)[4], int p) {
  const int q = p >> 1, sh = (p & 1) * 16;
  const uint32_t e0 = (r[0][q] >> sh) & 0xffffu, e1 = (r[1][q] >> sh) & 0xffffu;
  const uint32_t e2 = (r[2][q] >> sh) & 0xffffu, e3 = (r[3][q] >> sh) & 0xffffu;
  return __builtin_bit_cast(s4, u2{e0 | (e1 << 16), e2 | (e3 << 16)});
}

// RAGGED: windows from cumulative lengths (a separate instantiation, so that the uniform
// kernel carries none of its code).
template <bool KDA, typename ST, int BV, int TMAX, bool RAGGED>
__global__ __launch_bounds__(kThreads, fast_min_blocks(KDA, BV, TMAX, sizeof(ST) == 2))
void verify_fast_kernel(VerifyArgs a, FastLayout lay, RowWindows rw) {
  constexpr int DK = 128, KS = kKeyStride;
  // Tile split: thread (rg, cc) holds rows 4*(rg + RG*j) + i (j < QPT, i < 4) of column
  // quad cc, so that each load instruction of a wave covers whole 256-byte row segments
  // (rows of a 64-column tile); the dk reduction of the readout then runs over the row
  // groups within a wave (lane shuffles) and over the 4 waves (LDS).
  constexpr int CC = BV / 4, RG = kThreads / CC, QPT = DK / (4 * RG);
  constexpr int NV2 = 2 * TMAX;
  constexpr int VPP = (NV2 < 8) ? NV2 : 8;           // readout vectors per pass
  constexpr int NPASS = NV2 / VPP;
  static_assert(QPT >= 1 && DK % (4 * RG) == 0 && CC >= 8 && CC <= 32, "tile split");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  // GDN with a bf16 state and 128-column tiles: every readout vector is a scalar times a
  // bf16 input (q_t or k_t), so the readout runs on bf16 MFMAs with exact products, the
  // state straight from its loaded bytes (step 8).  A 16-lane group loads whole 256-byte
  // rows (8 columns a lane); wave w holds rows 32w + 16j + 4g + i (g = lane / 16, i < 4).
  constexpr bool BF16_MFMA = fast_bf16_mfma(KDA, sizeof(ST) == 2, BV, TMAX);
  // GDN with an fp32 state, 64-column tiles, windows 3-4: the same MFMA readout over the
  // state split into high and low bf16 parts (two MFMAs per block; step 8)
  constexpr bool F32_SPLIT = fast_f32_split(KDA, sizeof(ST) == 2, BV, TMAX);
  // KDA with an fp32 state, 64-column tiles, window 4: readout on bf16 MFMAs with both
  // operands split (step 8)
  constexpr bool KDA_SPLIT = fast_kda_split(KDA, sizeof(ST) == 2, BV, TMAX);
  // history keys in registers (when the plan says so, lay.kreg: rings of 17..64 records),
  // so that the LDS plan leaves room for a fourth workgroup per CU
  constexpr bool KREG = F32_SPLIT && TMAX == 8;
  constexpr int NTILE = BF16_MFMA ? 8 : QPT * 4;          // tile load instructions
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Lane mapping.  Column quad fastest (cc = lane % CC) makes 16 consecutive lanes read
  // one whole 256-byte row segment, the best load order; the MFMA readout needs it too
  // (its A operand).  With 3 or 4 window vectors per pass the FMA readout's row-group
  // sums dominate instead, so there a wave's RL = 64 / CC row groups sit on adjacent
  // lanes and sum by DPP quad operations (one load instruction still covers the same 4
  // row segments).
  constexpr bool MFMA_READOUT = (CC == 16 && TMAX >= 8);
  constexpr int RL = 64 / CC;                            // row groups per wave
  constexpr bool ADJ = !MFMA_READOUT && !F32_SPLIT && !KDA_SPLIT && TMAX >= 3;
  // fp32 state, 64-column tiles in this lane mapping: the fused fold on MFMAs (step 7; GDN
  // bf16, KDA fp32; KDA from window 2).  At window 1 it frees enough registers for six
  // workgroups per CU, which measured slower than five (28.3 against 27.7 us): the LDS
  // plan holds that kernel at five (fast_layout).
  constexpr bool MFMA_FOLD = sizeof(ST) == 4 && CC == 16 && !ADJ && (TMAX >= 2 || !KDA);
  const int cc = ADJ ? lane / RL : tid % CC;
  const int rg = ADJ ? wave * RL + lane % RL : tid / CC;
  const int lid = xcd_group_remap(blockIdx.x, a.nblocks, a.G * a.NV);
  const int vt = umod(lid, a.NV);
  const int h = umod(udiv(lid, a.NV), a.hv);
  const int row = udiv(lid, a.NV * a.hv);
  const int slot = a.slot_idx[row];
  if (slot < 0 || slot >= a.num_slots) return;          // null row: no reads, no writes

  const int L = a.L, hv = a.hv, hk = a.hk, dv = a.dv;
  const int kh = udiv(h, a.G), col0 = vt * BV;
  int T;
  size_t tok0;
  // uniform decode (TMAX = 1) has T = 1 at compile time; every other window is read at run
  // time (a compile-time window of 2-4 would spill under the register caps above)
  row_window(RAGGED ? rw.cu_seqlens : nullptr, rw.ntok, (!RAGGED && TMAX == 1) ? 1 : a.T, row,
             &T, &tok0);
  const int XS = lay.xs_stride, CS = lay.cs;

  bf16* xkq = reinterpret_cast<bf16*>(smem + lay.xkq);
  bf16* xv = reinterpret_cast<bf16*>(smem + lay.xv);
  bf16* xg = reinterpret_cast<bf16*>(smem + lay.xg);
  bf16* hkeys = reinterpret_cast<bf16*>(smem + lay.hkeys);
  bf16* fkeys = reinterpret_cast<bf16*>(smem + lay.fkeys);
  float* hd = reinterpret_cast<float*>(smem + lay.hd);
  float* hg = reinterpret_cast<float*>(smem + lay.hg);
  float* gam_i = reinterpret_cast<float*>(smem + lay.gam_i);
  float* khat = reinterpret_cast<float*>(smem + lay.khat);
  float* Gamv = reinterpret_cast<float*>(smem + lay.Gam);
  float* xs = reinterpret_cast<float*>(smem + lay.xs);
  float* xr = reinterpret_cast<float*>(smem + lay.xr);
  float* Cs = reinterpret_cast<float*>(smem + lay.C);
  float* red = reinterpret_cast<float*>(smem + lay.red);
  float* hist = reinterpret_cast<float*>(smem + lay.hist);
  float* Am = reinterpret_cast<float*>(smem + lay.Am);
  float* Qm = reinterpret_cast<float*>(smem + lay.Qm);

  const bf16* qg = static_cast<const bf16*>(a.q);
  const bf16* kg = static_cast<const bf16*>(a.k);
  const bf16* vg = static_cast<const bf16*>(a.v);
  const bf16* bg = static_cast<const bf16*>(a.beta);
  const bf16* gg = static_cast<const bf16*>(a.gate);
  const bf16* rkg = static_cast<const bf16*>(a.ring_k);

  // 1. the cursor through the scalar cache, before anything writes memory.  The window
  // operands (HBM -> LDS, asynchronous; an empty ragged window copies nothing) do not
  // depend on it: KDA sends them while the cursor is on its way (43.5 against 45.3 us at
  // window 3), GDN after it (its window-3 decode measured 33.8 against 32.8 us that way).
  int n = a.cursor[slot];
  if constexpr (KDA) {
    dma_rows_256(qg + (tok0 * hk + kh) * DK, (size_t)hk * DK * 2, T, xkq, KS * 2);
    dma_rows_256(kg + (tok0 * hk + kh) * DK, (size_t)hk * DK * 2, T, xkq + T * KS, KS * 2);
    dma_rows(vg + (tok0 * hv + h) * dv + col0, (size_t)hv * dv * 2, BV * 2, T, xv);
    dma_rows_256(gg + (tok0 * hv + h) * DK, (size_t)hv * DK * 2, T, xg, KS * 2);
  }
  n = n < 0 ? 0 : (n > L ? L : n);
  const bool fold = n + T > L;                           // the window would overflow
  const int base = fold ? 0 : n;                         // write_pos
  const int nh = n;
  if (RAGGED && T == 0) {                                // an empty ragged window
    if (a.write_pos_out && h == 0 && vt == 0 && tid == 0) a.write_pos_out[row] = base;
    return;
  }
  // 2. (GDN) the window operands, and the committed history [0, n): HBM -> LDS,
  // asynchronous
  if constexpr (!KDA) {
    dma_rows_256(qg + (tok0 * hk + kh) * DK, (size_t)hk * DK * 2, T, xkq, KS * 2);
    dma_rows_256(kg + (tok0 * hk + kh) * DK, (size_t)hk * DK * 2, T, xkq + T * KS, KS * 2);
    dma_rows(vg + (tok0 * hv + h) * dv + col0, (size_t)hv * dv * 2, BV * 2, T, xv);
  }
  const bool kreg = KREG && lay.kreg;
  if (nh > 0) {
    if (!kreg)
      dma_rows_256(rkg + ((size_t)slot * L * hk + kh) * DK, (size_t)hk * DK * 2, nh, hkeys,
                   KS * 2);
    else if (fold)                                       // for the fold only, unpadded
      dma_rows_256(rkg + ((size_t)slot * L * hk + kh) * DK, (size_t)hk * DK * 2, nh, fkeys,
                   DK * 2);
    dma_rows(a.ring_d + ((size_t)slot * L * hv + h) * dv + col0, (size_t)hv * dv * 4, BV * 4,
             nh, hd);
    if (KDA)
      dma_rows(a.ring_g + ((size_t)slot * L * hv + h) * DK, (size_t)hv * DK * 4, DK * 4, nh, hg);
    else
      dma_words(a.ring_g + (size_t)slot * L * hv + h, (size_t)hv * 4, nh, hg);
  }
  code_fence();

  // (kreg, no fold) the history keys of this wave's score tile (step 5), HBM -> registers,
  // behind the variable-length copies so that their wait counts only the tile: record
  // 16 wave + lane % 16, dk 16 ks + 4 (lane / 16) .. +3 in kk[ks], the layout of the MFMA's
  // A operand.  Lanes past the history load record 0 (selected away in step 5).
  u2 kk[8];
  if constexpr (KREG) {
    if (kreg && !fold) {
      const int rec = 16 * wave + (lane & 15);
      const bf16* kp = rkg + (((size_t)slot * L + (rec < nh ? rec : 0)) * hk + kh) * DK +
                       4 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kk[ks] = *reinterpret_cast<const u2*>(kp + 16 * ks);
    }
  }
  // 3. the state tile: HBM -> registers, the last vector loads issued before the wait
  const ST* sg = static_cast<const ST*>(a.state) + (((size_t)slot * hv + h) * DK) * dv + col0;
  f4 s[QPT][4];
  u4 raw[2][4];
  if constexpr (BF16_MFMA) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        raw[j][i] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(
            sg + (uint32_t)((32 * wave + 16 * j + 4 * (lane >> 4) + i) * dv + 8 * (lane & 15))));
    }
  } else {
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[j][i] = load4_nt(sg + (uint32_t)((4 * (rg + RG * j) + i) * dv + 4 * cc));
    }
  }
  code_fence();
  // the window's betas and (GDN) gates through the scalar cache, issued behind the loads:
  // the history copies wait only for the cursor (a wait for one scalar load is a wait for
  // all of them), and these land while the copies do
  float beta_s[TMAX], gate_s[TMAX], Gp[TMAX];
  if constexpr (TMAX <= 3) {
    // a short window: the loads under their branches, a round trip each, hide behind the
    // tile (window 3 decodes measured 32.7 us so against 33.4 us batched)
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      beta_s[t] = t < T ? load_bf16_uniform(bg + (tok0 + t) * hv + h) : 0.f;
      gate_s[t] = (!KDA && t < T) ? load_bf16_uniform(gg + (tok0 + t) * hv + h) : 0.f;
    }
  } else {
    // a long one: every word is loaded (a short ragged window repeats its last token,
    // 1 <= T here) and the empty asm needs them all at once, so one wait covers them (the
    // large-ring verify at window 8 measured 233 against 293 us with a wait per load)
    constexpr int NW = KDA ? TMAX : 2 * TMAX;            // words: betas, then (GDN) gates
    uint32_t wd[NW];
    int hi[NW];                                          // the value is the word's high half
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const int e = (tok0 + (t < T ? t : T - 1)) * hv + h;
      wd[t] = load_word_uniform(bg + e, hi[t]);
      if constexpr (!KDA) wd[TMAX + t] = load_word_uniform(gg + e, hi[TMAX + t]);
    }
    pin_words<NW>(wd);
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      // the values, not the words and their halves, live on from here: left to itself
      // the compiler keeps the words, and spills
      beta_s[t] = t < T ? pin_uniform(bf16_half(wd[t], hi[t])) : 0.f;
      if constexpr (!KDA)
        gate_s[t] = t < T ? pin_uniform(bf16_half(wd[TMAX + t], hi[TMAX + t])) : 0.f;
      else
        gate_s[t] = 0.f;
    }
  }
  lds_barrier<NTILE>();                                  // every copy but the tile is in LDS
  // fp32 state, on a fold: the arrival of this workgroup at its key group's counter (step 7
  // explains it), now that its reads of the ring are complete, so that the round trip of
  // the atomic overlaps the scores.  (bf16 state arrives in step 7: the result, read
  // there, would otherwise hold its readout until the whole tile had landed.)
  constexpr bool EARLY_ARRIVAL = sizeof(ST) == 4;
  int arrived = 0;
  if (EARLY_ARRIVAL && fold && wave == 0 && lane == 0) arrived = arrive(a, row, kh);

  const int nvec = 2 * T, hrows = fold ? 0 : nh;
  const int l16 = lane & 15, g4 = lane >> 4;

  // 4. decays and readout vectors (q_t at row 2t, k_t at row 2t+1).  GDN: window prefix
  // decays Gp[t] = prod_{w<=t} alpha_w from the gate registers, total history decay Gam,
  // suffix decay of each record; KDA: per key channel, in LDS.
  float Gam = 1.f;
  {
    float g = 1.f;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      g *= gate_s[t];
      Gp[t] = g;
    }
  }
  if (!KDA) {
    if (L <= 16) {
      // Suffix products of the gates within each 16-lane row by DPP (row_shl k: lane i
      // reads lane i + k of its row; lanes past the row end keep 1): lane i of a row ends
      // with prod_{i<=j<nh} alpha_j, so lane 0 holds Gam and lane i + 1 gamma_i.
      const int li = lane & 15;
      float v = li < nh ? hg[li] : 1.f;
      v *= dpp_one<0x101>(v);
      v *= dpp_one<0x102>(v);
      v *= dpp_one<0x104>(v);
      v *= dpp_one<0x108>(v);
      Gam = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
      const float ex = dpp_one<0x101>(v);
      if (wave == 2 && lane < nh) gam_i[lane] = ex;
    } else if (L <= 64) {
      // Rings up to 64 records: the same scan in each 16-lane row, then the rows joined
      // through their totals (lanes 0, 16, 32, 48): the product over (i, nh) is row i/16's
      // partial from lane i + 1 times the totals of the rows after it.
      const int rw = lane >> 4;
      float v = lane < nh ? hg[lane] : 1.f;
      v *= dpp_one<0x101>(v);
      v *= dpp_one<0x102>(v);
      v *= dpp_one<0x104>(v);
      v *= dpp_one<0x108>(v);
      const float t0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
      const float t1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
      const float t2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
      const float t3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
      const float f2 = t3, f1 = t2 * t3, f0 = t1 * f1;
      Gam = t0 * f0;
      const float F = rw == 0 ? f0 : rw == 1 ? f1 : rw == 2 ? f2 : 1.f;
      const float ex = dpp_one<0x101>(v) * F;
      if (wave == 2 && lane < nh) gam_i[lane] = ex;
    } else {
      for (int i = 0; i < nh; ++i) Gam *= hg[i];
    }
    // (the MFMA readouts of the split fp32 state and of a bf16 state take q, k raw)
    if (!F32_SPLIT && !BF16_MFMA && tid < DK) {
      float xq[TMAX], xk[TMAX];
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {                   // rows < 2*TMAX: in bounds
        xq[t] = to_f32(xkq[t * KS + tid]);
        xk[t] = to_f32(xkq[(T + t) * KS + tid]);
      }
      const float scale = fold ? 1.f : Gam;
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        if (t < T) {
          xr[(2 * t) * XS + tid] = (scale * Gp[t]) * xq[t];
          xr[(2 * t + 1) * XS + tid] = (scale * Gp[t]) * xk[t];
        }
      }
      for (int m = nvec; m < lay.nvec_pad; ++m) xr[m * XS + tid] = 0.f;
    } else if (wave == 2 && L > 64) {
      // gamma_i = prod_{i<j<nh} alpha_j for rings past 64 records (rings up to 64 have
      // theirs from the scan above)
      for (int i = lane; i < nh; i += 64) {
        float g = 1.f;
        for (int j = i + 1; j < nh; ++j) g *= hg[j];
        gam_i[i] = g;
      }
    }
  } else {
    if (tid < DK) {
      float run = 1.f;
      for (int t = 0; t < T; ++t) {
        run *= to_f32(xg[t * KS + tid]);
        const float q = run * to_f32(xkq[t * KS + tid]);
        const float k = run * to_f32(xkq[(T + t) * KS + tid]);
        xs[t * XS + tid] = q;
        xs[(T + t) * XS + tid] = k;
      }
      float g = 1.f;
#pragma unroll 4
      for (int i = nh - 1; i >= 0; --i) {            // khat replaces the gates in place
        const float al = hg[i * DK + tid];
        khat[i * DK + tid] = g * to_f32(hkeys[i * KS + tid]);
        g *= al;
      }
      Gamv[tid] = g;
      const float scale = fold ? 1.f : g;
      if constexpr (KDA_SPLIT) {
        // readout vectors in xs order (q_0.., then k_0..) as bf16 parts, x = hi + mid + e
        // with |e| <= 2^-17 |x|: hi rows [0, 2T), mid rows [nvec_pad, nvec_pad + 2T), XS
        // elements apart, in the space of the fp32 vectors
        bf16* xb = reinterpret_cast<bf16*>(xr);
        for (int v = 0; v < 2 * T; ++v) {
          const float x = scale * xs[v * XS + tid];
          const uint32_t w = __float_as_uint(x);
          xb[v * XS + tid] = bf16(w >> 16);
          xb[(lay.nvec_pad + v) * XS + tid] = bf16_rne(x - __uint_as_float(w & 0xffff0000u));
        }
      } else {
        for (int t = 0; t < T; ++t) {
          xr[(2 * t) * XS + tid] = scale * xs[t * XS + tid];
          xr[(2 * t + 1) * XS + tid] = scale * xs[(T + t) * XS + tid];
        }
        for (int m = nvec; m < lay.nvec_pad; ++m) xr[m * XS + tid] = 0.f;
      }
    }
    lds_barrier();
  }

  // 5. scores.  Rows: history records 0..hrows-1 (not on a fold), then (GDN) the window
  // keys; columns: the window vectors q_0..q_{T-1}, k_0..k_{T-1}.
  if (!KDA) {
    // undecayed dot products; the decays are applied where the scores are used
    const int R = hrows + T, RT = (R + 15) >> 4, CT = (nvec + 15) >> 4;   // CT is 1 or 2
    for (int tile = wave; tile < RT * CT; tile += kWaves) {
      const int rt = CT == 1 ? tile : tile >> 1, ct = CT == 1 ? 0 : tile & 1;
      const int ra = rt * 16 + l16, m = ct * 16 + l16;
      const bool aok = ra < R, bok = m < nvec;
      // operands from rows that always exist; rows outside the tile are selected away
      // (kreg: a history row's keys are this lane's registers, tile == wave here, for the
      // R <= L <= 64 rows of a window that does not fold make at most four row tiles)
      const bool areg = kreg && ra < hrows;
      const bf16* ap = (ra < hrows && !kreg) ? hkeys + ra * KS
                                             : xkq + (T + (aok && !areg ? ra - hrows : 0)) * KS;
      const bf16* bp = xkq + (bok ? m : 0) * KS;
      const s4 zero = s4{0, 0, 0, 0};
      f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int half = 0; half < 2; ++half) {              // two batches of LDS reads
        s4 av[DK / 32], bv[DK / 32];
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          const int k0 = (half * (DK / 32) + kb) * 16 + 4 * g4;
          av[kb] = *reinterpret_cast<const s4*>(ap + k0);
          if constexpr (KREG)
            if (areg) av[kb] = __builtin_bit_cast(s4, kk[half * (DK / 32) + kb]);
          bv[kb] = *reinterpret_cast<const s4*>(bp + k0);
        }
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
          acc = mfma_bf16_16x16x16(aok ? av[kb] : zero, bok ? bv[kb] : zero, acc);
      }
      if (bok) {
        const bool isq = m < T;
        const int t = isq ? m : m - T;
        const int r0 = rt * 16 + 4 * g4;
        // (windows of 8 and more) the window decays G(u, t) of this lane's rows u = r0 + j -
        // hrows, from the last row up, each from the one after it (rows of the history
        // take unused values); shorter windows form each on its own, in fewer registers
        float decs[4];
        if (TMAX >= 8 && r0 + 3 >= hrows) {
          float p = gate_product(gate_s, r0 + 3 - hrows, t);
          decs[3] = p;
#pragma unroll
          for (int j = 2; j >= 0; --j) {
            const int u = r0 + j - hrows;
            if (u < t) p *= pick(gate_s, u + 1);
            decs[j] = p;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = r0 + j;
          if (rr < hrows) {
            Cs[rr * CS + m] = acc[j];
          } else if (rr < R) {
            const int u = rr - hrows;
            const float dec = TMAX >= 8 ? decs[j] : gate_product(gate_s, u, t);
            if (isq) {
              if (u <= t) Qm[t * TMAX + u] = acc[j] * dec;
            } else if (u < t) {
              Am[t * TMAX + u] = pick(beta_s, t) * (acc[j] * dec);
            }
          }
        }
      }
    }
  } else {
    // history scores: fp32 MFMAs over the whole of dk, one 16 x 16 tile per wave, from
    // wave 3 down (waves 0 and 1 take the window pairs below), so the scores land in LDS
    // complete and their readers read one value per score
    const int RT = (hrows + 15) >> 4, CT = (nvec + 15) >> 4;
    for (int tile = kWaves - 1 - wave; tile < RT * CT; tile += kWaves) {
      const int rt = CT == 1 ? tile : tile >> 1, ct = CT == 1 ? 0 : tile & 1;
      const int ra = rt * 16 + l16, m = ct * 16 + l16;
      const bool aok = ra < hrows, bok = m < nvec;
      const float* ap = khat + (aok ? ra : 0) * DK;
      const float* bp = xs + (bok ? m : 0) * XS;
      f4 acc = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < DK / 32; ++q) {                  // eight K steps at a time
        float av[8], bv[8];
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          av[st] = ap[32 * q + 4 * st + g4];
          bv[st] = bp[32 * q + 4 * st + g4];
        }
#pragma unroll
        for (int st = 0; st < 8; ++st)
          acc = mfma_16x16x4(aok ? av[st] : 0.f, bok ? bv[st] : 0.f, acc);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) Cs[(rt * 16 + 4 * g4 + j) * CS + m] = acc[j];
    }
    // window pairs: per-channel decays between u and t, 16 lanes per pair
    const int npair = T * (T + 1) / 2, grp = tid >> 4, e = tid & 15;
    for (int p = grp; p < npair; p += kThreads / 16) {
      int t = 0;
      while ((t + 1) * (t + 2) / 2 <= p) ++t;
      const int u = p - t * (t + 1) / 2;
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < 2; ++c4) {
        const int r = 8 * e + 4 * c4;
        f4 dec = f4{1.f, 1.f, 1.f, 1.f};
        for (int w = u + 1; w <= t; ++w) dec *= bf16x4(xg + w * KS + r);
        const f4 kd = bf16x4(xkq + (T + u) * KS + r) * dec;
        const f4 a4 = bf16x4(xkq + t * KS + r) * kd, b4 = bf16x4(xkq + (T + t) * KS + r) * kd;
        sq += (a4[0] + a4[1]) + (a4[2] + a4[3]);
        sk += (b4[0] + b4[1]) + (b4[2] + b4[3]);
      }
      // sums over the 16 lanes of the pair by DPP (quads, half rows, then the row mirror)
      sq = adjacent_sum<8>(sq);
      sk = adjacent_sum<8>(sk);
      sq += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sq), 0x140, 0xF, 0xF, false));
      sk += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sk), 0x140, 0xF, 0xF, false));
      if (e == 0) {
        Qm[t * TMAX + u] = sq;
        if (u < t) Am[t * TMAX + u] = pick(beta_s, t) * sk;
      }
    }
    // the window's gates to the ring, on a window that does not fold (rows past the
    // history, which no workgroup reads this launch), by wave 2 while they are in LDS:
    // the split readout's plan reuses their space from the next step on.  (On a fold the
    // key group's last arriver writes them from the inputs, step 10.)
    if (!fold && h % a.G == 0 && vt == 0 && wave == 2) {
      for (int i = lane; i < T * DK; i += 64) {
        const int t = i / DK, r = i - t * DK;
        a.ring_g[(((size_t)slot * L + base + t) * hv + h) * DK + r] = to_f32(xg[t * KS + r]);
      }
    }
  }
  lds_barrier();

  // 6. (many window vectors) history part of the readout, before the tile is touched:
  //   hist[m][c] = sum_i d_i[c] w_i[m],  w_i[m] = gamma_i G_t(m) (k_i . x_m)  (GDN; KDA: the
  //   decayed keys' scores khat_i . x_m), vectors m in readout order.  An MFMA contraction over the
  //   records: A = d_i of 16 columns, B = w_i of 16 vectors, four records per step; wave w
  //   takes the column blocks w, w + 4, ...  (With few vectors the readout itself adds
  //   the history part, step 8.)
  const int NP = lay.nvec_pad;
  if ((MFMA_READOUT || BF16_MFMA || F32_SPLIT || KDA_SPLIT) && hrows > 0) {
    constexpr int NCB = BV / 16, NVB = (NV2 + 15) / 16;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      const int mv = vb * 16 + l16;                        // this lane's vector (B column)
      const bool mok = mv < nvec;
      const int tv = mv >> 1, colm = (mv & 1) ? T + tv : tv;
      // G_tv = prod_{w<=tv} alpha_w (windows of 8 and more: Gp[tv], by selection)
      const float Gm = KDA ? 1.f : TMAX >= 8 ? pick(Gp, tv) : gate_product(gate_s, -1, tv);
      for (int cb = wave; cb < NCB; cb += kWaves) {
        f4 acc = f4{0.f, 0.f, 0.f, 0.f};
        // four steps of four records at a time: their LDS reads go out together
        for (int ks0 = 0; 4 * ks0 < hrows; ks0 += 4) {
          float av[4], bv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int rec = 4 * (ks0 + u) + g4;
            const bool ok = rec < hrows;
            const int rs = ok ? rec : 0;                   // a row that exists; selected away
            const float dv_ = hd[rs * BV + cb * 16 + l16];
            float w;
            if (KDA) {
              w = Cs[rs * CS + (mok ? colm : 0)];
            } else {
              w = (Cs[rs * CS + (mok ? colm : 0)] * gam_i[rs]) * Gm;
            }
            av[u] = ok ? dv_ : 0.f;
            bv[u] = (ok && mok) ? w : 0.f;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) acc = mfma_16x16x4(av[u], bv[u], acc);
        }
        // lane holds columns cb*16 + 4*g4 + j of vector vb*16 + l16
        if (mv < NP) store4(hist + mv * BV + cb * 16 + 4 * g4, acc);
      }
    }
  }

  // 7. rows that overflow.  On a fused fold the window's keys and gates go to rows
  // 0..T-1, which other workgroups of the key group may still read: only the last of
  // them to get past its copies writes them (no spinning).  Only read-before-write
  // ordering is at stake, no data passes through the counter: every increment follows
  // its workgroup's completed reads (the copies landed before the first barrier), and the
  // writes follow the return of the last increment, so a relaxed device-scope atomic
  // suffices.  Wave 0 increments and reads the returned value.
  bool last = false;
  if constexpr (EARLY_ARRIVAL) {
    // fp32 state (arrival issued in step 3): every path first waits for the tile, before
    // any write.  The readout below is code shared by rows that fold and rows that do not,
    // and a wait there for tile loads still in flight would, on a fold, also wait for the
    // state writes issued before it (the counter covers stores too): a full HBM round trip
    // under load.  An fp32 tile has in practice landed by now.
    wait_vmem();
    last = fold && wave == 0 && __shfl(arrived, 0) == a.G * a.NV - 1;
  } else if (fold && wave == 0) {
    // bf16 state: a bf16 tile (twice the columns, smaller loads) is still arriving, and its
    // readout gains more from consuming it load by load; only the fold path waits, for the
    // returned value, which, vector-memory operations completing in order, also waits for
    // the tile.
    if (lane == 0)
      arrived = __hip_atomic_fetch_add(a.group_counter + (size_t)row * hk + kh, 1,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = __shfl(arrived, 0) == a.G * a.NV - 1;
  }
  if (fold && BF16_MFMA) {
    // S <- Gam (.) S + sum_i gamma_i k_i d_i^T in fp32, four rows at a time, then one
    // bf16 rounding: the rounded bytes are written back and kept for the readout
    ST* so = static_cast<ST*>(a.state) + (((size_t)slot * hv + h) * DK) * dv + col0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r0 = 32 * wave + 16 * j + 4 * (lane >> 4);
      float f[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f[i][2 * q] = __uint_as_float(raw[j][i][q] << 16) * Gam;
          f[i][2 * q + 1] = __uint_as_float(raw[j][i][q] & 0xffff0000u) * Gam;
        }
      }
      for (int rec = 0; rec < nh; ++rec) {
        const f4 d0 = load4(hd + rec * BV + 8 * (lane & 15));
        const f4 d1 = load4(hd + rec * BV + 8 * (lane & 15) + 4);
        const f4 kq = bf16x4(hkeys + rec * KS + r0) * gam_i[rec];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            f[i][c] += kq[i] * d0[c];
            f[i][4 + c] += kq[i] * d1[c];
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          raw[j][i][q] = uint32_t(bf16_rne(f[i][2 * q])) |
                         (uint32_t(bf16_rne(f[i][2 * q + 1])) << 16);
        __builtin_nontemporal_store(
            raw[j][i], reinterpret_cast<u4*>(so + (uint32_t)((r0 + i) * dv + 8 * (lane & 15))));
      }
    }
  } else if (fold) {
    // S <- Gam (.) S + sum_i gamma_i k_i d_i^T in the registers, then one write
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int r0 = 4 * (rg + RG * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[j][i] *= KDA ? Gamv[r0 + i] : Gam;
    }
    if constexpr (MFMA_FOLD && KDA) {
      // S += Khat D^T over records on v_mfma_f32_16x16x4_f32, the tile registers the
      // accumulators (lane l: rows 16 wave + 64 j + 4 (l / 16) + i at column 4 (l % 16)
      // + jj, element i of D[4 (l / 16) + i][l % 16]): A = the decayed keys khat_i (fp32),
      // B = d_i, lane group l / 16 taking record rb + l / 16; records past n are selected
      // to zero.
      const int lc = lane & 15, lg = lane >> 4;
      for (int rb = 0; rb < nh; rb += 4) {
        const int rec = rb + lg;
        const bool ok = rec < nh;
        const int rs = ok ? rec : 0;
        float ka[QPT];
#pragma unroll
        for (int j = 0; j < QPT; ++j) ka[j] = ok ? khat[rs * DK + 16 * wave + 64 * j + lc] : 0.f;
        const f4 dq = load4(hd + rs * BV + 4 * lc);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float b = ok ? dq[jj] : 0.f;
#pragma unroll
          for (int j = 0; j < QPT; ++j) {
            f4 acc = f4{s[j][0][jj], s[j][1][jj], s[j][2][jj], s[j][3][jj]};
            acc = mfma_16x16x4(ka[j], b, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) s[j][i][jj] = acc[i];
          }
        }
      }
    } else if constexpr (MFMA_FOLD) {
      // S += K (gamma (.) D)^T over records in blocks of 16 on v_mfma_f32_16x16x16_bf16.
      // The tile registers are the accumulators: for fixed (j, jj), lane l holds rows
      // 16 wave + 64 j + 4 (l / 16) + i at column 4 (l % 16) + jj, which is element i of
      // D[4 (l / 16) + i][l % 16] of a 16 x 16 block.  A = the keys of the block's rows
      // (bf16, exact), B = gamma_i d_i in three bf16 parts (error <= 2^-24), lane group
      // l / 16 taking records 4 (l / 16) .. +3 of the block; records past n are selected
      // to zero, never read into the product.
      const int lc = lane & 15, lg = lane >> 4;
      const bf16* fk = kreg ? fkeys : hkeys;
      const int fks = kreg ? DK : KS;
      for (int rb = 0; rb < nh; rb += 16) {
        int recs[4];
        bool ok[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rec = rb + 4 * lg + e;
          ok[e] = rec < nh;
          recs[e] = ok[e] ? rec : 0;
        }
        s4 ka[QPT];
#pragma unroll
        for (int j = 0; j < QPT; ++j) {
          const int row = 16 * wave + 64 * j + lc;
          s4 kv;
#pragma unroll
          for (int e = 0; e < 4; ++e) kv[e] = ok[e] ? short(fk[recs[e] * fks + row]) : short(0);
          ka[j] = kv;
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[e] = ok[e] ? hd[recs[e] * BV + 4 * lc + jj] * gam_i[recs[e]] : 0.f;
          s4 bh, bm, bl;
          split4x3(x, bh, bm, bl);
#pragma unroll
          for (int j = 0; j < QPT; ++j) {
            f4 acc = f4{s[j][0][jj], s[j][1][jj], s[j][2][jj], s[j][3][jj]};
            acc = mfma_bf16_16x16x16(ka[j], bh, acc);
            acc = mfma_bf16_16x16x16(ka[j], bm, acc);
            acc = mfma_bf16_16x16x16(ka[j], bl, acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) s[j][i][jj] = acc[i];
          }
        }
      }
    } else {
#pragma unroll 4
      for (int i = 0; i < nh; ++i) {
        const f4 dq = load4(hd + i * BV + 4 * cc) * (KDA ? 1.f : gam_i[i]);
#pragma unroll
        for (int j = 0; j < QPT; ++j) {
          const int r0 = 4 * (rg + RG * j);
          const f4 kq = KDA ? load4(khat + i * DK + r0) : bf16x4(hkeys + i * KS + r0);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) s[j][ii] += kq[ii] * dq;
        }
      }
    }
    ST* so = static_cast<ST*>(a.state) + (((size_t)slot * hv + h) * DK) * dv + col0;
    if constexpr (EARLY_ARRIVAL) {
      store_tile<QPT, RG>(so, s, rg, cc, dv);
    } else {
      // stored rounded to bf16; the readout below uses the rounded values
#pragma unroll
      for (int j = 0; j < QPT; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          store4_nt(so + (uint32_t)((4 * (rg + RG * j) + i) * dv + 4 * cc), s[j][i]);
          s[j][i] = round4<ST>(s[j][i]);
        }
      }
    }
  }

  constexpr bool SPREAD = TMAX >= 8;
  // 8. tile part of the readout, S^T xr_m over this thread's rows; each wave's partial
  // goes to LDS, and the thread of column c gathers P_m = sum of the 4 partials (+ the
  // history part) into registers.
  float Pv[NV2];
#pragma unroll
  for (int m = 0; m < NV2; ++m) Pv[m] = 0.f;
  if constexpr (BF16_MFMA) {
    // R_v = S^T x_v for the raw inputs x_v = xkq row v (q_0.., then k_0..) on bf16 MFMAs:
    // A = 16 vectors x this lane group's 4 rows, B = the same 4 rows x 16 columns
    // (column 8 n + p of the tile in MFMA p).  Lane l ends with vector 4 (l / 16) + e at
    // columns 8 (l % 16) + p in element e of accumulator p; P = (scale G_t) R + history.
    const int lc = lane & 15, lg = lane >> 4;
    f4 D[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) D[p] = f4{0.f, 0.f, 0.f, 0.f};
    const s4 zero4 = s4{0, 0, 0, 0};
    const bool vok = lc < nvec;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const s4 xa = *reinterpret_cast<const s4*>(xkq + (vok ? lc : 0) * KS + 32 * wave + 16 * j +
                                                 4 * lg);
      const s4 av = vok ? xa : zero4;
#pragma unroll
      for (int p = 0; p < 8; ++p) D[p] = mfma_bf16_16x16x16(av, column_of(raw[j], p), D[p]);
    }
    // per-wave partial sums to LDS, in readout order (q_t at 2t, k_t at 2t + 1).  The
    // buffer reuses the history records, which every wave has finished reading here.
    const int NPd = lay.nvec_pad;
    lds_barrier();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = 4 * lg + e;
      if (v < nvec) {
        const int m = v < T ? 2 * v : 2 * (v - T) + 1;
        float* dst = red + (wave * NPd + m) * BV + 8 * lc;
        store4(dst, f4{D[0][e], D[1][e], D[2][e], D[3][e]});
        store4(dst + 4, f4{D[4][e], D[5][e], D[6][e], D[7][e]});
      }
    }
    lds_barrier();
    if (SPREAD || tid < BV) {
      const float scale = fold ? 1.f : Gam;
#pragma unroll
      for (int m = 0; m < NV2; ++m) {
        if (m < nvec) {
          float p = (red[m * BV + tid % BV] + red[(NPd + m) * BV + tid % BV]) +
                    (red[(2 * NPd + m) * BV + tid % BV] + red[(3 * NPd + m) * BV + tid % BV]);
          p *= scale * Gp[m >> 1];
          if (hrows > 0) p += hist[m * BV + tid % BV];
          Pv[m] = p;
        }
      }
    }
  } else if constexpr (F32_SPLIT) {
    // R_v = S^T x_v for the raw inputs x_v = xkq row v on bf16 MFMAs, S = hi + lo: lane l
    // holds rows 16 wave + 64 j + 4 (l / 16) + i at columns 4 (l % 16) + p, so the four
    // lane groups of a wave cover 16 consecutive rows (the K block of j); MFMA p takes
    // column 4 n + p of the tile at B column n.  Lane l ends with vector 4 (l / 16) + e
    // at column 4 (l % 16) + p in element e of accumulator p.
    const int lc = lane & 15, lg = lane >> 4;
    f4 D[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) D[p] = f4{0.f, 0.f, 0.f, 0.f};
    const s4 zero4 = s4{0, 0, 0, 0};
    const bool vok = lc < nvec;
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const s4 xa = *reinterpret_cast<const s4*>(xkq + (vok ? lc : 0) * KS + 4 * (rg + RG * j));
      const s4 av = vok ? xa : zero4;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        s4 bh, bl;
        split4(s[j][0][p], s[j][1][p], s[j][2][p], s[j][3][p], bh, bl);
        D[p] = mfma_bf16_16x16x16(av, bh, D[p]);
        D[p] = mfma_bf16_16x16x16(av, bl, D[p]);
      }
    }
    const int NPd = lay.nvec_pad;
    // windows 5..8: the partials reuse the history region, which every wave has finished
    // reading here
    if constexpr (TMAX == 8) lds_barrier();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = 4 * lg + e;
      if (v < nvec) {
        const int m = v < T ? 2 * v : 2 * (v - T) + 1;
        store4(red + (wave * NPd + m) * BV + 4 * lc, f4{D[0][e], D[1][e], D[2][e], D[3][e]});
      }
    }
    lds_barrier();
    if constexpr (SPREAD && BV == 64) {
      // every thread needs the sums of its column: wave w forms those of vectors
      // 4 w .. 4 w + 3 (not all of them, as one thread per column would), then they pass
      // through the first partial plane
      const float scale = fold ? 1.f : Gam;
      const int c = tid % BV;
      float mine[NV2 / 4];
#pragma unroll
      for (int q = 0; q < NV2 / 4; ++q) {
        const int m = 4 * wave + q;
        float p = (red[m * BV + c] + red[(NPd + m) * BV + c]) +
                  (red[(2 * NPd + m) * BV + c] + red[(3 * NPd + m) * BV + c]);
        p *= scale * pick(Gp, m >> 1);
        if (hrows > 0) p += hist[m * BV + c];
        mine[q] = p;
      }
      lds_barrier();
#pragma unroll
      for (int q = 0; q < NV2 / 4; ++q) red[(4 * wave + q) * BV + c] = mine[q];
      lds_barrier();
#pragma unroll
      for (int m = 0; m < NV2; ++m)
        if (m < nvec) Pv[m] = red[m * BV + c];
    } else if (SPREAD || tid < BV) {
      const float scale = fold ? 1.f : Gam;
#pragma unroll
      for (int m = 0; m < NV2; ++m) {
        if (m < nvec) {
          float p = (red[m * BV + tid % BV] + red[(NPd + m) * BV + tid % BV]) +
                    (red[(2 * NPd + m) * BV + tid % BV] + red[(3 * NPd + m) * BV + tid % BV]);
          p *= scale * Gp[m >> 1];
          if (hrows > 0) p += hist[m * BV + tid % BV];
          Pv[m] = p;
        }
      }
    }
  } else if constexpr (KDA_SPLIT) {
    // R_v = S^T x_v, x_v the decayed vectors (xs order) = hi + mid, S = hi + lo: three
    // bf16 MFMAs per block (hi.hi, hi.lo, mid.hi), lane layout as in the split readout
    // above; the decays are inside x, so P = R + the history part.
    const int lc = lane & 15, lg = lane >> 4;
    const bf16* xb = reinterpret_cast<const bf16*>(xr);
    const int NPd = lay.nvec_pad;
    f4 D[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) D[p] = f4{0.f, 0.f, 0.f, 0.f};
    const s4 zero4 = s4{0, 0, 0, 0};
    const bool vok = lc < nvec;
    const int vrow = vok ? lc : 0;
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int r = 4 * (rg + RG * j);
      const s4 xh = *reinterpret_cast<const s4*>(xb + vrow * XS + r);
      const s4 xm = *reinterpret_cast<const s4*>(xb + (NPd + vrow) * XS + r);
      const s4 ah = vok ? xh : zero4, am = vok ? xm : zero4;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        s4 bh, bl;
        split4(s[j][0][p], s[j][1][p], s[j][2][p], s[j][3][p], bh, bl);
        D[p] = mfma_bf16_16x16x16(ah, bh, D[p]);
        D[p] = mfma_bf16_16x16x16(ah, bl, D[p]);
        D[p] = mfma_bf16_16x16x16(am, bh, D[p]);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = 4 * lg + e;
      if (v < nvec) {
        const int m = v < T ? 2 * v : 2 * (v - T) + 1;
        store4(red + (wave * NPd + m) * BV + 4 * lc, f4{D[0][e], D[1][e], D[2][e], D[3][e]});
      }
    }
    lds_barrier();
    if (SPREAD || tid < BV) {
#pragma unroll
      for (int m = 0; m < NV2; ++m) {
        if (m < nvec) {
          float p = (red[m * BV + tid % BV] + red[(NPd + m) * BV + tid % BV]) +
                    (red[(2 * NPd + m) * BV + tid % BV] + red[(3 * NPd + m) * BV + tid % BV]);
          if (hrows > 0) p += hist[m * BV + tid % BV];
          Pv[m] = p;
        }
      }
    }
  } else if constexpr (MFMA_READOUT) {
    // Many window vectors: an MFMA contraction over the tile rows.  The registers are
    // already an A operand: lane l holds column 4*(l%16) + jj of the rows of row group
    // 4*wave + l/16, so for fixed (j, i, jj) A[m][k] = S[row(k)][4m + jj] with K = the
    // wave's 4 row groups; B[k][n] = xr_n[row(k)].  Lane l ends with P of vector l%16 at
    // columns 16*(l/16) + 4e + jj (element e of accumulator jj).
    constexpr int NVB = (NV2 + 15) / 16;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      if (vb * 16 >= nvec) break;
      const int n = vb * 16 + l16;
      const bool nok = n < lay.nvec_pad;
      const float* xrow = xr + (nok ? n : 0) * XS;
      f4 D[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) D[jj] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < QPT; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xb = xrow[4 * (rg + RG * j) + i];
          const float b = nok ? xb : 0.f;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) D[jj] = mfma_16x16x4(s[j][i][jj], b, D[jj]);
        }
      }
      if (nok) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          store4(red + (wave * lay.nvec_pad + n) * BV + 16 * g4 + 4 * e,
                 f4{D[0][e], D[1][e], D[2][e], D[3][e]});
      }
    }
    lds_barrier();
    if (SPREAD || tid < BV) {
      const int NPd = lay.nvec_pad;
#pragma unroll
      for (int m = 0; m < NV2; ++m) {
        if (m < nvec) {
          float p = (red[m * BV + tid % BV] + red[(NPd + m) * BV + tid % BV]) +
                    (red[(2 * NPd + m) * BV + tid % BV] + red[(3 * NPd + m) * BV + tid % BV]);
          if (hrows > 0) p += hist[m * BV + tid % BV];
          Pv[m] = p;
        }
      }
    }
  } else {
    // Few window vectors: FMAs over this thread's rows, then lane sums across the row
    // groups of the wave, one pass of VPP vectors at a time.
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int m0 = ps * VPP;
      if (m0 >= nvec) break;
      if (ps > 0) lds_barrier();                   // the previous pass's partials are read
      f4 acc[VPP];
#pragma unroll
      for (int mm = 0; mm < VPP; ++mm) acc[mm] = f4{0.f, 0.f, 0.f, 0.f};
      // history part first (it needs no tile): row group rg takes records rg, rg + RG, ...
      // and adds d_i[4 columns] * w_i[m], w_i[m] = gamma_i G_t(m) (k_i . x_m) (KDA: the
      // decayed keys' scores); the lane sums below reduce it with the tile part
      for (int i = rg; i < hrows; i += RG) {
        const f4 dq = load4(hd + i * BV + 4 * cc);
        const float gi = KDA ? 1.f : gam_i[i];
#pragma unroll
        for (int mm = 0; mm < VPP; ++mm) {
          const int mv = m0 + mm, t = mv >> 1, col = (mv & 1) ? T + t : t;
          if (mv < nvec) {
            float w;
            if (KDA) {
              w = Cs[i * CS + col];
            } else {
              w = (Cs[i * CS + col] * gi) * Gp[t];
            }
            acc[mm] += dq * w;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < QPT; ++j) {
        const int rq = rg + RG * j;
#pragma unroll
        for (int mm = 0; mm < VPP; ++mm) {
          const f4 x = load4(xr + (m0 + mm) * XS + 4 * rq);
          acc[mm] += s[j][0] * x[0];
          acc[mm] += s[j][1] * x[1];
          acc[mm] += s[j][2] * x[2];
          acc[mm] += s[j][3] * x[3];
        }
      }
      // sum the RL row groups of the wave: adjacent lanes by DPP, or lanes CC apart by
      // permlane swaps
#pragma unroll
      for (int mm = 0; mm < VPP; ++mm) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float v = acc[mm][jj];
          if constexpr (ADJ) {
            v = adjacent_sum<RL>(v);
          } else {
            if constexpr (CC <= 8) v = xor_sum<8>(v);
            if constexpr (CC <= 16) v = xor_sum<16>(v);
            v = xor_sum<32>(v);
          }
          acc[mm][jj] = v;
        }
      }
      if (ADJ ? lane % RL == 0 : lane < CC) {
#pragma unroll
        for (int mm = 0; mm < VPP; ++mm) store4(red + (wave * VPP + mm) * BV + 4 * cc, acc[mm]);
      }
      lds_barrier();
      if (SPREAD || tid < BV) {
#pragma unroll
        for (int mm = 0; mm < VPP; ++mm) {
          const int m = m0 + mm;
          if (m < nvec) {
            Pv[m] = (red[mm * BV + tid % BV] + red[(VPP + mm) * BV + tid % BV]) +
                    (red[(2 * VPP + mm) * BV + tid % BV] + red[(3 * VPP + mm) * BV + tid % BV]);
          }
        }
      }
    }
  }

  // 9. per column: forward substitution over the window, outputs, ring deltas.  Windows of
  // 8 and more: every thread solves its column (tid % BV), and the kThreads / BV threads of
  // a column share its 2T stores, which would otherwise queue behind one another in one
  // wave.
  if (SPREAD || tid < BV) {
    constexpr int NQ = SPREAD ? kThreads / BV : 1;
    const int c = tid % BV, col = col0 + c, grp = tid / BV;
    float d[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        float U = beta_s[t] * (to_f32(xv[t * BV + c]) - Pv[2 * t + 1]);
#pragma unroll
        for (int u = 0; u < t; ++u) U = fmaf(-Am[t * TMAX + u], d[u], U);
        d[t] = U;
      }
    }
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        float o = Pv[2 * t];
#pragma unroll
        for (int u = 0; u <= t; ++u) o = fmaf(Qm[t * TMAX + u], d[u], o);
        if (t % NQ == grp) {
          a.out[((tok0 + t) * hv + h) * dv + col] = o * a.scale;
          a.ring_d[(((size_t)slot * L + base + t) * hv + h) * dv + col] = d[t];
        }
      }
    }
  }

  // 10. wave 0: write_pos, and the window's keys and gates.  The keys are shared by the
  // key group: one workgroup of it writes them.  GDN's gates are per head: each head's
  // first column tile writes its own, except on a fold, where the rows written are rows
  // other workgroups of the key group may still be reading, so the last of them writes all
  // of the group's, one lane per (token, head).  (KDA: G = 1, the same workgroup; its
  // gates, rows of dk, were written during the scores unless the window folds.)
  if (wave == 0) {
    if (a.write_pos_out && h == 0 && vt == 0 && lane == 0) a.write_pos_out[row] = base;
    const bool writer = fold ? last : (h % a.G == 0 && vt == 0);
    if (writer) {
      bf16* rk = static_cast<bf16*>(a.ring_k);
      for (int i = lane; i < T * (DK / 8); i += 64) {           // 16-byte chunks
        const int t = i / (DK / 8), c8 = (i - t * (DK / 8)) * 8;
        *reinterpret_cast<uint4*>(rk + (((size_t)slot * L + base + t) * hk + kh) * DK + c8) =
            *reinterpret_cast<const uint4*>(xkq + (T + t) * KS + c8);
      }
      if (KDA) {
        if (fold) {                                      // (not folding: step 5)
          for (int i = lane; i < T * DK; i += 64) {
            const int t = i / DK, r = i - t * DK;
            a.ring_g[(((size_t)slot * L + t) * hv + h) * DK + r] =
                to_f32(gg[((tok0 + t) * hv + h) * DK + r]);
          }
        }
      } else if (fold) {
        for (int i = lane; i < T * a.G; i += 64) {
          const int t = i / a.G, hh = kh * a.G + (i - t * a.G);
          a.ring_g[((size_t)slot * L + t) * hv + hh] = to_f32(gg[(tok0 + t) * hv + hh]);
        }
      }
      if (fold && lane == 0)
        __hip_atomic_store(a.group_counter + (size_t)row * hk + kh, 0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!KDA && !fold && vt == 0 && lane < T)                     // (gate_s: this head's)
      a.ring_g[((size_t)slot * L + base + lane) * hv + h] = pick(gate_s, lane);
  }
}

template <bool KDA, typename ST, int BV, int TMAX>
static hipError_t run_fast(const VerifyArgs& a, const FastLayout& lay, const RowWindows& w,
                           hipStream_t s) {
  auto k = w.cu_seqlens ? verify_fast_kernel<KDA, ST, BV, TMAX, true>
                        : verify_fast_kernel<KDA, ST, BV, TMAX, false>;
  if (lay.total > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lay.total);
  hipLaunchKernelGGL(k, dim3(a.nblocks), dim3(kThreads), lay.total, s, a, lay, w);
  return hipGetLastError();
}

template <bool KDA, typename ST, int BV>
static hipError_t fast_tmax(int tmax, const VerifyArgs& a, const FastLayout& lay,
                            const RowWindows& w, hipStream_t s) {
  switch (tmax) {
    case 1: return run_fast<KDA, ST, BV, 1>(a, lay, w, s);
    case 2: return run_fast<KDA, ST, BV, 2>(a, lay, w, s);
    case 3: return run_fast<KDA, ST, BV, 3>(a, lay, w, s);
    case 4: return run_fast<KDA, ST, BV, 4>(a, lay, w, s);
    case 8: return run_fast<KDA, ST, BV, 8>(a, lay, w, s);
    case 16: return run_fast<KDA, ST, BV, 16>(a, lay, w, s);
  }
  return hipErrorInvalidValue;
}

template <bool KDA, typename ST>
static hipError_t fast_bv(int bv, int tmax, const VerifyArgs& a, const FastLayout& lay,
                          const RowWindows& w, hipStream_t s) {
  switch (bv) {
    case 32: return fast_tmax<KDA, ST, 32>(tmax, a, lay, w, s);
    case 64: return fast_tmax<KDA, ST, 64>(tmax, a, lay, w, s);
    case 128: return fast_tmax<KDA, ST, 128>(tmax, a, lay, w, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_verify_fast(bool kda, int state_bf16, int bv, int tmax, const VerifyArgs& a,
                              const FastLayout& lay, const RowWindows& w, hipStream_t s) {
  if (kda) return state_bf16 ? fast_bv<true, bf16>(bv, tmax, a, lay, w, s)
                             : fast_bv<true, float>(bv, tmax, a, lay, w, s);
  return state_bf16 ? fast_bv<false, bf16>(bv, tmax, a, lay, w, s)
                    : fast_bv<false, float>(bv, tmax, a, lay, w, s);
}

}  // namespace rs
