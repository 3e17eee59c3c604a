// Commit fold and materialize for dk = 128 with bf16 keys (the Qwen3.5-shaped GDN and KDA
// layers), gfx950.
//
// Same method as fold_kernel in rs_kernels.hip: for a slot with nrec records,
//   S <- Gam (.) S + sum_{i < nrec} khat_i d_i^T,  khat_i = gamma_i (.) k_i,
// gamma_i = prod_{i<j<nrec} alpha_j, Gam = prod_{j<nrec} alpha_j (per key channel for KDA),
// written back in place (commit fold, nrec = fold_len) or as an fp32 copy (materialize,
// nrec = cursor).  The difference is where the tile lives: the [128 x BV] tile goes from
// HBM (non-temporal loads) straight into fp32 MFMA accumulators, four consecutive
// columns of one row per lane, and the rank-nrec update runs on v_mfma_f32_16x16x4_f32
// with the records as the contraction index (A = d_i of 16 columns, B = khat_i of 16
// rows).  Records come in by HBM->LDS copies; a wave owns 32 rows of the tile.  Records at
// or past nrec are selected to zero before the MFMA, never read from the ring.
#include <type_traits>

#include "rs_device.h"
#include "rs_internal.h"

namespace rs {

template <bool KDA, typename ST, typename OT, int BV, bool MATERIALIZE>
__global__ __launch_bounds__(kThreads) void fold_fast_kernel(FoldArgs a, FoldFastLayout lay) {
  constexpr int DK = 128, KS = kKeyStride;
  constexpr int NCB = BV / 16;                 // 16-column blocks of the tile
  constexpr int RBW = DK / 16 / kWaves;        // 16-row blocks per wave
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, q4 = lane >> 4;
  const int lid = xcd_group_remap(blockIdx.x, a.nblocks, a.G * a.NV);
  const int vt = umod(lid, a.NV);
  const int h = umod(udiv(lid, a.NV), a.hv);
  const int row = udiv(lid, a.NV * a.hv);
  const int slot = a.slot_idx[row];
  if (slot < 0 || slot >= a.num_slots) return;          // null row: no reads, no writes
  const int L = a.L, dv = a.dv, hv = a.hv, hk = a.hk;
  int n = a.nrec[slot];
  n = n < 0 ? 0 : (n > L ? L : n);
  if (!MATERIALIZE && n == 0) return;                   // nothing to commit
  const int kh = udiv(h, a.G), col0 = vt * BV;

  bf16* hkeys = reinterpret_cast<bf16*>(smem + lay.hkeys);
  float* hd = reinterpret_cast<float*>(smem + lay.hd);
  float* hg = reinterpret_cast<float*>(smem + lay.hg);
  float* gam_i = reinterpret_cast<float*>(smem + lay.gam_i);
  float* Gamv = reinterpret_cast<float*>(smem + lay.Gam);

  // 1. records [0, n): keys, this tile's deltas, gates -> LDS, asynchronous
  if (n > 0) {
    const bf16* rkg = static_cast<const bf16*>(a.ring_k);
    dma_rows_256(rkg + ((size_t)slot * L * hk + kh) * DK, (size_t)hk * DK * 2, n, hkeys,
                 KS * 2);
    dma_rows(a.ring_d + ((size_t)slot * L * hv + h) * dv + col0, (size_t)hv * dv * 4, BV * 4, n,
             hd);
    if (KDA)
      dma_rows(a.ring_g + ((size_t)slot * L * hv + h) * DK, (size_t)hv * DK * 4, DK * 4, n, hg);
    else
      dma_words(a.ring_g + (size_t)slot * L * hv + h, (size_t)hv * 4, n, hg);
  }
  code_fence();

  // 2. the state tile -> accumulators: lane holds row rb*16 + i16, columns cb*16 + 4*q4 ..+3
  const ST* src =
      static_cast<const ST*>(a.state_in) + (((size_t)slot * hv + h) * DK) * dv + col0;
  f4 acc[RBW][NCB];
#pragma unroll
  for (int rbi = 0; rbi < RBW; ++rbi) {
    const int r = (wave * RBW + rbi) * 16 + i16;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      acc[rbi][cb] = load4_nt(src + (uint32_t)(r * dv + cb * 16 + 4 * q4));
  }
  code_fence();
  lds_barrier<RBW * NCB>();                              // the records are in LDS

  // 3. decays.  GDN: Gam (every thread), gamma_i (thread i).  KDA: per key channel, the
  // gates of record i are replaced in place by khat_i = gamma_i (.) k_i.
  float Gam = 1.f;
  if (!KDA) {
    for (int i = 0; i < n; ++i) Gam *= hg[i];
    for (int i = tid; i < n; i += kThreads) {
      float g = 1.f;
      for (int j = i + 1; j < n; ++j) g *= hg[j];
      gam_i[i] = g;
    }
  } else if (tid < DK) {
    float g = 1.f;
    for (int i = n - 1; i >= 0; --i) {
      const float al = hg[i * DK + tid];
      hg[i * DK + tid] = g * to_f32(hkeys[i * KS + tid]);
      g *= al;
    }
    Gamv[tid] = g;
  }
  lds_barrier();

  // 4. S <- Gam (.) S, then the rank-n update on MFMA, four records per step
#pragma unroll
  for (int rbi = 0; rbi < RBW; ++rbi) {
    const float gr = KDA ? Gamv[(wave * RBW + rbi) * 16 + i16] : Gam;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[rbi][cb] *= gr;
  }
  for (int ks = 0; ks < (n + 3) >> 2; ++ks) {
    const int rec = 4 * ks + q4;
    const bool ok = rec < n;
    const int rs = ok ? rec : 0;                         // a row that exists; selected away
    const float gsc = KDA ? 1.f : gam_i[rs];
    float av[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const float dval = hd[rs * BV + cb * 16 + i16] * gsc;
      av[cb] = ok ? dval : 0.f;
    }
#pragma unroll
    for (int rbi = 0; rbi < RBW; ++rbi) {
      const int r = (wave * RBW + rbi) * 16 + i16;
      const float kv = KDA ? hg[rs * DK + r] : to_f32(hkeys[rs * KS + r]);
      const float b = ok ? kv : 0.f;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) acc[rbi][cb] = mfma_16x16x4(av[cb], b, acc[rbi][cb]);
    }
  }

  // 5. one write: the state in place (its dtype, RNE) or the fp32 materialized copy.  The
  // accumulators hold 16 rows x 4 columns per 16-column block, so a store straight from
  // them would write each row in 64-byte pieces (measured: 1.36x the state's bytes reach
  // HBM).  Each wave instead passes its 16-row blocks through LDS, over the record region
  // (dead once every wave is past the update), and stores whole row segments: BV / 4 lanes
  // per row, as the verify does.
  OT* dst = MATERIALIZE
      ? static_cast<OT*>(a.state_out) + (((size_t)row * hv + h) * DK) * dv + col0
      : static_cast<OT*>(a.state_out) + (((size_t)slot * hv + h) * DK) * dv + col0;
  constexpr int SST = BV + 4;                  // staging row stride (floats): no bank repeats
  constexpr int CPR = BV / 4, RPI = 64 / CPR;  // lanes per row, rows per store instruction
  lds_barrier();                               // every wave has read its last record
  float* stg = reinterpret_cast<float*>(smem + lay.stage) + wave * 16 * SST;
  const int sr = lane / CPR, sq = lane % CPR;
#pragma unroll
  for (int rbi = 0; rbi < RBW; ++rbi) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) store4(stg + i16 * SST + cb * 16 + 4 * q4, acc[rbi][cb]);
    asm volatile("" ::: "memory");             // one wave: LDS operations stay in order
    const int r0 = (wave * RBW + rbi) * 16;
#pragma unroll
    for (int k = 0; k < 16 / RPI; ++k) {
      const int rr = k * RPI + sr;
      store4_nt(dst + (uint32_t)((r0 + rr) * dv + 4 * sq), load4(stg + rr * SST + 4 * sq));
    }
    asm volatile("" ::: "memory");
  }
}

// Commit fold and materialize of a bf16 state in 128-column tiles.  The MFMA fold above
// keeps the tile as MFMA accumulators, whose lane layout would read a bf16 row in 32-byte
// pieces.  Here a 16-lane group reads whole 256-byte rows (8 columns a lane; wave w holds
// rows 32w + 16j + 4g + i, g = lane / 16), and the rank-nrec update runs on the VALU in
// fp32, four rows at a time, with one bf16 rounding per element at the end.  Same method,
// records and decays as fold_fast_kernel.
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

template <bool KDA, bool MATERIALIZE>
__global__ __launch_bounds__(kThreads, 4) void fold_bf16_kernel(FoldArgs a, FoldFastLayout lay) {
  constexpr int DK = 128, KS = kKeyStride, BV = 128;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lc = lane & 15, lg = lane >> 4;
  const int lid = xcd_group_remap(blockIdx.x, a.nblocks, a.G * a.NV);
  const int vt = umod(lid, a.NV);
  const int h = umod(udiv(lid, a.NV), a.hv);
  const int row = udiv(lid, a.NV * a.hv);
  const int slot = a.slot_idx[row];
  if (slot < 0 || slot >= a.num_slots) return;          // null row: no reads, no writes
  const int L = a.L, dv = a.dv, hv = a.hv, hk = a.hk;
  int n = a.nrec[slot];
  n = n < 0 ? 0 : (n > L ? L : n);
  if (!MATERIALIZE && n == 0) return;                   // nothing to commit
  const int kh = udiv(h, a.G), col0 = vt * BV;

  bf16* hkeys = reinterpret_cast<bf16*>(smem + lay.hkeys);
  float* hd = reinterpret_cast<float*>(smem + lay.hd);
  float* hg = reinterpret_cast<float*>(smem + lay.hg);
  float* gam_i = reinterpret_cast<float*>(smem + lay.gam_i);
  float* Gamv = reinterpret_cast<float*>(smem + lay.Gam);

  // 1. records [0, n) -> LDS, asynchronous
  if (n > 0) {
    const bf16* rkg = static_cast<const bf16*>(a.ring_k);
    dma_rows_256(rkg + ((size_t)slot * L * hk + kh) * DK, (size_t)hk * DK * 2, n, hkeys,
                 KS * 2);
    dma_rows(a.ring_d + ((size_t)slot * L * hv + h) * dv + col0, (size_t)hv * dv * 4, BV * 4, n,
             hd);
    if (KDA)
      dma_rows(a.ring_g + ((size_t)slot * L * hv + h) * DK, (size_t)hv * DK * 4, DK * 4, n, hg);
    else
      dma_words(a.ring_g + (size_t)slot * L * hv + h, (size_t)hv * 4, n, hg);
  }
  code_fence();

  // 2. the state tile -> registers, 16 bytes (8 bf16) per load
  const bf16* src =
      static_cast<const bf16*>(a.state_in) + (((size_t)slot * hv + h) * DK) * dv + col0;
  u4 raw[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      raw[j][i] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(
          src + (uint32_t)((32 * wave + 16 * j + 4 * lg + i) * dv + 8 * lc)));
  }
  code_fence();
  lds_barrier<8>();                                      // the records are in LDS

  // 3. decays, as in fold_fast_kernel
  float Gam = 1.f;
  if (!KDA) {
    for (int i = 0; i < n; ++i) Gam *= hg[i];
    for (int i = tid; i < n; i += kThreads) {
      float g = 1.f;
      for (int j = i + 1; j < n; ++j) g *= hg[j];
      gam_i[i] = g;
    }
  } else if (tid < DK) {
    float g = 1.f;
    for (int i = n - 1; i >= 0; --i) {
      const float al = hg[i * DK + tid];
      hg[i * DK + tid] = g * to_f32(hkeys[i * KS + tid]);
      g *= al;
    }
    Gamv[tid] = g;
  }
  lds_barrier();

  // 4. S <- Gam (.) S + sum_i khat_i d_i^T, four rows at a time, then one write
  bf16* dst16 = static_cast<bf16*>(a.state_out) + (((size_t)slot * hv + h) * DK) * dv + col0;
  float* dst32 = static_cast<float*>(a.state_out) + (((size_t)row * hv + h) * DK) * dv + col0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r0 = 32 * wave + 16 * j + 4 * lg;
    float f[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gr = KDA ? Gamv[r0 + i] : Gam;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[i][2 * q] = __uint_as_float(raw[j][i][q] << 16) * gr;
        f[i][2 * q + 1] = __uint_as_float(raw[j][i][q] & 0xffff0000u) * gr;
      }
    }
    for (int rec = 0; rec < n; ++rec) {
      const f4 d0 = load4(hd + rec * BV + 8 * lc);
      const f4 d1 = load4(hd + rec * BV + 8 * lc + 4);
      const f4 kq = KDA ? load4(hg + rec * DK + r0)
                        : load4(hkeys + rec * KS + r0) * gam_i[rec];
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
      const uint32_t off = (uint32_t)((r0 + i) * dv + 8 * lc);
      if constexpr (MATERIALIZE) {
        store4_nt(dst32 + off, f4{f[i][0], f[i][1], f[i][2], f[i][3]});
        store4_nt(dst32 + off + 4, f4{f[i][4], f[i][5], f[i][6], f[i][7]});
      } else {
        u4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = uint32_t(bf16_rne(f[i][2 * q])) | (uint32_t(bf16_rne(f[i][2 * q + 1])) << 16);
        __builtin_nontemporal_store(w, reinterpret_cast<u4*>(dst16 + off));
      }
    }
  }
}

hipError_t launch_fold_bf16(bool kda, bool materialize, const FoldArgs& a,
                            const FoldFastLayout& lay, hipStream_t s) {
  auto k = kda ? (materialize ? fold_bf16_kernel<true, true> : fold_bf16_kernel<true, false>)
               : (materialize ? fold_bf16_kernel<false, true> : fold_bf16_kernel<false, false>);
  if (lay.total > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lay.total);
  hipLaunchKernelGGL(k, dim3(a.nblocks), dim3(kThreads), lay.total, s, a, lay);
  return hipGetLastError();
}

template <bool KDA, typename ST, int BV, bool MAT>
static hipError_t run_fold_fast(const FoldArgs& a, const FoldFastLayout& lay, hipStream_t s) {
  using OT = typename std::conditional<MAT, float, ST>::type;
  auto k = fold_fast_kernel<KDA, ST, OT, BV, MAT>;
  if (lay.total > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lay.total);
  hipLaunchKernelGGL(k, dim3(a.nblocks), dim3(kThreads), lay.total, s, a, lay);
  return hipGetLastError();
}

template <bool KDA, typename ST, bool MAT>
static hipError_t fold_fast_bv(int bv, const FoldArgs& a, const FoldFastLayout& lay,
                               hipStream_t s) {
  switch (bv) {
    case 32: return run_fold_fast<KDA, ST, 32, MAT>(a, lay, s);
    case 64: return run_fold_fast<KDA, ST, 64, MAT>(a, lay, s);
    case 128: return run_fold_fast<KDA, ST, 128, MAT>(a, lay, s);
  }
  return hipErrorInvalidValue;
}

template <bool KDA, typename ST>
static hipError_t fold_fast_mat(int bv, bool mat, const FoldArgs& a, const FoldFastLayout& lay,
                                hipStream_t s) {
  return mat ? fold_fast_bv<KDA, ST, true>(bv, a, lay, s)
             : fold_fast_bv<KDA, ST, false>(bv, a, lay, s);
}

hipError_t launch_fold_fast(bool kda, int state_bf16, int bv, bool materialize,
                            const FoldArgs& a, const FoldFastLayout& lay, hipStream_t s) {
  if (kda) return state_bf16 ? fold_fast_mat<true, bf16>(bv, materialize, a, lay, s)
                             : fold_fast_mat<true, float>(bv, materialize, a, lay, s);
  return state_bf16 ? fold_fast_mat<false, bf16>(bv, materialize, a, lay, s)
                    : fold_fast_mat<false, float>(bv, materialize, a, lay, s);
}

}  // namespace rs
