// Verify for dk = 128 with bf16 inputs (the Qwen3.5-shaped GDN and KDA layers), gfx950.
//
// Same method as verify_kernel in rs_kernels.hip; the difference is how the workgroup
// spends its time.  The [128 x BV] state tile is the only large operand, and it streams
// straight into registers (four rows x four columns per thread, 256-byte row segments per
// 16 lanes) as one compile-time block of loads, issued after every small operand has
// been queued by direct HBM->LDS copies.  One explicit wait for "all but the tile" then
// lets the scalar work (decays, window pair products, history scores) run while the
// tile is still in flight.
//
// History is not replayed into the tile.  With H = Gam (.) S + sum_i khat_i d_i^T
// (khat_i = gamma_i (.) k_i), the readout splits into
//   H^T x = S^T (Gam (.) x) + sum_i d_i (khat_i . x),
// a pass over the registers plus nh scores per window vector (sglang commit 5: history
// terms only when write_pos is nonzero).  A row whose window would overflow the ring
// instead folds its prefix into the registers, writes the state back once and reads
// out with no history.
#include "rs_device.h"
#include "rs_internal.h"

namespace rs {

// A bf16 value at a workgroup-uniform address, through the scalar data cache.
__device__ __forceinline__ float load_bf16_uniform(const bf16* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const __attribute__((address_space(4))) uint32_t* w =
      (const __attribute__((address_space(4))) uint32_t*)(a & ~uintptr_t(3));
  const uint32_t v = *w;
  return __uint_as_float((a & 2) ? (v & 0xffff0000u) : (v << 16));
}

__device__ __forceinline__ f4 bf16x4(const bf16* p) { return load4(p); }

template <bool KDA, typename ST, int BV, int TMAX>
__global__ __launch_bounds__(kThreads) void verify_fast_kernel(VerifyArgs a, FastLayout lay) {
  constexpr int DK = 128;
  constexpr int CC = BV / 4, RG = kThreads / CC, NQ = DK / 4, QPT = NQ / RG;
  constexpr int VPP = (2 * TMAX < 8) ? 2 * TMAX : 8;
  constexpr int CS = 2 * TMAX;                 // row stride of the score matrix
  static_assert(NQ % RG == 0 && QPT >= 1, "tile split");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cc = tid % CC, rg = tid / CC;
  const int lid = xcd_remap(blockIdx.x, a.nblocks);
  const int vt = lid % a.NV;
  const int h = (lid / a.NV) % a.hv;
  const int row = lid / (a.NV * a.hv);
  const int slot = a.slot_idx[row];
  if (slot < 0 || slot >= a.num_slots) return;          // null row: no reads, no writes

  const int T = a.T, L = a.L, hv = a.hv, hk = a.hk, dv = a.dv;
  const int kh = h / a.G, col0 = vt * BV;
  const size_t tok0 = (size_t)row * T;
  const int XS = lay.xs_stride;

  bf16* xkq = reinterpret_cast<bf16*>(smem + lay.xkq);
  bf16* xv = reinterpret_cast<bf16*>(smem + lay.xv);
  bf16* xg = reinterpret_cast<bf16*>(smem + lay.xg);
  bf16* hkeys = reinterpret_cast<bf16*>(smem + lay.hkeys);
  float* hd = reinterpret_cast<float*>(smem + lay.hd);
  float* hg = reinterpret_cast<float*>(smem + lay.hg);
  float* khat = reinterpret_cast<float*>(smem + lay.khat);
  float* gam_i = reinterpret_cast<float*>(smem + lay.gam_i);
  float* Gam = reinterpret_cast<float*>(smem + lay.Gam);
  float* xs = reinterpret_cast<float*>(smem + lay.xs);
  float* xr = reinterpret_cast<float*>(smem + lay.xr);
  float* Cs = reinterpret_cast<float*>(smem + lay.C);
  float* P = reinterpret_cast<float*>(smem + lay.P);
  float* red = reinterpret_cast<float*>(smem + lay.red);
  float* Am = reinterpret_cast<float*>(smem + lay.Am);
  float* Qm = reinterpret_cast<float*>(smem + lay.Qm);
  float* bw = reinterpret_cast<float*>(smem + lay.bw);
  float* gw = reinterpret_cast<float*>(smem + lay.gw);
  int* flags = reinterpret_cast<int*>(smem + lay.flags);

  const bf16* qg = static_cast<const bf16*>(a.q);
  const bf16* kg = static_cast<const bf16*>(a.k);
  const bf16* vg = static_cast<const bf16*>(a.v);
  const bf16* bg = static_cast<const bf16*>(a.beta);
  const bf16* gg = static_cast<const bf16*>(a.gate);
  const bf16* rkg = static_cast<const bf16*>(a.ring_k);

  // 1. scalars through the scalar cache, before anything writes memory: the cursor, and
  // the window's betas and (GDN) gates
  int n = a.cursor[slot];
  n = n < 0 ? 0 : (n > L ? L : n);
  const bool fold = n + T > L;                           // the window would overflow
  const int base = fold ? 0 : n;                         // write_pos
  const int nh = n;
  float beta_s[TMAX], gate_s[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    beta_s[t] = t < T ? load_bf16_uniform(bg + (tok0 + t) * hv + h) : 0.f;
    gate_s[t] = (!KDA && t < T) ? load_bf16_uniform(gg + (tok0 + t) * hv + h) : 0.f;
  }

  // 2. window operands and the committed history [0, n): HBM -> LDS, asynchronous
  dma_rows(qg + (tok0 * hk + kh) * DK, (size_t)hk * DK * 2, DK * 2, T, xkq);
  dma_rows(kg + (tok0 * hk + kh) * DK, (size_t)hk * DK * 2, DK * 2, T, xkq + T * DK);
  dma_rows(vg + (tok0 * hv + h) * dv + col0, (size_t)hv * dv * 2, BV * 2, T, xv);
  if (KDA) dma_rows(gg + (tok0 * hv + h) * DK, (size_t)hv * DK * 2, DK * 2, T, xg);
  if (nh > 0) {
    dma_rows(rkg + ((size_t)slot * L * hk + kh) * DK, (size_t)hk * DK * 2, DK * 2, nh, hkeys);
    dma_rows(a.ring_d + ((size_t)slot * L * hv + h) * dv + col0, (size_t)hv * dv * 4, BV * 4,
             nh, hd);
    if (KDA)
      dma_rows(a.ring_g + ((size_t)slot * L * hv + h) * DK, (size_t)hv * DK * 4, DK * 4, nh, hg);
    else
      dma_words(a.ring_g + (size_t)slot * L * hv + h, (size_t)hv * 4, nh, hg);
  }
  code_fence();

  // 3. the state tile: HBM -> registers, the last vector loads issued before the wait
  const ST* sg = static_cast<const ST*>(a.state) + (((size_t)slot * hv + h) * DK) * dv + col0;
  f4 s[QPT][4];
#pragma unroll
  for (int j = 0; j < QPT; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[j][i] = load4(sg + (size_t)(4 * (rg + RG * j) + i) * dv + 4 * cc);
  }
  code_fence();

  if (tid == 0) {
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        bw[t] = beta_s[t];
        gw[t] = gate_s[t];
      }
    }
  }
  lds_barrier<QPT * 4>();                                // every copy but the tile is in LDS

  // 4. decays: window prefix products and scaled window vectors; history suffix products
  if (tid < DK) {
    float run = 1.f;
    for (int t = 0; t < T; ++t) {
      run *= KDA ? to_f32(xg[t * DK + tid]) : gw[t];
      xs[t * XS + tid] = run * to_f32(xkq[t * DK + tid]);
      xs[(T + t) * XS + tid] = run * to_f32(xkq[(T + t) * DK + tid]);
    }
    for (int m = 2 * T; m < lay.nvec_pad; ++m) xs[m * XS + tid] = 0.f;
    if (KDA) {
      float g = 1.f;
      for (int i = nh - 1; i >= 0; --i) {
        khat[i * XS + tid] = g * to_f32(hkeys[i * DK + tid]);
        g *= hg[i * DK + tid];
      }
      Gam[tid] = g;
    }
  }
  if (!KDA) {
    // gamma_i = prod_{i<j<nh} alpha_j, each thread on its own record; Gam = gamma_0 alpha_0
    const int i = kThreads - 1 - tid;
    if (i < nh) {
      float g = 1.f;
      for (int j = i + 1; j < nh; ++j) g *= hg[j];
      gam_i[i] = g;
      if (i == 0) Gam[0] = g * hg[0];
    }
    if (nh == 0 && tid == kThreads - 1) Gam[0] = 1.f;
  }
  lds_barrier();

  // 5. readout vectors, window pair scalars, history scores
  if (!fold && tid < DK) {
    const float G = KDA ? Gam[tid] : Gam[0];
    for (int m = 0; m < lay.nvec_pad; ++m) xr[m * XS + tid] = G * xs[m * XS + tid];
  }
  {
    const int npair = T * T, ndots = npair + (fold ? 0 : nh * 2 * T);
    for (int d = tid; d < ndots; d += kThreads) {
      if (d < npair) {
        const int t = d / T, u = d - t * T;
        if (u <= t) {
          const bf16* qt = xkq + t * DK;
          const bf16* kt = xkq + (T + t) * DK;
          const bf16* ku = xkq + (T + u) * DK;
          float sq = 0.f, sk = 0.f;
          if (KDA) {
            for (int r = 0; r < DK; r += 4) {
              f4 dec = f4{1.f, 1.f, 1.f, 1.f};
              for (int w = u + 1; w <= t; ++w) dec *= bf16x4(xg + w * DK + r);
              const f4 kd = bf16x4(ku + r) * dec;
              const f4 a4 = bf16x4(qt + r) * kd, b4 = bf16x4(kt + r) * kd;
              sq += (a4[0] + a4[1]) + (a4[2] + a4[3]);
              sk += (b4[0] + b4[1]) + (b4[2] + b4[3]);
            }
          } else {
            float dec = 1.f;
            for (int w = u + 1; w <= t; ++w) dec *= gw[w];
            for (int r = 0; r < DK; r += 4) {
              const f4 k4 = bf16x4(ku + r);
              const f4 a4 = bf16x4(qt + r) * k4, b4 = bf16x4(kt + r) * k4;
              sq += (a4[0] + a4[1]) + (a4[2] + a4[3]);
              sk += (b4[0] + b4[1]) + (b4[2] + b4[3]);
            }
            sq *= dec;
            sk *= dec;
          }
          Qm[t * TMAX + u] = sq;
          if (u < t) Am[t * TMAX + u] = bw[t] * sk;
        }
      } else {
        const int e = d - npair, i = e / (2 * T), m = e - i * (2 * T);
        const float* xm = xs + m * XS;
        float sc = 0.f;
        if (KDA) {
          const float* ki = khat + i * XS;
          for (int r = 0; r < DK; r += 4) {
            const f4 p4 = load4(ki + r) * load4(xm + r);
            sc += (p4[0] + p4[1]) + (p4[2] + p4[3]);
          }
        } else {
          const bf16* ki = hkeys + i * DK;
          for (int r = 0; r < DK; r += 4) {
            const f4 p4 = bf16x4(ki + r) * load4(xm + r);
            sc += (p4[0] + p4[1]) + (p4[2] + p4[3]);
          }
          sc *= gam_i[i];
        }
        Cs[i * CS + m] = sc;
      }
    }
  }
  lds_barrier();

  // This workgroup has read every ring record it needs (the copies have landed in LDS).
  // On a fused fold the window's keys and gates go to rows 0..T-1, which other workgroups
  // of the key group may still read: only the last of them to get here writes them (no
  // spinning).  Only read-before-write ordering is at stake, no data passes through the
  // counter: every increment follows its workgroup's completed reads, and the writes
  // follow the return of the last increment, so a relaxed device-scope atomic suffices.
  // The flag reaches the other threads through the barriers of the readout.
  if (fold && tid == 0) {
    const int old = __hip_atomic_fetch_add(a.group_counter + (size_t)row * hk + kh, 1,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    flags[0] = (old == a.G * a.NV - 1);
  }

  // 6. rows that overflow: fold the prefix into the registers and write the state once
  if (fold) {
    const float G0 = KDA ? 0.f : Gam[0];
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int r0 = 4 * (rg + RG * j);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[j][i] *= KDA ? Gam[r0 + i] : G0;
    }
    for (int i = 0; i < nh; ++i) {
      const f4 dq = load4(hd + i * BV + 4 * cc);
      const float gi = KDA ? 1.f : gam_i[i];
#pragma unroll
      for (int j = 0; j < QPT; ++j) {
        const int r0 = 4 * (rg + RG * j);
        const f4 kq = KDA ? load4(khat + i * XS + r0) : bf16x4(hkeys + i * DK + r0) * gi;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) s[j][ii] += kq[ii] * dq;
      }
    }
    ST* so = static_cast<ST*>(a.state) + (((size_t)slot * hv + h) * DK) * dv + col0;
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        store4(so + (size_t)(4 * (rg + RG * j) + i) * dv + 4 * cc, s[j][i]);
        s[j][i] = round4<ST>(s[j][i]);
      }
    }
  }

  // 7. readout P[m][c] = H^T x_m over the tile registers (+ history scores), reduced over
  // the row groups of a wave by butterflies, then over the 4 waves through LDS
  const float* xv_read = fold ? xs : xr;
  const int nvec = 2 * T;
  for (int m0 = 0; m0 < nvec; m0 += VPP) {
    f4 acc[VPP];
#pragma unroll
    for (int m = 0; m < VPP; ++m) acc[m] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int rq = rg + RG * j;
#pragma unroll
      for (int m = 0; m < VPP; ++m) {
        const f4 x = load4(xv_read + (m0 + m) * XS + 4 * rq);
        acc[m] += s[j][0] * x[0];
        acc[m] += s[j][1] * x[1];
        acc[m] += s[j][2] * x[2];
        acc[m] += s[j][3] * x[3];
      }
    }
    if (!fold) {
      for (int i = rg; i < nh; i += RG) {
        const f4 dq = load4(hd + i * BV + 4 * cc);
#pragma unroll
        for (int m = 0; m < VPP; ++m) {
          const float c = (m0 + m < nvec) ? Cs[i * CS + m0 + m] : 0.f;
          acc[m] += dq * c;
        }
      }
    }
#pragma unroll
    for (int off = CC; off < 64; off <<= 1) {
#pragma unroll
      for (int m = 0; m < VPP; ++m) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[m][jj] += __shfl_xor(acc[m][jj], off);
      }
    }
    if (lane < CC) {
#pragma unroll
      for (int m = 0; m < VPP; ++m) store4(red + (wave * VPP + m) * BV + 4 * cc, acc[m]);
    }
    lds_barrier();
    for (int i = tid; i < VPP * BV; i += kThreads) {
      const int m = i / BV, c = i - m * BV;
      if (m0 + m < nvec)
        P[(m0 + m) * BV + c] = (red[m * BV + c] + red[(VPP + m) * BV + c]) +
                               (red[(2 * VPP + m) * BV + c] + red[(3 * VPP + m) * BV + c]);
    }
    lds_barrier();
  }

  // 8. per column: forward substitution over the window, outputs, ring deltas
  if (tid < BV) {
    const int c = tid, col = col0 + c;
    float d[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        float U = bw[t] * (to_f32(xv[t * BV + c]) - P[(T + t) * BV + c]);
#pragma unroll
        for (int u = 0; u < t; ++u) U = fmaf(-Am[t * TMAX + u], d[u], U);
        d[t] = U;
      }
    }
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        float o = P[t * BV + c];
#pragma unroll
        for (int u = 0; u <= t; ++u) o = fmaf(Qm[t * TMAX + u], d[u], o);
        a.out[((tok0 + t) * hv + h) * dv + col] = o;
        a.ring_d[(((size_t)slot * L + base + t) * hv + h) * dv + col] = d[t];
      }
    }
  }
  if (a.write_pos_out && h == 0 && vt == 0 && tid == 0) a.write_pos_out[row] = base;

  // 9. the window's keys and gates (shared by the key group / by the head's tiles)
  const bool writer = fold ? (flags[0] != 0) : (h % a.G == 0 && vt == 0);
  if (writer) {
    bf16* rk = static_cast<bf16*>(a.ring_k);
    for (int i = tid; i < T * (DK / 8); i += kThreads) {        // 16-byte chunks
      const int t = i / (DK / 8), c8 = (i - t * (DK / 8)) * 8;
      *reinterpret_cast<uint4*>(rk + (((size_t)slot * L + base + t) * hk + kh) * DK + c8) =
          *reinterpret_cast<const uint4*>(xkq + (T + t) * DK + c8);
    }
    if (KDA) {
      for (int i = tid; i < T * DK; i += kThreads) {
        const int t = i / DK, r = i - t * DK;
        a.ring_g[(((size_t)slot * L + base + t) * hv + h) * DK + r] = to_f32(xg[t * DK + r]);
      }
    } else if (tid == 0) {
      for (int t = 0; t < T; ++t)
        for (int g = 0; g < a.G; ++g) {
          const int hh = kh * a.G + g;
          a.ring_g[((size_t)slot * L + base + t) * hv + hh] =
              load_bf16_uniform(gg + (tok0 + t) * hv + hh);
        }
    }
    if (fold && tid == 0)
      __hip_atomic_store(a.group_counter + (size_t)row * hk + kh, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool KDA, typename ST, int BV, int TMAX>
static hipError_t run_fast(const VerifyArgs& a, const FastLayout& lay, hipStream_t s) {
  auto k = verify_fast_kernel<KDA, ST, BV, TMAX>;
  if (lay.total > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lay.total);
  hipLaunchKernelGGL(k, dim3(a.nblocks), dim3(kThreads), lay.total, s, a, lay);
  return hipGetLastError();
}

template <bool KDA, typename ST, int BV>
static hipError_t fast_tmax(int tmax, const VerifyArgs& a, const FastLayout& lay, hipStream_t s) {
  switch (tmax) {
    case 1: return run_fast<KDA, ST, BV, 1>(a, lay, s);
    case 2: return run_fast<KDA, ST, BV, 2>(a, lay, s);
    case 4: return run_fast<KDA, ST, BV, 4>(a, lay, s);
    case 8: return run_fast<KDA, ST, BV, 8>(a, lay, s);
    case 16: return run_fast<KDA, ST, BV, 16>(a, lay, s);
  }
  return hipErrorInvalidValue;
}

template <bool KDA, typename ST>
static hipError_t fast_bv(int bv, int tmax, const VerifyArgs& a, const FastLayout& lay,
                          hipStream_t s) {
  switch (bv) {
    case 32: return fast_tmax<KDA, ST, 32>(tmax, a, lay, s);
    case 64: return fast_tmax<KDA, ST, 64>(tmax, a, lay, s);
    case 128: return fast_tmax<KDA, ST, 128>(tmax, a, lay, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_verify_fast(bool kda, int state_bf16, int bv, int tmax, const VerifyArgs& a,
                              const FastLayout& lay, hipStream_t s) {
  if (kda) return state_bf16 ? fast_bv<true, bf16>(bv, tmax, a, lay, s)
                             : fast_bv<true, float>(bv, tmax, a, lay, s);
  return state_bf16 ? fast_bv<false, bf16>(bv, tmax, a, lay, s)
                    : fast_bv<false, float>(bv, tmax, a, lay, s);
}

}  // namespace rs
