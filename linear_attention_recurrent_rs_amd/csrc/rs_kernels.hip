// ReplaySSM kernels for gfx950: verify (GDN / KDA), commit fold, materialize, cursor advance.
//
// One workgroup (256 threads, 4 waves) owns one (value tile, value head, request row):
// a [dk x BV] tile of that row's canonical state S.  The tile comes from HBM once, by
// direct-to-LDS 16-byte loads into a bank-swizzled LDS tile.  History records are
// replayed into an fp32 copy of the tile by one routine, fold_tile (fp32 MFMA rank-n
// update), used alike by the fused in-verify fold, the commit fold and materialize
// (LightLLM: decode and the separate fold walk the history with one device function).
//
// Window math (per value column s, a dk-vector; H = state after history):
//   s_t = a_t (.) s_{t-1} + k_t d_t,  d_t = b_t (v_t - (a_t (.) s_{t-1}) . k_t),  o_t = s_t . q_t
// With G_t = prod_{w<=t} a_w and dec(u,t) = prod_{u<w<=t} a_w (products over the causal
// range only, never a division):
//   d_t = b_t (v_t - H . (G_t (.) k_t)) - sum_{u<t} A[t][u] d_u,  A[t][u] = b_t k_t . (dec(u,t) (.) k_u)
//   o_t = H . (G_t (.) q_t) + sum_{u<=t} Q[t][u] d_u,              Q[t][u] = q_t . (dec(u,t) (.) k_u)
// i.e. the unit-lower-triangular solve (I + A) D = U of the WY/UT form.  Every sum over
// window positions runs over the causal range by construction, so draft u's inputs reach
// only d_t, o_t with t >= u (sglang commit 3: select, never multiply by zero).
#include "rs_device.h"
#include "rs_internal.h"

namespace rs {

// ------------------------------------------------------------------ tile load
// Issue the [dk x BV] tile whose (row 0, col 0) is at g (row stride gld elements) into the
// swizzled LDS tile.  Asynchronous: wait_vmem() + barrier before reading it.
template <typename ST, int BV>
__device__ __forceinline__ void issue_tile(const ST* g, int gld, ST* lds, int dk) {
  using TL = Tile<ST, BV>;
  const int nch = dk * TL::kCpr;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  char* lds_bytes = reinterpret_cast<char*>(lds);
  for (int p0 = wave * 64; p0 < nch; p0 += kThreads) {
    const int p = p0 + lane;
    if (p < nch) {
      int r, chunk;
      TL::slot_source(p, r, chunk);
      load_lds_16(g + (size_t)r * gld + chunk * TL::kEpc, lds_bytes + (size_t)p0 * 16);
    }
  }
}

// ------------------------------------------------------------------ history
// Records [0, nh) of one slot: keys of key head kh (to fp32), gates of value head h, and
// the deltas of this tile's columns [col0, col0 + BV).  Loads never reach past nh.
template <bool KDA, typename AT, int BV>
__device__ __forceinline__ void load_history(const AT* ring_k, const float* ring_d,
                                             const float* ring_g, int slot, int L, int hk,
                                             int hv, int kh, int h, int dk, int dv, int col0,
                                             int nh, float* khat, float* dhist, float* hg) {
  const int tid = threadIdx.x;
  for (int i = tid; i < nh * dk; i += kThreads) {
    const int rec = i / dk, r = i - rec * dk;
    khat[i] = to_f32(ring_k[(((size_t)slot * L + rec) * hk + kh) * dk + r]);
  }
  for (int i = tid; i < nh * BV; i += kThreads) {
    const int rec = i / BV, c = i - rec * BV;
    dhist[i] = ring_d[(((size_t)slot * L + rec) * hv + h) * dv + col0 + c];
  }
  if (KDA) {
    for (int i = tid; i < nh * dk; i += kThreads) {
      const int rec = i / dk, r = i - rec * dk;
      hg[i] = ring_g[(((size_t)slot * L + rec) * hv + h) * dk + r];
    }
  } else {
    for (int i = tid; i < nh; i += kThreads) hg[i] = ring_g[((size_t)slot * L + i) * hv + h];
  }
}

// khat_i <- gamma_i (.) k_i with gamma_i = prod_{i<j<nh} alpha_j (suffix products), and
// gam = prod_{j<nh} alpha_j, per key channel.  One thread per channel (tid < dk).
template <bool KDA>
__device__ __forceinline__ void history_decays(float* khat, const float* hg, float* gam,
                                               int nh, int dk) {
  const int r = threadIdx.x;
  if (r < dk) {
    float run = 1.f;
    for (int i = nh - 1; i >= 0; --i) {
      khat[i * dk + r] *= run;
      run *= KDA ? hg[i * dk + r] : hg[i];
    }
    gam[r] = run;
  }
}

// ------------------------------------------------------------------ fold
// H = gam (.) S + sum_{i<nh} khat_i d_i^T on the LDS tile, as fp32 MFMA over the record
// index (records >= nh are selected to zero before the MFMA, never loaded from the ring).
// Wave w owns row blocks w, w+4, ...; a 16x16 accumulator holds columns (cb*16 +
// 4*(l/16) + i) of row (rb*16 + l%16), i.e. four consecutive columns of one row per lane.
// dst32 (nullable): fp32 LDS tile receiving H (rounded to OT when gdst is set, so that it
// holds what was stored).  gdst (nullable): global [dk x BV] destination, row stride gld.
template <typename ST, typename OT, int BV>
__device__ __forceinline__ void fold_tile(const ST* src, float* dst32, const float* khat,
                                          const float* dhist, const float* gam, int nh, int dk,
                                          OT* gdst, int gld) {
  constexpr int NCB = BV / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, q4 = lane >> 4;
  const int nks = (nh + 3) >> 2;
  for (int rb = wave; rb < dk / 16; rb += kWaves) {
    const int r = rb * 16 + i16;
    const float g = gam[r];
    f4 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = load4(src + Tile<ST, BV>::at(r, cb * 16 + 4 * q4)) * g;
    for (int ks = 0; ks < nks; ++ks) {
      const int rec = ks * 4 + q4;
      const bool ok = rec < nh;
      const float b = ok ? khat[rec * dk + rb * 16 + i16] : 0.f;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const float av = ok ? dhist[rec * BV + cb * 16 + i16] : 0.f;
        acc[cb] = mfma_16x16x4(av, b, acc[cb]);
      }
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int c = cb * 16 + 4 * q4;
      f4 v = acc[cb];
      if (gdst) {
        store4(gdst + (size_t)r * gld + c, v);
        v = round4<OT>(v);
      }
      if (dst32) store4(dst32 + Tile<float, BV>::at(r, c), v);
    }
  }
}

// ------------------------------------------------------------------ readout
// P[m][c] = sum_r H[r][c] xs[m][r] for m < nvec.  Thread (cc = tid % (BV/4), rg) owns
// columns 4cc..4cc+3 and row quads rg, rg + RG, ...; partial sums are reduced across the
// row groups of a wave by butterflies, then across the 4 waves through LDS.
template <typename ET, int BV, int VPP>
__device__ __forceinline__ void readout(const ET* tile, const float* xs, int xs_stride, int dk,
                                        int nvec, float* P, float* red) {
  constexpr int CC = BV / 4, RG = kThreads / CC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cc = tid % CC, rg = tid / CC;
  const int nq = dk / 4;
  for (int m0 = 0; m0 < nvec; m0 += VPP) {
    f4 acc[VPP];
#pragma unroll
    for (int m = 0; m < VPP; ++m) acc[m] = f4{0.f, 0.f, 0.f, 0.f};
    for (int rq = rg; rq < nq; rq += RG) {
      const f4 s0 = load4(tile + Tile<ET, BV>::at(4 * rq + 0, 4 * cc));
      const f4 s1 = load4(tile + Tile<ET, BV>::at(4 * rq + 1, 4 * cc));
      const f4 s2 = load4(tile + Tile<ET, BV>::at(4 * rq + 2, 4 * cc));
      const f4 s3 = load4(tile + Tile<ET, BV>::at(4 * rq + 3, 4 * cc));
#pragma unroll
      for (int m = 0; m < VPP; ++m) {
        const f4 x = load4(xs + (m0 + m) * xs_stride + 4 * rq);
        acc[m] += s0 * x[0];
        acc[m] += s1 * x[1];
        acc[m] += s2 * x[2];
        acc[m] += s3 * x[3];
      }
    }
#pragma unroll
    for (int off = CC; off < 64; off <<= 1) {
#pragma unroll
      for (int m = 0; m < VPP; ++m) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] += __shfl_xor(acc[m][j], off);
      }
    }
    if (lane < CC) {
#pragma unroll
      for (int m = 0; m < VPP; ++m) store4(red + (wave * VPP + m) * BV + 4 * cc, acc[m]);
    }
    __syncthreads();
    for (int i = tid; i < VPP * BV; i += kThreads) {
      const int m = i / BV, c = i - m * BV;
      if (m0 + m < nvec) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += red[(w * VPP + m) * BV + c];
        P[(m0 + m) * BV + c] = s;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ verify
template <bool KDA, typename AT, typename ST, int BV, int TMAX>
__global__ __launch_bounds__(kThreads) void verify_kernel(VerifyArgs a, RowWindows rw) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int VPP = (2 * TMAX < 8) ? 2 * TMAX : 8;
  const int tid = threadIdx.x;
  const int lid = xcd_remap(blockIdx.x, a.nblocks);
  const int vt = umod(lid, a.NV);
  const int h = umod(udiv(lid, a.NV), a.hv);
  const int row = udiv(lid, a.NV * a.hv);
  const int slot = a.slot_idx[row];
  if (slot < 0 || slot >= a.num_slots) return;          // null row: no reads, no writes

  const int L = a.L, dk = a.dk, dv = a.dv, hv = a.hv, hk = a.hk;
  const int kh = udiv(h, a.G), col0 = vt * BV;
  int T;
  size_t tok0;
  row_window(rw.cu_seqlens, rw.ntok, a.T, row, &T, &tok0);
  int n = a.cursor[slot];
  n = n < 0 ? 0 : (n > L ? L : n);
  const bool fold = n + T > L;                           // the window would overflow
  const int base = fold ? 0 : n;                         // write_pos
  const int nh = n;                                      // records replayed over S
  if (T == 0) {                                          // an empty ragged window
    if (a.write_pos_out && h == 0 && vt == 0 && tid == 0) a.write_pos_out[row] = base;
    return;
  }

  ST* tile_raw = reinterpret_cast<ST*>(smem + a.lay.tile_raw);
  float* tile32 = reinterpret_cast<float*>(smem + a.lay.tile32);
  float* khat = reinterpret_cast<float*>(smem + a.lay.khat);
  float* dhist = reinterpret_cast<float*>(smem + a.lay.dhist);
  float* hg = reinterpret_cast<float*>(smem + a.lay.hg);
  float* xraw = reinterpret_cast<float*>(smem + a.lay.xraw);
  float* xs = reinterpret_cast<float*>(smem + a.lay.xs);
  float* gw = reinterpret_cast<float*>(smem + a.lay.gw);
  float* bw = reinterpret_cast<float*>(smem + a.lay.bw);
  float* gam = reinterpret_cast<float*>(smem + a.lay.gam);
  float* P = reinterpret_cast<float*>(smem + a.lay.P);
  float* red = reinterpret_cast<float*>(smem + a.lay.red);
  float* Am = reinterpret_cast<float*>(smem + a.lay.Am);
  float* Qm = reinterpret_cast<float*>(smem + a.lay.Qm);
  int* flags = reinterpret_cast<int*>(smem + a.lay.flags);
  const int XS = a.lay.xs_stride;

  const AT* qg = static_cast<const AT*>(a.q);
  const AT* kg = static_cast<const AT*>(a.k);
  const AT* vg = static_cast<const AT*>(a.v);
  const AT* bg = static_cast<const AT*>(a.beta);
  const AT* gg = static_cast<const AT*>(a.gate);
  ST* state_tile = static_cast<ST*>(a.state) + (((size_t)slot * hv + h) * dk) * dv + col0;

  // 1. the state tile: HBM -> LDS, asynchronous
  issue_tile<ST, BV>(state_tile, dv, tile_raw, dk);

  // 2. window inputs and the committed history
  for (int i = tid; i < 2 * T * dk; i += kThreads) {
    const int m = i / dk, r = i - m * dk;
    const AT* src = m < T ? qg : kg;
    const int t = m < T ? m : m - T;
    xraw[m * XS + r] = to_f32(src[((tok0 + t) * hk + kh) * dk + r]);
  }
  if (KDA) {
    for (int i = tid; i < T * dk; i += kThreads) {
      const int t = i / dk, r = i - t * dk;
      gw[i] = to_f32(gg[((tok0 + t) * hv + h) * dk + r]);
    }
  } else if (tid < T) {
    gw[tid] = to_f32(gg[(tok0 + tid) * hv + h]);
  }
  if (tid < T) bw[tid] = to_f32(bg[(tok0 + tid) * hv + h]);
  if (nh > 0)
    load_history<KDA, AT, BV>(static_cast<const AT*>(a.ring_k), a.ring_d, a.ring_g, slot, L,
                              hk, hv, kh, h, dk, dv, col0, nh, khat, dhist, hg);
  __syncthreads();

  // 3. this workgroup has read every ring record it needs.  On a fused fold the window's
  // keys and gates go to rows 0..T-1, which the other workgroups of the key group may
  // still read: only the last of them to get here writes them (no spinning).
  if (fold && tid == 0) {
    const int old = __hip_atomic_fetch_add(a.group_counter + (size_t)row * hk + kh, 1,
                                           __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    flags[0] = (old == a.G * a.NV - 1);
  }

  // 4. decays: history suffix products, window prefix products, scaled window vectors
  if (nh > 0) history_decays<KDA>(khat, hg, gam, nh, dk);
  if (tid < dk) {
    float run = 1.f;
    for (int t = 0; t < T; ++t) {
      run *= KDA ? gw[t * dk + tid] : gw[t];
      xs[t * XS + tid] = run * xraw[t * XS + tid];
      xs[(T + t) * XS + tid] = run * xraw[(T + t) * XS + tid];
    }
    for (int m = 2 * T; m < a.lay.nvec_pad; ++m) xs[m * XS + tid] = 0.f;
  }
  // window pair scalars, one thread per (t, u), u <= t
  {
    const int p = kThreads - 1 - tid;
    if (p < T * T) {
      const int t = p / T, u = p - t * T;
      if (u <= t) {
        const float* qt = xraw + t * XS;
        const float* kt = xraw + (T + t) * XS;
        const float* ku = xraw + (T + u) * XS;
        float sq = 0.f, sk = 0.f;
        if (KDA) {
          for (int r = 0; r < dk; ++r) {
            float dec = 1.f;
            for (int w = u + 1; w <= t; ++w) dec *= gw[w * dk + r];
            const float kd = ku[r] * dec;
            sq = fmaf(qt[r], kd, sq);
            sk = fmaf(kt[r], kd, sk);
          }
        } else {
          float dec = 1.f;
          for (int w = u + 1; w <= t; ++w) dec *= gw[w];
          for (int r = 0; r < dk; ++r) {
            sq = fmaf(qt[r], ku[r], sq);
            sk = fmaf(kt[r], ku[r], sk);
          }
          sq *= dec;
          sk *= dec;
        }
        Qm[t * TMAX + u] = sq;
        if (u < t) Am[t * TMAX + u] = bw[t] * sk;
      }
    }
  }
  wait_vmem();
  __syncthreads();

  // 5. history replay (and, on overflow, the fold written back to S), then the readout
  if (nh > 0) {
    fold_tile<ST, ST, BV>(tile_raw, tile32, khat, dhist, gam, nh, dk, fold ? state_tile : nullptr, dv);
    __syncthreads();
    readout<float, BV, VPP>(tile32, xs, XS, dk, 2 * T, P, red);
  } else {
    readout<ST, BV, VPP>(tile_raw, xs, XS, dk, 2 * T, P, red);
  }

  // 6. per column: forward substitution over the window, outputs, ring deltas
  if (tid < BV) {
    const int c = tid, col = col0 + c;
    float d[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        const float vv = to_f32(vg[((tok0 + t) * hv + h) * dv + col]);
        float U = bw[t] * (vv - P[(T + t) * BV + c]);
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
        a.out[((tok0 + t) * hv + h) * dv + col] = o * a.scale;
        a.ring_d[(((size_t)slot * L + base + t) * hv + h) * dv + col] = d[t];
      }
    }
  }
  if (a.write_pos_out && h == 0 && vt == 0 && tid == 0) a.write_pos_out[row] = base;

  // 7. the window's keys and gates (shared by the key group / by the head's tiles)
  const bool writer = fold ? (flags[0] != 0) : (h % a.G == 0 && vt == 0);
  if (writer) {
    AT* rk = static_cast<AT*>(a.ring_k);
    for (int i = tid; i < T * dk; i += kThreads) {
      const int t = i / dk, r = i - t * dk;
      rk[(((size_t)slot * L + base + t) * hk + kh) * dk + r] = kg[((tok0 + t) * hk + kh) * dk + r];
    }
    if (KDA) {
      for (int i = tid; i < T * dk; i += kThreads) {
        const int t = i / dk, r = i - t * dk;
        a.ring_g[(((size_t)slot * L + base + t) * hv + h) * dk + r] =
            to_f32(gg[((tok0 + t) * hv + h) * dk + r]);
      }
    } else {
      for (int i = tid; i < T * a.G; i += kThreads) {
        const int t = i / a.G, hh = kh * a.G + (i - t * a.G);
        a.ring_g[((size_t)slot * L + base + t) * hv + hh] = to_f32(gg[(tok0 + t) * hv + hh]);
      }
    }
    if (fold && tid == 0)
      __hip_atomic_store(a.group_counter + (size_t)row * hk + kh, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------------ commit fold / materialize
// MATERIALIZE = false: S[s] <- fold(S[s], ring[s, 0:fold_len[s]]) in place, skipped when
// fold_len is 0.  MATERIALIZE = true: out[row] <- fold(S[s], ring[s, 0:cursor[s]]) in fp32.
template <bool KDA, typename AT, typename ST, int BV, bool MATERIALIZE>
__global__ __launch_bounds__(kThreads) void fold_kernel(FoldArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lid = xcd_remap(blockIdx.x, a.nblocks);
  const int vt = umod(lid, a.NV);
  const int h = umod(udiv(lid, a.NV), a.hv);
  const int row = udiv(lid, a.NV * a.hv);
  const int slot = a.slot_idx[row];
  if (slot < 0 || slot >= a.num_slots) return;
  const int L = a.L, dk = a.dk, dv = a.dv, hv = a.hv;
  int n = a.nrec[slot];
  n = n < 0 ? 0 : (n > L ? L : n);
  if (!MATERIALIZE && n == 0) return;
  const int kh = udiv(h, a.G), col0 = vt * BV;

  ST* tile_raw = reinterpret_cast<ST*>(smem + a.lay.tile_raw);
  float* khat = reinterpret_cast<float*>(smem + a.lay.khat);
  float* dhist = reinterpret_cast<float*>(smem + a.lay.dhist);
  float* hg = reinterpret_cast<float*>(smem + a.lay.hg);
  float* gam = reinterpret_cast<float*>(smem + a.lay.gam);

  const ST* src = static_cast<const ST*>(a.state_in) + (((size_t)slot * hv + h) * dk) * dv + col0;
  issue_tile<ST, BV>(src, dv, tile_raw, dk);
  if (n > 0)
    load_history<KDA, AT, BV>(static_cast<const AT*>(a.ring_k), a.ring_d, a.ring_g, slot, L,
                              a.hk, hv, kh, h, dk, dv, col0, n, khat, dhist, hg);
  __syncthreads();
  if (n > 0) {
    history_decays<KDA>(khat, hg, gam, n, dk);
  } else if (threadIdx.x < dk) {
    gam[threadIdx.x] = 1.f;
  }
  wait_vmem();
  __syncthreads();
  if (MATERIALIZE) {
    float* dst = static_cast<float*>(a.state_out) + (((size_t)row * hv + h) * dk) * dv + col0;
    fold_tile<ST, float, BV>(tile_raw, nullptr, khat, dhist, gam, n, dk, dst, dv);
  } else {
    ST* dst = static_cast<ST*>(a.state_out) + (((size_t)slot * hv + h) * dk) * dv + col0;
    fold_tile<ST, ST, BV>(tile_raw, nullptr, khat, dhist, gam, n, dk, dst, dv);
  }
}

// ------------------------------------------------------------------ cursor advance
__global__ __launch_bounds__(kThreads) void advance_kernel(AdvanceArgs a) {
  const int r = blockIdx.x * kThreads + threadIdx.x;
  if (r >= a.B) return;
  const int s = a.slot_idx[r];
  if (s < 0 || s >= a.num_slots) return;
  int n = a.cursor[s];
  n = n < 0 ? 0 : (n > a.L ? a.L : n);
  int T;
  size_t tok0;
  row_window(a.cu_seqlens, a.ntok, a.T, r, &T, &tok0);
  int acc = a.accept[r];
  acc = acc < 0 ? 0 : (acc > T ? T : acc);
  const int base = (n + T > a.L) ? 0 : n;
  const int m = base + acc;
  int fl = 0;
  switch (a.policy) {
    case 1: fl = m; break;                                            // every commit
    case 2: fl = (m + a.next_T > a.L) ? m : 0; break;                 // lazy
    case 3: fl = (a.force_mask == nullptr || a.force_mask[r]) ? m : 0; break;  // force
    default: fl = 0; break;
  }
  a.fold_len[s] = fl;
  a.cursor[s] = fl ? 0 : m;
}

// ------------------------------------------------------------------ launchers
template <typename K>
static void set_lds_limit(K kernel, int bytes) {
  if (bytes > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <bool KDA, typename AT, typename ST, int BV, int TMAX>
static hipError_t run_verify(const VerifyArgs& a, const RowWindows& w, hipStream_t s) {
  auto k = verify_kernel<KDA, AT, ST, BV, TMAX>;
  set_lds_limit(k, a.lay.total);
  hipLaunchKernelGGL(k, dim3(a.nblocks), dim3(kThreads), a.lay.total, s, a, w);
  return hipGetLastError();
}

template <bool KDA, typename AT, typename ST, int BV>
static hipError_t verify_tmax(int tmax, const VerifyArgs& a, const RowWindows& w, hipStream_t s) {
  switch (tmax) {
    case 1: return run_verify<KDA, AT, ST, BV, 1>(a, w, s);
    case 2: return run_verify<KDA, AT, ST, BV, 2>(a, w, s);
    case 4: return run_verify<KDA, AT, ST, BV, 4>(a, w, s);
    case 8: return run_verify<KDA, AT, ST, BV, 8>(a, w, s);
    case 16: return run_verify<KDA, AT, ST, BV, 16>(a, w, s);
  }
  return hipErrorInvalidValue;
}

template <bool KDA, typename AT, typename ST>
static hipError_t verify_bv(int bv, int tmax, const VerifyArgs& a, const RowWindows& w, hipStream_t s) {
  switch (bv) {
    case 16: return verify_tmax<KDA, AT, ST, 16>(tmax, a, w, s);
    case 32: return verify_tmax<KDA, AT, ST, 32>(tmax, a, w, s);
    case 64: return verify_tmax<KDA, AT, ST, 64>(tmax, a, w, s);
    case 128: return verify_tmax<KDA, AT, ST, 128>(tmax, a, w, s);
  }
  return hipErrorInvalidValue;
}

template <bool KDA>
static hipError_t verify_types(int act_bf16, int state_bf16, int bv, int tmax,
                               const VerifyArgs& a, const RowWindows& w, hipStream_t s) {
  if (act_bf16) {
    return state_bf16 ? verify_bv<KDA, bf16, bf16>(bv, tmax, a, w, s)
                      : verify_bv<KDA, bf16, float>(bv, tmax, a, w, s);
  }
  return state_bf16 ? verify_bv<KDA, float, bf16>(bv, tmax, a, w, s)
                    : verify_bv<KDA, float, float>(bv, tmax, a, w, s);
}

hipError_t launch_verify(bool kda, int act_bf16, int state_bf16, int bv, int tmax,
                         const VerifyArgs& a, const RowWindows& w, hipStream_t s) {
  return kda ? verify_types<true>(act_bf16, state_bf16, bv, tmax, a, w, s)
             : verify_types<false>(act_bf16, state_bf16, bv, tmax, a, w, s);
}

template <bool KDA, typename AT, typename ST, int BV, bool MAT>
static hipError_t run_fold(const FoldArgs& a, hipStream_t s) {
  auto k = fold_kernel<KDA, AT, ST, BV, MAT>;
  set_lds_limit(k, a.lay.total);
  hipLaunchKernelGGL(k, dim3(a.nblocks), dim3(kThreads), a.lay.total, s, a);
  return hipGetLastError();
}

template <bool KDA, typename AT, typename ST, bool MAT>
static hipError_t fold_bv(int bv, const FoldArgs& a, hipStream_t s) {
  switch (bv) {
    case 16: return run_fold<KDA, AT, ST, 16, MAT>(a, s);
    case 32: return run_fold<KDA, AT, ST, 32, MAT>(a, s);
    case 64: return run_fold<KDA, AT, ST, 64, MAT>(a, s);
    case 128: return run_fold<KDA, AT, ST, 128, MAT>(a, s);
  }
  return hipErrorInvalidValue;
}

template <bool KDA, bool MAT>
static hipError_t fold_types(int act_bf16, int state_bf16, int bv, const FoldArgs& a,
                             hipStream_t s) {
  if (act_bf16) {
    return state_bf16 ? fold_bv<KDA, bf16, bf16, MAT>(bv, a, s)
                      : fold_bv<KDA, bf16, float, MAT>(bv, a, s);
  }
  return state_bf16 ? fold_bv<KDA, float, bf16, MAT>(bv, a, s)
                    : fold_bv<KDA, float, float, MAT>(bv, a, s);
}

hipError_t launch_fold(bool kda, int act_bf16, int state_bf16, int bv, bool materialize,
                       const FoldArgs& a, hipStream_t s) {
  if (kda) {
    return materialize ? fold_types<true, true>(act_bf16, state_bf16, bv, a, s)
                       : fold_types<true, false>(act_bf16, state_bf16, bv, a, s);
  }
  return materialize ? fold_types<false, true>(act_bf16, state_bf16, bv, a, s)
                     : fold_types<false, false>(act_bf16, state_bf16, bv, a, s);
}

hipError_t launch_advance(const AdvanceArgs& a, hipStream_t s) {
  const int blocks = (a.B + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(advance_kernel, dim3(blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace rs
