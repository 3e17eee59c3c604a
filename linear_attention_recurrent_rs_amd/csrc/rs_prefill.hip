// Chunked prefill of GDN layers (dk = 128, bf16 inputs, 64-column tiles), gfx950: each
// row's prompt runs from the slot's canonical state, which is then overwritten with the
// state after the last prompt token, and the cursor is set to 0 (LightLLM page, commit
// messages: prefill writes the canonical SSM directly and leaves the cursor at zero).
//
// One workgroup per (value tile, value head, row), as the verify; the state tile stays in
// registers for the whole prompt, which it walks in chunks of C = 16 tokens.  Within a
// chunk, with G_t the prefix product of the gates, dec(u,t) = prod_{u<w<=t} alpha_w, and S
// the state before the chunk (the same WY/UT form the verify uses for its window):
//   U_t  = beta_t (v_t - G_t S^T k_t)
//   (I + A) D = U,   A[t][u] = beta_t dec(u,t) (k_t . k_u) for u < t
//   o_t  = scale (G_t S^T q_t + sum_{u<=t} dec(u,t) (q_t . k_u) D_u)
//   S   <- G_{C-1} S + sum_u dec(u, C-1) k_u D_u^T.
// Every term is a dense contraction and runs on MFMA: the readout S^T [q; k] on bf16 MFMAs
// over the state split into high and low bf16 parts (|error| <= 2^-16 per element), the
// scores q.k and k.k on bf16 MFMAs (exact products of the bf16 inputs), D = (I + A)^-1 U
// and the outputs on fp32 MFMAs, and the state update on bf16 MFMAs with the keys exact
// and the decayed D in three bf16 parts (|error| <= 2^-24).  (I + A)^-1, a 16 x 16 unit
// lower-triangular inverse, is a forward substitution on 16 lanes.  Every token of a
// prompt is real, so contracting over the chunk's token index is sound here (the verify,
// whose rejected drafts may hold anything, never does); tokens past the end of a prompt's
// last chunk are selected away, never multiplied by zero.
//
// Register layout: wave w owns columns 16 w .. 16 w + 15 of the tile over all 128 rows;
// lane l holds column 16 w + l % 16 at rows 16 m + 4 (l / 16) + i (m < 8, i < 4), which is
// the MFMA accumulator layout of the 16 x 16 block (m, w).  So the readout sums over all
// rows inside one wave (no cross-wave reduction), and the solved D, which comes out of the
// fp32 MFMAs in the same layout, is the state update's operand without leaving registers.
// The tile enters and leaves through LDS, so that HBM sees whole 256-byte row segments.
#include "rs_device.h"
#include "rs_internal.h"
#include "rs_prefill.h"

namespace rs {

namespace {

constexpr int kDK = 128, kBV = 64, kC = 16, kKS = kKeyStride;
constexpr int kStageStride = kBV + 4;            // fp32, conflict-free column reads

// LDS plan (bytes).  The staging tile aliases everything else (used only at the start and
// the end, behind barriers).
struct PrefillLds {
  static constexpr int q = 0;                                     // [2][16][KS] bf16
  static constexpr int k = q + 2 * kC * kKS * 2;                  // [2][16][KS] bf16
  static constexpr int v = k + 2 * kC * kKS * 2;                  // [2][16][64] bf16
  static constexpr int beta = v + 2 * kC * kBV * 2;               // [2][16] fp32
  static constexpr int gate = beta + 2 * kC * 4;                  // [2][16] fp32
  static constexpr int Am = gate + 2 * kC * 4;                    // [16][16] fp32
  static constexpr int Qm = Am + kC * kC * 4;                     // [16][16] fp32
  static constexpr int Ti = Qm + kC * kC * 4;                     // [16][16] fp32
  static constexpr int Gp = Ti + kC * kC * 4;                     // [16] fp32
  static constexpr int gs = Gp + kC * 4;                          // [16] fp32
  static constexpr int O = gs + kC * 4;                           // [16][64] fp32
  static constexpr int end = O + kC * kBV * 4;
  static constexpr int stage = 0;                                 // [128][68] fp32
  static constexpr int stage_end = kDK * kStageStride * 4;
  static constexpr int total = end > stage_end ? end : stage_end;
};

}  // namespace

int prefill_lds_bytes() { return PrefillLds::total; }

// Four workgroups per CU (128 VGPRs, a few spilled): a batch of 16 prompts (1024
// workgroups) then runs in one round instead of a round and a third, which measured
// 347 -> 223 us; the spills cost less than the idle second round.
template <typename ST>
__global__ __launch_bounds__(kThreads, 4) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  using L = PrefillLds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lc = lane & 15, lg = lane >> 4;
  const int lid = xcd_group_remap(blockIdx.x, a.nblocks, a.G * a.NV);
  const int vt = umod(lid, a.NV);
  const int h = umod(udiv(lid, a.NV), a.hv);
  const int row = udiv(lid, a.NV * a.hv);
  const int slot = a.slot_idx[row];
  if (slot < 0 || slot >= a.num_slots) return;          // null row: no reads, no writes
  int P;
  size_t tok0;
  row_window(a.cu_seqlens, a.ntok, a.ntok, row, &P, &tok0);
  if (P == 0) {                                          // an empty prompt: S as it is
    if (h == 0 && vt == 0 && tid == 0) a.cursor[slot] = 0;
    return;
  }
  const int hv = a.hv, hk = a.hk, dv = a.dv, kh = udiv(h, a.G), col0 = vt * kBV;
  const bf16* qg = static_cast<const bf16*>(a.q);
  const bf16* kg = static_cast<const bf16*>(a.k);
  const bf16* vg = static_cast<const bf16*>(a.v);
  const bf16* bg = static_cast<const bf16*>(a.beta);
  const bf16* gg = static_cast<const bf16*>(a.gate);
  float* stage = reinterpret_cast<float*>(smem + L::stage);

  // 1. the state tile: HBM -> LDS in whole rows (16 lanes per 256-byte row segment), then
  // into the column layout
  ST* sg = static_cast<ST*>(a.state) + (((size_t)slot * hv + h) * kDK) * dv + col0;
  {
    const int q4 = tid & 15, r0 = tid >> 4;
    f4 t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = load4_nt(sg + (uint32_t)((r0 + 16 * k) * dv + 4 * q4));
#pragma unroll
    for (int k = 0; k < 8; ++k) store4(stage + (r0 + 16 * k) * kStageStride + 4 * q4, t[k]);
  }
  lds_barrier<0>();
  f4 S[8];                                               // rows 16 m + 4 lg + i, column c
  const int c = 16 * wave + lc;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) S[m][i] = stage[(16 * m + 4 * lg + i) * kStageStride + c];
  }
  lds_barrier<0>();                                      // the staging tile is free again
  // the chunk buffers start as zeros, so that rows past a prompt's end hold finite values
  for (int i = tid; i < L::beta / 16; i += kThreads)
    reinterpret_cast<uint4*>(smem)[i] = uint4{0, 0, 0, 0};
  lds_barrier<0>();

  // chunk inputs: q and k rows of the key head, this tile's v columns -> LDS (copies);
  // betas and gates of this head -> registers of lanes 0..15 of wave 0 (2-byte values)
  auto issue = [&](int ch, int buf) {
    const int t0 = ch * kC, n = min(kC, P - t0);
    const size_t tk = tok0 + t0;
    dma_rows_256(qg + (tk * hk + kh) * kDK, (size_t)hk * kDK * 2, n,
                 smem + L::q + buf * kC * kKS * 2, kKS * 2);
    dma_rows_256(kg + (tk * hk + kh) * kDK, (size_t)hk * kDK * 2, n,
                 smem + L::k + buf * kC * kKS * 2, kKS * 2);
    dma_rows(vg + (tk * hv + h) * dv + col0, (size_t)hv * dv * 2, kBV * 2, n,
             smem + L::v + buf * kC * kBV * 2);
  };
  float nb = 0.f, ng = 1.f;                              // wave 0, lane t < 16: token t
  auto issue_scalars = [&](int ch) {
    const int t0 = ch * kC, n = min(kC, P - t0);
    if (wave == 0 && lane < kC) {
      const bool ok = lane < n;
      const size_t e = (tok0 + t0 + (ok ? lane : 0)) * hv + h;
      const float b = to_f32(bg[e]), g = to_f32(gg[e]);
      nb = ok ? b : 0.f;
      ng = ok ? g : 1.f;                                 // past the prompt: no decay
    }
  };
  issue(0, 0);
  issue_scalars(0);
  const int nch = (P + kC - 1) / kC;
  float* Am = reinterpret_cast<float*>(smem + L::Am);
  float* Qm = reinterpret_cast<float*>(smem + L::Qm);
  float* Ti = reinterpret_cast<float*>(smem + L::Ti);
  float* Gp = reinterpret_cast<float*>(smem + L::Gp);
  float* gs = reinterpret_cast<float*>(smem + L::gs);
  float* Os = reinterpret_cast<float*>(smem + L::O);

  for (int ch = 0; ch < nch; ++ch) {
    const int buf = ch & 1, t0 = ch * kC, n = min(kC, P - t0);
    const bf16* xq = reinterpret_cast<const bf16*>(smem + L::q + buf * kC * kKS * 2);
    const bf16* xk = reinterpret_cast<const bf16*>(smem + L::k + buf * kC * kKS * 2);
    const bf16* xv = reinterpret_cast<const bf16*>(smem + L::v + buf * kC * kBV * 2);
    float* xb = reinterpret_cast<float*>(smem + L::beta + buf * kC * 4);
    float* xg = reinterpret_cast<float*>(smem + L::gate + buf * kC * 4);
    // 2. this chunk's inputs have landed (every wave's copies and scalar loads; also the
    // previous chunk's output stores)
    wait_vmem();
    if (wave == 0 && lane < kC) {
      xb[lane] = nb;
      xg[lane] = ng;
    }
    lds_barrier<0>();
    if (ch + 1 < nch) {                                  // the next chunk, in flight meanwhile
      issue(ch + 1, buf ^ 1);
      issue_scalars(ch + 1);
    }

    // 3. readout R_x = S^T x for the 16 q and 16 k rows (A = x, B = S in hi/lo parts):
    // lane ends with R[token 4 lg + i][column c]
    f4 Rq = f4{0.f, 0.f, 0.f, 0.f}, Rk = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      s4 bh, bl;
      split4(S[m][0], S[m][1], S[m][2], S[m][3], bh, bl);
      const s4 aq = *reinterpret_cast<const s4*>(xq + lc * kKS + 16 * m + 4 * lg);
      const s4 ak = *reinterpret_cast<const s4*>(xk + lc * kKS + 16 * m + 4 * lg);
      Rq = mfma_bf16_16x16x16(aq, bh, Rq);
      Rq = mfma_bf16_16x16x16(aq, bl, Rq);
      Rk = mfma_bf16_16x16x16(ak, bh, Rk);
      Rk = mfma_bf16_16x16x16(ak, bl, Rk);
    }

    // 4. wave 0: A = beta_t dec(u,t) k_t.k_u (u < t); wave 1: Q = dec(u,t) q_t.k_u (u <= t);
    // wave 2: prefix products G_t and exclusive suffix products dec(u, n-1) of the gates
    if (wave <= 1) {
      f4 g = f4{0.f, 0.f, 0.f, 0.f};
      const bf16* xa = wave == 0 ? xk : xq;
#pragma unroll
      for (int s = 0; s < kDK / 16; ++s) {
        const s4 av = *reinterpret_cast<const s4*>(xa + lc * kKS + 16 * s + 4 * lg);
        const s4 bv = *reinterpret_cast<const s4*>(xk + lc * kKS + 16 * s + 4 * lg);
        g = mfma_bf16_16x16x16(av, bv, g);
      }
      // dec(u, t) for t = 4 lg .. 4 lg + 3: the first by a product over (u, 4 lg], then
      // one more gate per step (products over the causal range only, never a quotient)
      const int u = lc;
      float dec = 1.f;
      for (int w = u + 1; w <= 4 * lg; ++w) dec *= xg[w];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * lg + i;
        if (i > 0 && t > u) dec *= xg[t];
        const bool live = t < n;
        if (wave == 0) Am[t * kC + u] = (live && u < t) ? xb[t] * (g[i] * dec) : 0.f;
        else Qm[t * kC + u] = (live && u <= t) ? g[i] * dec : 0.f;
      }
    } else if (wave == 2 && lane < kC) {
      // inclusive prefix products by DPP row shifts (lane t reads lane t - k; lanes before
      // the row start get 1), then the suffix products the same way in the other direction
      float p = xg[lane];
      p *= __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(p), 0x111, 0xF, 0xF, false));
      p *= __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(p), 0x112, 0xF, 0xF, false));
      p *= __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(p), 0x114, 0xF, 0xF, false));
      p *= __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(p), 0x118, 0xF, 0xF, false));
      float q = xg[lane];                                  // inclusive suffix products
      q *= __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(q), 0x101, 0xF, 0xF, false));
      q *= __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(q), 0x102, 0xF, 0xF, false));
      q *= __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(q), 0x104, 0xF, 0xF, false));
      q *= __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(q), 0x108, 0xF, 0xF, false));
      const float ex = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(q), 0x101, 0xF, 0xF, false));
      Gp[lane] = p;
      gs[lane] = lane < n ? ex : 0.f;                      // gates past the prompt are 1
    }
    lds_barrier<63>();

    // 5. U (every wave, registers) and, on wave 0, the inverse of (I + A) by forward
    // substitution, column u on lane u: x_u = 1, x_t = -sum_{u<=w<t} A[t][w] x_w
    f4 U;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * lg + i;
      const float vt_ = to_f32(xv[t * kBV + c]);
      U[i] = t < n ? xb[t] * (vt_ - Gp[t] * Rk[i]) : 0.f;
    }
    if (wave == 0 && lane < kC) {
      float x[kC];
#pragma unroll
      for (int t = 0; t < kC; ++t) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < t; ++w) acc = fmaf(Am[t * kC + w], x[w], acc);
        x[t] = t == lane ? 1.f : (t < lane ? 0.f : -acc);
      }
#pragma unroll
      for (int t = 0; t < kC; ++t) Ti[t * kC + lane] = x[t];
    }
    lds_barrier<63>();

    // 6. D = (I + A)^-1 U and O = G (.) R_q + Q D on fp32 MFMAs; K entry 4 lg + i of this
    // lane is its own register i (U, then D), the A operand row lc from LDS
    f4 D = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) D = mfma_16x16x4(Ti[lc * kC + 4 * lg + i], U[i], D);
    f4 O;
#pragma unroll
    for (int i = 0; i < 4; ++i) O[i] = Gp[4 * lg + i] * Rq[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) O = mfma_16x16x4(Qm[lc * kC + 4 * lg + i], D[i], O);
#pragma unroll
    for (int i = 0; i < 4; ++i) Os[(4 * lg + i) * kBV + c] = O[i] * a.scale;

    // 7. S <- G_{n-1} S + sum_u dec(u, n-1) k_u D_u^T: A = the keys of the block's 16 rows
    // (tokens past the prompt selected to zero), B = the decayed D in three bf16 parts
    {
      float dw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) dw[e] = gs[4 * lg + e] * D[e];
      s4 bh, bm, bl;
      split4x3(dw, bh, bm, bl);
      const float Gl = Gp[n - 1];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        s4 ka;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * lg + e;
          ka[e] = t < n ? short(xk[t * kKS + 16 * m + lc]) : short(0);
        }
        f4 acc = S[m] * Gl;
        acc = mfma_bf16_16x16x16(ka, bh, acc);
        acc = mfma_bf16_16x16x16(ka, bm, acc);
        acc = mfma_bf16_16x16x16(ka, bl, acc);
        S[m] = acc;
      }
    }
    lds_barrier<63>();                                   // every wave's outputs are in LDS
    // 8. the chunk's outputs, whole 256-byte rows per 16 lanes
    {
      const int t = tid >> 4, q4 = tid & 15;
      if (t < n)
        store4(a.out + ((tok0 + t0 + t) * hv + h) * dv + col0 + 4 * q4,
               *reinterpret_cast<const f4*>(Os + t * kBV + 4 * q4));
    }
  }

  // 9. the final state: registers -> LDS -> whole rows to HBM (bf16: rounded once), and
  // the cursor to 0
  lds_barrier<0>();                                      // every wave is past its last LDS read
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) stage[(16 * m + 4 * lg + i) * kStageStride + c] = S[m][i];
  }
  lds_barrier<63>();
  {
    const int q4 = tid & 15, r0 = tid >> 4;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      store4_nt(sg + (uint32_t)((r0 + 16 * k) * dv + 4 * q4),
                load4(stage + (r0 + 16 * k) * kStageStride + 4 * q4));
  }
  if (h == 0 && vt == 0 && tid == 0) a.cursor[slot] = 0;
}

hipError_t launch_prefill(bool state_bf16, const PrefillArgs& a, hipStream_t s) {
  auto k = state_bf16 ? prefill_kernel<bf16> : prefill_kernel<float>;
  const int lds = prefill_lds_bytes();
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  hipLaunchKernelGGL(k, dim3(a.nblocks), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace rs
