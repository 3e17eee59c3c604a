// Short causal convolution before the recurrence, with a per-slot window state, and the
// rollback of that window at commit (gfx950).
//
// The LightLLM page ("feat: add ReplaySSM state modes for GDN and KDA") keeps a conv state
// beside the canonical SSM (PR description: Conv/SSM state management, MTP accept and
// rollback; commit messages: page save and PD/DP copy "the accepted conv window", a
// restored slot receives the canonical conv and SSM state); the sglang GDN ReplaySSM spec
// verify PR rolls the conv back in the GDN ring commit (commit 4).  The convolution itself
// is not on the pages; this is the depthwise causal form a GDN layer applies to its mixed
// q/k/v channels:
//   y_t[c] = act( sum_{j<K} w[c][j] x_{t-K+1+j}[c] + b[c] ),   tap K-1 on the current input,
// with the slot's state holding its last K-1 committed inputs, oldest first.  The verify
// reads the state and writes the window's outputs; the commit moves the state to the K-1
// inputs ending at the last accepted draft.
//
// Both kernels are streaming: one thread owns 16 bytes of channels of one request row (8
// bf16 or 4 fp32 channels), so a wave reads 1 KB of contiguous channels per window row.
// The verify loads every window row up front (the window bound is a compile-time power of
// two), then slides the K taps over state ++ window in registers, accumulating in fp32.
#include "rs_device.h"
#include "rs_conv.h"
#include "rs_internal.h"

namespace rs {

namespace {

// 16 bytes of channels as loaded (4 fp32 or 8 bf16 channels), unpacked at use.
template <typename T> struct Chunk;
template <> struct Chunk<float> {
  static constexpr int N = 4;
  __device__ static float get(const uint4& r, int i) {
    return __uint_as_float(i == 0 ? r.x : i == 1 ? r.y : i == 2 ? r.z : r.w);
  }
};
template <> struct Chunk<bf16> {
  static constexpr int N = 8;
  __device__ static float get(const uint4& r, int i) {
    const uint32_t w = (i >> 1) == 0 ? r.x : (i >> 1) == 1 ? r.y : (i >> 1) == 2 ? r.z : r.w;
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// x * sigmoid(x) = x / (1 + e^-x) on the hardware exp2 and reciprocal (each within about
// an ulp): e^-x = 2^(-x log2 e); x -> -inf gives x * 0 = -0, x -> +inf gives x.
__device__ __forceinline__ float silu(float x) {
  const float e = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.f + e);
}

// N fp32 values to 16 or 32 bytes of the output dtype (bf16: round to nearest even).
template <int N>
__device__ __forceinline__ void store_out(void* p, bool out_bf16, const float (&v)[N]) {
  if (out_bf16) {
    uint32_t w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i)
      w[i] = uint32_t(bf16_rne(v[2 * i])) | (uint32_t(bf16_rne(v[2 * i + 1])) << 16);
    if constexpr (N == 8) {
      *reinterpret_cast<uint4*>(p) = uint4{w[0], w[1], w[2], w[3]};
    } else {
      *reinterpret_cast<uint2*>(p) = uint2{w[0], w[1]};
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<f4*>(static_cast<float*>(p) + i) = f4{v[i], v[i + 1], v[i + 2], v[i + 3]};
  }
}

}  // namespace

template <typename AT, int K, int TMAX>
__global__ __launch_bounds__(kThreads) void conv_verify_kernel(ConvArgs a, RowWindows rw) {
  using CH = Chunk<AT>;
  constexpr int N = CH::N;
  const int groups = a.C / N;
  const long gid = (long)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= (long)a.B * groups) return;
  const int row = (int)(gid / groups), c0 = (int)(gid % groups) * N;
  const int slot = a.slot_idx[row];
  if (slot < 0 || slot >= a.num_slots) return;          // null row: no reads, no writes
  int T;
  size_t tok0;
  row_window(rw.cu_seqlens, rw.ntok, a.T, row, &T, &tok0);
  if (T == 0) return;
  const AT* x = static_cast<const AT*>(a.x);
  const AT* wt = static_cast<const AT*>(a.weight);
  const AT* st = static_cast<const AT*>(a.state) + (size_t)slot * (K - 1) * a.C;
  // every load first: the window rows, the state rows, the taps and the bias
  uint4 xr[TMAX], sr[K - 1];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) xr[t] = t < T ? load16(x + (tok0 + t) * a.C + c0) : uint4{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < K - 1; ++j) sr[j] = load16(st + (size_t)j * a.C + c0);
  float w[N][K], b[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
#pragma unroll
    for (int j = 0; j < K; ++j) w[i][j] = to_f32(wt[(size_t)(c0 + i) * K + j]);
  }
  const uint4 br = a.bias ? load16(static_cast<const AT*>(a.bias) + c0) : uint4{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < N; ++i) b[i] = CH::get(br, i);
  // slide the taps: win holds the K-1 inputs before token t, oldest first
  float win[K - 1][N];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
#pragma unroll
    for (int i = 0; i < N; ++i) win[j][i] = CH::get(sr[j], i);
  }
  char* yb = static_cast<char*>(a.y);
  const int ob = a.out_bf16 ? 2 : 4;
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t < T) {
      float y[N], cur[N];
#pragma unroll
      for (int i = 0; i < N; ++i) {
        cur[i] = CH::get(xr[t], i);
        float acc = b[i];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) acc = fmaf(w[i][j], win[j][i], acc);
        acc = fmaf(w[i][K - 1], cur[i], acc);
        y[i] = a.silu ? silu(acc) : acc;
      }
      store_out<N>(yb + ((tok0 + t) * a.C + c0) * ob, a.out_bf16, y);
#pragma unroll
      for (int i = 0; i < N; ++i) {
#pragma unroll
        for (int j = 0; j + 1 < K - 1; ++j) win[j][i] = win[j + 1][i];
        win[K - 2][i] = cur[i];
      }
    }
  }
}

// The commit: state <- inputs [a, a + K - 1) of state ++ window, for live rows with a > 0.
// Every value is read before the first write (the state is updated in place).
// Layer l (blockIdx.y) of a layer-major stack: its states and window inputs sit
// state_layer_stride and x_layer_stride elements after layer l - 1's.
template <typename AT, int K>
__global__ __launch_bounds__(kThreads) void conv_commit_kernel(ConvArgs a, RowWindows rw) {
  constexpr int N = 16 / int(sizeof(AT));
  const int groups = a.C / N;
  const long gid = (long)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= (long)a.B * groups) return;
  const int row = (int)(gid / groups), c0 = (int)(gid % groups) * N;
  const int slot = a.slot_idx[row];
  if (slot < 0 || slot >= a.num_slots) return;
  int T;
  size_t tok0;
  row_window(rw.cu_seqlens, rw.ntok, a.T, row, &T, &tok0);
  int acc = a.accept[row];
  acc = acc < 0 ? 0 : (acc > T ? T : acc);
  if (acc == 0) return;
  const size_t layer = blockIdx.y;
  AT* st = static_cast<AT*>(a.state_rw) + layer * a.state_layer_stride +
           (size_t)slot * (K - 1) * a.C + c0;
  const AT* x = static_cast<const AT*>(a.x) + layer * a.x_layer_stride + tok0 * a.C + c0;
  uint4 keep[K - 1];
#pragma unroll
  for (int i = 0; i < K - 1; ++i) {
    const int j = acc + i;                               // index into state ++ window
    const AT* src = j < K - 1 ? st + (size_t)j * a.C : x + (size_t)(j - (K - 1)) * a.C;
    keep[i] = *reinterpret_cast<const uint4*>(src);
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < K - 1; ++i) *reinterpret_cast<uint4*>(st + (size_t)i * a.C) = keep[i];
}

template <typename AT, int K>
static hipError_t conv_verify_t(int tmax, const ConvArgs& a, const RowWindows& w, hipStream_t s) {
  constexpr int N = 16 / int(sizeof(AT));
  const long threads = (long)a.B * (a.C / N);
  const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
  switch (tmax) {
    case 1: hipLaunchKernelGGL((conv_verify_kernel<AT, K, 1>), grid, dim3(kThreads), 0, s, a, w); break;
    case 2: hipLaunchKernelGGL((conv_verify_kernel<AT, K, 2>), grid, dim3(kThreads), 0, s, a, w); break;
    case 4: hipLaunchKernelGGL((conv_verify_kernel<AT, K, 4>), grid, dim3(kThreads), 0, s, a, w); break;
    case 8: hipLaunchKernelGGL((conv_verify_kernel<AT, K, 8>), grid, dim3(kThreads), 0, s, a, w); break;
    case 16: hipLaunchKernelGGL((conv_verify_kernel<AT, K, 16>), grid, dim3(kThreads), 0, s, a, w); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename AT>
static hipError_t conv_verify_k(int width, int tmax, const ConvArgs& a, const RowWindows& w,
                                hipStream_t s) {
  switch (width) {
    case 2: return conv_verify_t<AT, 2>(tmax, a, w, s);
    case 3: return conv_verify_t<AT, 3>(tmax, a, w, s);
    case 4: return conv_verify_t<AT, 4>(tmax, a, w, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv_verify(bool act_bf16, int width, int tmax, const ConvArgs& a,
                              const RowWindows& w, hipStream_t s) {
  return act_bf16 ? conv_verify_k<bf16>(width, tmax, a, w, s)
                  : conv_verify_k<float>(width, tmax, a, w, s);
}

template <typename AT>
static hipError_t conv_commit_k(int width, const ConvArgs& a, const RowWindows& w,
                                hipStream_t s) {
  constexpr int N = 16 / int(sizeof(AT));
  const long threads = (long)a.B * (a.C / N);
  const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads), (unsigned)a.layers);
  switch (width) {
    case 2: hipLaunchKernelGGL((conv_commit_kernel<AT, 2>), grid, dim3(kThreads), 0, s, a, w); break;
    case 3: hipLaunchKernelGGL((conv_commit_kernel<AT, 3>), grid, dim3(kThreads), 0, s, a, w); break;
    case 4: hipLaunchKernelGGL((conv_commit_kernel<AT, 4>), grid, dim3(kThreads), 0, s, a, w); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_conv_commit(bool act_bf16, int width, const ConvArgs& a, const RowWindows& w,
                              hipStream_t s) {
  return act_bf16 ? conv_commit_k<bf16>(width, a, w, s) : conv_commit_k<float>(width, a, w, s);
}

}  // namespace rs
