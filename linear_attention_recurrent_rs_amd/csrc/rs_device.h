// Device helpers shared by the ReplaySSM kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rs {

constexpr int kThreads = 256;   // threads per workgroup: 4 waves of 64
constexpr int kWaves = 4;
constexpr int kXcds = 8;        // MI355X: 8 XCDs, workgroups dispatched round-robin

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint16_t bf16;

// ------------------------------------------------------------------ number formats

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return __uint_as_float(uint32_t(x) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ bf16 bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16(u >> 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return bf16_rne(x); }

// The value a state element holds once stored in type T (identity for fp32).
template <typename T> __device__ __forceinline__ float stored_value(float x) {
  return to_f32(from_f32<T>(x));
}

// Four consecutive elements as floats / from floats.
__device__ __forceinline__ f4 load4(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ f4 load4(const bf16* p) {
  uint2 u = *reinterpret_cast<const uint2*>(p);
  f4 r;
  r[0] = __uint_as_float(u.x << 16);
  r[1] = __uint_as_float(u.x & 0xffff0000u);
  r[2] = __uint_as_float(u.y << 16);
  r[3] = __uint_as_float(u.y & 0xffff0000u);
  return r;
}
__device__ __forceinline__ void store4(float* p, f4 v) { *reinterpret_cast<f4*>(p) = v; }
__device__ __forceinline__ void store4(bf16* p, f4 v) {
  uint2 u;
  u.x = uint32_t(bf16_rne(v[0])) | (uint32_t(bf16_rne(v[1])) << 16);
  u.y = uint32_t(bf16_rne(v[2])) | (uint32_t(bf16_rne(v[3])) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}
// The same, with the non-temporal hint: data streamed once, kept out of the caches' way.
__device__ __forceinline__ f4 load4_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
}
__device__ __forceinline__ f4 load4_nt(const bf16* p) {
  const u2 u = __builtin_nontemporal_load(reinterpret_cast<const u2*>(p));
  f4 r;
  r[0] = __uint_as_float(u[0] << 16);
  r[1] = __uint_as_float(u[0] & 0xffff0000u);
  r[2] = __uint_as_float(u[1] << 16);
  r[3] = __uint_as_float(u[1] & 0xffff0000u);
  return r;
}
__device__ __forceinline__ void store4_nt(float* p, f4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p));
}
__device__ __forceinline__ void store4_nt(bf16* p, f4 v) {
  u2 u;
  u[0] = uint32_t(bf16_rne(v[0])) | (uint32_t(bf16_rne(v[1])) << 16);
  u[1] = uint32_t(bf16_rne(v[2])) | (uint32_t(bf16_rne(v[3])) << 16);
  __builtin_nontemporal_store(u, reinterpret_cast<u2*>(p));
}
template <typename T> __device__ __forceinline__ f4 round4(f4 v) {
  f4 r;
  r[0] = stored_value<T>(v[0]); r[1] = stored_value<T>(v[1]);
  r[2] = stored_value<T>(v[2]); r[3] = stored_value<T>(v[3]);
  return r;
}

// ------------------------------------------------------------------ LDS state tile
// A [rows x bv] tile of element type T, stored as 16-byte chunks.  Chunk c of row r sits
// at chunk slot (c ^ (r % cpr)) of that row (cpr = chunks per row, a power of two), so
// that 16 lanes reading one chunk column of 16 consecutive rows, or 16 consecutive chunks
// of one row, hit distinct bank groups.
template <typename T, int BV>
struct Tile {
  static constexpr int kCpr = BV * int(sizeof(T)) / 16;   // chunks per row
  static constexpr int kEpc = 16 / int(sizeof(T));         // elements per chunk
  static_assert(kCpr >= 1 && (kCpr & (kCpr - 1)) == 0, "chunks per row must be 2^n");
  // element offset of (row r, column c), c % 4 == 0 (four columns never straddle chunks)
  __device__ __forceinline__ static int at(int r, int c) {
    int chunk = c / kEpc;
    return r * BV + ((chunk ^ (r & (kCpr - 1))) * kEpc) + (c % kEpc);
  }
  // global chunk held by linear LDS chunk slot p (inverse of the swizzle)
  __device__ __forceinline__ static void slot_source(int p, int& r, int& chunk) {
    r = p / kCpr;
    chunk = (p % kCpr) ^ (r & (kCpr - 1));
  }
};

// ------------------------------------------------------------------ lane sums
// v[l] + v[l ^ m] for m = 8, 16, 32 without the LDS pipe.  gfx950's permlane swaps trade
// rows (16 lanes) between two registers: with both operands v, permlane16_swap returns
// (rows 0,0,2,2 ; rows 1,1,3,3) and permlane32_swap (rows 0,1,0,1 ; rows 2,3,2,3), whose
// sums are the xor-16 and xor-32 partner sums.  Within a row, rotating by 8 reaches l ^ 8.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <int M>
__device__ __forceinline__ float xor_sum(float v) {
  const unsigned u = __float_as_uint(v);
  if constexpr (M == 8) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, int(u), 0x128, 0xF, 0xF, false));
  } else if constexpr (M == 16) {
    const u32x2 p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
  } else {
    static_assert(M == 32, "partner distance 8, 16 or 32");
    const u32x2 p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
}

// ------------------------------------------------------------------ index arithmetic
// Quotient and remainder of non-negative x by a workgroup-uniform d >= 1.  Head counts and
// tile counts are powers of two in practice: then a shift and a mask, instead of the
// general division (a reciprocal on the VALU and a correction on the SALU, about 25
// dependent instructions) that would otherwise sit in front of a workgroup's first load.
__device__ __forceinline__ int udiv(int x, int d) {
  return (d & (d - 1)) == 0 ? (x >> __builtin_ctz((unsigned)d)) : x / d;
}
__device__ __forceinline__ int umod(int x, int d) {
  return (d & (d - 1)) == 0 ? (x & (d - 1)) : x % d;
}

// ------------------------------------------------------------------ grid order
// Hardware hands workgroup p to XCD p % 8.  Return a logical index so that each XCD
// receives one contiguous range of logical indices (neighbouring value heads of one
// request, which share key heads and history keys, then share an L2).  Bijective on
// [0, n) for any n.
__device__ __forceinline__ int xcd_remap(int p, int n) {
  int xcd = p % kXcds, idx = p / kXcds;
  int per = n / kXcds, extra = n % kXcds;
  return xcd * per + (xcd < extra ? xcd : extra) + idx;
}

// Same, for work in groups of gs consecutive logical indices that share data (the tiles
// of the value heads of one key group): whole groups go round-robin over the XCDs, so a
// group shares one L2 and every XCD gets an even share of rows.  Needs n to be a multiple
// of 8 * gs (else the contiguous mapping above).  Bijective on [0, n).
__device__ __forceinline__ int xcd_group_remap(int p, int n, int gs) {
  if (umod(n, kXcds * gs) != 0) return xcd_remap(p, n);
  const int xcd = p % kXcds, q = p / kXcds;
  return (udiv(q, gs) * kXcds + xcd) * gs + umod(q, gs);
}

// ------------------------------------------------------------------ MFMA
// D(16x16) += A(16x4) B(4x16), fp32.  Lane l supplies A[l%16][l/16] and B[l/16][l%16];
// it holds D[4*(l/16)+i][l%16] in element i of the accumulator.
__device__ __forceinline__ f4 mfma_16x16x4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

typedef short s4 __attribute__((ext_vector_type(4)));
// D(16x16) += A(16x16) B(16x16), bf16 operands (products exact in fp32), fp32 accumulate.
// Lane l supplies four K entries of row l%16 of A and the same four K entries of column
// l%16 of B; it holds D[4*(l/16)+i][l%16] in element i of the accumulator.  Which four K
// entries a lane holds is immaterial as long as A and B agree.
__device__ __forceinline__ f4 mfma_bf16_16x16x16(s4 a, s4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ bf16 splits of fp32 values
// (operands of bf16 MFMAs standing in for fp32 products)
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));

// Four fp32 values (K entries 0..3 of an MFMA operand) split into bf16 parts, x = hi + lo
// + e with |e| <= 2^-16 |x|: hi keeps the upper 16 bits (truncation), lo is the exact
// remainder rounded to nearest even (one v_cvt_pk_bf16_f32 per pair).
__device__ __forceinline__ void split4(float x0, float x1, float x2, float x3, s4& hi, s4& lo) {
  const uint32_t w0 = __float_as_uint(x0), w1 = __float_as_uint(x1);
  const uint32_t w2 = __float_as_uint(x2), w3 = __float_as_uint(x3);
  hi = __builtin_bit_cast(s4, u2{(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)});
  const f2 r01 = {x0 - __uint_as_float(w0 & 0xffff0000u), x1 - __uint_as_float(w1 & 0xffff0000u)};
  const f2 r23 = {x2 - __uint_as_float(w2 & 0xffff0000u), x3 - __uint_as_float(w3 & 0xffff0000u)};
  lo = __builtin_bit_cast(s4, u2{__builtin_bit_cast(uint32_t, __builtin_convertvector(r01, b2)),
                                 __builtin_bit_cast(uint32_t, __builtin_convertvector(r23, b2))});
}

// Four fp32 values split into three bf16 parts, x = hi + mid + lo + e with
// |e| <= 2^-24 |x|: hi and mid keep the upper 16 bits of x and of the exact remainder,
// lo is the final remainder rounded to nearest even.
__device__ __forceinline__ void split4x3(const float (&x)[4], s4& hi, s4& mid, s4& lo) {
  uint32_t h[4], m[4];
  f2 r[2];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t w = __float_as_uint(x[e]);
    h[e] = w & 0xffff0000u;
    const float r1 = x[e] - __uint_as_float(h[e]);
    m[e] = __float_as_uint(r1) & 0xffff0000u;
    r[e >> 1][e & 1] = r1 - __uint_as_float(m[e]);
  }
  hi = __builtin_bit_cast(s4, u2{(h[0] >> 16) | h[1], (h[2] >> 16) | h[3]});
  mid = __builtin_bit_cast(s4, u2{(m[0] >> 16) | m[1], (m[2] >> 16) | m[3]});
  lo = __builtin_bit_cast(s4, u2{__builtin_bit_cast(uint32_t, __builtin_convertvector(r[0], b2)),
                                 __builtin_bit_cast(uint32_t, __builtin_convertvector(r[1], b2))});
}

// Direct HBM -> LDS copy of 16 bytes per lane: lane l writes lds_wave_base + 16*l.
__device__ __forceinline__ void load_lds_16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base,
                                   16, 0, 0);
}
// Same, 4 bytes per lane: lane l writes lds_wave_base + 4*l.
__device__ __forceinline__ void load_lds_4(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base,
                                   4, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory operations
// of this wave are outstanding and leaves the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS traffic that waits for this wave's LDS operations and for all
// but its last N vector-memory operations, and no more: unlike __syncthreads(), loads
// still in flight (a state tile streaming into registers) stay in flight.  Writes that
// reach LDS through HBM->LDS copies count as vector-memory operations.  The memory
// clobbers keep the compiler from moving LDS accesses across the barrier.
template <int N = 63>
__device__ __forceinline__ void lds_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Keep the compiler from moving memory operations or scheduling instructions across.
__device__ __forceinline__ void code_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Asynchronous copy of nrows rows of row_bytes (a multiple of 16) from global memory (row r
// at g + r * gstride bytes) into LDS, rows packed back to back at dst.  All threads of the
// workgroup take part; wait_vmem*() + a barrier before reading dst.
__device__ __forceinline__ void dma_rows(const void* g, size_t gstride, int row_bytes,
                                         int nrows, void* dst) {
  const int cpr = row_bytes >> 4, n = nrows * cpr;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char* gb = static_cast<const char*>(g);
  char* db = static_cast<char*>(dst);
  for (int p0 = wave * 64; p0 < n; p0 += kThreads) {
    const int p = p0 + lane;
    if (p < n) {
      const int r = p / cpr, c = p - r * cpr;
      load_lds_16(gb + (size_t)r * gstride + c * 16, db + p0 * 16);
    }
  }
}

// Asynchronous copy of nrows rows of 256 bytes (row r at g + r * gstride bytes) into LDS
// rows dst_stride bytes apart (a padded stride spreads equal columns of consecutive rows
// over different banks).  One row per wave instruction, 16 lanes of 16 bytes.
__device__ __forceinline__ void dma_rows_256(const void* g, size_t gstride, int nrows,
                                             void* dst, int dst_stride) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char* gb = static_cast<const char*>(g);
  char* db = static_cast<char*>(dst);
  for (int r = wave; r < nrows; r += kWaves)
    if (lane < 16) load_lds_16(gb + (size_t)r * gstride + lane * 16, db + r * dst_stride);
}

// Asynchronous gather of n 4-byte words (word i at g + i * gstride bytes) into LDS dst[i].
__device__ __forceinline__ void dma_words(const void* g, size_t gstride, int n, void* dst) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char* gb = static_cast<const char*>(g);
  char* db = static_cast<char*>(dst);
  for (int p0 = wave * 64; p0 < n; p0 += kThreads) {
    const int p = p0 + lane;
    if (p < n) load_lds_4(gb + (size_t)p * gstride, db + p0 * 4);
  }
}

}  // namespace rs
