// Device-side helpers for the gfx950 kernels: vector types, MFMA wrappers,
// conversions, wave/workgroup reductions, batch descriptor lookups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp2 {

// Bounds-checking builds (FP2_DEBUG_BOUNDS): each call that reads page ids or
// a CSR first runs a check kernel that sets bits of an error word (1: a page
// id outside [0, num_pages); 2: a CSR entry outside its row's blocks or out of
// order; 4: CSR row pointers out of order or past the causal count), and every
// kernel that reads them returns at once while the word is set, so that a bad
// input is reported instead of read past.  Release builds pass a null word and
// the guard compiles to nothing.
#ifdef FP2_DEBUG_BOUNDS
#define FP2_BOUNDS_GUARD(word) \
  do {                                                                                    \
    if ((word) != nullptr && *reinterpret_cast<const volatile uint32_t*>(word) != 0u) return; \
  } while (0)
#else
#define FP2_BOUNDS_GUARD(word) ((void)(word))
#endif


typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// MFMA: D(32x32 f32) += A(32xK) * B(Kx32).
// Operand layout (wave64): lane l supplies row (l%32) of A and column (l%32)
// of B, over K-slice [k0 + (l/32)*K/2, k0 + (l/32+1)*K/2).  Result: lane l
// holds column l%32, rows 8*(i/4) + 4*(l/32) + (i%4) for i = 0..15.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16: lane l holds A row l%16 and B column l%16 at k = 8(l/16)
// .. 8(l/16)+7, and D rows 4(l/16) .. 4(l/16)+3 of column l%16
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f16_32x32x16(half8 a, half8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// OCP e4m3 x e4m3, K = 64 (format code 0 = fp8 e4m3 for both operands;
// E8M0 scale 127 = 1.0, i.e. unscaled).
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------------------
// Conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;  // v_cvt_pk_bf16_f32: round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// two floats -> packed fp16 (round toward zero; exact for values that fp16 holds)
__device__ __forceinline__ uint32_t pack_f16x2_rtz(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 4 OCP e4m3 bytes -> 4 floats (hardware conversion; gfx950 uses the OCP format)
__device__ __forceinline__ f32x4 e4m3x4_to_f32(uint32_t w) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  return f32x4{lo[0], lo[1], hi[0], hi[1]};
}

// ---------------------------------------------------------------------------
// Reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Combine the values of lanes l and l^32 (the two halves of a score column).
// v_permlane32_swap returns {v[l % 32], v[l % 32 + 32]} in either order, so a
// symmetric combine of the pair is the same for both halves (checked on gfx950).
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// lane l <-> lane l^32 (cross-lane crossbar; used where only the partner's value is wanted)
__device__ __forceinline__ float swap_halves(float v) { return __shfl_xor(v, 32, 64); }

// Tree reductions over N register values (N a power of two): depth log2(N)
// instead of a serial chain.
template <int N>
__device__ __forceinline__ float tree_max(const float* x) {
  if constexpr (N == 1) return x[0];
  else return fmaxf(tree_max<N / 2>(x), tree_max<N / 2>(x + N / 2));
}
template <int N>
__device__ __forceinline__ float tree_sum(const float* x) {
  if constexpr (N == 1) return x[0];
  else return tree_sum<N / 2>(x) + tree_sum<N / 2>(x + N / 2);
}

// ---------------------------------------------------------------------------
// Token position -> (page index within the sequence, slot) for any page size,
// without an integer division: a shift for powers of two, else a float
// reciprocal estimate corrected by one step (exact for pos < 2^22; the host
// caps sequences at 2^21 tokens).
// ---------------------------------------------------------------------------
struct PageMap {
  int ps;      // page size
  int shift;   // log2(ps) when ps is a power of two, else -1
  float inv;   // 1.0f / ps

  static PageMap make(int page_size) {
    PageMap m;
    m.ps = page_size;
    m.shift = -1;
    for (int s = 0; s < 31; ++s)
      if ((1 << s) == page_size) m.shift = s;
    m.inv = 1.0f / (float)page_size;
    return m;
  }
  __device__ __forceinline__ void split(int pos, int& page, int& slot) const {
    if (shift >= 0) {
      page = pos >> shift;
      slot = pos & (ps - 1);
      return;
    }
    int q = (int)((float)pos * inv);
    int r = pos - q * ps;
    if (r < 0) { --q; r += ps; }
    else if (r >= ps) { ++q; r -= ps; }
    page = q;
    slot = r;
  }
};

// Load of a value that is uniform across the wave and read-only for the whole
// kernel, through the scalar memory path (constant address space): it does
// not share the vector-memory counter with in-flight vector loads.
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)(p))[i];
}

// ---------------------------------------------------------------------------
// Batch descriptors: index of the sequence owning global block `gb`, given
// the prefix-sum array cu[0..n] (cu[s] <= gb < cu[s+1]).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int n, int gb) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= gb) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace fp2
