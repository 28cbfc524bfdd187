// Device-side helpers shared by the gfx950 kernels: element types, bf16
// packing, cross-lane moves (DPP and permlane swaps of CDNA4) and exp2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Storage element tags.
struct F32 {
  static constexpr int kBytes = 4;
};
struct BF16 {
  static constexpr int kBytes = 2;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}

// Two fp32 -> packed bf16x2 (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Two fp32 -> packed bf16x2 with the hardware converter (round to nearest even).
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// fp32 += a.bf16x2 . b.bf16x2 (two products summed into an fp32 accumulator).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Element i of read-only data that no kernel writes while it runs (block
// tables), read through the constant address space: with a wave-uniform index
// it becomes a scalar load, whose wait (lgkmcnt) leaves the vector loads in
// flight alone, even in kernels that store to global memory before it.
__device__ __forceinline__ int32_t load_ro_i32(const int32_t* p, long long i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// log2 of sum_j 2^(s_j) for a softmax state with running max m (log2 units)
// and sum l = sum_j 2^(s_j - m); -inf for an empty state.
__device__ __forceinline__ float state_lse2(float m, float l) {
  return l > 0.f ? m + fast_log2(l) : -__builtin_inff();
}

// ---- cross-lane moves -------------------------------------------------------
// DPP controls (gfx9 encoding).
enum : int {
  kDppQuadXor1 = 0xB1,      // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,      // quad_perm [2,3,0,1]
  kDppRowRor8 = 0x128,      // row_ror:8  == lane ^ 8 inside a 16-lane row
  kDppRowMirror = 0x140,    // lane i <-> 15 - i inside a row
  kDppRowHalfMirror = 0x141 // lane i <-> 7 - i inside each half row
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}

// permlane32_swap: lanes 0..31 of the result pair hold (x_own, x_of_lane+32);
// lanes 32..63 hold (y_of_lane-32, y_own).  So r.x + r.y is, in the low half,
// x summed over the lane pair and, in the high half, y summed over it.
__device__ __forceinline__ float swap_add32(float x, float y) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Same between even and odd 16-lane rows (lanes l and l ^ 16).
__device__ __forceinline__ float swap_add16(float x, float y) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float shfl_xor32(float x) {
  // value of lane ^ 32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

// value of lane ^ 16
__device__ __forceinline__ float shfl_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (threadIdx.x & 16) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppRowMirror>(x));
  x = fmaxf(x, shfl_xor16(x));
  return fmaxf(x, shfl_xor32(x));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  x += shfl_xor16(x);
  return x + shfl_xor32(x);
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Streaming read (non-temporal hint): each K/V byte is read once per call.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

}  // namespace pa
