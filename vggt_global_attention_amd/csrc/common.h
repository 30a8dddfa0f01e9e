// Device-side building blocks shared by the gfx950 kernels of libvggtattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vggt {

typedef _Float16 f16;
typedef __bf16 bf16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSpecial = 17;   // 1 camera + 16 register tokens per frame
constexpr int kDh = 64;        // head width supported by the kernels
constexpr int kXcds = 8;       // MI355X: 8 accelerator complex dies, one L2 each

// Workspace row -> X row map.  With v = w - base (no row if v < 0), rows are
// grouped: group g = v / grp_stride, slot t = v % grp_stride; the row is a
// real token iff t < grp_valid and g < ngroups, and then reads X row
// g * src_stride + t.
//   global:   one group of N rows           (grp_stride = rows, src_stride = 0)
//   frame:    S groups of T rows, padded to a multiple of 64
//   register: S groups of the 17 special rows, packed
//   a window of global rows [base, base + n) -> output rows 0..n-1
struct RowMap {
  int64_t grp_stride;
  int64_t src_stride;
  int32_t grp_valid;
  int32_t ngroups;
  int64_t base;
  __device__ __forceinline__ int64_t src(int64_t w) const {
    const int64_t v = w - base;
    if (v < 0) return -1;
    int64_t g = v / grp_stride;
    int64_t t = v - g * grp_stride;
    return (t < grp_valid && g < ngroups) ? g * src_stride + t : -1;
  }
};

// Scalars the kernels exchange through the workspace (all written by the
// prep stage before they are read).
struct Scalars {
  float xnorm;     // max L2 norm over the X rows of the set(s)
  float wvnorm;    // max L2 norm over the V rows of Wqkv
  float woabs;     // max |Wo|
  float pad;
  float kmax[1];   // [H] max L2 norm of the normalised, rotated fp16 keys per head
};

// Blocks are handed to the 8 XCDs round-robin; remap so that each XCD works
// through one contiguous range of logical block ids (shared operands then
// stay in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  int xcd = b & (kXcds - 1);
  int slot = b >> 3;
  int per = nblocks >> 3;
  int rem = nblocks & (kXcds - 1);
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Power-of-two exponent e such that bound * 2^e <= 2^14 (clamped); 0 if the
// bound is zero or not finite.
__device__ __forceinline__ int range_exponent(float bound) {
  if (!(bound > 0.f) || !(bound < 3.0e38f)) return 0;
  int e = (int)floorf(14.f - log2f(bound));
  return e < -60 ? -60 : (e > 60 ? 60 : e);
}

// Max-reduce across the four 16-lane groups that hold one MFMA column.
__device__ __forceinline__ float max_across_groups(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float sum_across_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ void atomic_max_nonneg(float* p, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(p), __float_as_uint(v));
}

}  // namespace vggt
