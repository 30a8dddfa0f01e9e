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
// prep stage before they are read).  The workspace starts with them, so the
// status word sits at byte VGGT_ATTN_STATUS_OFFSET of every workspace.  A
// descriptor cache starts with the same header.
struct Scalars {
  float xnorm;      // max L2 norm over the X rows of the set(s); +inf if one is not finite
  float wvnorm;     // max L2 norm over the V rows of Wqkv; +inf if one is not finite
  float woabs;      // max |Wo|; +inf if an entry is not finite
  float pad;        // descriptor cache: exponent of the stored values (int bits)
  uint32_t status;  // VGGT_ATTN_RANGE_* bits the prep stage found (0: all in range)
  float kmax[1];    // [H] max L2 norm of the normalised, rotated fp16 keys per head
};
inline constexpr size_t scalars_bytes(int H) { return sizeof(float) * (5 + (size_t)H); }

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

// Exact floor(n / d) for 0 <= n < 2^31 and 1 <= d < 2^31 by one multiply:
// m = ceil(2^k / d) with k = 31 + l, l = ceil(log2 d).  The excess e = m d - 2^k
// is below d, so n m / 2^k = n / d + n e / (d 2^k) with n e / (d 2^k) < 2^-l <= 1/d,
// which never reaches the next multiple of 1/d (division by invariant integers
// using multiplication, after Granlund and Montgomery).  m <= 2^32 and
// n m < 2^64.
struct FastDiv {
  uint64_t m;
  int k;
  int d;
};

inline FastDiv fast_div(int64_t d) {
  if (d < 1) d = 1;
  if (d > 0x7fffffff) d = 0x7fffffff;  // every numerator is below d then: quotient 0
  int l = 0;
  while (((int64_t)1 << l) < d) ++l;
  const int k = 31 + l;
  return FastDiv{(((uint64_t)1 << k) + (uint64_t)d - 1) / (uint64_t)d, k, (int)d};
}

__host__ __device__ __forceinline__ int fdiv(int n, const FastDiv& f) {
  return (int)(((uint64_t)(uint32_t)n * f.m) >> f.k);
}

__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v + (v of lane l ^ 32), the same bits on both lanes (fp32 addition is
// commutative), through gfx950's v_permlane32_swap (a VALU op, no LDS).
__device__ __forceinline__ float add_xor32(float v) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// c + a.x b.x + a.y b.y in fp32 (v_dot2 of two 16-bit pairs)
__device__ __forceinline__ float dot2_acc(f16x2 a, f16x2 b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}
__device__ __forceinline__ float dot2_acc(bf16x2 a, bf16x2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// 16-bit operand types of the attention core and the output projection:
// fp16 (the default path) or bf16 (the bf16-operand variant).
template <bool B16>
struct Ops16 {
  typedef f16 T;
  typedef f16x2 T2;
  typedef f16x4 T4;
  typedef f16x8 T8;
};
template <>
struct Ops16<true> {
  typedef bf16 T;
  typedef bf16x2 T2;
  typedef bf16x4 T4;
  typedef bf16x8 T8;
};

__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Power-of-two exponent e such that bound * 2^e <= 2^14 (clamped to
// [-60, 60], so that the output projection's 2^-(e + s) stays a normal fp32
// number); 0 if the bound is zero or not finite.
__device__ __forceinline__ int range_exponent(float bound) {
  if (!(bound > 0.f) || !(bound < 3.0e38f)) return 0;
  int e = (int)floorf(14.f - log2f(bound));
  return e < -60 ? -60 : (e > 60 ? 60 : e);
}

// True when range_exponent cannot do its job for `bound`: the bound is not
// finite (or beyond 3e38), or the exponent it needs lies outside [-60, 60].
// A zero bound (all values zero) is in range.
__device__ __forceinline__ bool range_exponent_clamped(float bound) {
  if (bound == 0.f) return false;
  if (!(bound > 0.f) || !(bound < 3.0e38f)) return true;
  const float e = floorf(14.f - log2f(bound));
  return e < -60.f || e > 60.f;
}

// x if finite and non-negative-ordered into a running maximum, else +inf
// (fmaxf would drop a NaN): the bounds of the prep stage carry a non-finite
// input forward as +inf, which the status check then reports.
__device__ __forceinline__ float max_or_inf(float best, float x) {
  return x < INFINITY ? fmaxf(best, x) : INFINITY;
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
