// Descriptor key / value cache ("FlashVGGT: Efficient and Scalable Visual
// Geometry Transformers with Compressed Descriptor Attention", chatpaper.ai,
// abstract): every image token attends to a compact set of descriptor
// tokens, and chunked inference keeps the descriptors of earlier chunks.
//
// The cache holds the descriptors' keys (LayerNorm-ed, fp16, [H][cap][64]) and
// values (fp16, [H][64][cap], keys permuted inside aligned groups of 16), the
// layouts the attention kernel streams, behind a Scalars header.  The values
// carry one power-of-two scale 2^e for the whole cache, the same range guard
// as the blocks' values: e = range_exponent(max descriptor norm * max norm of
// the V rows of Wqkv), kept in the header's `pad` word.  Norm bounds only
// grow, so e only falls; an append that lowers it first multiplies the stored
// values by 2^(e_new - e_old) -- exact, a power of two -- and then writes the
// new ones at the new scale.  Every kernel reads the bounds from the header on
// the device: no host synchronisation anywhere.
#include "plan.h"

namespace vggt {

__device__ __forceinline__ int exp_bits_to_int(float f) { return __builtin_bit_cast(int, f); }
__device__ __forceinline__ float int_to_exp_bits(int e) { return __builtin_bit_cast(float, e); }

// Zero the whole cache; the header's exponent word gets the empty marker.
__global__ __launch_bounds__(256) void desc_init_kernel(u32x4* cache, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x) {
    u32x4 v = {0u, 0u, 0u, 0u};
    // header word 3 is Scalars::pad
    if (i == 0) v[3] = (uint32_t)kDescEmpty;
    cache[i] = v;
  }
}

// Rescale the stored values [H][64][0, nslots) when the exponent falls.  The
// exponent words are only read here; desc_commit_kernel writes them after.
__global__ __launch_bounds__(256) void desc_rescale_kernel(const Scalars* hdr, f16* vt,
                                                           int64_t cap_rows, int64_t nslots,
                                                           int nrows) {
  const int e_old = exp_bits_to_int(hdr->pad);
  const int e_new = range_exponent(hdr->xnorm * hdr->wvnorm);
  if (e_new >= e_old) return;
  const float f = ldexpf(1.f, e_new - e_old);
  const int64_t per_row = nslots / 8;
  const int64_t total = per_row * nrows;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per_row, c = (i - r * per_row) * 8;
    f16x8* p = reinterpret_cast<f16x8*>(vt + r * cap_rows + c);
    f16x8 v = *p;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (f16)((float)v[e] * f);
    *p = v;
  }
}

__global__ void desc_commit_kernel(Scalars* hdr) {
  if (threadIdx.x == 0) hdr->pad = int_to_exp_bits(range_exponent(hdr->xnorm * hdr->wvnorm));
}

// Copy the cache's bounds into a call's scalars: the value bound (so the
// output projection undoes the cache's scale) and the per-head key norms (the
// attention kernel's softmax bound); a non-finite descriptor (its norm is
// +inf) or a value bound out of the scale's reach adds its range bits.
__global__ void desc_load_kernel(const Scalars* hdr, Scalars* sc, int H) {
  const int t = threadIdx.x;
  if (t == 0) {
    const float xm = hdr->xnorm, vm = hdr->wvnorm;
    sc->xnorm = xm;
    sc->wvnorm = vm;
    uint32_t bits = 0;
    if (!(xm < INFINITY)) bits |= VGGT_ATTN_RANGE_X;
    if (!(vm < INFINITY)) bits |= VGGT_ATTN_RANGE_WQKV;
    if (!bits && (range_exponent_clamped(xm * vm) ||
                  (double)xm * vm * sc->woabs * (H * kDh) >= 3.0e38))
      bits |= VGGT_ATTN_RANGE_SCALE;
    sc->status |= bits;
  }
  for (int h = t; h < H; h += blockDim.x) sc->kmax[h] = hdr->kmax[h];
}

static int grid_cap(int64_t work, int per_block, int cap) {
  int64_t b = (work + per_block - 1) / per_block;
  if (b < 1) b = 1;
  return (int)(b < cap ? b : cap);
}

hipError_t launch_desc_init(char* cache, const DescLayout& L, int H, hipStream_t st) {
  (void)H;
  const int64_t n16 = (int64_t)(L.total / 16);
  hipLaunchKernelGGL(desc_init_kernel, dim3(grid_cap(n16, 256, 4096)), dim3(256), 0, st,
                     reinterpret_cast<u32x4*>(cache), n16);
  return hipGetLastError();
}

hipError_t launch_desc_append(char* cache, const DescLayout& L, int H, int d, float eps,
                              int64_t count, const bf16* D, int64_t m, const bf16* Wqkv,
                              const float* kg, const float* kb, hipStream_t st) {
  Scalars* hdr = reinterpret_cast<Scalars*>(cache);
  // 1. bounds: max norm of the new descriptor rows and of the V rows of Wqkv
  hipError_t e = launch_rownorm_max(D, m, d, RowMap{INT64_MAX / 2, 0, (int32_t)m, 1, 0},
                                    &hdr->xnorm, st);
  if (e != hipSuccess) return e;
  e = launch_rownorm_max(Wqkv + (int64_t)2 * d * d, d, d, RowMap{INT64_MAX / 2, 0, d, 1, 0},
                         &hdr->wvnorm, st);
  if (e != hipSuccess) return e;
  // 2. values already stored move to the new scale (whole groups of 16 slots:
  //    a key below `count` may sit in a slot at or above it)
  if (count > 0) {
    const int64_t nslots = (count + 15) / 16 * 16;
    const int nrows = H * kDh;
    hipLaunchKernelGGL(desc_rescale_kernel, dim3(grid_cap(nslots / 8 * nrows, 256, 4096)),
                       dim3(256), 0, st, (const Scalars*)hdr,
                       reinterpret_cast<f16*>(cache + L.off_v), L.cap_rows, nslots, nrows);
  }
  hipLaunchKernelGGL(desc_commit_kernel, dim3(1), dim3(64), 0, st, hdr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 3. keys and values of the new rows, at positions count .. count + m - 1
  return launch_desc_kv(cache, L, H, d, eps, count, D, m, Wqkv, kg, kb, st);
}

hipError_t launch_desc_load(const Plan& p, const Ptrs& a, hipStream_t st) {
  hipLaunchKernelGGL(desc_load_kernel, dim3(1), dim3(64), 0, st,
                     reinterpret_cast<const Scalars*>(a.cache), ws_scalars(p, a), p.H);
  return hipGetLastError();
}

}  // namespace vggt
