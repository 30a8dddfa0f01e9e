// Prep-stage kernels (all HBM-bound and small next to the GEMMs and the
// attention core):
//   * clear the workspace scalars (and the subsampled mode's sums) and
//     tabulate cos/sin of the 2D RoPE angles;
//   * range bounds: max L2 norm of the X rows of the attention set(s), of the
//     V rows of Wqkv, and max |Wo| -- they pick exact power-of-two scales that
//     keep V, O and Wo inside fp16 range for the attention and output kernels;
//   * an fp16 copy of Wo scaled by 2^s (the output GEMM runs on fp16 MFMA);
//   * the register-mode patch-row copy Y = X.
#include "plan.h"

namespace vggt {

// RoPE table entry (pos, i) = (cos, sin)(pos * base^(-i/16)) for the 16
// frequencies of a 32-feature half of a 64-wide head; angles in double.
// Also clears `nsums` floats at `sums` (subsampled mode: the discarded-token
// sums the CORE stage accumulates).
__global__ void prep_kernel(float* scal, int nscal, float* sums, int nsums, float2* rope, int npos,
                            float base) {
  for (int i = threadIdx.x; i < nscal; i += blockDim.x) scal[i] = 0.f;
  for (int i = threadIdx.x; i < nsums; i += blockDim.x) sums[i] = 0.f;
  for (int i = threadIdx.x; i < npos * 16; i += blockDim.x) {
    int pos = i >> 4, f = i & 15;
    double theta = pow((double)base, -(double)f / 16.0);
    double sn, cs;
    sincos((double)pos * theta, &sn, &cs);
    rope[i] = make_float2((float)cs, (float)sn);
  }
}

// Max over rows of the L2 norm of a bf16 row of `len` elements (len a
// multiple of 8).  Rows are workspace rows mapped through `map`; unmapped
// rows are skipped.  Each wave walks rows w, w + nwaves, ... (four at a time,
// loads issued together); the workgroup reduces in LDS and issues a single
// atomic.
__global__ __launch_bounds__(256) void rownorm_max_kernel(const bf16* base, int64_t nrows,
                                                          int len, RowMap map, float* out) {
  __shared__ float red[4];
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  float best = 0.f;
  for (int64_t w0 = wave; w0 < nrows; w0 += 4 * nwaves) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t w = w0 + u * nwaves;
      const int64_t src = w < nrows ? map.src(w) : -1;
      if (src < 0) continue;
      const bf16* row = base + src * len;
      for (int c = lane * 8; c < len; c += 512) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(row + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = (float)v[e];
          acc[u] = fmaf(f, f, acc[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float a = acc[u];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o);
      best = fmaxf(best, sqrtf(a));
    }
  }
  if (lane == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (m > 0.f) atomic_max_nonneg(out, m);
  }
}

__global__ __launch_bounds__(256) void absmax_kernel(const bf16* x, int64_t n8, float* out) {
  __shared__ float red[4];
  float best = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    bf16x8 v = reinterpret_cast<const bf16x8*>(x)[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) best = fmaxf(best, fabsf((float)v[e]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) best = fmaxf(best, __shfl_xor(best, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (m > 0.f) atomic_max_nonneg(out, m);
  }
}

// Wo (bf16) -> fp16 * 2^s with s chosen from max|Wo| so the largest entry
// lands near 2^14; exact for every entry within 2^-24 of the largest.
__global__ __launch_bounds__(256) void wo_convert_kernel(const bf16* wo, int64_t n8,
                                                         const Scalars* sc, f16* out) {
  const int s = range_exponent(sc->woabs);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    bf16x8 v = reinterpret_cast<const bf16x8*>(wo)[i];
    f16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (f16)ldexpf((float)v[e], s);
    reinterpret_cast<f16x8*>(out)[i] = o;
  }
}

// Register mode, Y != X: copy the patch rows (tokens 17..T-1) of every frame.
// Each thread moves four 16-byte chunks per step (loads first, then stores).
__global__ __launch_bounds__(256) void patch_copy_kernel(const bf16* X, bf16* Y, int S,
                                                         int64_t frame_elems, int64_t skip_elems) {
  const int64_t per = (frame_elems - skip_elems) / 8;  // 16-byte chunks per frame
  const int64_t total = per * S;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < total; i0 += 4 * stride) {
    u32x4 v[4];
    int64_t off[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      const int64_t s = i / per, c = i - s * per;
      off[u] = i < total ? s * frame_elems + skip_elems + c * 8 : -1;
      if (off[u] >= 0) v[u] = *reinterpret_cast<const u32x4*>(X + off[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (off[u] >= 0) *reinterpret_cast<u32x4*>(Y + off[u]) = v[u];
  }
}

// Residual update between the blocks of a layer schedule: for rows whose
// index modulo `period` is below `active`, Z = X + gamma * Y per channel (fp32
// fma, one rounding to bf16); other rows Z = X.  Optionally also writes Z into
// a strided cache (row r at C + r * c_stride).  Eight channels per step.
__global__ __launch_bounds__(256) void residual_kernel(const bf16* X, const bf16* Y, bf16* Z,
                                                       int64_t rows, int d, const float* gamma,
                                                       int period, int active, bf16* C,
                                                       int64_t c_stride) {
  const int per_row = d / 8;
  const int64_t total = rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per_row;
    const int c = (int)(i - r * per_row) * 8;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(X + r * d + c);
    bf16x8 z = x;
    if ((int)(r % period) < active) {
      const bf16x8 y = *reinterpret_cast<const bf16x8*>(Y + r * d + c);
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + c);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + c + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        z[e] = (bf16)fmaf(e < 4 ? g0[e & 3] : g1[e & 3], (float)y[e], (float)x[e]);
    }
    *reinterpret_cast<bf16x8*>(Z + r * d + c) = z;
    if (C) *reinterpret_cast<bf16x8*>(C + r * c_stride + c) = z;
  }
}

static int grid_for(int64_t work, int per_block, int cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (int)(g > cap ? cap : g);
}

hipError_t launch_prep(const Plan& p, const Ptrs& a, hipStream_t st) {
  Scalars* sc = ws_scalars(p, a);
  const bool sub = p.mode == VGGT_ATTN_MODE_SUBSAMPLED;
  hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<float*>(sc),
                     4 + p.H, sub ? ws_sums(p, a) : nullptr, sub ? 128 * p.H : 0, ws_rope(p, a),
                     p.rope_npos, p.base);
  // Descriptor mode: no values are projected here; the bounds of the cached
  // values are copied in after the Wo conversion (launch_desc_load).
  if (p.mode != VGGT_ATTN_MODE_DESCRIPTOR) {
    // X rows of the set(s): walk the workspace rows through the row map.
    hipLaunchKernelGGL(rownorm_max_kernel, dim3(grid_for(p.rows, 16, 2048)), dim3(256), 0, st,
                       a.X, p.rows, p.d, p.map, &sc->xnorm);
    RowMap ident{INT64_MAX / 2, 0, p.d, 1};
    hipLaunchKernelGGL(rownorm_max_kernel, dim3(grid_for(p.d, 16, 2048)), dim3(256), 0, st,
                       a.Wqkv + (int64_t)2 * p.d * p.d, (int64_t)p.d, p.d, ident, &sc->wvnorm);
  }
  const int64_t n8 = (int64_t)p.d * p.d / 8;
  hipLaunchKernelGGL(absmax_kernel, dim3(grid_for(n8, 1024, 256)), dim3(256), 0, st, a.Wo, n8,
                     &sc->woabs);
  hipLaunchKernelGGL(wo_convert_kernel, dim3(grid_for(n8, 256, 2048)), dim3(256), 0, st, a.Wo,
                     n8, (const Scalars*)sc, ws_wo(p, a));
  if (p.mode == VGGT_ATTN_MODE_DESCRIPTOR) return launch_desc_load(p, a, st);
  return hipGetLastError();
}

hipError_t launch_rownorm_max(const bf16* X, int64_t rows, int d, RowMap map, float* out,
                              hipStream_t st) {
  hipLaunchKernelGGL(rownorm_max_kernel, dim3(grid_for(rows, 16, 2048)), dim3(256), 0, st, X, rows,
                     d, map, out);
  return hipGetLastError();
}

hipError_t launch_patch_copy(const Plan& p, const Ptrs& a, hipStream_t st) {
  if (p.T <= kSpecial) return hipSuccess;
  const int64_t frame = (int64_t)p.T * p.d, skip = (int64_t)kSpecial * p.d;
  const int64_t work = (frame - skip) / 8 * p.S;
  hipLaunchKernelGGL(patch_copy_kernel, dim3(grid_for(work, 1024, 4096)), dim3(256), 0, st, a.X,
                     a.Y, p.S, frame, skip);
  return hipGetLastError();
}

hipError_t launch_residual(const bf16* X, const bf16* Y, bf16* Z, int64_t rows, int d,
                           const float* gamma, int period, int active, bf16* C, int64_t c_stride,
                           hipStream_t st) {
  const int64_t work = rows * (d / 8);
  hipLaunchKernelGGL(residual_kernel, dim3(grid_for(work, 256, 8192)), dim3(256), 0, st, X, Y, Z,
                     rows, d, gamma, period, active, C, c_stride);
  return hipGetLastError();
}

}  // namespace vggt
