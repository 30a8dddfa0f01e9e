// Prep-stage kernels (all HBM-bound and small next to the GEMMs and the
// attention core), two launches per call:
//   * bounds_kernel: cos/sin of the 2D RoPE angles, the subsampled mode's
//     sums cleared, and the range bounds -- max L2 norm of the X rows of the
//     attention set(s), of the V rows of Wqkv, and max |Wo| -- as one partial
//     maximum per workgroup (no atomics, nothing to clear first);
//   * wo_convert_kernel: reduces the partial maxima into the workspace
//     scalars (exact power-of-two scales that keep V, O and Wo inside fp16
//     range), sets the range status bits (non-finite inputs, affines or
//     bounds that no pre-scale brings into fp16 range) and writes the fp16
//     copy of Wo scaled by 2^s (the output GEMM runs on fp16 MFMA);
// plus the register-mode patch-row copy Y = X and the residual update of a
// layer schedule.
#include "plan.h"

namespace vggt {

// RoPE table entry (pos, i) = (cos, sin)(pos * base^(-i/16)) for the 16
// frequencies of a 32-feature half of a 64-wide head; angles in double.
__device__ __forceinline__ float2 rope_entry(int i, float base) {
  const int pos = i >> 4, f = i & 15;
  const double theta = pow((double)base, -(double)f / 16.0);
  double sn, cs;
  sincos((double)pos * theta, &sn, &cs);
  return make_float2((float)cs, (float)sn);
}

// Largest L2 norm of the bf16 rows of `len` elements (a multiple of 8) that
// waves wave0, wave0 + nwaves, ... of the grid walk (four rows at a time,
// loads issued together); rows are mapped through `map`, unmapped rows
// skipped; +inf once a row holds a non-finite value or its squared norm
// overflows fp32.  Per-lane result (every lane of a wave holds the wave's
// value).
__device__ __forceinline__ float rows_norm_max(const bf16* base, int64_t nrows, int len,
                                               const RowMap& map, int64_t wave0, int64_t nwaves,
                                               int lane) {
  float best = 0.f;
  for (int64_t w0 = wave0; w0 < nrows; w0 += 4 * nwaves) {
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
      best = max_or_inf(best, sqrtf(a));
    }
  }
  return best;
}

// Maximum of v over a 256-thread workgroup (result in thread 0).
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();  // `red` may still be read from a previous call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

struct BoundsArgs {
  const bf16* X;      // rows through map (skipped when null)
  int64_t rows;
  RowMap map;
  const bf16* Wqkv;   // [3d][d]: V rows for the bound (skipped when X is null), Q and K rows
                      // checked for non-finite values
  const bf16* Wo;     // [d][d]
  int d;
  float* part;        // [kBoundsX] X, [kBoundsV] Wv, [kBoundsO] Wo, [kBoundsV] Wq / Wk partials
  float2* rope;
  int nrope;          // table entries (positions x 16)
  float base;
  float* sums;        // subsampled mode: cleared
  int nsums;
};

// One launch: RoPE table, cleared sums and the partial bound maxima.  Every
// workgroup takes part in the X rows; the first kBoundsV in the V rows of
// Wqkv, the first kBoundsO in |Wo|.  The grid has at least kBoundsO
// workgroups and at most kBoundsX.
__global__ __launch_bounds__(256) void bounds_kernel(BoundsArgs b) {
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t gtid = (int64_t)blockIdx.x * 256 + tid, gthreads = (int64_t)gridDim.x * 256;
  for (int64_t i = gtid; i < b.nrope; i += gthreads) b.rope[i] = rope_entry((int)i, b.base);
  for (int64_t i = gtid; i < b.nsums; i += gthreads) b.sums[i] = 0.f;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (tid >> 6);
  float xm = 0.f, vm = 0.f, om = 0.f, qkm = 0.f;
  const RowMap ident{INT64_MAX / 2, 0, 3 * b.d, 1, 0};
  if (b.X) {
    xm = rows_norm_max(b.X, b.rows, b.d, b.map, wave, (int64_t)gridDim.x * 4, lane);
    if (blockIdx.x < kBoundsV)
      vm = rows_norm_max(b.Wqkv + (int64_t)2 * b.d * b.d, b.d, b.d, ident, wave,
                         (int64_t)kBoundsV * 4, lane);
  }
  if (blockIdx.x < kBoundsV)
    qkm = rows_norm_max(b.Wqkv, 2 * b.d, b.d, ident, wave, (int64_t)kBoundsV * 4, lane);
  if (blockIdx.x < kBoundsO) {
    const int64_t n8 = (int64_t)b.d * b.d / 8;
    for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < n8; i += (int64_t)kBoundsO * 256) {
      const bf16x8 v = reinterpret_cast<const bf16x8*>(b.Wo)[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) om = max_or_inf(om, fabsf((float)v[e]));
    }
  }
  xm = block_max(xm, red);
  vm = block_max(vm, red);
  om = block_max(om, red);
  qkm = block_max(qkm, red);
  if (tid == 0) {
    b.part[blockIdx.x] = xm;
    if (blockIdx.x < kBoundsV) b.part[kBoundsX + blockIdx.x] = vm;
    if (blockIdx.x < kBoundsO) b.part[kBoundsX + kBoundsV + blockIdx.x] = om;
    if (blockIdx.x < kBoundsV) b.part[kBoundsX + kBoundsV + kBoundsO + blockIdx.x] = qkm;
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
      best = max_or_inf(best, sqrtf(a));
    }
  }
  if (lane == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (m > 0.f) atomic_max_nonneg(out, m);
  }
}

// The per-head QK-norm affines of a call (k_gamma / k_beta null in
// descriptor mode, whose keys come from the cache) and whether the range bits
// are ORed into the status word (keep) or replace it.
struct AffineArgs {
  const float* qg;
  const float* qb;
  const float* kg;
  const float* kb;
  int keep;
  int desc;  // descriptor mode: the value bounds are the cache's (checked when they are loaded)
  int bf16;  // the Wo copy in bf16 (bf16 attention operands), else fp16
};

// Largest per-feature bound 8 |gamma| + |beta| over an [H][64] affine (a
// LayerNorm-ed feature is at most sqrt(63) < 8 in magnitude); +inf if an entry
// is not finite.  Result in every thread of the workgroup.
__device__ __forceinline__ float affine_bound(const float* g, const float* b, int n, float* red) {
  float a = 0.f;
  if (g)
    for (int i = threadIdx.x; i < n; i += 256) a = max_or_inf(a, 8.f * fabsf(g[i]) + fabsf(b[i]));
  return block_max(a, red);
}

// Wo (bf16) -> fp16 * 2^s with s chosen from max|Wo| so the largest entry
// lands near 2^14; exact for every entry within 2^-24 of the largest.  Every
// workgroup reduces the |Wo| partial maxima itself; workgroup 0 also writes
// the scalars: the three bounds, cleared key norms (the QKV epilogue takes
// their maximum) and the range status.  nx = X partials written by the
// bounds kernel.
__global__ __launch_bounds__(256) void wo_convert_kernel(const bf16* wo, int64_t n8,
                                                         const float* part, int nx, Scalars* sc,
                                                         int H, void* out, AffineArgs af) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const float woabs = block_max(tid < kBoundsO ? part[kBoundsX + kBoundsV + tid] : 0.f, red);
  if (blockIdx.x == 0) {
    float xm = 0.f;
    for (int i = tid; i < nx; i += 256) xm = fmaxf(xm, part[i]);
    xm = block_max(xm, red);
    const float vm = block_max(tid < kBoundsV ? part[kBoundsX + tid] : 0.f, red);
    const float qkm =
        block_max(tid < kBoundsV ? part[kBoundsX + kBoundsV + kBoundsO + tid] : 0.f, red);
    const float aq = affine_bound(af.qg, af.qb, H * kDh, red);
    const float ak = affine_bound(af.kg, af.kb, H * kDh, red);
    if (tid == 0) {
      sc->xnorm = xm;
      sc->wvnorm = vm;
      sc->woabs = woabs;
      sc->pad = 0.f;
      // Every bound is +inf when its input holds a non-finite value.
      uint32_t bits = 0;
      if (!(xm < INFINITY)) bits |= VGGT_ATTN_RANGE_X;
      if (!(vm < INFINITY) || !(qkm < INFINITY)) bits |= VGGT_ATTN_RANGE_WQKV;
      if (!(woabs < INFINITY)) bits |= VGGT_ATTN_RANGE_WO;
      // q / k features are at most 8 |gamma| + |beta| after the LayerNorm:
      // keep them well inside fp16 (65504)
      if (!(aq < 32768.f) || !(ak < 32768.f)) bits |= VGGT_ATTN_RANGE_AFFINE;
      if (!bits && !af.desc) {
        // v and Wo need a power-of-two scale within 2^+-60; |y| is at most
        // d max|o| max|Wo| <= d max||x|| max||w_v|| max|Wo| and must stay
        // below bf16's largest value
        if (range_exponent_clamped(xm * vm) || range_exponent_clamped(woabs) ||
            (double)xm * vm * woabs * (H * kDh) >= 3.0e38)
          bits |= VGGT_ATTN_RANGE_SCALE;
      }
      sc->status = bits | (af.keep ? sc->status : 0u);
    }
    for (int i = tid; i < H; i += 256) sc->kmax[i] = 0.f;
  }
  const int s = range_exponent(woabs);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    bf16x8 v = reinterpret_cast<const bf16x8*>(wo)[i];
    if (af.bf16) {
      // exact: a power-of-two scale inside bf16's exponent range
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)ldexpf((float)v[e], s);
      reinterpret_cast<bf16x8*>(out)[i] = o;
    } else {
      f16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (f16)ldexpf((float)v[e], s);
      reinterpret_cast<f16x8*>(out)[i] = o;
    }
  }
}

// Register mode, Y != X: copy the patch rows (tokens 17..T-1) of every frame.
// Blocks (x, y): x walks the frame's patch rows in 16-byte chunks, y the
// frames; each thread moves four chunks per step (loads first, then stores),
// consecutive lanes on consecutive chunks, and no index needs a division.
// Non-temporal loads and stores: the gigabytes streamed through once would
// only evict useful lines (s500 copy alone: 6.1 TB/s, against 5.6 with plain
// accesses and 5.1 for the runtime's device-to-device copy).
__global__ __launch_bounds__(256) void patch_copy_kernel(const bf16* X, bf16* Y, int S,
                                                         int64_t frame_elems, int64_t skip_elems,
                                                         int64_t per) {
  const int64_t step = (int64_t)gridDim.x * 256 * 4;
  for (int s = blockIdx.y; s < S; s += gridDim.y) {
    const u32x4* src = reinterpret_cast<const u32x4*>(X + (int64_t)s * frame_elems + skip_elems);
    u32x4* dst = reinterpret_cast<u32x4*>(Y + (int64_t)s * frame_elems + skip_elems);
    for (int64_t c0 = (int64_t)blockIdx.x * 256 * 4 + threadIdx.x; c0 < per; c0 += step) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c0 + u * 256 < per) v[u] = __builtin_nontemporal_load(src + c0 + u * 256);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c0 + u * 256 < per) __builtin_nontemporal_store(v[u], dst + c0 + u * 256);
    }
  }
}

// Residual update between the blocks of a layer schedule: for rows whose
// index modulo `period` is below `active`, Z = X + gamma * Y per channel (fp32
// fma, one rounding to bf16); other rows Z = X.  Optionally also writes Z into
// a strided cache (row r at C + r * c_stride).  Eight channels per step.
// `only_active`: the loop visits the active rows alone (Z == X and no cache:
// the other rows would be copied onto themselves).
__global__ __launch_bounds__(256) void residual_kernel(const bf16* X, const bf16* Y, bf16* Z,
                                                       int64_t rows, int d, const float* gamma,
                                                       int period, int active, bf16* C,
                                                       int64_t c_stride, int only_active) {
  const int per_row = d / 8;
  const int64_t vrows = only_active ? rows / period * active : rows;  // visited rows
  const int64_t total = vrows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t v = i / per_row;
    const int c = (int)(i - v * per_row) * 8;
    const int64_t r = only_active ? v / active * period + v % active : v;
    // streamed once: non-temporal accesses (as the patch copy)
    const bf16x8 x = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(X + r * d + c));
    bf16x8 z = x;
    if ((int)(r % period) < active) {
      const bf16x8 y = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(Y + r * d + c));
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + c);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + c + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        z[e] = (bf16)fmaf(e < 4 ? g0[e & 3] : g1[e & 3], (float)y[e], (float)x[e]);
    }
    __builtin_nontemporal_store(z, reinterpret_cast<bf16x8*>(Z + r * d + c));
    if (C) __builtin_nontemporal_store(z, reinterpret_cast<bf16x8*>(C + r * c_stride + c));
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
  // Descriptor mode: no values are projected here; the bounds of the cached
  // values are copied in after the Wo conversion (launch_desc_load).  X's
  // rows are still checked for non-finite values (its queries).
  const bool desc = p.mode == VGGT_ATTN_MODE_DESCRIPTOR;
  BoundsArgs b;
  b.X = a.X;
  b.rows = p.rows;
  b.map = p.map;
  b.Wqkv = a.Wqkv;
  b.Wo = a.Wo;
  b.d = p.d;
  b.part = reinterpret_cast<float*>(a.ws + p.off_bounds);
  b.rope = ws_rope(p, a);
  b.nrope = p.rope_npos * 16;
  b.base = p.base;
  b.sums = sub ? ws_sums(p, a) : nullptr;
  b.nsums = sub ? 128 * p.H : 0;
  int grid = grid_for(p.rows, 16, kBoundsX);
  if (grid < kBoundsO) grid = kBoundsO;
  hipLaunchKernelGGL(bounds_kernel, dim3(grid), dim3(256), 0, st, b);
  const int64_t n8 = (int64_t)p.d * p.d / 8;
  const AffineArgs af{a.qg, a.qb, desc ? nullptr : a.kg, desc ? nullptr : a.kb,
                      p.keep_status ? 1 : 0, desc ? 1 : 0, p.bf16_ops ? 1 : 0};
  hipLaunchKernelGGL(wo_convert_kernel, dim3(grid_for(n8, 256, 2048)), dim3(256), 0, st, a.Wo,
                     n8, (const float*)b.part, grid, sc, p.H, ws_wo(p, a), af);
  if (desc) return launch_desc_load(p, a, st);
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
  const int64_t per = (frame - skip) / 8;  // 16-byte chunks per frame
  // about 4 chunks per thread per frame (at most 2^20 blocks); frames spread
  // over y (at most 65,535)
  int64_t bx = (per + 256 * 4 - 1) / (256 * 4);
  if (bx > (1 << 20)) bx = 1 << 20;
  const int by = p.S < 65535 ? p.S : 65535;
  hipLaunchKernelGGL(patch_copy_kernel, dim3((unsigned)bx, (unsigned)by), dim3(256), 0, st, a.X,
                     a.Y, p.S, frame, skip, per);
  return hipGetLastError();
}

hipError_t launch_residual(const bf16* X, const bf16* Y, bf16* Z, int64_t rows, int d,
                           const float* gamma, int period, int active, bf16* C, int64_t c_stride,
                           hipStream_t st) {
  // in place without a cache, rows outside the active ones stay as they are
  const int only_active = (X == Z && C == nullptr && active < period && rows % period == 0) ? 1 : 0;
  const int64_t work = (only_active ? rows / period * active : rows) * (d / 8);
  hipLaunchKernelGGL(residual_kernel, dim3(grid_for(work, 256, 8192)), dim3(256), 0, st, X, Y, Z,
                     rows, d, gamma, period, active, C, c_stride, only_active);
  return hipGetLastError();
}

}  // namespace vggt
