// AVGGT subsampled global attention: the key / value side ("AVGGT: Rethinking
// Global Attention for Accelerating VGGT", gist.science summary, technical
// summary section 2B).
//
// After the QKV stage has written k and v^T for every token, the CORE stage of
// the subsampled mode first
//   * gathers the kept tokens -- the 17 specials of every frame and the
//     top-left patch of every sub_h x sub_w window of the grid -- into compact
//     key / value buffers laid out exactly like the full ones (k row-major,
//     v^T feature-major with key bits 2 and 3 swapped inside aligned groups of
//     16, now by compact index), zero-padded to a multiple of 64 keys;
//   * sums the keys and the values of the discarded tokens per head (fp32),
//     from which the attention kernel takes the mean key / value pair.
// The kernels are memory-bound and small: the kept set is ~1/7 of the tokens
// at 3 x 3 windows, the sums read k and v^T once.
#include "plan.h"

namespace vggt {

struct SubsampleGeom {
  int T, gw, sub_h, sub_w;
  int kept_frame;  // kept tokens per frame
  int ncw;         // kept patch columns per grid row
};

// Token index (in the global set) of compact key c.
__device__ __forceinline__ int64_t kept_token(const SubsampleGeom& g, int64_t c) {
  const int64_t s = c / g.kept_frame;
  const int u = (int)(c - s * g.kept_frame);
  if (u < kSpecial) return s * g.T + u;
  const int pidx = u - kSpecial, a = pidx / g.ncw, b = pidx - a * g.ncw;
  return s * g.T + kSpecial + (int64_t)(a * g.sub_h) * g.gw + b * g.sub_w;
}

// True iff token w of the global set (w < N) is a discarded patch.
__device__ __forceinline__ bool discarded(const SubsampleGeom& g, int64_t w) {
  const int t = (int)(w % g.T);
  if (t < kSpecial) return false;
  const int pidx = t - kSpecial, r = pidx / g.gw, c = pidx - r * g.gw;
  return (r % g.sub_h) != 0 || (c % g.sub_w) != 0;
}

// Storage slot of key x inside its aligned group of 16 (bits 2 and 3 swapped).
__device__ __forceinline__ int64_t vt_slot(int64_t x) {
  return (x & ~(int64_t)15) | (((x >> 2) & 1) << 3) | (((x >> 3) & 1) << 2) | (x & 3);
}

// One workgroup per (64 compact keys, head).  The 64 token indices are
// computed once into LDS.  K: 512 16-byte chunks, two per thread.
__global__ __launch_bounds__(256) void sga_gather_kernel(const f16* k, const f16* vt, int64_t rows,
                                                         f16* kc, f16* vc, int64_t kv_rows, int Lk,
                                                         SubsampleGeom g) {
  __shared__ int64_t tok[64];
  const int hd = blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  if (threadIdx.x < 64) {
    const int64_t c = c0 + threadIdx.x;
    tok[threadIdx.x] = c < Lk ? kept_token(g, c) : -1;
  }
  __syncthreads();
  const f16* kh = k + (int64_t)hd * rows * kDh;
  const f16* vh = vt + (int64_t)hd * kDh * rows;
  f16* kch = kc + (int64_t)hd * kv_rows * kDh;
  f16* vch = vc + (int64_t)hd * kDh * kv_rows;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ch = threadIdx.x + 256 * i, row = ch >> 3, col = ch & 7;
    const int64_t w = tok[row];
    u32x4 v = {0, 0, 0, 0};
    if (w >= 0) v = *reinterpret_cast<const u32x4*>(kh + w * kDh + col * 8);
    *reinterpret_cast<u32x4*>(kch + (c0 + row) * kDh + col * 8) = v;
  }
  // V^T: lane = compact key, each wave walks 16 features; a load instruction
  // reads one feature row near 64 kept tokens, a store writes 128 contiguous
  // bytes (slot order inside groups of 16).
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t w = tok[lane];
  const int64_t src = w >= 0 ? vt_slot(w) : 0;
  f16* dcol = vch + c0 + vt_slot(lane);
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int e = wv * 16 + i;
    const f16 x = w >= 0 ? vh[(int64_t)e * rows + src] : (f16)0.f;
    dcol[(int64_t)e * kv_rows] = x;
  }
}

// Per head: sum over the discarded tokens of k (64 features) and of v
// (64 features, in the scaled domain of v^T).  One workgroup per (1024
// tokens, head): 64 threads first classify the block's tokens into a 16-bit
// mask per group of 16 (LDS), then every thread sums its share.  Each
// workgroup writes its 128 partial sums; sga_sum_final_kernel adds the
// partials of a head in a fixed order, so the result is deterministic.
__global__ __launch_bounds__(256) void sga_sum_kernel(const f16* k, const f16* vt, int64_t rows,
                                                      int64_t N, float* partial, SubsampleGeom g) {
  __shared__ float red[32][65];
  __shared__ uint32_t dmask[64];
  const int hd = blockIdx.y;
  const int64_t w0 = (int64_t)blockIdx.x * 1024;
  const f16* kh = k + (int64_t)hd * rows * kDh;
  const f16* vh = vt + (int64_t)hd * kDh * rows;
  const int tid = threadIdx.x;
  if (tid < 64) {
    uint32_t m = 0;
    const int64_t wg = w0 + tid * 16;
    for (int u = 0; u < 16; ++u)
      if (wg + u < N && discarded(g, wg + u)) m |= 1u << u;
    dmask[tid] = m;
  }
  __syncthreads();
  auto is_disc = [&](int lw) { return (dmask[lw >> 4] >> (lw & 15)) & 1u; };

  // keys: thread = (row group tid>>3, 16-byte column tid&7), rows w0 + (tid>>3) + 32 i
  float ks[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int col = tid & 7, rg = tid >> 3;
  for (int i = 0; i < 32; ++i) {
    const int lw = rg + 32 * i;
    if (is_disc(lw)) {
      const f16x8 v = *reinterpret_cast<const f16x8*>(kh + (w0 + lw) * kDh + col * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) ks[e] += (float)v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][col * 8 + e] = ks[e];
  __syncthreads();
  float* out = partial + ((int64_t)hd * gridDim.x + blockIdx.x) * 128;
  if (tid < 64) {
    float s = 0.f;
    for (int r = 0; r < 32; ++r) s += red[r][tid];
    out[tid] = s;
  }

  // values: each wave walks 16 features; per feature a lane reads 16 bytes
  // at slots 8*lane and 512 + 8*lane (two coalesced 1 KB reads per wave).
  // Slot x of v^T holds key vt_slot(x) (the swap is its own inverse).  A key
  // below N can sit in a slot at or above N inside the last group of 16, so
  // whole groups are read (slots < roundup(N, 16) <= rows); keys at or past N
  // are never marked discarded.
  const int lane = tid & 63, wv = tid >> 6;
  const int64_t nslots = (N + 15) & ~(int64_t)15;
  uint32_t take[2];  // discarded-key bits of this lane's two 8-slot chunks
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int lx = c * 512 + lane * 8;
    take[c] = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) take[c] |= is_disc((int)vt_slot(lx + u)) << u;
    if (w0 + lx >= nslots) take[c] = 0;
  }
  for (int i = 0; i < 16; ++i) {
    const int e = wv * 16 + i;
    const f16* vrow = vh + (int64_t)e * rows + w0;
    float vs = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (take[c] == 0) continue;
      const f16x8 v = *reinterpret_cast<const f16x8*>(vrow + c * 512 + lane * 8);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if ((take[c] >> u) & 1u) vs += (float)v[u];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) vs += __shfl_xor(vs, o);
    if (lane == 0) out[64 + e] = vs;
  }
}

// Fixed-order sum of the per-block partials of one head: thread (half, f)
// adds blocks half, half + 2, ... of feature f; the two halves then meet in
// LDS.
__global__ __launch_bounds__(256) void sga_sum_final_kernel(const float* partial, int nblk,
                                                            float* sums) {
  __shared__ float red[128];
  const int hd = blockIdx.x, f = threadIdx.x & 127, half = threadIdx.x >> 7;
  const float* p = partial + (int64_t)hd * nblk * 128 + f;
  float s = 0.f;
#pragma unroll 8
  for (int b = half; b < nblk; b += 2) s += p[(int64_t)b * 128];
  if (half == 1) red[f] = s;
  __syncthreads();
  if (half == 0) sums[hd * 128 + f] = s + red[f];
}

hipError_t launch_subsample(const Plan& p, const Ptrs& a, hipStream_t st) {
  SubsampleGeom g;
  g.T = p.T;
  g.gw = p.gw;
  g.sub_h = p.sub_h;
  g.sub_w = p.sub_w;
  g.ncw = (p.gw + p.sub_w - 1) / p.sub_w;
  g.kept_frame = kSpecial + ((p.gh + p.sub_h - 1) / p.sub_h) * g.ncw;
  const int64_t N = (int64_t)p.S * p.T;
  const unsigned gx = (unsigned)((p.Lk + 63) / 64);
  hipLaunchKernelGGL(sga_gather_kernel, dim3(gx, p.H), dim3(256), 0, st, ws_k(p, a), ws_v(p, a),
                     p.rows, ws_kloop(p, a), ws_vloop(p, a), p.kv_rows, p.Lk, g);
  if (p.nD > 0) {
    const unsigned sx = (unsigned)((N + 1023) / 1024);
    float* partial = reinterpret_cast<float*>(a.ws + p.off_part);
    hipLaunchKernelGGL(sga_sum_kernel, dim3(sx, p.H), dim3(256), 0, st, ws_k(p, a), ws_v(p, a),
                       p.rows, N, partial, g);
    hipLaunchKernelGGL(sga_sum_final_kernel, dim3(p.H), dim3(256), 0, st, (const float*)partial,
                       (int)sx, ws_sums(p, a));
  }
  return hipGetLastError();
}

}  // namespace vggt
