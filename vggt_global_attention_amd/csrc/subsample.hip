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

// One workgroup per (64 compact keys, head).  K: 512 16-byte chunks, two per
// thread.  V^T: 64 features x 64 keys, thread = (feature, 16-key group): the
// 16 values of a group are gathered into registers and stored as two
// 16-byte chunks in slot order.
__global__ __launch_bounds__(256) void sga_gather_kernel(const f16* k, const f16* vt, int64_t rows,
                                                         f16* kc, f16* vc, int64_t kv_rows, int Lk,
                                                         SubsampleGeom g) {
  const int hd = blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * 64;
  const f16* kh = k + (int64_t)hd * rows * kDh;
  const f16* vh = vt + (int64_t)hd * kDh * rows;
  f16* kch = kc + (int64_t)hd * kv_rows * kDh;
  f16* vch = vc + (int64_t)hd * kDh * kv_rows;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ch = threadIdx.x + 256 * i, row = ch >> 3, col = ch & 7;
    const int64_t c = c0 + row;
    u32x4 v = {0, 0, 0, 0};
    if (c < Lk) v = *reinterpret_cast<const u32x4*>(kh + kept_token(g, c) * kDh + col * 8);
    *reinterpret_cast<u32x4*>(kch + c * kDh + col * 8) = v;
  }
  const int e = threadIdx.x >> 2;             // feature
  const int64_t gb = c0 + (threadIdx.x & 3) * 16;  // first key of the 16-group
  f16 val[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t c = gb + u;
    val[vt_slot(u)] = c < Lk ? vh[(int64_t)e * rows + vt_slot(kept_token(g, c))] : (f16)0.f;
  }
  f16x8 lo, hi;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    lo[u] = val[u];
    hi[u] = val[8 + u];
  }
  f16* dst = vch + (int64_t)e * kv_rows + gb;
  *reinterpret_cast<f16x8*>(dst) = lo;
  *reinterpret_cast<f16x8*>(dst + 8) = hi;
}

// Per head: sum over the discarded tokens of k (64 features) and of v
// (64 features, in the scaled domain of v^T).  One workgroup per (1024
// tokens, head) writes its 128 partial sums; sga_sum_final_kernel adds the
// partials of a head in a fixed order, so the result is deterministic.
__global__ __launch_bounds__(256) void sga_sum_kernel(const f16* k, const f16* vt, int64_t rows,
                                                      int64_t N, float* partial, SubsampleGeom g) {
  __shared__ float red[32][65];
  const int hd = blockIdx.y;
  const int64_t w0 = (int64_t)blockIdx.x * 1024;
  const f16* kh = k + (int64_t)hd * rows * kDh;
  const f16* vh = vt + (int64_t)hd * kDh * rows;
  const int tid = threadIdx.x;

  // keys: thread = (row group tid>>3, 16-byte column tid&7), rows w0 + (tid>>3) + 32 i
  float ks[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int col = tid & 7, rg = tid >> 3;
  for (int i = 0; i < 32; ++i) {
    const int64_t w = w0 + rg + 32 * i;
    if (w < N && discarded(g, w)) {
      const f16x8 v = *reinterpret_cast<const f16x8*>(kh + w * kDh + col * 8);
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

  // values: thread = (feature tid>>2, quarter tid&3 of the 1024 slots); slot
  // x of v^T holds key vt_slot(x) (the swap is its own inverse).  A key below
  // N can sit in a slot at or above N inside the last group of 16, so the
  // walk covers whole groups (slots < roundup(N, 16) <= rows).
  const int e = tid >> 2, qt = tid & 3;
  const int64_t nslots = (N + 15) & ~(int64_t)15;
  float vs = 0.f;
  for (int i = 0; i < 32; ++i) {
    const int64_t x0 = w0 + qt * 256 + i * 8;
    if (x0 >= nslots) break;
    const f16x8 v = *reinterpret_cast<const f16x8*>(vh + (int64_t)e * rows + x0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t w = vt_slot(x0 + u);
      if (w < N && discarded(g, w)) vs += (float)v[u];
    }
  }
  vs += __shfl_xor(vs, 1);
  vs += __shfl_xor(vs, 2);
  if (qt == 0) out[64 + e] = vs;
}

__global__ __launch_bounds__(128) void sga_sum_final_kernel(const float* partial, int nblk,
                                                            float* sums) {
  const int hd = blockIdx.x, f = threadIdx.x;
  const float* p = partial + (int64_t)hd * nblk * 128 + f;
  float s = 0.f;
  for (int b = 0; b < nblk; ++b) s += p[(int64_t)b * 128];
  sums[hd * 128 + f] = s;
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
    hipLaunchKernelGGL(sga_sum_final_kernel, dim3(p.H), dim3(128), 0, st, (const float*)partial,
                       (int)sx, ws_sums(p, a));
  }
  return hipGetLastError();
}

}  // namespace vggt
