// HTTM head-wise temporal token merging ("HTTM: Head-wise Temporal Token
// Merging for Faster VGGT", 10100.com, sections 02, 04 and 05): the CORE stage
// of the merged mode merges every head's tokens before the attention kernel
// and gives every token its merged token's output after it.
//
// Reading (the page names the parts, not the rule): frames in runs of F and
// the patch grid in windows of wh x ww make spatio-temporal blocks; per head
// and block the patches of the run's first frame are the destinations, the
// other frames' patches the sources; a source's similarity to a destination
// is the dot product of their keys in that head (the stored fp16 keys, summed
// in fp32 in feature order); each source takes its most similar destination
// (ties: the first) and the r sources of highest similarity (ties: the first)
// merge.  A merged token's query and key are its members' means and its value
// their sum (with the key's size n entering the attention's row sum, the
// value sum is n times the mean: a merged key counts n times); the special
// tokens never merge.
//
// Merged order, the same in every head: the 17 S special tokens frame by
// frame, then block by block (frame run, window row, window column) each
// destination and then the block's unmerged sources.  Every block's place
// follows from the geometry alone, so no head waits for another.
//
// One workgroup per (strip, head), a strip being one frame run x one window
// row with all its windows: the strip's keys sit in LDS for the similarities
// (at most kMergeStripMax tokens), then its values and its queries for the
// member sums; its merged tokens are contiguous, so their value columns are
// written to the transposed value buffer as whole runs.
#include "plan.h"

namespace vggt {

struct MergeArgs {
  const f16* q;      // [H][rows][64] normalised, rotated, scaled queries
  const f16* k;      // [H][rows][64] normalised, rotated keys
  const f16* v;      // [H][rows][64] values x 2^kv (token-major in this mode)
  f16* qc;           // [H][kv_rows][64] merged queries
  f16* kc;           // [H][kv_rows][64] merged keys
  f16* vc;           // [H][64][kv_rows] merged value sums x 2^-shift, keys permuted in 16-groups
  f16* nw;           // [H][kv_rows] merged token sizes, 0 past M
  int32_t* owner;    // [H][S*T] merged token of every token
  int64_t rows, kv_rows, M, per_run;
  int S, T, gh, gw;
  int F, wh, ww, r, shift;
  int nwr;           // window rows (0 without patches)
};

// Place of merged token x in the transposed value buffer (bits 2 and 3
// swapped inside every aligned group of 16, the order the attention kernel's
// MFMA consumes probabilities).
__device__ __forceinline__ int64_t vslot(int64_t x) {
  return (x & ~(int64_t)15) | (((x >> 2) & 1) << 3) | (((x >> 3) & 1) << 2) | (x & 3);
}

constexpr int kKeyStride = 72;  // halves per LDS key row (64 + 8: rows 4 banks apart)

__global__ __launch_bounds__(256) void httm_merge_kernel(MergeArgs a) {
  __shared__ __attribute__((aligned(16))) f16 keys[kMergeStripMax * kKeyStride];
  __shared__ float score[kMergeStripMax];
  __shared__ short best[kMergeStripMax];
  __shared__ unsigned char merged[kMergeStripMax];
  __shared__ short mlist[kMergeStripMax];       // strip tokens in member order
  __shared__ short mstart[kMergeStripMax + 1];  // first mlist slot of each local merged token
  const int h = blockIdx.y, item = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t N = (int64_t)a.S * a.T;
  const f16* qh = a.q + (int64_t)h * a.rows * kDh;
  const f16* kh = a.k + (int64_t)h * a.rows * kDh;
  const f16* vh = a.v + (int64_t)h * a.rows * kDh;
  f16* qch = a.qc + (int64_t)h * a.kv_rows * kDh;
  f16* kch = a.kc + (int64_t)h * a.kv_rows * kDh;
  f16* vch = a.vc + (int64_t)h * kDh * a.kv_rows;
  f16* nwh = a.nw + (int64_t)h * a.kv_rows;
  int32_t* own = a.owner + (int64_t)h * N;
  const float vscale = __builtin_amdgcn_ldexpf(1.f, -a.shift);

  // workgroup (frame run fr, window row wr); the window-row-0 workgroup of a
  // run also passes the run's special tokens through, the first one also
  // pads the merged set
  const int nwr1 = a.nwr > 0 ? a.nwr : 1;
  const int fr = item / nwr1, wr = item - fr * nwr1;
  const int f0 = fr * a.F, nf = a.S - f0 < a.F ? a.S - f0 : a.F;
  if (wr == 0) {
    // special tokens: merged token s * 17 + t, size 1
    for (int idx = tid; idx < nf * kSpecial * 8; idx += 256) {
      const int sl = idx >> 3, c = idx & 7, fi = sl / kSpecial, t = sl - fi * kSpecial;
      const int64_t tok = (int64_t)(f0 + fi) * a.T + t, m = (int64_t)(f0 + fi) * kSpecial + t;
      const u32x4 qv = *reinterpret_cast<const u32x4*>(qh + tok * kDh + c * 8);
      const u32x4 kv = *reinterpret_cast<const u32x4*>(kh + tok * kDh + c * 8);
      const f16x8 vv = *reinterpret_cast<const f16x8*>(vh + tok * kDh + c * 8);
      *reinterpret_cast<u32x4*>(qch + m * kDh + c * 8) = qv;
      *reinterpret_cast<u32x4*>(kch + m * kDh + c * 8) = kv;
      const int64_t col = vslot(m);
#pragma unroll
      for (int e = 0; e < 8; ++e) vch[(int64_t)(c * 8 + e) * a.kv_rows + col] = (f16)((float)vv[e] * vscale);
      if (c == 0) {
        nwh[m] = (f16)1.f;
        own[tok] = (int32_t)m;
      }
    }
    if (fr == 0) {
      // the attention kernel reads whole 64-key tiles: merged tokens M ..
      // the tile's end are finite zeros of size 0
      const int64_t end = (a.M + kAttnBK - 1) / kAttnBK * kAttnBK;
      const f16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int64_t idx = tid; idx < (end - a.M) * 8; idx += 256) {
        const int64_t m = a.M + (idx >> 3);
        const int c = (int)(idx & 7);
        *reinterpret_cast<f16x8*>(qch + m * kDh + c * 8) = z;
        *reinterpret_cast<f16x8*>(kch + m * kDh + c * 8) = z;
        const int64_t col = vslot(m);
#pragma unroll
        for (int e = 0; e < 8; ++e) vch[(int64_t)(c * 8 + e) * a.kv_rows + col] = (f16)0.f;
        if (c == 0) nwh[m] = (f16)0.f;
      }
    }
  }
  if (a.nwr == 0) return;  // no patches: nothing merges

  // the strip: frame run fr x window row wr, every window column
  const int r0 = wr * a.wh, rh = a.gh - r0 < a.wh ? a.gh - r0 : a.wh;
  const int gw = a.gw, ww = a.ww;
  const int nt = nf * rh * gw;            // strip tokens: local (i * rh + row) * gw + col
  const int nd_row = rh * gw;             // tokens of one frame of the strip
  const int64_t base = (int64_t)kSpecial * a.S + fr * a.per_run +
                       merged_run_count(nf, a.gh, gw, a.wh, ww, a.r, wr);
  auto token_of = [&](int l) -> int64_t {
    const int i = l / nd_row, rest = l - i * nd_row, row = rest / gw, col = rest - row * gw;
    return (int64_t)(f0 + i) * a.T + kSpecial + (int64_t)(r0 + row) * gw + col;
  };
  // the strip's rows of one head's k, v or q into LDS, row stride kKeyStride
  auto stage = [&](const f16* src) {
    constexpr int kBatch = 4;
    for (int i0 = tid; i0 < nt * 8; i0 += 256 * kBatch) {
      u32x4 x[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int idx = i0 + b * 256;
        if (idx < nt * 8) x[b] = *reinterpret_cast<const u32x4*>(src + token_of(idx >> 3) * kDh + (idx & 7) * 8);
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const int idx = i0 + b * 256;
        if (idx < nt * 8) *reinterpret_cast<u32x4*>(&keys[(idx >> 3) * kKeyStride + (idx & 7) * 8]) = x[b];
      }
    }
  };
  // 1. the strip's keys into LDS; its values and queries into registers
  //    meanwhile (thread tid holds chunks tid + 256 b), for the member sums
  constexpr int kPre = (kMergeStripMax * 8 + 255) / 256;
  u32x4 vpre[kPre], qpre[kPre];
#pragma unroll
  for (int b = 0; b < kPre; ++b) {
    const int idx = tid + b * 256;
    if (idx < nt * 8) {
      const int64_t off = token_of(idx >> 3) * kDh + (idx & 7) * 8;
      vpre[b] = *reinterpret_cast<const u32x4*>(vh + off);
      qpre[b] = *reinterpret_cast<const u32x4*>(qh + off);
    }
  }
  stage(kh);
  __syncthreads();
  // 2. every source's most similar destination of its window (sequential
  //    fp32 sum over the features; the fp16 products are exact in fp32)
  for (int l = nd_row + tid; l < nt; l += 256) {
    const int rest = l % nd_row, row = rest / gw, col = rest - row * gw;
    const int c0 = col / ww * ww, cw = gw - c0 < ww ? gw - c0 : ww;
    float bs = 0.f;
    int bj = -1;
    float ks[8][8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const f16x8 x = *reinterpret_cast<const f16x8*>(&keys[l * kKeyStride + c * 8]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ks[c][e] = (float)x[e];
    }
    for (int dr = 0; dr < rh; ++dr)
      for (int dc = 0; dc < cw; ++dc) {
        const f16* kd = &keys[(dr * gw + c0 + dc) * kKeyStride];
        float sim = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const f16x8 y = *reinterpret_cast<const f16x8*>(kd + c * 8);
#pragma unroll
          for (int e = 0; e < 8; ++e) sim = fmaf(ks[c][e], (float)y[e], sim);
        }
        if (bj < 0 || sim > bs) {
          bs = sim;
          bj = dr * cw + dc;
        }
      }
    score[l] = bs;
    best[l] = (short)bj;
  }
  __syncthreads();
  // 3. the r best sources of each window merge (ties: the earlier source in
  //    frame, row, column order)
  for (int l = nd_row + tid; l < nt; l += 256) {
    const int i = l / nd_row, rest = l - i * nd_row, row = rest / gw, col = rest - row * gw;
    const int c0 = col / ww * ww, cw = gw - c0 < ww ? gw - c0 : ww;
    const int me = ((i - 1) * rh + row) * cw + (col - c0);  // index among the window's sources
    int rank = 0;
    for (int i2 = 1; i2 < nf; ++i2)
      for (int r2 = 0; r2 < rh; ++r2)
        for (int q2 = 0; q2 < cw; ++q2) {
          const int l2 = i2 * nd_row + r2 * gw + c0 + q2;
          const int other = ((i2 - 1) * rh + r2) * cw + q2;
          rank += (score[l2] > score[l] || (score[l2] == score[l] && other < me)) ? 1 : 0;
        }
    merged[l] = rank < a.r ? 1 : 0;
  }
  __syncthreads();
  // 4. every strip token's merged token, and the member lists: mlist holds
  //    the strip's tokens merged token by merged token, each in member order
  //    (its destination, then its sources in frame, row, column order), and
  //    mstart[x] is where local merged token x begins.  A window's merged
  //    tokens: its destinations (each with the sources merged into it), then
  //    its unmerged sources; its member slots begin at the strip tokens of
  //    the windows before it.
  int cnt = 0;
  for (int c = 0; c < gw; c += ww) cnt += (int)merged_block_count(nf, rh * (gw - c < ww ? gw - c : ww), a.r);
  for (int l = tid; l < nt; l += 256) {
    const int i = l / nd_row, rest = l - i * nd_row, row = rest / gw, col = rest - row * gw;
    const int c0 = col / ww * ww, cw = gw - c0 < ww ? gw - c0 : ww, nd = rh * cw;
    const int ns = (nf - 1) * nd, nm = ns < a.r ? ns : a.r;
    int xw = 0;  // local index of the window's first merged token
    for (int c = 0; c < c0; c += ww) xw += (int)merged_block_count(nf, rh * (gw - c < ww ? gw - c : ww), a.r);
    const int wstart = nf * rh * c0;
    const bool src_merged = i > 0 && merged[l];
    const int me = i == 0 ? -1 : ((i - 1) * rh + row) * cw + (col - c0);
    const int j = i == 0 ? row * cw + (col - c0) : (src_merged ? best[l] : -1);
    int below = 0, same_before = 0, unmerged_before = 0;
    for (int i2 = 1; i2 < nf; ++i2)
      for (int r2 = 0; r2 < rh; ++r2)
        for (int q2 = 0; q2 < cw; ++q2) {
          const int l2 = i2 * nd_row + r2 * gw + c0 + q2;
          const int other = ((i2 - 1) * rh + r2) * cw + q2;
          if (merged[l2]) {
            const int b2 = best[l2];
            below += b2 < j ? 1 : 0;
            same_before += (b2 == j && other < me) ? 1 : 0;
          } else {
            unmerged_before += other < me ? 1 : 0;
          }
        }
    int x, slot;
    if (i == 0) {
      x = xw + j;
      slot = wstart + j + below;
      mstart[x] = (short)slot;
    } else if (src_merged) {
      x = xw + j;
      slot = wstart + j + below + 1 + same_before;
    } else {
      x = xw + nd + unmerged_before;
      slot = wstart + nd + nm + unmerged_before;
      mstart[x] = (short)slot;
    }
    mlist[slot] = (short)l;
    own[token_of(l)] = (int32_t)(base + x);
  }
  if (tid == 0) mstart[cnt] = (short)nt;
  __syncthreads();
  // 5. the strip's merged tokens, from rows staged in LDS (the keys still
  //    there, then the values, then the queries): every staging copy is one
  //    16-byte load per thread and step, all in flight together.  Member
  //    sums in member order (the destination, then its sources in frame,
  //    row, column order), in fp32.
  f16* rows_lds = keys;  // [nt][kKeyStride]
  // member sum of 8 features (chunk c) of local merged token m from the
  // staged rows; returns the member count
  auto chunk_sum = [&](int m, int c, float* acc) -> int {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const int k0 = mstart[m], k1 = mstart[m + 1];
    for (int k = k0; k < k1; ++k) {
      const f16x8 x = *reinterpret_cast<const f16x8*>(&rows_lds[mlist[k] * kKeyStride + c * 8]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (float)x[e];
    }
    return k1 - k0;
  };
  auto unstage = [&](const u32x4* pre) {
#pragma unroll
    for (int b = 0; b < kPre; ++b) {
      const int idx = tid + b * 256;
      if (idx < nt * 8) *reinterpret_cast<u32x4*>(&rows_lds[(idx >> 3) * kKeyStride + (idx & 7) * 8]) = pre[b];
    }
  };
  // 5a. key means (the keys are still staged); item = 8 m + chunk
  for (int idx = tid; idx < cnt * 8; idx += 256) {
    const int m = idx >> 3, c = idx & 7;
    float acc[8];
    const float inv = 1.f / (float)chunk_sum(m, c, acc);
    f16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (f16)(acc[e] * inv);
    *reinterpret_cast<f16x8*>(kch + (base + m) * kDh + c * 8) = o;
  }
  __syncthreads();
  // 5b. value sums x 2^-shift into the transposed buffer and the sizes; item =
  //     chunk * cnt + m, so a wave's lanes write consecutive merged tokens
  //     (whole runs of each feature row)
  unstage(vpre);
  __syncthreads();
  for (int idx = tid; idx < cnt * 8; idx += 256) {
    const int c = idx / cnt, m = idx - c * cnt;
    float acc[8];
    const int n = chunk_sum(m, c, acc);
    const int64_t col = vslot(base + m);
#pragma unroll
    for (int e = 0; e < 8; ++e) vch[(int64_t)(c * 8 + e) * a.kv_rows + col] = (f16)(acc[e] * vscale);
    if (c == 0) nwh[base + m] = (f16)(float)n;
  }
  __syncthreads();
  // 5c. query means; item = 8 m + chunk
  unstage(qpre);
  __syncthreads();
  for (int idx = tid; idx < cnt * 8; idx += 256) {
    const int m = idx >> 3, c = idx & 7;
    float acc[8];
    const float inv = 1.f / (float)chunk_sum(m, c, acc);
    f16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (f16)(acc[e] * inv);
    *reinterpret_cast<f16x8*>(qch + (base + m) * kDh + c * 8) = o;
  }
}

// Unmerging: every token's output rows (the q buffer, which the output
// projection reads) take their merged token's output, times 2^shift (the
// merged values' scale).  One thread per 16-byte chunk.
__global__ __launch_bounds__(256) void httm_unmerge_kernel(const f16* oc, const int32_t* owner,
                                                           f16* q, int64_t rows, int64_t kv_rows,
                                                           int64_t N, int H, float scale) {
  const int64_t total = (int64_t)H * N * 8;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int c = (int)(idx & 7);
    const int64_t ht = idx >> 3, h = ht / N, t = ht - h * N;
    const int64_t m = owner[h * N + t];
    const f16x8 o = *reinterpret_cast<const f16x8*>(oc + (h * kv_rows + m) * kDh + c * 8);
    f16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (f16)((float)o[e] * scale);
    *reinterpret_cast<f16x8*>(q + (h * rows + t) * kDh + c * 8) = r;
  }
}

hipError_t launch_merge(const Plan& p, const Ptrs& a, hipStream_t st) {
  MergeArgs m;
  m.q = ws_q(p, a);
  m.k = ws_k(p, a);
  m.v = ws_v(p, a);
  m.qc = ws_qc(p, a);
  m.kc = ws_kloop(p, a);
  m.vc = ws_vloop(p, a);
  m.nw = ws_nw(p, a);
  m.owner = ws_owner(p, a);
  m.rows = p.rows;
  m.kv_rows = p.kv_rows;
  m.M = p.L;
  m.per_run = p.hper_run;
  m.S = p.S;
  m.T = p.T;
  m.gh = p.gh;
  m.gw = p.gw;
  m.F = p.hf;
  m.wh = p.hwh;
  m.ww = p.hww;
  m.r = p.hr;
  m.shift = p.hshift;
  m.nwr = p.gw > 0 ? (p.gh + p.hwh - 1) / p.hwh : 0;
  const int runs = (p.S + p.hf - 1) / p.hf;
  hipLaunchKernelGGL(httm_merge_kernel, dim3((unsigned)(runs * (m.nwr > 0 ? m.nwr : 1)), (unsigned)p.H),
                     dim3(256), 0, st, m);
  return hipGetLastError();
}

hipError_t launch_unmerge(const Plan& p, const Ptrs& a, hipStream_t st) {
  const int64_t N = (int64_t)p.S * p.T, work = (int64_t)p.H * N * 8;
  int64_t grid = (work + 255) / 256;
  if (grid > 16384) grid = 16384;
  hipLaunchKernelGGL(httm_unmerge_kernel, dim3((unsigned)grid), dim3(256), 0, st,
                     (const f16*)ws_qc(p, a), (const int32_t*)ws_owner(p, a), ws_q(p, a), p.rows,
                     p.kv_rows, N, p.H, ldexpf(1.f, p.hshift));
  return hipGetLastError();
}

}  // namespace vggt
