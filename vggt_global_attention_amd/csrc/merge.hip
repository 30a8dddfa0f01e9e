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
// (at most kMergeStripMax tokens), its merged tokens are contiguous, so their
// value columns are written to the transposed value buffer as whole runs.
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
  int nwr, nstrips;  // window rows, strips (frame runs x window rows)
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
  __shared__ short pos[kMergeStripMax];
  __shared__ unsigned char merged[kMergeStripMax];
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

  if (item < a.S) {
    // the special tokens of frame `item`: merged tokens item * 17 + t, size 1
    for (int t = wave; t < kSpecial; t += 4) {
      const int64_t tok = (int64_t)item * a.T + t, m = (int64_t)item * kSpecial + t;
      qch[m * kDh + lane] = qh[tok * kDh + lane];
      kch[m * kDh + lane] = kh[tok * kDh + lane];
      vch[(int64_t)lane * a.kv_rows + vslot(m)] = (f16)((float)vh[tok * kDh + lane] * vscale);
      if (lane == 0) {
        nwh[m] = (f16)1.f;
        own[tok] = (int32_t)m;
      }
    }
    return;
  }
  if (item == a.S + a.nstrips) {
    // the attention kernel reads whole 64-key tiles: merged tokens M .. the
    // tile's end are finite zeros of size 0
    const int64_t end = (a.M + kAttnBK - 1) / kAttnBK * kAttnBK;
    for (int64_t m = a.M + wave; m < end; m += 4) {
      qch[m * kDh + lane] = (f16)0.f;
      kch[m * kDh + lane] = (f16)0.f;
      vch[(int64_t)lane * a.kv_rows + vslot(m)] = (f16)0.f;
      if (lane == 0) nwh[m] = (f16)0.f;
    }
    return;
  }

  // strip: frame run fr, window row wr
  const int strip = item - a.S, fr = strip / a.nwr, wr = strip - fr * a.nwr;
  const int f0 = fr * a.F, nf = a.S - f0 < a.F ? a.S - f0 : a.F;
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
  // 1. the strip's keys into LDS (16 bytes per step)
  for (int idx = tid; idx < nt * 8; idx += 256) {
    const int l = idx >> 3, c = idx & 7;
    *reinterpret_cast<u32x4*>(&keys[l * kKeyStride + c * 8]) =
        *reinterpret_cast<const u32x4*>(kh + token_of(l) * kDh + c * 8);
  }
  __syncthreads();
  // 2. every source's most similar destination of its window (sequential
  //    fp32 sum over the features; the fp16 products are exact in fp32)
  for (int l = nd_row + tid; l < nt; l += 256) {
    const int rest = l % nd_row, row = rest / gw, col = rest - row * gw;
    const int c0 = col / ww * ww, cw = gw - c0 < ww ? gw - c0 : ww;
    float bs = 0.f;
    int bj = -1;
    for (int dr = 0; dr < rh; ++dr)
      for (int dc = 0; dc < cw; ++dc) {
        const f16* kd = &keys[(dr * gw + c0 + dc) * kKeyStride];
        const f16* ks = &keys[l * kKeyStride];
        float sim = 0.f;
        for (int c = 0; c < kDh; c += 8) {
          const f16x8 x = *reinterpret_cast<const f16x8*>(ks + c);
          const f16x8 y = *reinterpret_cast<const f16x8*>(kd + c);
#pragma unroll
          for (int e = 0; e < 8; ++e) sim = fmaf((float)x[e], (float)y[e], sim);
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
  // 4. merged token of every strip token: window base + destination, or
  //    window base + destinations + rank among the window's unmerged sources
  for (int l = tid; l < nt; l += 256) {
    const int i = l / nd_row, rest = l - i * nd_row, row = rest / gw, col = rest - row * gw;
    const int c0 = col / ww * ww, cw = gw - c0 < ww ? gw - c0 : ww, nd = rh * cw;
    int64_t b0 = base;
    for (int c = 0; c < c0; c += ww) b0 += merged_block_count(nf, rh * (gw - c < ww ? gw - c : ww), a.r);
    int64_t m;
    if (i == 0) {
      m = b0 + row * cw + (col - c0);
    } else if (merged[l]) {
      m = b0 + best[l];
    } else {
      const int me = ((i - 1) * rh + row) * cw + (col - c0);
      int before = 0;
      for (int i2 = 1; i2 < nf; ++i2)
        for (int r2 = 0; r2 < rh; ++r2)
          for (int q2 = 0; q2 < cw; ++q2) {
            const int l2 = i2 * nd_row + r2 * gw + c0 + q2;
            const int other = ((i2 - 1) * rh + r2) * cw + q2;
            before += (other < me && !merged[l2]) ? 1 : 0;
          }
      pos[l] = (short)before;
      m = b0 + nd + before;
    }
    own[token_of(l)] = (int32_t)m;
  }
  __syncthreads();
  // 5. the strip's merged tokens: one wave each, lane = feature.  Members:
  //    a destination and the sources merged into it, or one unmerged source.
  int64_t cnt = 0;
  for (int c = 0; c < gw; c += ww) cnt += merged_block_count(nf, rh * (gw - c < ww ? gw - c : ww), a.r);
  f16* vstage = keys;  // [64][cnt]: the value sums, staged for whole-run stores
  for (int m = wave; m < cnt; m += 4) {
    // find the window and the slot inside it
    int c0 = 0, cw = 0;
    int64_t slot = m;
    for (; c0 < gw; c0 += ww) {
      cw = gw - c0 < ww ? gw - c0 : ww;
      const int64_t n = merged_block_count(nf, rh * cw, a.r);
      if (slot < n) break;
      slot -= n;
    }
    const int nd = rh * cw;
    float sq = 0.f, sk = 0.f, sv = 0.f;
    int n = 0;
    auto add = [&](int l) {
      const int64_t tok = token_of(l);
      sq += (float)qh[tok * kDh + lane];
      sk += (float)kh[tok * kDh + lane];
      sv += (float)vh[tok * kDh + lane];
      ++n;
    };
    if (slot < nd) {
      const int j = (int)slot, dr = j / cw, dc = j - dr * cw;
      add(dr * gw + c0 + dc);
      for (int i2 = 1; i2 < nf; ++i2)
        for (int r2 = 0; r2 < rh; ++r2)
          for (int q2 = 0; q2 < cw; ++q2) {
            const int l2 = i2 * nd_row + r2 * gw + c0 + q2;
            if (merged[l2] && best[l2] == j) add(l2);
          }
    } else {
      const int want = (int)(slot - nd);
      for (int i2 = 1; i2 < nf; ++i2)
        for (int r2 = 0; r2 < rh; ++r2)
          for (int q2 = 0; q2 < cw; ++q2) {
            const int l2 = i2 * nd_row + r2 * gw + c0 + q2;
            if (!merged[l2] && pos[l2] == want) add(l2);
          }
    }
    const float inv = 1.f / (float)n;
    qch[(base + m) * kDh + lane] = (f16)(sq * inv);
    kch[(base + m) * kDh + lane] = (f16)(sk * inv);
    vstage[lane * cnt + m] = (f16)(sv * vscale);
    if (lane == 0) nwh[base + m] = (f16)(float)n;
  }
  __syncthreads();
  // 6. value columns: runs of the strip's merged tokens per feature row
  for (int64_t idx = tid; idx < kDh * cnt; idx += 256) {
    const int f = (int)(idx / cnt);
    const int64_t m = idx - f * cnt;
    vch[(int64_t)f * a.kv_rows + vslot(base + m)] = vstage[f * cnt + m];
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
  m.nstrips = (p.S + p.hf - 1) / p.hf * m.nwr;
  hipLaunchKernelGGL(httm_merge_kernel, dim3((unsigned)(p.S + m.nstrips + 1), (unsigned)p.H),
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
