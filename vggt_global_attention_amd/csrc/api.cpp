// C ABI of libvggtattn: argument checks, planning and stage dispatch.  Every
// check runs before the first HIP call, so a rejected call launches nothing.
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "entry.h"

namespace vggt {

static_assert(offsetof(Scalars, status) == VGGT_ATTN_STATUS_OFFSET,
              "the status word's offset is part of the ABI");

static int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

#ifdef VGGT_ATTN_TUNING
bool tuning_knob(const char* name, int* value) {
  const char* e = getenv(name);
  if (!e || !*e) return false;
  *value = atoi(e);
  return true;
}
#else
bool tuning_knob(const char*, int*) { return false; }
#endif

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Kept tokens per frame in subsampled mode: the 17 specials and the top-left
// cell of every sub_h x sub_w window of the grid.
static int64_t kept_per_frame(const vggt_attn_shape* s, int sub_h, int sub_w) {
  return kSpecial + (int64_t)((s->grid_h + sub_h - 1) / sub_h) * ((s->grid_w + sub_w - 1) / sub_w);
}

int make_plan(int mode, const vggt_attn_shape* s, const CallOpts& o, Plan* p) {
  int sub_h = o.sub_h, sub_w = o.sub_w;
  if (!s || !p) return VGGT_ATTN_EINVAL;
  if (mode != VGGT_ATTN_MODE_FRAME && mode != VGGT_ATTN_MODE_GLOBAL &&
      mode != VGGT_ATTN_MODE_REGISTER && mode != VGGT_ATTN_MODE_SUBSAMPLED &&
      mode != VGGT_ATTN_MODE_DESCRIPTOR && mode != VGGT_ATTN_MODE_MERGED)
    return VGGT_ATTN_EINVAL;
  if (s->S < 1 || s->H < 1 || s->d < 1 || s->grid_h < 0 || s->grid_w < 0) return VGGT_ATTN_ESHAPE;
  if (s->d != s->H * kDh || s->d % kGemmBN != 0) return VGGT_ATTN_ESHAPE;
  const int64_t patches = (int64_t)s->grid_h * s->grid_w;
  if (patches > (1 << 24) || (int64_t)s->T != kSpecial + patches) return VGGT_ATTN_ESHAPE;
  const int64_t N = (int64_t)s->S * s->T;
  if (N >= ((int64_t)1 << 31)) return VGGT_ATTN_ESHAPE;
  if (!(isfinite(s->rope_base) && s->rope_base > 0.f)) return VGGT_ATTN_ERANGE;
  if (!(isfinite(s->ln_eps) && s->ln_eps > 0.f)) return VGGT_ATTN_ERANGE;
  if (s->pos_offset < 0 || s->pos_offset > 65535) return VGGT_ATTN_ERANGE;
  const bool subsampled = mode == VGGT_ATTN_MODE_SUBSAMPLED;
  const bool desc = mode == VGGT_ATTN_MODE_DESCRIPTOR;
  const bool merged = mode == VGGT_ATTN_MODE_MERGED;
  // merged mode: frames == 0 sizes the workspace for the largest merged set
  // (nothing merges); a call passes its blocks and merges
  const bool msize = merged && o.httm_frames == 0;
  if (merged && !msize) {
    if (o.httm_frames < 1 || o.httm_wh < 1 || o.httm_ww < 1 || o.httm_r < 0) return VGGT_ATTN_ERANGE;
    const int64_t nf = o.httm_frames < s->S ? o.httm_frames : s->S;
    const int64_t wh = o.httm_wh < s->grid_h ? o.httm_wh : s->grid_h;
    if (nf * wh * s->grid_w > kMergeStripMax) return VGGT_ATTN_ERANGE;
  }
  if (desc && (o.desc_capacity < 0 || o.desc_capacity >= ((int64_t)1 << 31) ||
               o.desc_count < 0 || o.desc_count > o.desc_capacity))
    return VGGT_ATTN_ERANGE;
  if (!subsampled) sub_h = sub_w = 1;
  if (sub_h < 1 || sub_w < 1) return VGGT_ATTN_ERANGE;
  const bool window = o.q_count >= 0;
  if (window) {
    if (mode != VGGT_ATTN_MODE_GLOBAL) return VGGT_ATTN_EINVAL;
    if (o.q_begin < 0 || o.q_count < 1 || o.q_begin + o.q_count > N) return VGGT_ATTN_ERANGE;
  }

  memset(p, 0, sizeof(*p));
  p->mode = mode;
  p->S = s->S;
  p->T = s->T;
  p->d = s->d;
  p->H = s->H;
  p->gh = s->grid_h;
  p->gw = s->grid_w;
  p->off = s->pos_offset;
  p->base = s->rope_base;
  p->eps = s->ln_eps;
  p->keep_status = o.keep_status;
  // the bf16-operand variant serves the plain sets: frame, global (also a
  // query window of it) and register
  if (o.bf16_ops && mode != VGGT_ATTN_MODE_FRAME && mode != VGGT_ATTN_MODE_GLOBAL &&
      mode != VGGT_ATTN_MODE_REGISTER)
    return VGGT_ATTN_EINVAL;
  p->bf16_ops = o.bf16_ops;
  p->patch_copy = !o.no_patch_copy;
  const int64_t R = (int64_t)s->S * kSpecial;
  int64_t cover;  // workspace rows the attention kernel may touch
  if (mode == VGGT_ATTN_MODE_GLOBAL || subsampled || desc || merged) {
    p->nseq = 1;
    p->L = (int)N;
    p->seq_stride = round_up(N, kAttnBK);
    cover = p->seq_stride;
    p->attn_qb = 2;
    p->attn_waves = 8;
  } else if (mode == VGGT_ATTN_MODE_FRAME) {
    p->nseq = s->S;
    p->L = s->T;
    // q / k rows: frames padded to 16 rows; the last frame's last key tile
    // (64 rows from a multiple of 64) must stay inside the buffer
    p->seq_stride = round_up(s->T, kFrameRowAlign);
    cover = p->seq_stride * (s->S - 1) + round_up(s->T, kAttnBK);
    p->attn_qb = 1;
    p->attn_waves = 4;
  } else {
    p->nseq = 1;
    p->L = (int)R;
    p->seq_stride = round_up(R, kAttnBK);
    cover = p->seq_stride;
    p->attn_qb = 1;
    p->attn_waves = 4;
  }
  // Tuning override of the attention tile (tuning build only).
  bool tile_forced = false;
  int knob = 0;
  if (tuning_knob("VGGT_ATTN_QB", &knob) && (knob == 1 || knob == 2)) {
    p->attn_qb = knob;
    tile_forced = true;
  }
  if (tuning_knob("VGGT_ATTN_WAVES", &knob) && (knob == 4 || knob == 8)) {
    p->attn_waves = knob;
    tile_forced = true;
  }
  p->rows = row_padding(cover);
  if (p->rows >= ((int64_t)1 << 31)) return VGGT_ATTN_ESHAPE;  // kernels index rows in 32 bits
  p->sub_h = sub_h;
  p->sub_w = sub_w;
  if (subsampled) {
    p->Lk = (int)(kept_per_frame(s, sub_h, sub_w) * s->S);
    p->kv_rows = round_up(p->Lk, kKvAlign);
    p->kv_seq_stride = round_up(p->Lk, kAttnBK);
    p->nD = (int)(N - p->Lk);
    // the subsampled kernel has a single tile shape
    p->attn_qb = 2;
    p->attn_waves = 8;
  } else if (merged) {
    // queries, keys and values: the merged tokens (as many as the tokens when
    // only sizing)
    int64_t M = N;
    if (!msize) {
      const int F = o.httm_frames, r = o.httm_r;
      const int nwr = s->grid_w > 0 ? (s->grid_h + o.httm_wh - 1) / o.httm_wh : 0;
      const int full = s->S / F, rest = s->S % F;
      p->hper_run = merged_run_count(F, s->grid_h, s->grid_w, o.httm_wh, o.httm_ww, r, nwr);
      M = (int64_t)kSpecial * s->S + full * p->hper_run +
          (rest ? merged_run_count(rest, s->grid_h, s->grid_w, o.httm_wh, o.httm_ww, r, nwr) : 0);
      p->hf = F;
      p->hwh = o.httm_wh;
      p->hww = o.httm_ww;
      p->hr = r;
      // a merged token has at most 1 + min(r, (F - 1) wh ww) members: its
      // value sum carries 2^-hshift so that it stays inside fp16
      const int64_t cells = (int64_t)(o.httm_wh < s->grid_h ? o.httm_wh : s->grid_h) *
                            (o.httm_ww < s->grid_w ? o.httm_ww : s->grid_w);
      const int64_t src = (int64_t)((F < s->S ? F : s->S) - 1) * cells;
      const int64_t nmax = 1 + (src < r ? src : (int64_t)r);
      while (((int64_t)1 << p->hshift) < nmax) ++p->hshift;
    }
    p->L = (int)M;
    p->Lk = (int)M;
    p->kv_rows = round_up(M, kKvAlign);
    p->kv_seq_stride = round_up(M, kAttnBK);
    p->nD = 0;
  } else if (desc) {
    // keys / values: the first desc_count entries of the caller's cache
    p->desc = desc_layout(s->H, o.desc_capacity > 0 ? o.desc_capacity : 1);
    p->Lk = (int)o.desc_count;
    p->kv_rows = p->desc.cap_rows;
    p->kv_seq_stride = round_up(o.desc_count, kAttnBK);
    p->nD = 0;
  } else {
    p->Lk = p->L;  // (a query window below moves L, never the keys)
    p->kv_rows = p->rows;
    p->kv_seq_stride = p->seq_stride;
    p->nD = 0;
  }
  // v^T columns: frames padded to whole 64-key tiles; elsewhere the rows
  p->vt_rows = p->rows;
  p->vt_seq_stride = p->seq_stride;
  if (mode == VGGT_ATTN_MODE_FRAME) {
    p->vt_seq_stride = round_up(s->T, kAttnBK);
    p->vt_rows = round_up((int64_t)s->S * p->vt_seq_stride, 256);
  }
  if (p->kv_rows > kMaxKvRows || p->vt_rows > kMaxKvRows) return VGGT_ATTN_ESHAPE;
  if (mode == VGGT_ATTN_MODE_GLOBAL || subsampled || desc || merged) {
    p->map = RowMap{p->rows, 0, (int32_t)N, 1, 0};
  } else if (mode == VGGT_ATTN_MODE_FRAME) {
    p->map = RowMap{p->seq_stride, s->T, s->T, s->S, 0};
  } else {
    p->map = RowMap{kSpecial, s->T, kSpecial, s->S, 0};
  }
  p->out_map = p->map;
  p->q0 = 0;
  p->window = window;
  if (window) {
    // keys: every token; queries and outputs: rows [q_begin, q_begin + q_count)
    p->q0 = (int)o.q_begin;
    p->L = (int)(o.q_begin + o.q_count);
    p->out_map = RowMap{p->rows, 0, (int32_t)o.q_count, 1, o.q_begin};
  }
  // Small global-type grids (global sets, query windows, descriptor
  // attention): when the 8-wave tile would give fewer workgroups than the
  // device has CUs, the 4-wave tile of one query block per wave runs four
  // times as many, up to three per CU.  Both tiles compute every row the
  // same way, bit for bit.
  const int64_t cus = o.cus > 0 ? o.cus : 256;
  if ((mode == VGGT_ATTN_MODE_GLOBAL || desc || merged) && !tile_forced &&
      (int64_t)(p->L - p->q0 + 511) / 512 * s->H < cus) {
    p->attn_qb = 1;
    p->attn_waves = 4;
  }
  // Register sets (one set of 17 S rows) take 64 queries per wave on 4-wave
  // workgroups while that grid still has a workgroup per CU (measured at
  // S = 500, 8,500 rows: 0.29 against 0.32 ms with 32 queries per wave, and
  // 0.30 ms on 8-wave workgroups); smaller sets keep 32 queries per wave for
  // the workgroup count.
  if (mode == VGGT_ATTN_MODE_REGISTER && !tile_forced && (R + 255) / 256 * s->H >= cus) {
    p->attn_qb = 2;
  }
  p->rope_npos = (s->grid_h > s->grid_w ? s->grid_h : s->grid_w) + s->pos_offset;
  if (p->rope_npos < 1) p->rope_npos = 1;

  size_t off = 0;
  p->off_scal = off;
  off += round_up((int64_t)scalars_bytes(s->H), 256);
  p->off_bounds = off;  // partial maxima of the prep stage
  off += round_up((int64_t)sizeof(float) * kBoundsParts, 256);
  p->off_rope = off;
  off += round_up((int64_t)p->rope_npos * 16 * sizeof(float2), 256);
  p->off_wo = off;
  off += round_up((int64_t)s->d * s->d * 2, 256);
  const size_t qkv = (size_t)s->H * (size_t)p->rows * kDh * 2;
  p->off_q = off;
  off += qkv;
  if (desc) {
    // queries only: keys and values come from the cache
    p->off_k = p->off_v = p->off_q;
  } else {
    p->off_k = off;
    off += qkv;
    p->off_v = off;
    off += (size_t)s->H * (size_t)p->vt_rows * kDh * 2;
  }
  if (merged) {
    // merged queries, keys, values and key sizes, kv_rows per head (sized for
    // the largest set when only sizing), and every token's merged token
    const size_t mq = (size_t)s->H * (size_t)p->kv_rows * kDh * 2;
    p->off_qc = off;
    off += mq;
    p->off_kc = off;
    off += mq;
    p->off_vc = off;
    off += mq;
    p->off_nw = off;
    off += round_up((int64_t)s->H * p->kv_rows * 2, 256);
    p->off_owner = off;
    off += round_up((int64_t)s->H * N * 4, 256);
  }
  if (subsampled) {
    // compact keys / values sized for the largest kept set (sub_h = sub_w = 1:
    // every token), so the workspace size does not depend on the windows
    p->off_kc = off;
    off += qkv;
    p->off_vc = off;
    off += qkv;
    p->off_sums = off;  // [H][128] fp32: sums of discarded keys, then values
    off += round_up((int64_t)s->H * 128 * sizeof(float), 256);
    p->off_part = off;  // [H][ceil(N/1024)][128] fp32 partial sums
    off += round_up((int64_t)s->H * ((N + 1023) / 1024) * 128 * sizeof(float), 256);
  }
  // Partial results of a split attention tail (global sets, query windows,
  // subsampled and register sets; not frames, whose sets are short, nor the
  // descriptor mode, whose key count is not known when its workspace is
  // sized).  Sized from the shape alone, not the device; in subsampled mode
  // from the kept keys, largest with 1 x 1 windows, the size the workspace
  // query reports.
  // The region is sized for the largest need over the attention tiles (128,
  // 256 or 512 queries per workgroup), so that the size does not depend on
  // which tile the device's CU count picks.
  p->split_cap = 0;
  p->off_split = off;
  if (mode == VGGT_ATTN_MODE_GLOBAL || mode == VGGT_ATTN_MODE_REGISTER || subsampled || merged) {
    int64_t ways = (p->Lk + kAttnBK - 1) / kAttnBK / kSplitMinTiles;
    if (ways > kSplitMaxWays) ways = kSplitMaxWays;
    if (ways >= 2) {
      auto units = [&](int64_t bq) {
        const int64_t W = (p->L - p->q0 + bq - 1) / bq * s->H * p->nseq;
        const int64_t cap = kSplitMaxRows / bq;
        return W * ways < cap ? W * ways : cap;
      };
      int64_t region = 0;
      for (int64_t bq = 128; bq <= 512; bq *= 2) {
        const int64_t b = units(bq) * bq * (kDh + 2) * (int64_t)sizeof(float);
        if (b > region) region = b;
      }
      p->split_cap = (int)units((int64_t)p->attn_waves * p->attn_qb * 32);
      off += round_up(region, 256);
    }
  }
  p->total = off;
  return VGGT_ATTN_OK;
}

}  // namespace vggt

namespace vggt {

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

int check_call(int mode, const vggt_attn_shape* shape, const CallOpts& o, const void* X,
               const void* Wqkv, const void* Wo, const float* qg, const float* qb, const float* kg,
               const float* kb, void* Y, void* ws, size_t ws_bytes, Plan* plan) {
  CallOpts oc = o;
  oc.cus = device_cu_count();
  int st = make_plan(mode, shape, oc, plan);
  if (st != VGGT_ATTN_OK) return st;
  const bool desc = mode == VGGT_ATTN_MODE_DESCRIPTOR;
  // descriptor mode: keys come from the cache, so no key affine is passed
  if (!X || !Wqkv || !Wo || !qg || !qb || (!desc && (!kg || !kb)) || !Y || !ws)
    return VGGT_ATTN_EINVAL;
  if (desc) {
    if (!o.cache) return VGGT_ATTN_EINVAL;
    if (o.desc_capacity < 1 || o.desc_count < 1) return VGGT_ATTN_ERANGE;
    if (!aligned(o.cache, 256)) return VGGT_ATTN_EALIGN;
    if (o.cache_bytes < plan->desc.total) return VGGT_ATTN_EWORKSPACE;
  }
  if (!aligned(X, 16) || !aligned(Y, 16) || !aligned(Wqkv, 16) || !aligned(Wo, 16) ||
      !aligned(qg, 4) || !aligned(qb, 4) || !aligned(kg, 4) || !aligned(kb, 4) || !aligned(ws, 256))
    return VGGT_ATTN_EALIGN;
  if (ws_bytes < plan->total) return VGGT_ATTN_EWORKSPACE;
  const size_t nx = (size_t)plan->S * plan->T * plan->d * 2;
  const size_t ny = plan->window ? (size_t)(plan->L - plan->q0) * plan->d * 2 : nx;
  const size_t nw = (size_t)3 * plan->d * plan->d * 2, no = (size_t)plan->d * plan->d * 2;
  const size_t ng = (size_t)plan->H * kDh * 4;
  const bool in_place = (mode == VGGT_ATTN_MODE_REGISTER && Y == X);
  if (!in_place && overlap(Y, ny, X, nx)) return VGGT_ATTN_EINVAL;
  if (overlap(Y, ny, Wqkv, nw) || overlap(Y, ny, Wo, no) || overlap(Y, ny, qg, ng) ||
      overlap(Y, ny, qb, ng) || overlap(Y, ny, kg, ng) || overlap(Y, ny, kb, ng) ||
      overlap(Y, ny, ws, plan->total))
    return VGGT_ATTN_EINVAL;
  if (desc && (overlap(Y, ny, o.cache, plan->desc.total) ||
               overlap(ws, plan->total, o.cache, plan->desc.total)))
    return VGGT_ATTN_EINVAL;
  // The workspace is written by the library: it must not hold any input.
  if (overlap(ws, plan->total, X, nx) || overlap(ws, plan->total, Wqkv, nw) ||
      overlap(ws, plan->total, Wo, no) || overlap(ws, plan->total, qg, ng) ||
      overlap(ws, plan->total, qb, ng) || overlap(ws, plan->total, kg, ng) ||
      overlap(ws, plan->total, kb, ng))
    return VGGT_ATTN_EINVAL;
  return VGGT_ATTN_OK;
}

int run(int mode, const CallOpts& o, int first_stage, int last_stage,
        const vggt_attn_shape* shape, const void* X, const void* Wqkv, const void* Wo,
        const float* qg, const float* qb, const float* kg, const float* kb, void* Y, void* ws,
        size_t ws_bytes, void* stream) {
  Plan plan;
  int st = check_call(mode, shape, o, X, Wqkv, Wo, qg, qb, kg, kb, Y, ws, ws_bytes, &plan);
  if (st != VGGT_ATTN_OK) return st;
  Ptrs a{reinterpret_cast<const bf16*>(X), reinterpret_cast<const bf16*>(Wqkv),
         reinterpret_cast<const bf16*>(Wo), qg, qb, kg, kb, reinterpret_cast<bf16*>(Y),
         reinterpret_cast<char*>(ws), reinterpret_cast<char*>(const_cast<void*>(o.cache))};
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  for (int stage = first_stage; stage <= last_stage; ++stage) {
    hipError_t e = hipSuccess;
    switch (stage) {
      case VGGT_ATTN_STAGE_PREP: e = launch_prep(plan, a, hs); break;
      case VGGT_ATTN_STAGE_QKV: e = launch_qkv(plan, a, hs); break;
      case VGGT_ATTN_STAGE_CORE:
        if (plan.mode == VGGT_ATTN_MODE_SUBSAMPLED) e = launch_subsample(plan, a, hs);
        if (plan.mode == VGGT_ATTN_MODE_MERGED) e = launch_merge(plan, a, hs);
        if (e == hipSuccess) e = launch_core(plan, a, hs);
        if (e == hipSuccess && plan.mode == VGGT_ATTN_MODE_MERGED) e = launch_unmerge(plan, a, hs);
        break;
      case VGGT_ATTN_STAGE_OUT: e = launch_out(plan, a, hs); break;
    }
    if (e != hipSuccess) return VGGT_ATTN_EHIP;
  }
  return VGGT_ATTN_OK;
}

int check_residual(const void* X, const void* Y, const void* Z, int64_t rows, int d,
                   const float* gamma, int period, int active, const void* C, int64_t c_stride) {
  if (!X || !Y || !Z || !gamma) return VGGT_ATTN_EINVAL;
  if (rows < 0 || d < 8 || d % 8 != 0 || period < 1 || active < 0) return VGGT_ATTN_ESHAPE;
  if (C && (c_stride < d || c_stride % 8 != 0)) return VGGT_ATTN_ESHAPE;
  if (!aligned(X, 16) || !aligned(Y, 16) || !aligned(Z, 16) || !aligned(gamma, 16) ||
      (C && !aligned(C, 16)))
    return VGGT_ATTN_EALIGN;
  const size_t n = (size_t)rows * d * 2, ng = (size_t)d * 4;
  // Z may be X itself; no other overlap between the buffers
  if (overlap(Z, n, Y, n) || overlap(Z, n, gamma, ng) || (Z != X && overlap(Z, n, X, n)))
    return VGGT_ATTN_EINVAL;
  if (C) {
    const size_t nc = rows ? ((size_t)(rows - 1) * c_stride + d) * 2 : 0;
    if (overlap(C, nc, X, n) || overlap(C, nc, Y, n) || overlap(C, nc, Z, n) ||
        overlap(C, nc, gamma, ng))
      return VGGT_ATTN_EINVAL;
  }
  return VGGT_ATTN_OK;
}

}  // namespace vggt

using namespace vggt;

extern "C" {

size_t vggt_attn_workspace_bytes(int mode, const vggt_attn_shape* shape) {
  Plan plan;
  if (make_plan(mode, shape, CallOpts(), &plan) != VGGT_ATTN_OK) return 0;
  return plan.total;
}

#define VGGT_ARGS                                                                          \
  const vggt_attn_shape *shape, const void *X, const void *Wqkv, const void *Wo,            \
      const float *q_gamma, const float *q_beta, const float *k_gamma, const float *k_beta, \
      void *Y, void *workspace, size_t workspace_bytes, void *stream
#define VGGT_PASS \
  shape, X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y, workspace, workspace_bytes, stream

int vggt_attn_frame(VGGT_ARGS) {
  return run(VGGT_ATTN_MODE_FRAME, CallOpts(), VGGT_ATTN_STAGE_PREP, VGGT_ATTN_STAGE_OUT, VGGT_PASS);
}

int vggt_attn_global(VGGT_ARGS) {
  return run(VGGT_ATTN_MODE_GLOBAL, CallOpts(), VGGT_ATTN_STAGE_PREP, VGGT_ATTN_STAGE_OUT, VGGT_PASS);
}

int vggt_attn_global_register(VGGT_ARGS) {
  return run(VGGT_ATTN_MODE_REGISTER, CallOpts(), VGGT_ATTN_STAGE_PREP, VGGT_ATTN_STAGE_OUT, VGGT_PASS);
}

int vggt_attn_bf16ops(int mode, int stage, VGGT_ARGS) {
  if (mode != VGGT_ATTN_MODE_FRAME && mode != VGGT_ATTN_MODE_GLOBAL &&
      mode != VGGT_ATTN_MODE_REGISTER)
    return VGGT_ATTN_EINVAL;
  if (stage != VGGT_ATTN_STAGE_ALL && (stage < VGGT_ATTN_STAGE_PREP || stage > VGGT_ATTN_STAGE_OUT))
    return VGGT_ATTN_EINVAL;
  CallOpts o;
  o.bf16_ops = true;
  if (stage == VGGT_ATTN_STAGE_ALL) return run(mode, o, VGGT_ATTN_STAGE_PREP, VGGT_ATTN_STAGE_OUT, VGGT_PASS);
  return run(mode, o, stage, stage, VGGT_PASS);
}

int vggt_attn_stage(int mode, int stage, VGGT_ARGS) {
  if (stage < VGGT_ATTN_STAGE_PREP || stage > VGGT_ATTN_STAGE_OUT) return VGGT_ATTN_EINVAL;
  // these modes need windows / a cache / blocks: they have stage entries of their own
  if (mode == VGGT_ATTN_MODE_SUBSAMPLED || mode == VGGT_ATTN_MODE_DESCRIPTOR ||
      mode == VGGT_ATTN_MODE_MERGED)
    return VGGT_ATTN_EINVAL;
  return run(mode, CallOpts(), stage, stage, VGGT_PASS);
}

int vggt_attn_global_subsampled(const vggt_attn_shape* shape, int32_t sub_h, int32_t sub_w,
                                const void* X, const void* Wqkv, const void* Wo,
                                const float* q_gamma, const float* q_beta,
                                const float* k_gamma, const float* k_beta, void* Y,
                                void* workspace, size_t workspace_bytes, void* stream) {
  CallOpts o;
  o.sub_h = sub_h;
  o.sub_w = sub_w;
  return run(VGGT_ATTN_MODE_SUBSAMPLED, o, VGGT_ATTN_STAGE_PREP, VGGT_ATTN_STAGE_OUT, VGGT_PASS);
}

int vggt_attn_subsampled_stage(int stage, const vggt_attn_shape* shape, int32_t sub_h,
                               int32_t sub_w, const void* X, const void* Wqkv, const void* Wo,
                               const float* q_gamma, const float* q_beta, const float* k_gamma,
                               const float* k_beta, void* Y, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (stage < VGGT_ATTN_STAGE_PREP || stage > VGGT_ATTN_STAGE_OUT) return VGGT_ATTN_EINVAL;
  CallOpts o;
  o.sub_h = sub_h;
  o.sub_w = sub_w;
  return run(VGGT_ATTN_MODE_SUBSAMPLED, o, stage, stage, VGGT_PASS);
}

static CallOpts merged_opts(int32_t frames, int32_t win_h, int32_t win_w, int32_t r) {
  CallOpts o;
  // 0 frames would mean "sizing only" to the planner: a call passes >= 1
  o.httm_frames = frames < 1 ? -1 : frames;
  o.httm_wh = win_h;
  o.httm_ww = win_w;
  o.httm_r = r;
  return o;
}

int vggt_attn_global_merged(const vggt_attn_shape* shape, int32_t frames, int32_t win_h,
                            int32_t win_w, int32_t r, const void* X, const void* Wqkv,
                            const void* Wo, const float* q_gamma, const float* q_beta,
                            const float* k_gamma, const float* k_beta, void* Y, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return run(VGGT_ATTN_MODE_MERGED, merged_opts(frames, win_h, win_w, r), VGGT_ATTN_STAGE_PREP,
             VGGT_ATTN_STAGE_OUT, VGGT_PASS);
}

int vggt_attn_merged_stage(int stage, const vggt_attn_shape* shape, int32_t frames, int32_t win_h,
                           int32_t win_w, int32_t r, const void* X, const void* Wqkv,
                           const void* Wo, const float* q_gamma, const float* q_beta,
                           const float* k_gamma, const float* k_beta, void* Y, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (stage < VGGT_ATTN_STAGE_PREP || stage > VGGT_ATTN_STAGE_OUT) return VGGT_ATTN_EINVAL;
  return run(VGGT_ATTN_MODE_MERGED, merged_opts(frames, win_h, win_w, r), stage, stage, VGGT_PASS);
}

int vggt_attn_global_rows(const vggt_attn_shape* shape, int64_t row_begin, int64_t row_count,
                          const void* X, const void* Wqkv, const void* Wo, const float* q_gamma,
                          const float* q_beta, const float* k_gamma, const float* k_beta,
                          void* Y_rows, void* workspace, size_t workspace_bytes, void* stream) {
  CallOpts o;
  o.q_begin = row_begin;
  o.q_count = row_count < 0 ? 0 : row_count;  // negative counts are out of range, not "all"
  void* Y = Y_rows;
  return run(VGGT_ATTN_MODE_GLOBAL, o, VGGT_ATTN_STAGE_PREP, VGGT_ATTN_STAGE_OUT, VGGT_PASS);
}

int vggt_attn_global_rows_stage(int stage, const vggt_attn_shape* shape, int64_t row_begin,
                                int64_t row_count, const void* X, const void* Wqkv, const void* Wo,
                                const float* q_gamma, const float* q_beta, const float* k_gamma,
                                const float* k_beta, void* Y_rows, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (stage < VGGT_ATTN_STAGE_PREP || stage > VGGT_ATTN_STAGE_OUT) return VGGT_ATTN_EINVAL;
  CallOpts o;
  o.q_begin = row_begin;
  o.q_count = row_count < 0 ? 0 : row_count;
  void* Y = Y_rows;
  return run(VGGT_ATTN_MODE_GLOBAL, o, stage, stage, VGGT_PASS);
}

int vggt_attn_residual(const void* X, const void* Y, void* Z, int64_t rows, int32_t d,
                       const float* gamma, int32_t period, int32_t active, void* C,
                       int64_t c_stride, void* stream) {
  const int st = check_residual(X, Y, Z, rows, d, gamma, period, active, C, c_stride);
  if (st != VGGT_ATTN_OK || rows == 0) return st;
  hipError_t e = launch_residual(reinterpret_cast<const bf16*>(X), reinterpret_cast<const bf16*>(Y),
                                 reinterpret_cast<bf16*>(Z), rows, d, gamma, period, active,
                                 reinterpret_cast<bf16*>(C), c_stride,
                                 reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VGGT_ATTN_OK : VGGT_ATTN_EHIP;
}

size_t vggt_attn_desc_cache_bytes(const vggt_attn_shape* shape, int64_t capacity) {
  Plan plan;
  CallOpts o;
  o.desc_capacity = capacity;
  if (capacity < 1 || make_plan(VGGT_ATTN_MODE_DESCRIPTOR, shape, o, &plan) != VGGT_ATTN_OK)
    return 0;
  return plan.desc.total;
}

int vggt_attn_desc_cache_init(const vggt_attn_shape* shape, int64_t capacity, void* cache,
                              size_t cache_bytes, void* stream) {
  Plan plan;
  CallOpts o;
  o.desc_capacity = capacity;
  int st = make_plan(VGGT_ATTN_MODE_DESCRIPTOR, shape, o, &plan);
  if (st != VGGT_ATTN_OK) return st;
  if (capacity < 1) return VGGT_ATTN_ERANGE;
  if (!cache) return VGGT_ATTN_EINVAL;
  if (!aligned(cache, 256)) return VGGT_ATTN_EALIGN;
  if (cache_bytes < plan.desc.total) return VGGT_ATTN_EWORKSPACE;
  hipError_t e = launch_desc_init(reinterpret_cast<char*>(cache), plan.desc, plan.H,
                                  reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VGGT_ATTN_OK : VGGT_ATTN_EHIP;
}

int vggt_attn_desc_append(const vggt_attn_shape* shape, int64_t capacity, int64_t count,
                          const void* D, int64_t m, const void* Wqkv, const float* k_gamma,
                          const float* k_beta, void* cache, size_t cache_bytes, void* stream) {
  Plan plan;
  CallOpts o;
  o.desc_capacity = capacity;
  int st = make_plan(VGGT_ATTN_MODE_DESCRIPTOR, shape, o, &plan);
  if (st != VGGT_ATTN_OK) return st;
  if (capacity < 1 || count < 0 || m < 1 || count > capacity - m) return VGGT_ATTN_ERANGE;
  if (!D || !Wqkv || !k_gamma || !k_beta || !cache) return VGGT_ATTN_EINVAL;
  if (!aligned(D, 16) || !aligned(Wqkv, 16) || !aligned(k_gamma, 4) || !aligned(k_beta, 4) ||
      !aligned(cache, 256))
    return VGGT_ATTN_EALIGN;
  if (cache_bytes < plan.desc.total) return VGGT_ATTN_EWORKSPACE;
  const size_t nc = plan.desc.total, nd = (size_t)m * plan.d * 2;
  const size_t nw = (size_t)3 * plan.d * plan.d * 2, ng = (size_t)plan.H * kDh * 4;
  if (overlap(cache, nc, D, nd) || overlap(cache, nc, Wqkv, nw) ||
      overlap(cache, nc, k_gamma, ng) || overlap(cache, nc, k_beta, ng))
    return VGGT_ATTN_EINVAL;
  hipError_t e = launch_desc_append(reinterpret_cast<char*>(cache), plan.desc, plan.H, plan.d,
                                    plan.eps, count, reinterpret_cast<const bf16*>(D), m,
                                    reinterpret_cast<const bf16*>(Wqkv), k_gamma, k_beta,
                                    reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? VGGT_ATTN_OK : VGGT_ATTN_EHIP;
}

#define VGGT_DESC_ARGS                                                                      \
  const vggt_attn_shape *shape, int64_t capacity, int64_t count, const void *cache,         \
      size_t cache_bytes, const void *X, const void *Wqkv, const void *Wo,                  \
      const float *q_gamma, const float *q_beta, void *Y, void *workspace,                  \
      size_t workspace_bytes, void *stream

static CallOpts desc_opts(int64_t capacity, int64_t count, const void* cache, size_t cache_bytes) {
  CallOpts o;
  o.cache = cache;
  o.cache_bytes = cache_bytes;
  o.desc_capacity = capacity;
  o.desc_count = count;
  return o;
}

int vggt_attn_desc_attend(VGGT_DESC_ARGS) {
  return run(VGGT_ATTN_MODE_DESCRIPTOR, desc_opts(capacity, count, cache, cache_bytes),
             VGGT_ATTN_STAGE_PREP, VGGT_ATTN_STAGE_OUT, shape, X, Wqkv, Wo, q_gamma, q_beta,
             nullptr, nullptr, Y, workspace, workspace_bytes, stream);
}

int vggt_attn_desc_attend_stage(int stage, VGGT_DESC_ARGS) {
  if (stage < VGGT_ATTN_STAGE_PREP || stage > VGGT_ATTN_STAGE_OUT) return VGGT_ATTN_EINVAL;
  return run(VGGT_ATTN_MODE_DESCRIPTOR, desc_opts(capacity, count, cache, cache_bytes), stage,
             stage, shape, X, Wqkv, Wo, q_gamma, q_beta, nullptr, nullptr, Y, workspace,
             workspace_bytes, stream);
}

const char* vggt_attn_status_str(int status) {
  switch (status) {
    case VGGT_ATTN_OK: return "ok";
    case VGGT_ATTN_EINVAL: return "invalid argument (null pointer, unknown mode or stage, or forbidden aliasing)";
    case VGGT_ATTN_ESHAPE: return "unsupported shape (need Dh = 64, d % 128 == 0, T = 17 + grid_h*grid_w, S*T < 2^31)";
    case VGGT_ATTN_EALIGN: return "misaligned pointer (tensors 16 B, gamma/beta 4 B, workspace 256 B)";
    case VGGT_ATTN_EWORKSPACE: return "workspace smaller than vggt_attn_workspace_bytes()";
    case VGGT_ATTN_EHIP: return "HIP runtime error while enqueueing a kernel";
    case VGGT_ATTN_ERANGE:
      return "value out of range: rope_base / ln_eps must be finite and > 0, pos_offset in "
             "0..65535, sub_h / sub_w >= 1, row window inside the set; or (range status) a "
             "non-finite input or a bound beyond fp16 range";
    case VGGT_ATTN_ESCRATCH:
      return "the call needs more workspace than the static scratch of vggt_attn_block_noalloc "
             "(VGGT_ATTN_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int vggt_attn_range_status(const void* workspace, uint32_t* bits, void* stream) {
  if (!workspace || !aligned(workspace, 256)) return VGGT_ATTN_EINVAL;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  uint32_t word = 0;
  if (hipMemcpyAsync(&word, reinterpret_cast<const char*>(workspace) + VGGT_ATTN_STATUS_OFFSET,
                     sizeof(word), hipMemcpyDeviceToHost, hs) != hipSuccess ||
      hipStreamSynchronize(hs) != hipSuccess)
    return VGGT_ATTN_EHIP;
  if (bits) *bits = word;
  return word ? VGGT_ATTN_ERANGE : VGGT_ATTN_OK;
}

int vggt_attn_version(void) { return 10200; }

}  // extern "C"
