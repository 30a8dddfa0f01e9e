// Projection GEMMs of the attention block on gfx950 MFMA, with fused epilogues.
//
//   QKV: [q|k|v] = x Wqkv^T for every workspace row (bf16 x bf16 -> fp32),
//        then per (token, head): LayerNorm of q and k over the 64 features
//        with the per-head gamma/beta, 2D RoPE on patch tokens, q scaled by
//        log2(e)/sqrt(64) (the attention kernel works in base 2), fp16 store.
//        v is scaled by an exact power of two (range guard) and stored
//        transposed, key-major, for the attention kernel.
//   OUT: Y = O Wo^T (fp16 x fp16 -> fp32), exact power-of-two un-scaling,
//        bf16 store scattered to the X-row of every workspace row.
//
// Tile: 128 token rows x 128 output features x 64-deep k-steps, 4 waves, each
// wave a 64 x 64 block = one head for 64 tokens, so the LayerNorm and the RoPE
// pairs (feature i, i+16) of a (token, head) never leave the wave.  MFMA
// 32x32x16 computes the block transposed (features x tokens): lane l holds
// token l%32 of each 32-token block and features 8*(r/4) + 4*(l/32) + r%4
// (r = 0..15) of each 32-feature block -- 32 of the head's 64 features; the
// other 32 sit in lane l^32, and both RoPE partners (r, r+8) in the lane
// itself.  LDS tiles are 128-byte rows with the 16-byte chunk index XOR-ed with
// row bits 0..2 and bit 3 (conflict-free for 32-row operand reads);
// global->LDS goes through registers, each k-step loaded two k-steps ahead.
#include <stdlib.h>

#include <type_traits>

#include "plan.h"

namespace vggt {

struct GemmArgs {
  const void* A;  // weights [Nf][K], row-major (bf16 for QKV, fp16 for OUT)
  const void* B;  // QKV: X bf16 [S*T][d] through `map`; OUT: O fp16 [H][rows][64]
  int64_t rows;   // workspace rows (multiple of 128)
  int64_t vt_rows;  // QKV: columns of v^T [H][64][vt_rows]
  int vt_seq;       // QKV: 0, or the v^T column stride of a set (frame sets): workspace row
                    // w = s * seq_stride + t has its value at column s * vt_seq + t
  FastDiv dss;      // division by seq_stride (used when vt_seq != 0)
  int vt_sets;      // (vt_seq != 0) sets with a v^T column range: rows past them store no v^T
  int Nf, K;
  int fgroups;    // output-feature groups walked one after the other (divides Nf / 128)
  int64_t m_first;       // first workspace row of the token tiles (a multiple of the tile)
  int64_t q_lo, q_hi;    // QKV: q is needed only for rows [q_lo, q_hi)
  int f_off;             // QKV: feature index (in [q|k|v]) of A's first row
  int64_t dst_off;       // QKV: workspace row w is stored at row w + dst_off
  int real_only;         // QKV: rows without a token write nothing
  int v_rows;            // QKV: store v token-major, [H][rows][64] like q and k (the merged
                         // mode's merge stage reads it so), instead of transposed
  RowMap map;            // QKV: workspace row -> X row; OUT: workspace row -> Y row
  FastDiv dgrp, dT, dgw; // division by map.grp_stride, T and gw
  int T, gw, off, d;
  float eps;
  const float *qg, *qb, *kg, *kb;
  const float2* rope;
  Scalars* sc;
  f16 *q, *k, *vt;
  bf16* y;
};

// RowMap::src in 32-bit arithmetic: every workspace row and token index of a
// call is below 2^31 (checked on the host), so the 64-bit division of the
// generic map becomes one multiply by the precomputed FastDiv.
__device__ __forceinline__ int64_t row_src(const GemmArgs& g, int64_t w64) {
  const RowMap& m = g.map;
  const int v = (int)(w64 - m.base);
  if (v < 0) return -1;
  const int grp = fdiv(v, g.dgrp);
  const int t = v - grp * g.dgrp.d;
  return (t < m.grp_valid && grp < m.ngroups) ? (int64_t)(grp * (int)m.src_stride + t) : -1;
}

// v^T column of workspace row x (below 2^31).  For frame sets also the row's
// place t in its set and the set's padding columns [pad0, pad1): the columns
// past the set's last row up to the next multiple of 64, which no row maps to.
// They hold masked keys of the attention kernel's last tile, whose zero
// probabilities must meet finite values, so the epilogue writes zeros there
// with the set's last rows.  Rows past the last set (the buffer's tail
// padding) get column -1: no v^T store.  Identity (t = -1) for the other sets.
struct VtCol {
  int64_t col, pad0, pad1;
  int t;
};
__device__ __forceinline__ VtCol vt_column(const GemmArgs& g, int64_t x) {
  VtCol c{x, 0, 0, -1};
  if (g.vt_seq == 0) return c;
  const int x32 = (int)x;
  const int s = fdiv(x32, g.dss);
  c.t = x32 - s * g.dss.d;
  const int64_t base = (int64_t)s * g.vt_seq;
  c.col = s < g.vt_sets ? base + c.t : -1;
  c.pad0 = base + g.dss.d;
  c.pad1 = base + g.vt_seq;
  return c;
}

// Grid position of X row `src` for the RoPE of q and k: (row, column) plus the
// position offset for patch tokens, row -1 for the special tokens and for
// workspace rows without a token (no rotation).
__device__ __forceinline__ int2 rope_pos(const GemmArgs& g, int64_t src) {
  int2 pos = make_int2(-1, 0);
  if (src >= 0) {
    const int s32 = (int)src;
    const int t = s32 - fdiv(s32, g.dT) * g.T;
    if (t >= kSpecial) {
      const int pidx = t - kSpecial, r = fdiv(pidx, g.dgw);
      pos = make_int2(r + g.off, pidx - r * g.gw + g.off);
    }
  }
  return pos;
}

// q is pre-multiplied by log2(e)/sqrt(64): the attention kernel uses exp2.
constexpr float kQScale = 0.18033688011112042f;

// LayerNorm of one (token, head) over its 64 features -- this lane's 32 in
// a0 (features 8*(r/4) + 4*h + r%4) and a1 (the same + 32), the other 32 in
// lane l ^ 32 -- then the per-feature affine map (gm / bt, which carry q's
// softmax scale), 2D RoPE for patch tokens (pos.x >= 0: feature i of each
// half pairs with i + 16, registers r and r + 8 of the lane) and fp16
// conversion into o[fb][rq] = features fb*32 + 8*rq + 4*h .. +3.  NORM: also
// the squared L2 norm of the fp16 vector, summed over the lane pair.
template <bool NORM, typename T4>
__device__ __forceinline__ void ln_rope_16(const f32x16& a0, const f32x16& a1,
                                           const float (&gm)[2][16], const float (&bt)[2][16],
                                           float eps, const float2* rope, int2 pos, int h,
                                           T4 (&o)[2][4], float& n2) {
  typedef decltype(T4{}.xy) T2;
  float y[2][16];
  float s1 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s1 += a0[r] + a1[r];
  const float mean = add_xor32(s1) * (1.f / kDh);
  float s2 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    y[0][r] = a0[r] - mean;
    y[1][r] = a1[r] - mean;
    s2 = fmaf(y[0][r], y[0][r], s2);
    s2 = fmaf(y[1][r], y[1][r], s2);
  }
  const float var = add_xor32(s2) * (1.f / kDh);
  const float rstd = __builtin_amdgcn_rsqf(var + eps);
#pragma unroll
  for (int fb = 0; fb < 2; ++fb)
#pragma unroll
    for (int r = 0; r < 16; ++r) y[fb][r] = fmaf(y[fb][r] * rstd, gm[fb][r], bt[fb][r]);
  if (pos.x >= 0) {
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) {
      const float2* cs_row = rope + (fb == 0 ? pos.x : pos.y) * 16;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float2 cs = cs_row[8 * (r >> 2) + 4 * h + (r & 3)];
        const float a = y[fb][r], b = y[fb][r + 8];
        y[fb][r] = a * cs.x - b * cs.y;
        y[fb][r + 8] = b * cs.x + a * cs.y;
      }
    }
  }
  n2 = 0.f;
#pragma unroll
  for (int fb = 0; fb < 2; ++fb)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const f32x4 v = {y[fb][4 * rq], y[fb][4 * rq + 1], y[fb][4 * rq + 2], y[fb][4 * rq + 3]};
      o[fb][rq] = __builtin_convertvector(v, T4);
      if (NORM) {
        const T2 lo = {o[fb][rq][0], o[fb][rq][1]}, hi = {o[fb][rq][2], o[fb][rq][3]};
        n2 = dot2_acc(lo, lo, n2);
        n2 = dot2_acc(hi, hi, n2);
      }
    }
  if (NORM) n2 = add_xor32(n2);
}

// gamma / beta of the wave's head in the lane's feature order, times the
// output scale.
__device__ __forceinline__ void load_affine(const float* gam, const float* bet, float scale,
                                            int h, float (&gm)[2][16], float (&bt)[2][16]) {
#pragma unroll
  for (int fb = 0; fb < 2; ++fb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int f = fb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      gm[fb][r] = gam[f] * scale;
      bt[fb][r] = bet[f] * scale;
    }
}

// v of one (token, head) in the lane's feature order (as ln_rope_16 leaves
// q and k), times the range scale vs, to the operand type.
template <typename T4>
__device__ __forceinline__ void v_rows_16(const f32x16& a0, const f32x16& a1, float vs,
                                          T4 (&o)[2][4]) {
#pragma unroll
  for (int rq = 0; rq < 4; ++rq) {
    const f32x4 v0 = {a0[4 * rq] * vs, a0[4 * rq + 1] * vs, a0[4 * rq + 2] * vs, a0[4 * rq + 3] * vs};
    const f32x4 v1 = {a1[4 * rq] * vs, a1[4 * rq + 1] * vs, a1[4 * rq + 2] * vs, a1[4 * rq + 3] * vs};
    o[0][rq] = __builtin_convertvector(v0, T4);
    o[1][rq] = __builtin_convertvector(v1, T4);
  }
}

// Epilogues: the QKV projection and the output projection, each for fp16
// (default) or bf16 (the bf16-operand variant) attention operands: q, k and
// v stored in that type, the output projection's O and Wo read in it.
enum { kEpiQKV = 0, kEpiOut = 1, kEpiQKVB = 2, kEpiOutB = 3 };
constexpr bool epi_qkv(int e) { return e == kEpiQKV || e == kEpiQKVB; }
constexpr bool epi_b16(int e) { return e == kEpiQKVB || e == kEpiOutB; }

template <int EPI>
struct GemmTypes {
  // MFMA operands: X and Wqkv are bf16; O and Wo are the attention operand type
  typedef typename std::conditional<epi_qkv(EPI) || epi_b16(EPI), bf16x8, f16x8>::type V8;
  typedef Ops16<epi_b16(EPI)> Out;  // QKV: the stored q, k, v
};

__device__ __forceinline__ int swz(int row, int col) {
  return row * 128 + ((col ^ (row & 7) ^ ((row >> 3) & 1)) << 4);
}

// Epilogue of one wave's block: acc[fb][tb][r] holds feature
// fbase + fb*32 + fo(r) of token (workspace row) mbase + tb*32 + j, with
// fo(r) = 8*(r/4) + 4*h + r%4; the 64 features are one head (fb = 0 its first
// half).
template <int EPI, int TB>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, f32x16 (&acc)[2][TB],
                                              int64_t mbase, int fbase, int j, int h, int lane) {
  typedef typename GemmTypes<EPI>::Out::T OT;
  typedef typename GemmTypes<EPI>::Out::T2 OT2;
  typedef typename GemmTypes<EPI>::Out::T4 OT4;
  if (epi_qkv(EPI)) {
    const int fq = fbase + g.f_off;
    const int blk = fq / g.d;  // 0: q, 1: k, 2: v
    const int hd = (fq - blk * g.d) / kDh;
    if (blk < 2) {
      float gm[2][16], bt[2][16];
      load_affine((blk == 0 ? g.qg : g.kg) + hd * kDh, (blk == 0 ? g.qb : g.kb) + hd * kDh,
                  blk == 0 ? kQScale : 1.f, h, gm, bt);
      OT* dst = reinterpret_cast<OT*>(blk == 0 ? g.q : g.k) + (int64_t)hd * g.rows * kDh;
      auto block = [&](auto norm_c) {
        constexpr bool NORM = decltype(norm_c)::value;
        float kmx = 0.f;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const int64_t w = mbase + tb * 32 + j;
          const int64_t src = row_src(g, w);
          OT4 o[2][4];
          float n2;
          ln_rope_16<NORM>(acc[0][tb], acc[1][tb], gm, bt, g.eps, g.rope, rope_pos(g, src), h, o,
                           n2);
          if (!g.real_only || src >= 0) {
#pragma unroll
            for (int fb = 0; fb < 2; ++fb)
#pragma unroll
              for (int rq = 0; rq < 4; ++rq)
                *reinterpret_cast<OT4*>(dst + (w + g.dst_off) * kDh + fb * 32 + 8 * rq + 4 * h) =
                    o[fb][rq];
          }
          if (NORM && src >= 0) kmx = fmaxf(kmx, sqrtf(n2));
        }
        if (NORM) {
#pragma unroll
          for (int sh = 1; sh < 32; sh <<= 1) kmx = fmaxf(kmx, __shfl_xor(kmx, sh));
          if (lane == 0 && kmx > 0.f) atomic_max_nonneg(&g.sc->kmax[hd], kmx);
        }
      };
      if (blk == 1) {
        block(std::true_type());
      } else {
        block(std::false_type());
      }
    } else if (g.v_rows) {
      const float vs = __builtin_amdgcn_ldexpf(1.f, range_exponent(g.sc->xnorm * g.sc->wvnorm));
      OT* dst = reinterpret_cast<OT*>(g.vt) + (int64_t)hd * g.rows * kDh;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int64_t w = mbase + tb * 32 + j;
        OT4 o[2][4];
        v_rows_16(acc[0][tb], acc[1][tb], vs, o);
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
            *reinterpret_cast<OT4*>(dst + (w + g.dst_off) * kDh + fb * 32 + 8 * rq + 4 * h) =
                o[fb][rq];
      }
    } else {
      const int kv = range_exponent(g.sc->xnorm * g.sc->wvnorm);
      OT* dst = reinterpret_cast<OT*>(g.vt) + (int64_t)hd * kDh * g.vt_rows;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int64_t w = mbase + tb * 32 + j;
        if (g.real_only && row_src(g, w) < 0) continue;
        const VtCol vc = vt_column(g, w + g.dst_off);
        if (vc.col < 0) continue;
        const int64_t x = vc.col;
        // Key position inside its aligned group of 16: key 8a + 4c + b is
        // stored at 8c + 4a + b (bits 2 and 3 swapped), the order in which
        // the attention kernel's MFMA consumes probabilities.
        const int64_t pos = (x & ~(int64_t)15) | (((x >> 2) & 1) << 3) | (((x >> 3) & 1) << 2) | (x & 3);
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int e = fb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            dst[(int64_t)e * g.vt_rows + pos] = (OT)ldexpf(acc[fb][tb][r], kv);
          }
      }
      // A set's last row in this wave's rows: the whole wave zeroes the set's
      // padding columns of the 64 features, 16 bytes a lane (whole aligned
      // 16-groups, so the key order inside them is moot).  A 32-row block
      // holds at most one set end (sets have at least 32 rows).
      if (g.vt_seq != 0) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const int64_t w = mbase + tb * 32 + j;
          const VtCol vc = vt_column(g, w + g.dst_off);
          const uint64_t ends = __ballot(vc.col >= 0 && vc.t == g.dss.d - 1 &&
                                         !(g.real_only && row_src(g, w) < 0));
          if (ends == 0) continue;
          const int src = __builtin_ctzll(ends);
          const int64_t pad0 = __shfl(vc.pad0, src), pad1 = __shfl(vc.pad1, src);
          const int chunks = (int)((pad1 - pad0) >> 3);  // 16-byte chunks per feature row
          for (int i = lane; i < kDh * chunks; i += 64) {
            const int e = i / chunks, c = i - e * chunks;
            *reinterpret_cast<u32x4*>(dst + (int64_t)e * g.vt_rows + pad0 + c * 8) =
                u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
    }
  } else {
    const int kv = range_exponent(g.sc->xnorm * g.sc->wvnorm);
    const int ws = range_exponent(g.sc->woabs);
    const float scale = ldexpf(1.f, -(kv + ws));
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int64_t w = mbase + tb * 32 + j;
      const int64_t src = row_src(g, w);
      if (src < 0) continue;
      bf16* dst = g.y + src * g.d + fbase + 4 * h;
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          bf16x4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = (bf16)(acc[fb][tb][4 * rq + r] * scale);
          *reinterpret_cast<bf16x4*>(dst + fb * 32 + 8 * rq) = o;
        }
    }
  }
}

// Epilogue of the 256 x 256 kernel, staged through LDS: each wave first
// writes its finished 128-token x 64-feature block into its own 16 KB of the
// (by then idle) operand buffers, then stores it with 16-byte lanes along
// whole 128-byte rows -- q / k / O rows token-major, v^T feature-major --
// instead of the 8- and 2-byte scattered stores of gemm_epilogue, whose
// instruction count dominated the epilogue.  Token-major rows are swizzled
// by chunk ^ (token & 7), feature-major rows by chunk ^ (4 * bit 2 of the
// feature), which keeps both the writes and the reads free of bank conflicts.
// The descriptor append path (rows without a token must not be stored, keys
// not aligned to 16) keeps the direct stores for v^T.
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
}

template <int EPI>
__device__ __forceinline__ void gemm_epilogue_staged(const GemmArgs& g, f32x16 (&acc)[2][4],
                                                     int64_t mbase, int fbase, int j, int h,
                                                     int lane, char* lds) {
  constexpr int TB = 4;
  typedef typename GemmTypes<EPI>::Out::T OT;
  typedef typename GemmTypes<EPI>::Out::T2 OT2;
  typedef typename GemmTypes<EPI>::Out::T4 OT4;
  if (epi_qkv(EPI)) {
    const int fq = fbase + g.f_off;
    const int blk = fq / g.d;  // 0: q, 1: k, 2: v
    const int hd = (fq - blk * g.d) / kDh;
    if (blk == 2 && !g.v_rows && (g.real_only || (g.dst_off & 15) != 0)) {
      gemm_epilogue<EPI, TB>(g, acc, mbase, fbase, j, h, lane);
      return;
    }
    if (blk == 2 && g.v_rows) {
      // v token-major: the rows of q / k without LayerNorm and RoPE, scaled
      const float vs = __builtin_amdgcn_ldexpf(1.f, range_exponent(g.sc->xnorm * g.sc->wvnorm));
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int tl = tb * 32 + j;
        OT4 o[2][4];
        v_rows_16(acc[0][tb], acc[1][tb], vs, o);
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
            *reinterpret_cast<OT4*>(lds + tl * 128 + (((fb * 4 + rq) ^ (tl & 7)) << 4) + h * 8) =
                o[fb][rq];
      }
      lds_wave_sync();
      f16* dst = g.vt + (int64_t)hd * g.rows * kDh;
#pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int q = it * 64 + lane, tl = q >> 3, c = q & 7;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + tl * 128 + ((c ^ (tl & 7)) << 4));
        *reinterpret_cast<u32x4*>(dst + (mbase + tl + g.dst_off) * kDh + c * 8) = v;
      }
      return;
    }
    if (blk < 2) {
      float gm[2][16], bt[2][16];
      load_affine((blk == 0 ? g.qg : g.kg) + hd * kDh, (blk == 0 ? g.qb : g.kb) + hd * kDh,
                  blk == 0 ? kQScale : 1.f, h, gm, bt);
      // keys also record the largest norm of the stored vectors (the
      // attention kernel's logit bound); queries skip it
      auto block = [&](auto norm_c) {
        constexpr bool NORM = decltype(norm_c)::value;
        float kmx = 0.f;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const int tl = tb * 32 + j;
          const int64_t src = row_src(g, mbase + tl);
          OT4 o[2][4];
          float n2;
          ln_rope_16<NORM>(acc[0][tb], acc[1][tb], gm, bt, g.eps, g.rope, rope_pos(g, src), h, o,
                           n2);
          // features fb*32 + 8*rq + 4*h .. +3: 16-byte chunk fb*4 + rq, half h
#pragma unroll
          for (int fb = 0; fb < 2; ++fb)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq)
              *reinterpret_cast<OT4*>(lds + tl * 128 + (((fb * 4 + rq) ^ (tl & 7)) << 4) + h * 8) =
                  o[fb][rq];
          if (NORM && src >= 0) kmx = fmaxf(kmx, sqrtf(n2));
        }
        if (NORM) {
#pragma unroll
          for (int sh = 1; sh < 32; sh <<= 1) kmx = fmaxf(kmx, __shfl_xor(kmx, sh));
          if (lane == 0 && kmx > 0.f) atomic_max_nonneg(&g.sc->kmax[hd], kmx);
        }
      };
      if (blk == 1) {
        block(std::true_type());
      } else {
        block(std::false_type());
      }
      lds_wave_sync();
      OT* dst = reinterpret_cast<OT*>(blk == 0 ? g.q : g.k) + (int64_t)hd * g.rows * kDh;
#pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int q = it * 64 + lane, tl = q >> 3, c = q & 7;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + tl * 128 + ((c ^ (tl & 7)) << 4));
        const int64_t w = mbase + tl;
        if (!g.real_only || row_src(g, w) >= 0)
          *reinterpret_cast<u32x4*>(dst + (w + g.dst_off) * kDh + c * 8) = v;
      }
    } else {
      // 2^kv exactly: scaling by it and rounding to fp16 rounds once, as ldexp would
      const float vs = __builtin_amdgcn_ldexpf(1.f, range_exponent(g.sc->xnorm * g.sc->wvnorm));
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int tl = tb * 32 + j;
        // slot of token tl inside its aligned group of 16 (bits 2 and 3 swapped)
        const int slot = (tl & ~15) | (((tl >> 2) & 1) << 3) | (((tl >> 3) & 1) << 2) | (tl & 3);
        // feature e = fb*32 + 8*(r/4) + 4*h + r%4 has bit 2 = h, so the
        // chunk swizzle is the lane's own: one base address per lane
        char* base = lds + 4 * h * 256 + (((slot >> 3) ^ (h << 2)) << 4) + (slot & 7) * 2;
#pragma unroll
        for (int fb = 0; fb < 2; ++fb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const f32x2 v = {acc[fb][tb][r] * vs, acc[fb][tb][r + 1] * vs};
            const OT2 o = __builtin_convertvector(v, OT2);
            const int e0 = fb * 32 + 8 * (r >> 2) + (r & 3);  // feature minus 4*h
            *reinterpret_cast<OT*>(base + e0 * 256) = o[0];
            *reinterpret_cast<OT*>(base + (e0 + 1) * 256) = o[1];
          }
      }
      lds_wave_sync();
      // lane l stores the 8 keys of chunk c = l % 16 of feature rows l / 16,
      // + 4, ..: one v^T column (and padding choice) per lane
      const VtCol vc = vt_column(g, mbase + g.dst_off + (lane & 15) * 8);
      const bool pad = vc.col >= 0 && vc.t == g.dss.d - 8;  // the set's last chunk of 8 rows
      f16* dst = g.vt + (int64_t)hd * kDh * g.vt_rows;
#pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int q = it * 64 + lane, e = q >> 4, c = q & 15;
        const u32x4 v =
            *reinterpret_cast<const u32x4*>(lds + e * 256 + ((c ^ (((e >> 2) & 1) << 2)) << 4));
        if (vc.col >= 0) *reinterpret_cast<u32x4*>(dst + (int64_t)e * g.vt_rows + vc.col) = v;
        if (pad) {
          for (int64_t z = vc.pad0; z < vc.pad1; z += 8)
            *reinterpret_cast<u32x4*>(dst + (int64_t)e * g.vt_rows + z) = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  } else {
    const int kv = range_exponent(g.sc->xnorm * g.sc->wvnorm);
    const int ws = range_exponent(g.sc->woabs);
    const float scale = ldexpf(1.f, -(kv + ws));
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int tl = tb * 32 + j;
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          bf16x4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = (bf16)(acc[fb][tb][4 * rq + r] * scale);
          *reinterpret_cast<bf16x4*>(lds + tl * 128 + (((fb * 4 + rq) ^ (tl & 7)) << 4) + h * 8) = o;
        }
    }
    lds_wave_sync();
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int q = it * 64 + lane, tl = q >> 3, c = q & 7;
      const int64_t src = row_src(g, mbase + tl);
      if (src < 0) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(lds + tl * 128 + ((c ^ (tl & 7)) << 4));
      *reinterpret_cast<u32x4*>(g.y + src * g.d + fbase + c * 8) = v;
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs g) {
  typedef typename GemmTypes<EPI>::V8 V8;
  __shared__ __attribute__((aligned(16))) char smem[2][2][kGemmBM * 128];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int j = lane & 31, h = lane >> 5;

  // Block order.  Blocks go to the 8 XCDs round-robin (block b runs on XCD
  // b % 8).  When the token tiles split evenly, XCD x owns token tiles
  // [x*ntm/8, (x+1)*ntm/8) -- every X (or O) row is fetched from HBM by one
  // XCD only -- and walks them once per group of output features, all token
  // tiles of a group before the next group: the group's slice of the weights
  // (fgroups is picked on the host so that a slice is at most 3 MB) stays in
  // the XCD's L2 while the token tiles stream past, and X is read fgroups
  // times in all.  Otherwise fall back to one contiguous range of (token
  // tile, feature tile) per XCD.
  const int ntn = g.Nf / kGemmBN;
  const int ntm = gridDim.x / ntn;
  int64_t m0;
  int n0;
  if (ntm % kXcds == 0 && ntn % g.fgroups == 0) {
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int ntt = ntm / kXcds, pf = ntn / g.fgroups;
    const int fg = slot / (ntt * pf), rem = slot - fg * ntt * pf;
    m0 = (int64_t)(xcd * ntt + rem / pf) * kGemmBM;
    n0 = (fg * pf + rem % pf) * kGemmBN;
  } else {
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    m0 = (int64_t)(logical / ntn) * kGemmBM;
    n0 = (logical % ntn) * kGemmBN;
  }
  m0 += g.m_first;
  // query rows outside the window need no q (whole workgroup leaves)
  if (epi_qkv(EPI) && n0 + g.f_off < g.d && (m0 + kGemmBM <= g.q_lo || m0 >= g.q_hi)) return;

  const uint16_t* A = reinterpret_cast<const uint16_t*>(g.A) + (int64_t)n0 * g.K;
  const uint16_t* Bbase = reinterpret_cast<const uint16_t*>(g.B);

  // This thread's four A chunks and four B chunks per k-step.
  const uint16_t* aptr[4];
  const uint16_t* bptr[4];
  bool bval[4];
  int soff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, row = c >> 3, col = c & 7;
    soff[i] = swz(row, col);
    aptr[i] = A + (int64_t)row * g.K + col * 8;
    if (epi_qkv(EPI)) {
      const int64_t src = row_src(g, m0 + row);
      bval[i] = src >= 0;
      bptr[i] = Bbase + (bval[i] ? src : 0) * g.K + col * 8;
    } else {
      bval[i] = true;
      bptr[i] = Bbase + (m0 + row) * kDh + col * 8;
    }
  }

  // Global -> LDS staging: two register sets, so each k-step's loads are
  // issued two k-steps before they are stored (the X / O stream comes from
  // HBM; one k-step of MFMAs does not cover its latency).
  u32x4 ra[2][4], rb[2][4];
  auto gload = [&](int kt, u32x4 (&A4)[4], u32x4 (&B4)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) A4[i] = *reinterpret_cast<const u32x4*>(aptr[i] + kt * kGemmBK);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (epi_qkv(EPI)) {
        B4[i] = bval[i] ? *reinterpret_cast<const u32x4*>(bptr[i] + kt * kGemmBK) : u32x4{0, 0, 0, 0};
      } else {
        B4[i] = *reinterpret_cast<const u32x4*>(bptr[i] + (int64_t)kt * g.rows * kDh);
      }
    }
  };
  auto sstore = [&](int buf, const u32x4 (&A4)[4], const u32x4 (&B4)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&smem[buf][0][soff[i]]) = A4[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&smem[buf][1][soff[i]]) = B4[i];
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  auto compute = [&](int buf) {
    const char* As = smem[buf][0];
    const char* Bs = smem[buf][1];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      V8 af[2], bfr[2];
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
        af[fb] = *reinterpret_cast<const V8*>(As + swz(wn * 64 + fb * 32 + j, kc * 2 + h));
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        bfr[tb] = *reinterpret_cast<const V8*>(Bs + swz(wm * 64 + tb * 32 + j, kc * 2 + h));
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[fb][tb] = mfma32x32x16(af[fb], bfr[tb], acc[fb][tb]);
    }
  };

  // nk = K / 64 is even (K is a multiple of 128); the loop is unrolled by two
  // so that the register sets keep static indices.  At the top of step kt,
  // LDS buffer kt&1 holds k-step kt and set (kt+1)&1 has k-step kt+1 in flight.
  const int nk = g.K / kGemmBK;
  gload(0, ra[0], rb[0]);
  gload(1, ra[1], rb[1]);
  sstore(0, ra[0], rb[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    if (kt + 2 < nk) gload(kt + 2, ra[0], rb[0]);
    compute(0);
    sstore(1, ra[1], rb[1]);
    __syncthreads();
    if (kt + 3 < nk) gload(kt + 3, ra[1], rb[1]);
    compute(1);
    if (kt + 2 < nk) sstore(0, ra[0], rb[0]);
    __syncthreads();
  }

  gemm_epilogue<EPI, 2>(g, acc, m0 + wm * 64, n0 + wn * 64, j, h, lane);
}

// ---------------------------------------------------------------------------
// Main kernel: 256 token rows x 128 output features per workgroup, 4 waves of
// 128 x 64 (one head for 128 tokens; 8 MFMA blocks, 0.75 KB of LDS operand
// reads per MFMA instead of 1 KB), 32-deep k-steps, operands copied
// global -> LDS by the load unit itself (global_load_lds, 16 bytes per lane)
// three k-steps deep, so there is no register staging and no ds_write.  LDS
// rows are 64 bytes; chunk c of row r sits at chunk c ^ ((r >> 2) & 3), which
// spreads a 32-row operand read over all 16-byte bank groups.  A DMA
// instruction fills 16 consecutive rows (1 KB), lane i row i/4 and chunk i%4,
// so lane i fetches source chunk (i%4) ^ ((i/16) & 3).
// ---------------------------------------------------------------------------
constexpr int kDmaBM = 256, kDmaBN = 128, kDmaBK = 32, kDmaStages = 3;

__device__ __forceinline__ int swz64(int row, int col) {
  return row * 64 + ((col ^ ((row >> 2) & 3)) << 4);
}

__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_dma_kernel(GemmArgs g) {
  typedef typename GemmTypes<EPI>::V8 V8;
  constexpr int kAB = kDmaBN * 64;  // A stage: 128 feature rows x 64 B
  constexpr int kBB = kDmaBM * 64;  // B stage: 256 token rows x 64 B
  __shared__ __attribute__((aligned(1024))) char smem[kDmaStages][kAB + kBB];
  static_assert(sizeof(smem) >= 4 * 16384, "staged epilogue: 16 KB of LDS per wave");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int j = lane & 31, h = lane >> 5;

  // Block order: as gemm_kernel, with 256-row token tiles.
  const int ntn = g.Nf / kDmaBN;
  const int ntm = gridDim.x / ntn;
  int64_t m0;
  int n0;
  if (ntm % kXcds == 0 && ntn % g.fgroups == 0) {
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int ntt = ntm / kXcds, pf = ntn / g.fgroups;
    const int fg = slot / (ntt * pf), rem = slot - fg * ntt * pf;
    m0 = (int64_t)(xcd * ntt + rem / pf) * kDmaBM;
    n0 = (fg * pf + rem % pf) * kDmaBN;
  } else {
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    m0 = (int64_t)(logical / ntn) * kDmaBM;
    n0 = (logical % ntn) * kDmaBN;
  }
  m0 += g.m_first;
  // query rows outside the window need no q (whole workgroup leaves)
  if (epi_qkv(EPI) && n0 + g.f_off < g.d && (m0 + kDmaBM <= g.q_lo || m0 >= g.q_hi)) return;

  // DMA sources of this lane: A rows (q*4 + wave)*16 + lane/4 (q < 2), B rows
  // likewise (q < 4); column chunk (lane%4) ^ ((lane/16) & 3).
  const int lrow = lane >> 2, lcol = (lane & 3) ^ ((lane >> 4) & 3);
  const uint16_t* A = reinterpret_cast<const uint16_t*>(g.A);
  const uint16_t* Bb = reinterpret_cast<const uint16_t*>(g.B);
  const uint16_t* aptr[2];
  const uint16_t* bptr[4];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    aptr[q] = A + (int64_t)(n0 + (q * 4 + wave) * 16 + lrow) * g.K + lcol * 8;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t w = m0 + (q * 4 + wave) * 16 + lrow;
    if (epi_qkv(EPI)) {
      // rows without a token read X row 0: finite values whose outputs are
      // masked keys or never read
      const int64_t src = row_src(g, w);
      bptr[q] = Bb + (src >= 0 ? src : 0) * g.K + lcol * 8;
    } else {
      bptr[q] = Bb + w * kDh + lcol * 8;
    }
  }
  auto dma = [&](int kt, int stage) {
    char* base = &smem[stage][0];
#pragma unroll
    for (int q = 0; q < 2; ++q) dma16(aptr[q] + kt * kDmaBK, base + (q * 4 + wave) * 1024);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint16_t* src = epi_qkv(EPI)
                                ? bptr[q] + kt * kDmaBK
                                : bptr[q] + (int64_t)(kt >> 1) * g.rows * kDh + (kt & 1) * kDmaBK;
      dma16(src, base + kAB + (q * 4 + wave) * 1024);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  auto compute = [&](int stage) {
    const char* As = &smem[stage][0];
    const char* Bs = As + kAB;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      V8 af[2], bfr[4];
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
        af[fb] = *reinterpret_cast<const V8*>(As + swz64(wn * 64 + fb * 32 + j, kc * 2 + h));
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        bfr[tb] = *reinterpret_cast<const V8*>(Bs + swz64(wm * 128 + tb * 32 + j, kc * 2 + h));
#pragma unroll
      for (int fb = 0; fb < 2; ++fb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[fb][tb] = mfma32x32x16(af[fb], bfr[tb], acc[fb][tb]);
    }
  };

  // Six DMA instructions per wave per k-step.  At the end of step kt, step
  // kt+1 must have landed; step kt+2 may still be in flight (vmcnt <= 6).
  // The barrier is the bare s_barrier: a __syncthreads() would also wait for
  // every outstanding load, in-flight prefetch included.  Reuse is safe: the
  // buffer step kt+2 overwrites was last read in step kt-1, before the
  // barrier that closed it.
  // The waits also cover this wave's LDS reads (lgkmcnt(0)): the compiler may
  // sink the last MFMAs below the barrier, and no read of a stage may still be
  // in flight when another wave starts refilling it.
  constexpr int kVm6 = 0x0076, kVm0 = 0x0070;  // s_waitcnt vmcnt(6|0) lgkmcnt(0)
  const int nk = g.K / kDmaBK;
  dma(0, 0);
  dma(1, 1);
  __builtin_amdgcn_s_waitcnt(kVm6);
  __builtin_amdgcn_s_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 2 < nk;
    if (more) dma(kt + 2, (kt + 2) % kDmaStages);
    compute(kt % kDmaStages);
    if (more) __builtin_amdgcn_s_waitcnt(kVm6);
    else __builtin_amdgcn_s_waitcnt(kVm0);
    __builtin_amdgcn_s_barrier();
  }

  // the loop's last barrier: no wave reads the operand stages any more
  gemm_epilogue_staged<EPI>(g, acc, m0 + wm * 128, n0 + wn * 64, j, h, lane,
                            &smem[0][0] + wave * 16384);
}

// ---------------------------------------------------------------------------
// Wide kernel (output features a multiple of 256): 256 token rows x 256
// output features per workgroup, 8 waves of 128 x 64 (2 x 4), 64-deep
// k-steps; 160 KB of LDS: two 32 KB weight stages and three 32 KB token-row
// stages (token rows copied two k-steps ahead, weights one; measured at the
// s500 frame QKV shape against two stages of both: 3.86 vs 3.91 ms, s100
// QKV 0.77 vs 0.79 ms).  A DMA instruction moves 8 whole
// 128-byte rows (8 cache lines, all bytes used), and the 256 x 256 tile moves
// half the bytes per FLOP of the 256 x 128 one.  LDS rows use the 128-byte
// swizzle chunk ^ (row & 7) ^ ((row >> 3) & 1); lane i of a DMA instruction
// writes row i/8, chunk position i%8, so it fetches source chunk
// (i%8) ^ (i/8) ^ ((R0 >> 3) & 1) for the instruction's first row R0.
// (Measured alternatives at the s500 frame QKV shape: 32-deep k-steps in four
// stages, 4.60 ms; a per-tile rotation of the k order, no change; 4.40 ms
// here.)
// ---------------------------------------------------------------------------
constexpr int kWBM = 256, kWBN = 256, kWBK = 64;

template <int EPI>
__global__ __launch_bounds__(512, 1) void gemm_wide_kernel(GemmArgs g) {
  typedef typename GemmTypes<EPI>::V8 V8;
  constexpr int kAB = kWBN * 128;  // A stage: 256 feature rows x 128 B
  constexpr int kBB = kWBM * 128;  // B stage: 256 token rows x 128 B
  // Two A (weight) stages and three B (token row) stages, 160 KB: the token
  // rows are read from HBM for the first time and are copied two k-steps
  // ahead; the weight slice is L2-resident and is copied one step ahead.
  constexpr int kAStages = 2, kBStages = 3;
  __shared__ __attribute__((aligned(1024))) char smem[kAStages * kAB + kBStages * kBB];
  static_assert(sizeof(smem) >= 8 * 16384, "staged epilogue: 16 KB of LDS per wave");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;  // 2 token halves x 4 feature quarters
  const int j = lane & 31, h = lane >> 5;

  const int ntn = g.Nf / kWBN;
  const int ntm = gridDim.x / ntn;
  int64_t m0;
  int n0;
  if (ntm % kXcds == 0 && ntn % g.fgroups == 0) {
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int ntt = ntm / kXcds, pf = ntn / g.fgroups;
    const int fg = slot / (ntt * pf), rem = slot - fg * ntt * pf;
    m0 = (int64_t)(xcd * ntt + rem / pf) * kWBM;
    n0 = (fg * pf + rem % pf) * kWBN;
  } else {
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    m0 = (int64_t)(logical / ntn) * kWBM;
    n0 = (logical % ntn) * kWBN;
  }
  m0 += g.m_first;
  if (epi_qkv(EPI) && n0 + g.f_off < g.d && (m0 + kWBM <= g.q_lo || m0 >= g.q_hi)) return;

  // DMA: instruction q of wave w covers rows (q*8 + w)*8 .. +7 (q < 4) of A
  // and of B; lane row lane/8.
  const int lrow = lane >> 3;
  const uint16_t* A = reinterpret_cast<const uint16_t*>(g.A);
  const uint16_t* Bb = reinterpret_cast<const uint16_t*>(g.B);
  const uint16_t* aptr[4];
  const uint16_t* bptr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r0 = (q * 8 + wave) * 8;
    const int lcol = (lane & 7) ^ lrow ^ ((r0 >> 3) & 1);
    aptr[q] = A + (int64_t)(n0 + r0 + lrow) * g.K + lcol * 8;
    const int64_t w = m0 + r0 + lrow;
    if (epi_qkv(EPI)) {
      const int64_t src = row_src(g, w);  // rows without a token read X row 0 (finite, unused)
      bptr[q] = Bb + (src >= 0 ? src : 0) * g.K + lcol * 8;
    } else {
      bptr[q] = Bb + w * kDh + lcol * 8;
    }
  }
  auto dma_a = [&](int kt, int stage) {
    char* base = smem + stage * kAB;
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(aptr[q] + kt * kWBK, base + (q * 8 + wave) * 1024);
  };
  auto dma_b = [&](int kt, int stage) {
    char* base = smem + kAStages * kAB + stage * kBB;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint16_t* src = epi_qkv(EPI) ? bptr[q] + kt * kWBK
                                           : bptr[q] + (int64_t)kt * g.rows * kDh;
      dma16(src, base + (q * 8 + wave) * 1024);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nk = g.K / kWBK;
  // Operand fragments of one 16-deep k-chunk of a stage: the A rows of the
  // wave's two feature blocks and the B rows of its four token blocks.
  struct Frag {
    V8 a[2], b[4];
  };
  auto load = [&](int kt, int kc, Frag& f) {
    const char* As = smem + (kt & 1) * kAB;
    const char* Bs = smem + kAStages * kAB + (kt % kBStages) * kBB;
#pragma unroll
    for (int fb = 0; fb < 2; ++fb)
      f.a[fb] = *reinterpret_cast<const V8*>(As + swz(wn * 64 + fb * 32 + j, kc * 2 + h));
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      f.b[tb] = *reinterpret_cast<const V8*>(Bs + swz(wm * 128 + tb * 32 + j, kc * 2 + h));
  };
  // MFMAs i in [lo, hi) of a chunk's eight (feature block i / 4, token block
  // i % 4), fenced so that the compiler keeps them where they are written
  auto mma = [&](const Frag& f, int lo, int hi) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i >= lo && i < hi) acc[i >> 2][i & 3] = mfma32x32x16(f.a[i >> 2], f.b[i & 3], acc[i >> 2][i & 3]);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Per k-step each wave issues four DMA instructions for the next step's
  // weights, then four for the token rows two steps ahead.  At the end of
  // step kt, step kt+1 must have landed (weights and token rows); the token
  // rows of step kt+2 may still be in flight: vmcnt counts a wave's loads in
  // issue order, so vmcnt(4) leaves exactly those.  The four 16-deep k-chunks
  // of a stage are software pipelined: the fragments of chunk c+1 are read
  // from LDS between the second and third of chunk c's eight MFMAs, and after
  // the stage barrier the first chunk of the next stage is read there in the
  // last chunk.  A chunk's first MFMA then waits only for reads that were
  // issued six MFMAs earlier.  Bare s_barrier after an explicit wait that
  // also covers this wave's LDS reads (lgkmcnt(0), as in gemm_dma_kernel):
  // every read of a stage that a later copy overwrites was issued and
  // completed before that barrier (weights: the stage of step kt-1, refilled
  // in step kt; token rows: the stage of step kt-1, refilled for kt+2).
  constexpr int kVm0 = 0x0070, kVm4 = 0x0074;  // s_waitcnt vmcnt(0|4) lgkmcnt(0)
  dma_a(0, 0);
  dma_b(0, 0);
  if (nk > 1) {
    dma_b(1, 1);
    __builtin_amdgcn_s_waitcnt(kVm4);
  } else {
    __builtin_amdgcn_s_waitcnt(kVm0);
  }
  __builtin_amdgcn_s_barrier();
  Frag f0, f1;
  load(0, 0, f0);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) dma_a(kt + 1, (kt + 1) & 1);
    const bool ahead = kt + 2 < nk;
    if (ahead) dma_b(kt + 2, (kt + 2) % kBStages);
    mma(f0, 0, 2);
    load(kt, 1, f1);
    mma(f0, 2, 8);
    mma(f1, 0, 2);
    load(kt, 2, f0);
    mma(f1, 2, 8);
    mma(f0, 0, 2);
    load(kt, 3, f1);
    mma(f0, 2, 8);
    if (ahead) {
      __builtin_amdgcn_s_waitcnt(kVm4);
    } else {
      __builtin_amdgcn_s_waitcnt(kVm0);
    }
    __builtin_amdgcn_s_barrier();
    mma(f1, 0, 2);
    if (kt + 1 < nk) load(kt + 1, 0, f0);
    mma(f1, 2, 8);
  }

  // the loop's last barrier: no wave reads the operand stages any more
  gemm_epilogue_staged<EPI>(g, acc, m0 + wm * 128, n0 + wn * 64, j, h, lane,
                            smem + wave * 16384);
}

// Smallest number of output-feature groups (a divisor of the feature tile
// count) whose weight slice fits a 3 MB share of an XCD's 4 MB L2 (Wqkv at
// d = 1024 in two slices: measured against three 2 MB slices, QKV at s100
// 0.74 vs 0.77 ms and at s500 frame 3.71 vs 3.76 ms).
static int feature_groups(int nf, int k, int elem_bytes, int bn) {
  const int ntn = nf / bn;
  int v = 0;  // tuning override (must divide the tile count)
  if (tuning_knob("VGGT_GEMM_FGROUPS", &v) && v >= 1 && ntn % v == 0) return v;
  const int64_t bytes = (int64_t)nf * k * elem_bytes;
  for (int gcount = 1; gcount < ntn; ++gcount)
    if (ntn % gcount == 0 && bytes / gcount <= ((int64_t)3 << 20)) return gcount;
  return ntn;
}

// Kernel choice: 2 = wide (256 x 256, output features a multiple of 256),
// 1 = DMA 256 x 128, 0 = register-staged 128 x 128.  The DMA kernels need
// whole 256-row token tiles.  The tuning build's VGGT_GEMM = 0 | 1 | 2 picks
// the kind (a comparison switch).
static int gemm_kind(const Plan& p, int nf) {
  int kind = 2;
  bool forced = false;
  int v = 0;
  if (tuning_knob("VGGT_GEMM", &v) && v >= 0 && v <= 2) {
    kind = v;
    forced = true;
  }
  if (kind == 2 && nf % kWBN != 0) kind = 1;
  if (kind >= 1 && p.rows % kDmaBM != 0) kind = 0;
  // Few token rows (small sets): the smaller tiles that give more CUs a
  // workgroup, while the larger ones would leave most of them idle.
  if (!forced) {
    const int cus = device_cu_count();
    if (kind == 2 && (p.rows / kWBM) * (nf / kWBN) < cus) kind = 1;
    if (kind == 1 && (p.rows / kDmaBM) * (nf / kDmaBN) < cus) kind = 0;
  }
  return kind;
}

// The epilogues divide by the map's group stride, T and gw: set their
// multipliers once per launch.
static void set_divisors(GemmArgs& g) {
  g.dgrp = fast_div(g.map.grp_stride);
  g.dT = fast_div(g.T);
  g.dgw = fast_div(g.gw);
}

static GemmArgs base_args(const Plan& p, const Ptrs& a) {
  GemmArgs g{};
  g.rows = p.rows;
  g.vt_rows = p.vt_rows;
  g.vt_seq = p.vt_seq_stride != p.seq_stride ? (int)p.vt_seq_stride : 0;
  g.dss = fast_div(g.vt_seq != 0 ? (int)p.seq_stride : 1);
  g.vt_sets = p.nseq;
  g.map = p.map;
  g.T = p.T;
  g.gw = p.gw;
  g.off = p.off;
  g.d = p.d;
  g.eps = p.eps;
  g.qg = a.qg;
  g.qb = a.qb;
  g.kg = a.kg;
  g.kb = a.kb;
  g.rope = ws_rope(p, a);
  g.sc = ws_scalars(p, a);
  g.q = ws_q(p, a);
  g.k = ws_k(p, a);
  g.vt = ws_v(p, a);
  g.y = a.Y;
  g.m_first = 0;
  g.q_lo = p.q0;
  g.q_hi = p.window ? p.L : p.rows;
  g.v_rows = p.mode == VGGT_ATTN_MODE_MERGED ? 1 : 0;
  set_divisors(g);
  return g;
}

// One GEMM launch of `blocks` workgroups with the kernel family `kind`
// (2: 256 x 256 tiles, 1: DMA-fed, 0: plain).
template <int EPI>
static void launch_gemm(int kind, int blocks, const GemmArgs& g, hipStream_t st) {
  if (kind == 2) {
    hipLaunchKernelGGL(gemm_wide_kernel<EPI>, dim3(blocks), dim3(512), 0, st, g);
  } else if (kind == 1) {
    hipLaunchKernelGGL(gemm_dma_kernel<EPI>, dim3(blocks), dim3(256), 0, st, g);
  } else {
    hipLaunchKernelGGL(gemm_kernel<EPI>, dim3(blocks), dim3(256), 0, st, g);
  }
}

hipError_t launch_qkv(const Plan& p, const Ptrs& a, hipStream_t st) {
  GemmArgs g = base_args(p, a);
  g.A = a.Wqkv;
  g.B = a.X;
  // descriptor mode: queries only (the keys / values are in the cache)
  g.Nf = p.mode == VGGT_ATTN_MODE_DESCRIPTOR ? p.d : 3 * p.d;
  g.K = p.d;
  const int kind = gemm_kind(p, g.Nf);
  g.fgroups = feature_groups(g.Nf, g.K, 2, kind == 2 ? kWBN : kGemmBN);
  const int64_t bm = kind == 2 ? kWBM : kind == 1 ? kDmaBM : kGemmBM;
  const int64_t bn = kind == 2 ? kWBN : kind == 1 ? kDmaBN : kGemmBN;
  const int blocks = (int)(p.rows / bm) * (int)(g.Nf / bn);
  if (p.bf16_ops) {
    launch_gemm<kEpiQKVB>(kind, blocks, g, st);
  } else {
    launch_gemm<kEpiQKV>(kind, blocks, g, st);
  }
  return hipGetLastError();
}

hipError_t launch_patch_copy(const Plan& p, const Ptrs& a, hipStream_t st);

hipError_t launch_desc_kv(char* cache, const DescLayout& L, int H, int d, float eps,
                          int64_t count, const bf16* D, int64_t m, const bf16* Wqkv,
                          const float* kg, const float* kb, hipStream_t st) {
  // K and V rows of Wqkv over the m descriptor rows; tile rows past m read
  // row 0 and store nothing.  Descriptors carry no grid position: with T = 1
  // every row is token 0 of its "frame", which is never rotated.
  const int64_t tiles = (m + kWBM - 1) / kWBM;
  GemmArgs g{};
  g.A = Wqkv + (int64_t)d * d;
  g.B = D;
  g.rows = L.cap_rows;  // head stride of the cache arrays
  g.vt_rows = L.cap_rows;
  g.vt_seq = 0;
  g.dss = fast_div(1);
  g.vt_sets = 1;
  g.Nf = 2 * d;
  g.K = d;
  g.m_first = 0;
  g.q_lo = 0;
  g.q_hi = tiles * kWBM;
  g.f_off = d;
  g.dst_off = count;
  g.real_only = 1;
  g.map = RowMap{tiles * kWBM, 0, (int32_t)m, 1, 0};
  g.T = 1;
  g.gw = 1;
  set_divisors(g);
  g.off = 0;
  g.d = d;
  g.eps = eps;
  g.qg = nullptr;
  g.qb = nullptr;
  g.kg = kg;
  g.kb = kb;
  g.rope = nullptr;
  g.sc = reinterpret_cast<Scalars*>(cache);
  g.q = nullptr;
  g.k = reinterpret_cast<f16*>(cache + L.off_k);
  g.vt = reinterpret_cast<f16*>(cache + L.off_v);
  g.y = nullptr;
  int kind = 2;
  int v = 0;
  if (tuning_knob("VGGT_GEMM", &v) && v >= 0 && v < 2) kind = v;
  if (kind == 2 && g.Nf % kWBN != 0) kind = 1;
  const int bn = kind == 2 ? kWBN : kind == 1 ? kDmaBN : kGemmBN;
  g.fgroups = feature_groups(g.Nf, g.K, 2, bn);
  if (kind == 2) {
    hipLaunchKernelGGL(gemm_wide_kernel<kEpiQKV>, dim3((unsigned)(tiles * (g.Nf / kWBN))), dim3(512),
                       0, st, g);
  } else if (kind == 1) {
    hipLaunchKernelGGL(gemm_dma_kernel<kEpiQKV>,
                       dim3((unsigned)(tiles * (kWBM / kDmaBM) * (g.Nf / kDmaBN))), dim3(256), 0, st,
                       g);
  } else {
    hipLaunchKernelGGL(gemm_kernel<kEpiQKV>,
                       dim3((unsigned)(tiles * (kWBM / kGemmBM) * (g.Nf / kGemmBN))), dim3(256), 0,
                       st, g);
  }
  return hipGetLastError();
}

hipError_t launch_out(const Plan& p, const Ptrs& a, hipStream_t st) {
  GemmArgs g = base_args(p, a);
  g.A = ws_wo(p, a);
  g.B = ws_q(p, a);  // the attention kernel leaves O in place of q
  g.Nf = p.d;
  g.K = p.d;
  const int kind = gemm_kind(p, g.Nf);
  const int bn = kind == 2 ? kWBN : kGemmBN;
  g.fgroups = feature_groups(g.Nf, g.K, 2, bn);
  g.map = p.out_map;
  set_divisors(g);
  // token tiles covering the output rows: all rows, or the query window
  const int64_t bm = kind == 2 ? kWBM : kind == 1 ? kDmaBM : kGemmBM;
  const int64_t lo = p.window ? p.q0 / bm * bm : 0;
  const int64_t hi = p.window ? (p.L + bm - 1) / bm * bm : p.rows;
  g.m_first = lo;
  const int blocks = (int)((hi - lo) / bm) * (g.Nf / bn);
  if (p.bf16_ops) {
    launch_gemm<kEpiOutB>(kind, blocks, g, st);
  } else {
    launch_gemm<kEpiOut>(kind, blocks, g, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.mode == VGGT_ATTN_MODE_REGISTER && a.Y != a.X && p.patch_copy)
    return launch_patch_copy(p, a, st);
  return hipSuccess;
}

}  // namespace vggt
