// Attention core on gfx950: O = softmax(q k^T / sqrt(Dh)) v for every
// (attention set, head), Dh = 64, no mask inside a set.  The same code serves
// the per-frame sets (S sets of T tokens), the global set (S*T tokens) and the
// register set (17*S tokens): a set is just a run of workspace rows.
//
// MFMA layout.  Each wave keeps QB*32 queries in registers, as 2*QB blocks
// of 16, and per 64-key tile runs two MFMA 16x16x32 fp16 products, both
// computed transposed so no data moves between lanes:
//   S^T[key, query] = K[key, :] . Q[query, :]            (A = K tile, B = Q)
//   O^T[feat, query] += V^T[feat, key] . P^T[key, query] (A = V^T tile, B = P)
// Lane l holds query column l%16 of each block; the K rows are read in the
// permuted order given with Rows below, so that the probabilities a lane
// holds after the softmax are exactly the B operand of its PV step, given
// v^T's key order (the QKV kernel swaps key bits 2 and 3 inside every aligned
// group of 16).  16x16x32 rather than 32x32x16: the same work per tile at
// twice the MFMA issues but half the accumulator traffic per FLOP, which is
// what counts once random fp16 operands hold the chip at its power limit
// (measured: 3% faster at 103,100 tokens).
//
// Softmax (base 2: q carries log2(e)/sqrt(Dh)): online softmax with a
// per-query reference m; logits leave the MFMA already shifted (the
// accumulator starts at -m) and P = 2^(s-m) goes to fp16.  Two facts keep the max
// out of the steady state:
//   * bound = |q| * max_k |k| >= every logit of the row (Cauchy-Schwarz on
//     the LayerNorm-ed, rotated vectors), known before the first tile;
//   * fp16 holds P <= 2^15 without overflow and keeps full relative precision
//     for P >= 2^-14.
// The first tile takes the row max m0.  If bound - m0 <= 19, the reference is
// pinned at max(m0, bound - 15): no later logit can push P above 2^15, and the
// reference sits at most 4 above the row's largest logit (>= m0), so the top
// term of the row stays >= 2^-4 and the row's probabilities keep fp16's
// relative precision down to 2^-10 of it; the row is "settled" and its max is
// never taken again.  Rows that are not settled keep an online max and
// re-check the settle condition after each tile: over the first kEagerTiles
// tiles of a key range the reference follows the running max exactly (a
// first tile's max is a poor estimate of the row's: at 103,100 tokens with
// the workloads' QK-norm affine, 800 of 25,760 waves hold a row that the
// first tile leaves unsettled, 46 after 4 tiles, 2 after 16), later only
// lazily (when a logit exceeds m + 8).  Rows far below their bound -- peaked
// rows, or a loose bound when the QK-norm gain is large -- so run as ordinary
// online-softmax rows.  A wider settle gap would let the reference float up
// to (gap - 15) above the row max and push the bulk of the row's
// probabilities into fp16's subnormal range (per-row error 1e-2 at a gap of
// 29 with a QK-norm gain near 2).  Waves that stay unsettled cost more than
// their share: their workgroup runs at their pace, and a few slow workgroups
// stretch the end of the launch (measured at 103,100 tokens against the
// 29 gap: 16% slower when rows could settle only on their first tile, 7%
// with 4 eager tiles, 4% with 8, none with 16).  The row sum accumulates the fp16-rounded
// probabilities with v_dot2 (the same values the PV MFMA consumes).
//
// One kernel, attn_kernel<QB, NW, SGA>: NW waves and NW*QB*32 queries per
// workgroup (SGA: the subsampled global set, whose keys are a compact copy of
// the kept tokens, plus two per-row columns folded in at the end).  Global
// sets use 8 waves x 64 queries (512 queries share each K/V tile, one
// workgroup per CU); frame sets use 4 waves x 32 queries (small sets, ragged
// ends); register sets use 4 waves x 64 queries while that grid still gives
// every CU a workgroup, else 4 x 32.  Every shape runs the same per-row arithmetic, so a row
// comes out bit for bit the same whichever tile computes it.  The partly
// filled last round of a single-set grid runs as key ranges whose softmax
// states attn_merge_kernel combines (split tail, below).  Measured
// alternatives that did not pay on gfx950: an 8-wave "ping-pong" split (waves
// sharing a SIMD alternating MFMA and softmax phases between barriers),
// direct global->LDS loads three buffers deep (two deep is what the loop
// uses), and 128 queries per wave (spills).  With random fp16 operands this
// loop is power-bound: the shader clock settles near 1.9 GHz, so lowering the
// energy per FLOP (LDS bytes, accumulator traffic, non-MFMA instructions)
// matters as much as issue slots.
#include <atomic>
#include <type_traits>

#include "plan.h"

namespace vggt {

constexpr float kTau = 8.f;        // unsettled rows: rescale when a logit exceeds m + kTau
constexpr float kPinBelow = 15.f;  // settled rows: reference pinned at bound - kPinBelow (P <= 2^15)
constexpr float kSettleGap = 19.f; // settle once bound - m <= kSettleGap: the pinned reference
                                   // is at most kSettleGap - kPinBelow = 4 above the row max
constexpr int kEagerTiles = 16;    // unsettled rows follow the exact running max this long

struct AttnArgs {
  f16* q;              // [H][rows][64] scaled queries; overwritten with O
  const f16* k;        // [H][kv_rows][64] keys of the loop
  const f16* vt;       // [H][64][vt_rows], keys permuted inside aligned 16-groups
  int64_t rows;        // query rows per head; set s starts at row s * seq_stride
  int64_t seq_stride;
  int64_t kv_rows;     // key rows per head; set s starts at key s * kv_seq_stride
  int64_t kv_seq_stride;
  int64_t vt_rows;     // columns per v^T row; set s starts at column s * vt_seq_stride
  int64_t vt_seq_stride;
  int nseq, L, Lk, H, qtiles;  // sets, query end and keys per set, heads, query tiles
  FastDiv qt_div, h_div;       // division by qtiles and by H (scalar on the device)
  int q0;                      // first query row of a set (a window of the global set), else 0
  const Scalars* sc;
  // subsampled global set only: every token's key / value (for the diagonal)
  // and the per-head sums of the discarded keys and values (for the mean)
  const f16* k_all;    // [H][rows][64]
  const f16* vt_all;   // [H][64][rows]
  const float* sums;   // [H][128]
  int nD, T, gw, sub_h, sub_w;
  // split tail (split_p > 1): each XCD runs its contiguous range of
  // workgroups whole up to a multiple of its slots (xcd_slots) and the rest
  // as split_p key ranges each; the partial results of XCD x's tail unit v
  // go to unit x * umax + v of part ([units][BQ][64] fp32 O, then
  // [units][BQ] float2 (m, l), units = 8 * umax)
  int split_p, xcd_slots, umax;
  float* part;
  // merged mode only: the size of every merged key, [H][kv_rows] (0 past the
  // set); key j enters the softmax with weight nw[j] exp(logit)
  const f16* nw;
};

// LDS tiles are 64 rows x 128 bytes.  An MFMA operand read takes one 16-byte
// chunk per lane, 16 lanes at a time: 16 consecutive rows (v^T) or rows
// {0..7, 16..23} + 8 jj of a 32-row block (K, read in the permuted key order).
// XOR-ing the chunk index with row bits 0..2, bit 3 and bit 4 spreads either
// pattern over all banks (measured on gfx950 for consecutive rows: 5.2 cycles
// per ds_read_b128 per CU, against 8.8 with row bits 0..2 alone).
__device__ __forceinline__ int lds_slot(int row, int col) {
  return col ^ (row & 7) ^ ((row >> 3) & 1) ^ ((row >> 4) & 1);  // an involution in col
}
__device__ __forceinline__ int lds_swz(int row, int col) { return row * 128 + (lds_slot(row, col) << 4); }

// 16 bytes per lane global -> LDS by the load unit (buffer_load ... lds):
// lane i of the wave writes lds_wave_base + 16 i.  The source is a buffer
// resource -- a wave-uniform base in scalar registers -- plus the lane's byte
// offset in a vector register, so moving to the next tile costs scalar adds
// only, no per-lane 64-bit address arithmetic.  The resource spans 4 GB from
// `base` with no range clamping (every copy of the loop is in bounds).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t lane_off,
                                          void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_wave_base,
                                           16, lane_off, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// The tile.  Lane l: r = l % 16 (query of a 16-row block; A-row of an operand read),
// g = l / 16.  S^T blocks are 16 keys x 16 queries, accumulator i of lane l
// holding A-row 4g + i.  The K rows are read in a permuted order: A-row r of
// key block kb is key
//   32 (kb/2) + 16 (r/8) + 8 (kb%2) + 4 ((r/4)%2) + r%4,
// so accumulator i of block kb holds key 32(kb/2) + 16(g/2) + 8(kb%2) +
// 4(g%2) + i.  With v^T's key order (bits 2 and 3 swapped in each aligned
// group of 16), positions 32c + 8g .. +7 -- what lane group g feeds to the
// 32-key step c of the PV product -- are then exactly the keys of
// accumulators 0..3 of block 2c followed by those of block 2c + 1.
// O^T blocks are 16 features x 16 queries: accumulator i of block db holds
// feature 16 db + 4g + i.
// ---------------------------------------------------------------------------
template <int NB, typename T8 = f16x8>  // 16-row query blocks per wave, operand type
struct Rows {
  T8 qf[NB][2];     // B operand of S^T: q[row 16 qb + r][32 dc + 8 g .. +7]
  float bound[NB];  // upper bound of every logit of the row (-inf: no row)
  float m[NB];      // reference the logits are taken relative to
  float l[NB];      // partial row sum (this lane's keys)
  f32x4 negm[NB];   // -m broadcast
  f32x4 O[4][NB];   // O^T[16 db + 4 g + i][row 16 qb + r]
  unsigned settled; // bit qb: the row of query block qb is settled (its reference is final)
  bool track;       // wave-uniform: some row is not settled yet
};

// Reductions over the four 16-lane groups that hold one query row, through
// gfx950's permlane swaps (VALU; no LDS round trip and no wait): each lane's
// pair of results is its own value and that of lane l ^ 16 (then l ^ 32), in
// the same order on both lanes, so every lane of a row gets the same bits.
__device__ __forceinline__ float max_over_groups16(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups16(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS lane offsets of the operand reads: ka[kb % 2][dc] for K (block kb adds
// (kb / 2) * 4096), va[db % 2][c] for v^T (block db adds (db / 2) * 4096).
struct Lanes {
  int ka[2][2], va[2][2];
  __device__ __forceinline__ explicit Lanes(int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int dc = 0; dc < 2; ++dc)
        ka[jj][dc] = lds_swz(16 * (r >> 3) + 8 * jj + 4 * ((r >> 2) & 1) + (r & 3), 4 * dc + g);
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
      for (int c = 0; c < 2; ++c) va[par][c] = lds_swz(16 * par + r, 4 * c + g);
  }
  __device__ __forceinline__ void flip(int off) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        ka[a][b] ^= off;
        va[a][b] ^= off;
      }
  }
};

template <int NB, typename T8, typename T>
__device__ __forceinline__ void rows_init(Rows<NB, T8>& R, const T* qh, int64_t seq0, int qloc0, int L,
                                          int lane, float kmax) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int qb = 0; qb < NB; ++qb) {
    const int row = qloc0 + qb * 16 + r;
    const bool ok = row < L;
    float n2 = 0.f;
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      if (ok) {
        R.qf[qb][dc] = *reinterpret_cast<const T8*>(qh + (seq0 + row) * kDh + dc * 32 + g * 8);
      } else {
        R.qf[qb][dc] = __builtin_bit_cast(T8, u32x4{0u, 0u, 0u, 0u});
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = (float)R.qf[qb][dc][e];
        n2 = fmaf(f, f, n2);
      }
    }
    n2 = sum_over_groups16(n2);
    // 2^-10 relative margin covers the fp32 rounding of norms and dot products.
    R.bound[qb] = ok ? sqrtf(n2) * kmax * (1.f + 0x1p-10f) : -INFINITY;
    R.m[qb] = 0.f;
    R.l[qb] = 0.f;
    R.negm[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < 4; ++db) R.O[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  R.settled = 0u;
  R.track = true;
}

// The probabilities of one 64-key tile: S^T = K Q^T - m (MASK: keys at or
// beyond `valid` start from -inf, so their probability is exactly 0); where
// needed (below) the max of every row that is not settled moves or pins its
// reference first -- to the exact running max while `eager`, else only when
// the tile's max exceeds m + kTau; then P = 2^S in fp16 into pf, and the row
// sums (W: each key weighted by its size from the LDS tile Ns, else by 1).
// KB = 2 (a short last tile of at most 32 keys): key blocks 0 and 1 only,
// which hold keys 0..31, and the first PV step; the other probabilities are
// exactly zero, so the result is the same bit for bit.
template <bool MASK, int KB, bool W, int NB, typename T8>
__device__ __forceinline__ void tile_probs(Rows<NB, T8>& R, const Lanes& ln, const char* Ks,
                                           const f16* Ns, int lane, int valid, bool first,
                                           bool eager, T8 (&pf)[NB][2]) {
  static_assert(KB == 4 || KB == 2, "whole tile or its first 32 keys");
  constexpr bool B16 = std::is_same<T8, bf16x8>::value;
  static_assert(!(W && B16), "size-weighted rows run on fp16 operands");
  typedef typename Ops16<B16>::T T;
  typedef typename Ops16<B16>::T2 T2;
  constexpr int NC = KB / 2;  // 32-key PV steps
  const int g = lane >> 4;
  f32x4 S[KB][NB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    T8 kf[2];
#pragma unroll
    for (int dc = 0; dc < 2; ++dc)
      kf[dc] = *reinterpret_cast<const T8*>(Ks + ln.ka[kb & 1][dc] + (kb >> 1) * 4096);
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      f32x4 c = R.negm[qb];
      if (MASK) {
        const int key0 = 32 * (kb >> 1) + 16 * (g >> 1) + 8 * (kb & 1) + 4 * (g & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = key0 + i >= valid ? -INFINITY : c[i];
      }
      S[kb][qb] = mfma16x16x32(kf[0], R.qf[qb][0], c);
      S[kb][qb] = mfma16x16x32(kf[1], R.qf[qb][1], S[kb][qb]);
    }
  }
  if (first || R.track) {
    bool unsettled = false;
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      float mt = S[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; i += 2) mt = fmaxf(mt, fmaxf(S[kb][qb][i], S[kb][qb][i + 1]));
      mt = max_over_groups16(mt);  // row max of this tile, relative to m
      // a settled row keeps its reference whatever its wave does, so a row's
      // arithmetic never depends on the other rows of its wave
      const bool fixed = !first && ((R.settled >> qb) & 1u);
      float mn = (first || mt > (eager ? 0.f : kTau)) ? R.m[qb] + mt : R.m[qb];
      if (fixed) mn = R.m[qb];
      const bool settled = fixed || mn >= R.bound[qb] - kSettleGap;
      if (settled && !fixed) mn = fmaxf(mn, R.bound[qb] - kPinBelow);
      if (settled) R.settled |= 1u << qb;
      unsettled = unsettled || !settled;
      const float dl = mn - R.m[qb];
      if (dl != 0.f) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[kb][qb][i] -= dl;
        const float al = first ? 1.f : __builtin_amdgcn_exp2f(-dl);
        R.l[qb] *= al;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) R.O[db][qb][i] *= al;
      }
      R.m[qb] = mn;
      R.negm[qb] = f32x4{-mn, -mn, -mn, -mn};
    }
    R.track = __ballot(unsettled) != 0;
  }
  // W: row-sum weights of the lane's keys (key block kb holds keys key0(kb) .. +3)
  f16x4 wk[W ? KB : 1];
  if constexpr (W) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int key0 = 32 * (kb >> 1) + 16 * (g >> 1) + 8 * (kb & 1) + 4 * (g & 1);
      wk[kb] = *reinterpret_cast<const f16x4*>(Ns + key0);
    }
  }
#pragma unroll
  for (int qb = 0; qb < NB; ++qb)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      T8 v;
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const f32x2 e2 = {__builtin_amdgcn_exp2f(S[2 * c + half][qb][i]),
                            __builtin_amdgcn_exp2f(S[2 * c + half][qb][i + 1])};
          const T2 h2 = __builtin_convertvector(e2, T2);
          v[4 * half + i] = h2[0];
          v[4 * half + i + 1] = h2[1];
          if constexpr (W) {
            const f16x2 w2 = {wk[2 * c + half][i], wk[2 * c + half][i + 1]};
            R.l[qb] = dot2_acc(h2, w2, R.l[qb]);
          } else {
            R.l[qb] = dot2_acc(h2, T2{(T)1.f, (T)1.f}, R.l[qb]);
          }
        }
      pf[qb][c] = v;
    }
}

// One 64-key tile: its probabilities (tile_probs), then O^T += V^T P^T.
template <bool MASK, int KB = 4, bool W = false, int NB, typename T8>
__device__ __forceinline__ void tile_run(Rows<NB, T8>& R, const Lanes& ln, const char* Ks,
                                         const char* Vs, const f16* Ns, int lane, int valid,
                                         bool first, bool eager) {
  constexpr int NC = KB / 2;  // 32-key PV steps
  T8 pf[NB][2];
  tile_probs<MASK, KB, W>(R, ln, Ks, Ns, lane, valid, first, eager, pf);
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const T8 vf = *reinterpret_cast<const T8*>(Vs + ln.va[db & 1][c] + (db >> 1) * 4096);
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) R.O[db][qb] = mfma16x16x32(vf, pf[qb][c], R.O[db][qb]);
    }
}

// Subsampled global set: fold into each row's softmax the two columns the key
// loop does not hold -- the token's own key / value when the token itself was
// discarded (a kept token's diagonal is already in the loop), and the mean key
// / value pair of the discarded tokens, which stands for the row's other n_i
// discarded columns (logit + log2 n_i).  Rescales O and l to the new reference
// like one more online-softmax step, in fp32.  One query block (QBI) at a
// time, loads issued before the arithmetic that uses them.
template <int QBI, int NB>
__device__ __forceinline__ void sga_block(Rows<NB>& R, const AttnArgs& p, int hd, int qloc0, int lane) {
  const int r = lane & 15, g = lane >> 4;
  const int row = qloc0 + QBI * 16 + r;  // = token index: one set, identity row map
  if (row >= p.L) return;                // the row's four lane groups leave together
  const int t = row % p.T;
  bool kept = true;
  if (t >= kSpecial) {
    const int pidx = t - kSpecial, pr = pidx / p.gw, pc = pidx - pr * p.gw;
    kept = (pr % p.sub_h) == 0 && (pc % p.sub_w) == 0;
  }
  const float* sk = p.sums + hd * 128;
  const float* sv = sk + 64;
  // this lane's 16 features of the token's own key (q layout) and value (O layout)
  f16x8 kd[2];
  f16 vd[4][4];
  if (!kept) {
    const f16* krow = p.k_all + ((int64_t)hd * p.rows + row) * kDh + g * 8;
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) kd[dc] = *reinterpret_cast<const f16x8*>(krow + dc * 32);
    const int64_t slot = ((int64_t)row & ~(int64_t)15) | (((row >> 2) & 1) << 3) |
                         (((row >> 3) & 1) << 2) | (row & 3);
    const f16* vcol = p.vt_all + ((int64_t)hd * kDh + 4 * g) * p.rows + slot;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) vd[db][i] = vcol[(int64_t)(db * 16 + i) * p.rows];
  } else {
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) kd[dc] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) vd[db][i] = (f16)0.f;
  }
  float sd = 0.f, sm = 0.f;
#pragma unroll
  for (int dc = 0; dc < 2; ++dc) {
    const f32x4 k0 = *reinterpret_cast<const f32x4*>(sk + dc * 32 + g * 8);
    const f32x4 k1 = *reinterpret_cast<const f32x4*>(sk + dc * 32 + g * 8 + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float qv = (float)R.qf[QBI][dc][e];
      sd = fmaf(qv, (float)kd[dc][e], sd);
      sm = fmaf(qv, e < 4 ? k0[e & 3] : k1[e & 3], sm);
    }
  }
  sd = sum_over_groups16(sd);
  sm = sum_over_groups16(sm);
  const float inv = p.nD > 0 ? 1.f / (float)p.nD : 0.f;
  const int n = p.nD - (kept ? 0 : 1);
  const float s_d = kept ? -INFINITY : sd;
  const float s_m = n > 0 ? sm * inv + __log2f((float)n) : -INFINITY;
  const float mn = fmaxf(R.m[QBI], fmaxf(s_d, s_m));
  const float al = __builtin_amdgcn_exp2f(R.m[QBI] - mn);
  const float pd = __builtin_amdgcn_exp2f(s_d - mn), pm = __builtin_amdgcn_exp2f(s_m - mn);
  R.l[QBI] = R.l[QBI] * al + (g == 0 ? pd + pm : 0.f);
  const float pmi = pm * inv;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const f32x4 vb = *reinterpret_cast<const f32x4*>(sv + db * 16 + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      R.O[db][QBI][i] = fmaf(R.O[db][QBI][i], al, fmaf(pd, (float)vd[db][i], pmi * vb[i]));
  }
  R.m[QBI] = mn;
}

template <int NB>
__device__ __forceinline__ void sga_columns(Rows<NB>& R, const AttnArgs& p, int hd, int qloc0,
                                            int lane) {
  sga_block<0>(R, p, hd, qloc0, lane);
  __builtin_amdgcn_sched_barrier(0);
  sga_block<1>(R, p, hd, qloc0, lane);
  if constexpr (NB == 4) {
    __builtin_amdgcn_sched_barrier(0);
    sga_block<2>(R, p, hd, qloc0, lane);
    __builtin_amdgcn_sched_barrier(0);
    sga_block<3>(R, p, hd, qloc0, lane);
  }
}

template <int NB, typename T8, typename T>
__device__ __forceinline__ void rows_store(const Rows<NB, T8>& R, T* qh, int64_t seq0, int qloc0, int L,
                                           int lane) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int qb = 0; qb < NB; ++qb) {
    const float inv = 1.f / sum_over_groups16(R.l[qb]);
    const int row = qloc0 + qb * 16 + r;
    if (row < L) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        typename Ops16<std::is_same<T, bf16>::value>::T4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (T)(R.O[db][qb][i] * inv);
        *reinterpret_cast<decltype(o)*>(qh + (seq0 + row) * kDh + db * 16 + 4 * g) = o;
      }
    }
  }
}

template <int NB, typename T8>
__device__ __forceinline__ void rows_store_partial(const Rows<NB, T8>& R, float* po, float2* pml, int lrow0,
                                                   int lane) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int qb = 0; qb < NB; ++qb) {
    const float lt = sum_over_groups16(R.l[qb]);
    const int lr = lrow0 + qb * 16 + r;
#pragma unroll
    for (int db = 0; db < 4; ++db)
      *reinterpret_cast<f32x4*>(po + lr * kDh + db * 16 + 4 * g) = R.O[db][qb];
    if (g == 0) pml[lr] = make_float2(R.m[qb], lt);
  }
}

// Workgroup coordinates: (query tile, head, set) of the logical workgroup,
// and for a unit of the split tail its key range ks (else -1); `skip` marks
// the padding blocks of a split grid.
struct BlockCoord {
  int h, s, qt, ks, unit;
  bool skip;
};
__device__ __forceinline__ BlockCoord coord_of(const AttnArgs& p, int logical) {
  BlockCoord c;
  const int t2 = fdiv(logical, p.qt_div);
  c.qt = logical - t2 * p.qtiles;
  c.s = fdiv(t2, p.h_div);
  c.h = t2 - c.s * p.H;
  c.ks = -1;
  c.unit = -1;
  c.skip = false;
  return c;
}

// The logical workgroups of XCD x: the contiguous range xcd_remap gives it.
struct XcdRange {
  int base, n, whole, tail;  // first logical id, count, whole ones, split ones
};
__device__ __forceinline__ XcdRange xcd_range(const AttnArgs& p, int x) {
  const int W = p.qtiles * p.H * p.nseq;
  const int per = W >> 3, rem = W & (kXcds - 1);
  XcdRange r;
  r.n = per + (x < rem ? 1 : 0);
  r.base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  r.tail = r.n % p.xcd_slots;
  r.whole = r.n - r.tail;
  return r;
}

// Blocks go to the XCDs round-robin (block b to XCD b mod 8, in order of its
// slot b / 8).  Without a split each XCD walks its range in order; with one,
// slots [0, whole) of XCD x are its whole workgroups and the next tail *
// split_p slots their key ranges, on the XCD whose L2 already holds the
// range's keys and values.
__device__ __forceinline__ BlockCoord block_coord(const AttnArgs& p) {
  const int b = blockIdx.x;
  if (p.split_p <= 1) return coord_of(p, xcd_remap(b, gridDim.x));
  const int x = b & (kXcds - 1), slot = b >> 3;
  const XcdRange r = xcd_range(p, x);
  if (slot < r.whole) return coord_of(p, r.base + slot);
  const int v = slot - r.whole;
  BlockCoord c = coord_of(p, r.base + r.whole + (v < r.tail * p.split_p ? v / p.split_p : 0));
  if (v >= r.tail * p.split_p) {
    c.skip = true;  // padding: this XCD has fewer slots than the longest
    return c;
  }
  c.ks = v % p.split_p;
  c.unit = x * p.umax + v;
  return c;
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
// K / V^T tiles are double buffered in LDS and copied one tile ahead by the
// load unit (global_load_lds, no register staging), with one workgroup
// barrier per tile.
template <int QB, int NW, bool SGA, bool W, bool B16>
__global__ __launch_bounds__(NW * 64, (NW == 4 && QB == 1) ? 3 : 2) void attn_kernel(AttnArgs p) {
  constexpr int BQ = NW * QB * 32;
  static_assert(!(B16 && (SGA || W)), "the bf16-operand variant serves plain sets");
  typedef typename Ops16<B16>::T T;  // q, k, v, P and O
  // K / V^T tiles [buffer][K, V^T][64 rows x 128 bytes], then in merged mode
  // (W) the sizes of the tile's 64 keys, 1 KB per buffer (the first 128
  // bytes used; see issue()).  One LDS object: with a second one the
  // compiler waits for every outstanding LDS copy, the next tile's too,
  // before a tile's first LDS read.
  __shared__ __attribute__((aligned(16))) char smem_raw[2 * 2 * 64 * 128 + (W ? 2 * 1024 : 0)];
  auto& smem = *reinterpret_cast<char (*)[2][2][64 * 128]>(smem_raw);
  f16* const sizes_lds = reinterpret_cast<f16*>(smem_raw + 2 * 2 * 64 * 128);

  const int tid = threadIdx.x;
  // the wave index is uniform: LDS destinations and copy bases stay scalar
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // single-set grids may have a split tail
  constexpr bool kSplit = true;
  const BlockCoord bc = kSplit ? block_coord(p) : coord_of(p, xcd_remap(blockIdx.x, gridDim.x));
  if (kSplit && bc.skip) return;  // whole block: before any barrier
  const int64_t seq0 = (int64_t)bc.s * p.seq_stride;
  const int64_t kv0 = (int64_t)bc.s * p.kv_seq_stride;
  const int64_t vt0 = (int64_t)bc.s * p.vt_seq_stride;
  const int L = p.L;
  const int qloc0 = p.q0 + bc.qt * BQ + wave * QB * 32;
  const bool active = __builtin_amdgcn_readfirstlane(qloc0) < L;
  T* qh = reinterpret_cast<T*>(p.q) + (int64_t)bc.h * p.rows * kDh;
  const f16* kh = p.k + (int64_t)bc.h * p.kv_rows * kDh;
  const f16* vh = p.vt + (int64_t)bc.h * kDh * p.vt_rows;
  const f16* nh = W ? p.nw + (int64_t)bc.h * p.kv_rows + kv0 : nullptr;

  using LanesT = Lanes;
  typedef typename Ops16<B16>::T8 T8;

  // The tile loop for a wave of NB 16-row query blocks (2 QB, or one block
  // for a wave of a short last query tile, below).
  auto run = [&](auto nb_c) {
    constexpr int NB = decltype(nb_c)::value;
    Rows<NB, T8> R;
    rows_init(R, qh, seq0, qloc0, L, lane, p.sc->kmax[bc.h]);

    // key tiles [t0, t1): all of them, or one key range of a split workgroup
    // (only the range that ends the set has a masked last tile)
    const int ntiles = (p.Lk + 63) / 64;
    int t0 = 0, t1 = ntiles;
    if (bc.ks >= 0) {
      t0 = bc.ks * ntiles / p.split_p;
      t1 = (bc.ks + 1) * ntiles / p.split_p;
    }
    const int last_valid = t1 == ntiles ? p.Lk - 64 * (ntiles - 1) : 64;

    // K and v^T tiles are 64 rows of 128 bytes each.  The load unit copies them
    // straight into LDS: one instruction fills 8 consecutive rows (1 KB; lane i
    // lands in row i/8, slot i%8), so lane i fetches the source chunk that the
    // row swizzle puts in that slot.  Wave w fills rows [8 KI w, 8 KI (w+1)) of
    // both tiles.  A tile is complete once every wave has waited for its own
    // copies (vmcnt) and passed the workgroup barrier.
    constexpr int KI = 8 / NW;
    // Copy i of this wave fills rows 8 (wave KI + i) .. +7 of a tile.  Its
    // source is a wave-uniform base -- the first of those rows of K, or of v^T
    // at the tile's first key -- moved per tile by scalar adds, plus the lane's
    // byte offset within the eight rows: below 8 * 128 bytes for K, below
    // 8 vt_rows * 2 bytes for v^T (vt_rows <= 2^28 keeps it in 32 bits).
    uint32_t ok[KI], ov[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int row = 8 * (wave * KI + i) + (lane >> 3);
      const int col = lds_slot(row, lane & 7);
      ok[i] = (uint32_t)(((lane >> 3) * kDh + col * 8) * 2);
      ov[i] = (uint32_t)((lane >> 3) * 2) * (uint32_t)p.vt_rows + (uint32_t)(col * 16);
    }
    auto issue = [&](int tile, int buf) {
      const int64_t key0 = kv0 + (int64_t)tile * 64, col0 = vt0 + (int64_t)tile * 64;
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const int row0 = 8 * (wave * KI + i);
        lds_dma16(dma_rsrc(kh + (key0 + row0) * kDh), ok[i], &smem[buf][0][0] + (wave * KI + i) * 1024);
        lds_dma16(dma_rsrc(vh + (int64_t)row0 * p.vt_rows + col0), ov[i],
                  &smem[buf][1][0] + (wave * KI + i) * 1024);
      }
      // the 64 key sizes (128 bytes): every lane of every wave copies chunk
      // i % 8 to slot i, so slots 0..7 hold the sizes (the waves write the
      // same bytes; no branch around the copy)
      if (W) lds_dma16(dma_rsrc(nh + (int64_t)tile * 64), (uint32_t)((lane & 7) * 16), sizes_lds + buf * 512);
    };
    auto land = [&]() {
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): this wave's copies are in LDS
      __syncthreads();
    };

    const LanesT ln(lane);
    // One tile from LDS buffer BUF while the next tile moves into BUF ^ 1.  The
    // loop is unrolled by two so that BUF is a constant and every LDS address
    // is a lane offset plus an immediate; a scheduling barrier keeps the two
    // halves from being interleaved (which would only add live registers).
    auto step = [&](auto buf_c, int t) {
      constexpr int BUF = decltype(buf_c)::value;
      issue(t + 1, BUF ^ 1);
      if (active)
        tile_run<false, 4, W>(R, ln, smem[BUF][0], smem[BUF][1], sizes_lds + BUF * 512, lane, 64, t == t0,
                              t - t0 < kEagerTiles);
      land();
      __builtin_amdgcn_sched_barrier(0);
    };
    issue(t0, 0);
    land();
    // all tiles of the range but its last: no mask; tile t sits in LDS buffer
    // (t - t0) & 1
    // (Every tile shape runs this unrolled loop: 4-wave tiles of one row block
    // per wave fit it in 168 registers, three waves per SIMD, and those of two
    // row blocks in 256 with the short-tile path below left out.)
    int t = t0;
    for (; t + 2 < t1; t += 2) {
      step(std::integral_constant<int, 0>(), t);
      step(std::integral_constant<int, 1>(), t + 1);
    }
    if (t < t1 - 1) {
      step(std::integral_constant<int, 0>(), t);
      ++t;
    }
    // last tile of the range (t = t1 - 1): keys past the end of the set masked.  Small
    // sets on 4-wave tiles of one row block per wave (frames) often end in a
    // short tile -- 7 of 64 keys for a 26 x 39 frame -- whose second half is
    // skipped (its probabilities are exactly zero, so the result is the same bit
    // for bit); the two-row-block tile leaves that path out for its registers.
    if (active) {
      LanesT lb = ln;
      lb.flip(((t - t0) & 1) * 2 * 64 * 128);
      const bool first = t1 - t0 == 1, eager = t - t0 < kEagerTiles;
      const f16* Ns = sizes_lds + ((t - t0) & 1) * 512;
      if (NW == 4 && QB == 1 && last_valid <= 32) {
        tile_run<true, 2, W>(R, lb, smem[0][0], smem[0][1], Ns, lane, last_valid, first, eager);
      } else {
        tile_run<true, 4, W>(R, lb, smem[0][0], smem[0][1], Ns, lane, last_valid, first, eager);
      }
    }
    // the diagonal and mean columns enter once per row: in its last key range
    if constexpr (SGA) {
      if (active && (bc.ks < 0 || bc.ks == p.split_p - 1)) sga_columns(R, p, bc.h, qloc0, lane);
    }
    if (kSplit && bc.unit >= 0) {
      // a key range of a split workgroup: unnormalised state for the merge
      float* po = p.part + (int64_t)bc.unit * BQ * kDh;
      float2* pml = reinterpret_cast<float2*>(p.part + (int64_t)kXcds * p.umax * BQ * kDh) +
                    (int64_t)bc.unit * BQ;
      if (active) rows_store_partial(R, po, pml, wave * QB * 32, lane);
    } else if (active) {
      rows_store(R, qh, seq0, qloc0, L, lane);
    }
  };
  // A wave with at most 16 rows -- in the short last query tile of a frame
  // set (7 of 32 for a 26 x 39 frame), or with none -- runs one row block:
  // the same per-row arithmetic (bit for bit the same rows), half the MFMAs
  // and softmax work, so the short tile's workgroup leaves sooner.
  if constexpr (QB == 1 && !SGA) {
    if (L - qloc0 <= 16) {
      run(std::integral_constant<int, 1>());
      return;
    }
  }
  run(std::integral_constant<int, 2 * QB>());
}

// Merge of a split tail: for each query row of a split workgroup, the
// split_p key-range states (m_i, l_i, O_i) combine as one softmax over all
// keys, O = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i with M = max_i m_i,
// stored in fp16 in place of the row's q like an unsplit workgroup.  Blocks:
// (XCD x, tail workgroup i of x, 16 rows); 16 threads per row, 4 features
// each.
template <int BQ, bool B16>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs p) {
  constexpr int per_wg = BQ / 16;
  const int tail_max = p.umax / p.split_p;
  const int x = blockIdx.x / (tail_max * per_wg);
  const int rest = blockIdx.x - x * tail_max * per_wg;
  const int i = rest / per_wg;
  const int lr = (rest - i * per_wg) * 16 + (threadIdx.x >> 4);
  const int f = (threadIdx.x & 15) * 4;
  const XcdRange r = xcd_range(p, x);
  if (i >= r.tail) return;
  const BlockCoord c = coord_of(p, r.base + r.whole + i);
  const int row = p.q0 + c.qt * BQ + lr;
  if (row >= p.L) return;
  const float2* ml = reinterpret_cast<const float2*>(p.part + (int64_t)kXcds * p.umax * BQ * kDh);
  const int64_t u0 = (int64_t)x * p.umax + (int64_t)i * p.split_p;
  float M = -INFINITY;
  for (int k = 0; k < p.split_p; ++k) M = fmaxf(M, ml[(u0 + k) * BQ + lr].x);
  float l = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < p.split_p; ++k) {
    const float2 e = ml[(u0 + k) * BQ + lr];
    const float w = __builtin_amdgcn_exp2f(e.x - M);
    l = fmaf(w, e.y, l);
    const f32x4 oi = *reinterpret_cast<const f32x4*>(p.part + ((u0 + k) * BQ + lr) * kDh + f);
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) o[e4] = fmaf(w, oi[e4], o[e4]);
  }
  const float inv = 1.f / l;
  typedef typename Ops16<B16>::T T;
  typename Ops16<B16>::T4 out;
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4) out[e4] = (T)(o[e4] * inv);
  T* qh = reinterpret_cast<T*>(p.q) + (int64_t)c.h * p.rows * kDh;
  *reinterpret_cast<decltype(out)*>(qh + ((int64_t)c.s * p.seq_stride + row) * kDh + f) = out;
}

// Split tail.  Each XCD walks a contiguous range of the W workgroups on its
// slots (its CUs times the workgroups of the kernel that fit a CU); the last
// round of the range holds tail = n mod slots workgroups and leaves the other
// slots idle.  Running each of those as P key ranges (P units of 1/P the
// work, on the same XCD) shortens that round from one workgroup time to
// ceil(tail P / slots) / P.  P is the smallest that gets within 2% of the
// best, with at least kSplitMinTiles key tiles per range and 8 * tail * P
// units within the partial-result buffer.  The tuning build's VGGT_ATTN_SPLIT
// = P forces the key ranges per split workgroup (1: no split).
struct SplitPlan {
  int P = 1, xcd_slots = 0, umax = 0;
  int64_t grid = 0;
};

static SplitPlan choose_split(const Plan& p, int64_t W, int ntiles, int per_cu) {
  SplitPlan sp;
  sp.grid = W;
  const int64_t C = (int64_t)device_cu_count() * (per_cu > 0 ? per_cu : 1);
  if (p.split_cap <= 0 || C % kXcds != 0) return sp;
  const int64_t cpx = C / kXcds;
  const int64_t per = W / kXcds, rem = W % kXcds;
  int64_t tail = 0;  // the largest tail of any XCD
  for (int x = 0; x < kXcds; ++x) {
    const int64_t n = per + (x < rem ? 1 : 0), t = n % cpx;
    if (t > tail) tail = t;
  }
  if (tail == 0) return sp;
  auto allowed = [&](int P) {
    return kXcds * tail * P <= p.split_cap && ntiles / P >= kSplitMinTiles;
  };
  int best = 1;
  double best_t = 1.0;
  for (int P = 2; P <= kSplitMaxWays && allowed(P); ++P) {
    const double t = (double)((tail * P + cpx - 1) / cpx) / P;
    if (t < best_t - 0.02) {
      best_t = t;
      best = P;
    }
  }
  int forced = 0;
  if (tuning_knob("VGGT_ATTN_SPLIT", &forced)) {
    int P = forced;
    while (P > 1 && !allowed(P)) --P;
    if (P >= 1) best = P;
  }
  if (best <= 1) return sp;
  int64_t slots = 0;  // the longest XCD
  for (int x = 0; x < kXcds; ++x) {
    const int64_t n = per + (x < rem ? 1 : 0), t = n % cpx;
    if (n - t + t * best > slots) slots = n - t + t * best;
  }
  sp.P = best;
  sp.xcd_slots = (int)cpx;
  sp.umax = (int)(tail * best);
  sp.grid = slots * kXcds;
  return sp;
}

template <int QB, int NW, bool SGA, bool W = false, bool B16 = false>
static hipError_t launch_attn_t(const Plan& p, const Ptrs& a, hipStream_t st) {
  constexpr int BQ = NW * QB * 32;
  AttnArgs g{};
  // merged mode: the merged queries, keys and values, kv_rows rows per head
  g.q = W ? ws_qc(p, a) : ws_q(p, a);
  g.k = ws_kloop(p, a);
  g.vt = ws_vloop(p, a);
  g.rows = W ? p.kv_rows : p.rows;
  g.nw = W ? ws_nw(p, a) : nullptr;
  g.seq_stride = p.seq_stride;
  g.kv_rows = p.kv_rows;
  g.kv_seq_stride = p.kv_seq_stride;
  // v^T of the loop: the projection's own (frame, global, register sets) or a
  // compact copy (subsampled, merged, descriptor keys), which has the keys' rows
  const bool own_vt = !compact_kv(p) && p.mode != VGGT_ATTN_MODE_DESCRIPTOR;
  g.vt_rows = own_vt ? p.vt_rows : p.kv_rows;
  g.vt_seq_stride = own_vt ? p.vt_seq_stride : p.kv_seq_stride;
  g.nseq = p.nseq;
  g.L = p.L;
  g.Lk = p.Lk;
  g.H = p.H;
  g.q0 = p.q0;
  g.qtiles = (p.L - p.q0 + BQ - 1) / BQ;
  g.qt_div = fast_div(g.qtiles);
  g.h_div = fast_div(p.H);
  g.sc = ws_scalars(p, a);
  if (SGA) {
    g.k_all = ws_k(p, a);
    g.vt_all = ws_v(p, a);
    g.sums = ws_sums(p, a);
    g.nD = p.nD;
    g.T = p.T;
    g.gw = p.gw;
    g.sub_h = p.sub_h;
    g.sub_w = p.sub_w;
  }
  const int64_t blocks = (int64_t)g.qtiles * p.H * p.nseq;
  SplitPlan sp;
  sp.grid = blocks;
  if (p.split_cap > 0) {
    // workgroups of this kernel resident per CU (register / LDS bound)
    static std::atomic<int> occupancy{0};
    int per_cu = occupancy.load(std::memory_order_relaxed);
    if (per_cu == 0) {
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_kernel<QB, NW, SGA, W, B16>,
                                                       NW * 64, 0) != hipSuccess)
        per_cu = -1;
      occupancy.store(per_cu, std::memory_order_relaxed);
    }
    sp = choose_split(p, blocks, (p.Lk + 63) / 64, per_cu);
  }
  g.split_p = sp.P;
  g.xcd_slots = sp.xcd_slots;
  g.umax = sp.umax;
  g.part = reinterpret_cast<float*>(a.ws + p.off_split);
  hipLaunchKernelGGL((attn_kernel<QB, NW, SGA, W, B16>), dim3((unsigned)sp.grid), dim3(NW * 64), 0,
                     st, g);
  if (sp.P > 1) {
    const int tail_max = sp.umax / sp.P;
    hipLaunchKernelGGL((attn_merge_kernel<BQ, B16>), dim3((unsigned)(kXcds * tail_max * (BQ / 16))),
                       dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

hipError_t launch_core(const Plan& p, const Ptrs& a, hipStream_t st) {
  if (p.mode == VGGT_ATTN_MODE_SUBSAMPLED) return launch_attn_t<2, 8, true>(p, a, st);
  if (p.mode == VGGT_ATTN_MODE_MERGED) {
    if (p.attn_waves == 8) return launch_attn_t<2, 8, false, true>(p, a, st);
    return launch_attn_t<1, 4, false, true>(p, a, st);
  }
  if (p.bf16_ops) {
    // the bf16-operand variant of the plain sets (global, frame, register)
    if (p.attn_waves == 8) {
      if (p.attn_qb == 2) return launch_attn_t<2, 8, false, false, true>(p, a, st);
      if (p.attn_qb == 1) return launch_attn_t<1, 8, false, false, true>(p, a, st);
    } else {
      if (p.attn_qb == 2) return launch_attn_t<2, 4, false, false, true>(p, a, st);
      if (p.attn_qb == 1) return launch_attn_t<1, 4, false, false, true>(p, a, st);
    }
    return hipErrorInvalidValue;
  }
  if (p.attn_waves == 8) {
    if (p.attn_qb == 2) return launch_attn_t<2, 8, false>(p, a, st);
    if (p.attn_qb == 1) return launch_attn_t<1, 8, false>(p, a, st);
  } else {
    if (p.attn_qb == 2) return launch_attn_t<2, 4, false>(p, a, st);
    if (p.attn_qb == 1) return launch_attn_t<1, 4, false>(p, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace vggt
