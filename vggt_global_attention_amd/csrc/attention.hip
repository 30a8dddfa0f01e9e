// Attention core on gfx950: O = softmax(q k^T / sqrt(Dh)) v for every
// (attention set, head), Dh = 64, no mask inside a set.  One kernel serves the
// per-frame sets (S sets of T tokens), the global set (S*T tokens) and the
// register set (17*S tokens): a set is just a run of workspace rows.
//
// Work split: a workgroup owns BQ = NW*QB*16 query rows of one (set, head)
// and streams that set's keys/values through LDS in 64-key tiles (double
// buffered through registers, one barrier per tile).  Each wave keeps its
// QB*16 queries in registers and runs two MFMA 16x16x32 fp16 products per
// tile, both computed transposed so no data moves between lanes:
//   S^T[key, query] = K[key, :] . Q[query, :]      (A = K tile, B = Q)
//   O^T[feat, query] += V^T[feat, key] . P^T[key, query]  (A = V^T tile, B = P)
// With this orientation a lane holds one query column and, per 16-key block,
// keys 4*(lane/16) + 0..3.  Two adjacent key blocks give a lane the 8
// probabilities its B operand needs for a 32-key step, in the order
// (4c+0..3, 16+4c+0..3); the QKV kernel stores v^T with that same order inside
// every aligned group of 32 keys, so the PV product is exact.
//
// Softmax (base 2: q carries log2(e)/sqrt(Dh)): an online softmax with a
// per-query reference m.  Logits come out of the MFMA already shifted
// (accumulator initialised to -m).  A tile's row max is taken with one
// in-lane max and two cross-lane steps; m is only moved when a logit exceeds
// m + kTau, so P = 2^(s-m) <= 2^kTau always fits fp16 and O and the row sum
// are rescaled rarely.  Once m >= bound - kTauSkip, where bound =
// |q| * max|k| >= every logit (Cauchy-Schwarz on the LayerNorm-ed vectors),
// no later logit can push P past 2^kTauSkip and the max is no longer taken.
// The row sum accumulates the fp16-rounded probabilities with v_dot2
// (the same values the PV MFMA consumes).
#include "plan.h"

namespace vggt {

constexpr float kTau = 8.f;       // rescale when a logit exceeds m + kTau
constexpr float kTauSkip = 15.f;  // stop tracking the max once bound - m <= kTauSkip

struct AttnArgs {
  f16* q;            // [H][rows][64] scaled queries; overwritten with O
  const f16* k;      // [H][rows][64]
  const f16* vt;     // [H][64][rows], keys permuted inside aligned 32-groups
  int64_t rows;
  int64_t seq_stride;
  int nseq, L, H, qtiles;
  const Scalars* sc;
};

__device__ __forceinline__ int lds_swz(int row, int col) {
  return row * 128 + ((col ^ (row & 7)) << 4);
}

template <int QB, int NW>
__global__ __launch_bounds__(NW * 64, 2) void attn_kernel(AttnArgs p) {
  constexpr int BQ = NW * QB * 16;
  constexpr int NT = NW * 64;
  constexpr int CH = (2 * 512) / NT;  // 16-byte chunks per thread per K+V tile
  __shared__ __attribute__((aligned(16))) char smem[2][2][64 * 128];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, gq = lane >> 4;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = logical % p.qtiles;
  const int t2 = logical / p.qtiles;
  const int h = t2 % p.H;
  const int s = t2 / p.H;
  const int64_t seq0 = (int64_t)s * p.seq_stride;
  const int L = p.L;
  const int qloc0 = qt * BQ + wave * QB * 16;
  const bool wave_active = qloc0 < L;

  f16* qh = p.q + (int64_t)h * p.rows * kDh;
  const f16* kh = p.k + (int64_t)h * p.rows * kDh;
  const f16* vh = p.vt + (int64_t)h * kDh * p.rows;

  // ---- queries of this wave (B operand of S^T), their norms and bounds
  f16x8 qf[QB][2];
  float bound[QB];
  const float kmax = p.sc->kmax[h];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qloc0 + qb * 16 + j;
    const bool ok = row < L;
    float n2 = 0.f;
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      if (ok) {
        qf[qb][dc] = *reinterpret_cast<const f16x8*>(qh + (seq0 + row) * kDh + dc * 32 + gq * 8);
      } else {
        qf[qb][dc] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = (float)qf[qb][dc][e];
        n2 = fmaf(f, f, n2);
      }
    }
    n2 = sum_across_groups(n2);
    // 2^-10 relative margin covers the fp32 rounding of norms and dot products.
    bound[qb] = ok ? sqrtf(n2) * kmax * (1.f + 0x1p-10f) : -INFINITY;
  }

  float m[QB], l[QB];
  f32x4 negm[QB];
  f32x4 O[4][QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = 0.f;
    l[qb] = 0.f;
    negm[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int db = 0; db < 4; ++db) O[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool track = true;

  const int ntiles = (L + 63) / 64;
  const int last_valid = L - 64 * (ntiles - 1);

  // ---- K / V^T tile loader: chunk c < 512 is K (row c>>3, 16B col c&7),
  // chunk c >= 512 is V^T (feature row, 16B col).
  u32x4 rg[CH];
  int soff[CH];
  const f16* gsrc[CH];
  int64_t gstep[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + NT * i;
    const int cc = c & 511, row = cc >> 3, col = cc & 7;
    soff[i] = (c >> 9) * (64 * 128) + lds_swz(row, col);
    if (c < 512) {
      gsrc[i] = kh + (seq0 + row) * kDh + col * 8;
      gstep[i] = 64 * kDh;
    } else {
      gsrc[i] = vh + (int64_t)row * p.rows + seq0 + col * 8;
      gstep[i] = 64;
    }
  }
  auto gload = [&](int tile) {
#pragma unroll
    for (int i = 0; i < CH; ++i)
      rg[i] = *reinterpret_cast<const u32x4*>(gsrc[i] + (int64_t)tile * gstep[i]);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i)
      *reinterpret_cast<u32x4*>(&smem[buf][0][0] + soff[i]) = rg[i];
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    if (tile + 1 < ntiles) gload(tile + 1);

    if (wave_active) {
      const char* Ks = smem[buf][0];
      const char* Vs = smem[buf][1];
      // ---- S^T = K Q^T - m
      f32x4 S[4][QB];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f16x8 k0 = *reinterpret_cast<const f16x8*>(Ks + lds_swz(kb * 16 + j, gq));
        const f16x8 k1 = *reinterpret_cast<const f16x8*>(Ks + lds_swz(kb * 16 + j, 4 + gq));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          S[kb][qb] = mfma16x16x32(k0, qf[qb][0], negm[qb]);
          S[kb][qb] = mfma16x16x32(k1, qf[qb][1], S[kb][qb]);
        }
      }
      if (tile == ntiles - 1 && last_valid < 64) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kb * 16 + 4 * gq + r >= last_valid) {
#pragma unroll
              for (int qb = 0; qb < QB; ++qb) S[kb][qb][r] = -INFINITY;
            }
      }
      // ---- online max (first tile, then only while the bound leaves room)
      if (tile == 0 || track) {
        const bool first = tile == 0;
        float delta[QB];
        bool any = first;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float mt = fmaxf(fmaxf(S[0][qb][0], S[0][qb][1]), fmaxf(S[0][qb][2], S[0][qb][3]));
#pragma unroll
          for (int kb = 1; kb < 4; ++kb)
            mt = fmaxf(mt, fmaxf(fmaxf(S[kb][qb][0], S[kb][qb][1]), fmaxf(S[kb][qb][2], S[kb][qb][3])));
          mt = max_across_groups(mt);
          delta[qb] = first ? mt : (mt > kTau ? mt : 0.f);
          any = any || (delta[qb] != 0.f);
        }
        if (__ballot(any)) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const float dl = delta[qb];
            m[qb] += dl;
            negm[qb] = f32x4{-m[qb], -m[qb], -m[qb], -m[qb]};
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int r = 0; r < 4; ++r) S[kb][qb][r] -= dl;
            if (!first) {
              const float al = __builtin_amdgcn_exp2f(-dl);
              l[qb] *= al;
#pragma unroll
              for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) O[db][qb][r] *= al;
            }
          }
        }
        bool need = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) need = need || (m[qb] < bound[qb] - kTauSkip);
        track = __ballot(need) != 0;
      }
      // ---- P = 2^S in fp16, row sums, O^T += V^T P^T
      f16x8 pf[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          f16x8 v;
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              const f32x2 e2 = {__builtin_amdgcn_exp2f(S[2 * c + half][qb][r]),
                                __builtin_amdgcn_exp2f(S[2 * c + half][qb][r + 1])};
              const f16x2 h2 = __builtin_convertvector(e2, f16x2);
              v[half * 4 + r] = h2[0];
              v[half * 4 + r + 1] = h2[1];
              l[qb] = __builtin_amdgcn_fdot2(h2, f16x2{(f16)1.f, (f16)1.f}, l[qb], false);
            }
          pf[qb][c] = v;
        }
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const f16x8 vf = *reinterpret_cast<const f16x8*>(Vs + lds_swz(db * 16 + j, c * 4 + gq));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) O[db][qb] = mfma16x16x32(vf, pf[qb][c], O[db][qb]);
        }
    }

    if (tile + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store O (in place of q), valid rows only
  if (wave_active) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lt = sum_across_groups(l[qb]);
      const float inv = 1.f / lt;
      const int row = qloc0 + qb * 16 + j;
      if (row < L) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          f16x4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = (f16)(O[db][qb][r] * inv);
          *reinterpret_cast<f16x4*>(qh + (seq0 + row) * kDh + db * 16 + 4 * gq) = o;
        }
      }
    }
  }
}

template <int QB, int NW>
static hipError_t launch_attn_t(const Plan& p, const Ptrs& a, hipStream_t st) {
  constexpr int BQ = NW * QB * 16;
  AttnArgs g;
  g.q = ws_q(p, a);
  g.k = ws_k(p, a);
  g.vt = ws_v(p, a);
  g.rows = p.rows;
  g.seq_stride = p.seq_stride;
  g.nseq = p.nseq;
  g.L = p.L;
  g.H = p.H;
  g.qtiles = (p.L + BQ - 1) / BQ;
  g.sc = ws_scalars(p, a);
  const int64_t blocks = (int64_t)g.qtiles * p.H * p.nseq;
  hipLaunchKernelGGL((attn_kernel<QB, NW>), dim3((unsigned)blocks), dim3(NW * 64), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_core(const Plan& p, const Ptrs& a, hipStream_t st) {
  if (p.attn_qb == 4 && p.attn_waves == 4) return launch_attn_t<4, 4>(p, a, st);
  if (p.attn_qb == 2 && p.attn_waves == 4) return launch_attn_t<2, 4>(p, a, st);
  return hipErrorInvalidValue;
}

}  // namespace vggt
