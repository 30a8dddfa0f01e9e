// Host-side planning for one libvggtattn call: sequence layout in the
// workspace, workspace carve-up and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"
#include "libvggtattn.h"

namespace vggt {

constexpr int kGemmBM = 128;        // token rows per GEMM tile
constexpr int kGemmBN = 128;        // output features per GEMM tile (two heads)
constexpr int kGemmBK = 64;
constexpr int kAttnBK = 64;         // keys per attention tile
constexpr int kRowAlign = 256;      // workspace rows are padded to this

struct Plan {
  int mode;
  int S, T, d, H, gh, gw, off;
  float base, eps;
  // attention sets: nseq sequences of L tokens, sequence s starting at
  // workspace row s * seq_stride
  int nseq;
  int L;
  int64_t seq_stride;
  int64_t rows;        // workspace rows held by q/k/v (multiple of kRowAlign)
  RowMap map;          // workspace row -> X row
  int rope_npos;       // entries per axis of the RoPE table
  int attn_qb;         // 32-query blocks per wave in the attention kernel
  int attn_waves;      // waves per attention workgroup (4 or 8)
  // workspace carve-up (byte offsets)
  size_t off_scal, off_rope, off_wo, off_q, off_k, off_v, total;
};

struct Ptrs {
  const bf16* X;
  const bf16* Wqkv;
  const bf16* Wo;
  const float* qg;
  const float* qb;
  const float* kg;
  const float* kb;
  bf16* Y;
  char* ws;
};

// Fills `p`; returns VGGT_ATTN_OK or the shape / range status.
int make_plan(int mode, const vggt_attn_shape* s, Plan* p);

hipError_t launch_prep(const Plan& p, const Ptrs& a, hipStream_t st);
hipError_t launch_qkv(const Plan& p, const Ptrs& a, hipStream_t st);
hipError_t launch_core(const Plan& p, const Ptrs& a, hipStream_t st);
hipError_t launch_out(const Plan& p, const Ptrs& a, hipStream_t st);

inline Scalars* ws_scalars(const Plan& p, const Ptrs& a) {
  return reinterpret_cast<Scalars*>(a.ws + p.off_scal);
}
inline float2* ws_rope(const Plan& p, const Ptrs& a) {
  return reinterpret_cast<float2*>(a.ws + p.off_rope);
}
inline f16* ws_wo(const Plan& p, const Ptrs& a) { return reinterpret_cast<f16*>(a.ws + p.off_wo); }
inline f16* ws_q(const Plan& p, const Ptrs& a) { return reinterpret_cast<f16*>(a.ws + p.off_q); }
inline f16* ws_k(const Plan& p, const Ptrs& a) { return reinterpret_cast<f16*>(a.ws + p.off_k); }
inline f16* ws_v(const Plan& p, const Ptrs& a) { return reinterpret_cast<f16*>(a.ws + p.off_v); }

}  // namespace vggt
