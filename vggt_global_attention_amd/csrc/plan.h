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
// Workspace rows are padded to kRowAlign (8 XCDs x 256-row GEMM tiles, so
// each XCD walks whole token tiles) when that adds at most 1/64 of the rows,
// else to one 256-row tile (the GEMMs would compute more padding rows than
// the even XCD split saves).
constexpr int kRowAlign = 2048;
inline int64_t row_padding(int64_t cover) {
  const int64_t wide = (cover + kRowAlign - 1) / kRowAlign * kRowAlign;
  return wide - cover <= cover / 64 ? wide : (cover + 255) / 256 * 256;
}
// Key / value rows per head at most 2^28: the attention kernel's copies address
// eight v^T rows from one base with a 32-bit byte offset (8 * kv_rows * 2 < 2^32).
constexpr int64_t kMaxKvRows = (int64_t)1 << 28;
constexpr int kKvAlign = 256;       // compact key rows (subsampled mode) are padded to this
constexpr int kFrameRowAlign = 16;  // q / k rows of a frame set are padded to this
// Split attention tail: its partial-result buffer holds at most
// kSplitMaxRows query rows x key ranges; a split workgroup runs at most
// kSplitMaxWays key ranges of at least kSplitMinTiles key tiles each.
// Prep stage: per-workgroup partial maxima of the range bounds (X row norms
// over up to kBoundsX workgroups, V rows of Wqkv over kBoundsV, |Wo| over
// kBoundsO), reduced by the Wo conversion.
// The first kBoundsV workgroups also check the Q and K rows of Wqkv for
// non-finite values (their own partials, after the |Wo| ones).
constexpr int kBoundsX = 2048, kBoundsV = 64, kBoundsO = 128;
constexpr int kBoundsParts = kBoundsX + kBoundsV + kBoundsO + kBoundsV;
constexpr int kSplitMaxRows = 1 << 18;
constexpr int kSplitMaxWays = 32;
constexpr int kSplitMinTiles = 24;

// Options of the extended entry points.
struct CallOpts {
  int sub_h = 1, sub_w = 1;  // subsampled mode: windows
  int64_t q_begin = 0;       // global mode: first query row computed
  int64_t q_count = -1;      // global mode: query rows computed (-1: every row)
  // descriptor mode: the caller's key / value cache and its fill
  const void* cache = nullptr;
  size_t cache_bytes = 0;
  int64_t desc_capacity = 0;
  int64_t desc_count = 0;
  // CUs of the device the call runs on (tile choices); 0 when only sizing
  // the workspace, whose size never depends on the device
  int cus = 0;
  // the prep stage ORs its range bits into the workspace's status word
  // instead of replacing it (the blocks of a schedule after the first)
  bool keep_status = false;
  // bf16 attention operands (q, k, v, P, O and the Wo copy) instead of fp16
  bool bf16_ops = false;
  // register mode, Y != X: leave Y's patch rows unwritten (the layer schedule
  // reads only the special rows of a register block's output)
  bool no_patch_copy = false;
  // merged mode: frames per block, window rows / columns, merges per block
  // (frames == 0: only sizing the workspace, for the largest merged set)
  int httm_frames = 0, httm_wh = 0, httm_ww = 0, httm_r = 0;
};

// Descriptor key / value cache (caller-owned device buffer, 256-byte
// aligned): a Scalars header (xnorm = max norm of the appended descriptor
// rows, wvnorm = max norm of the V rows of Wqkv, pad = the power-of-two
// exponent the stored values carry, as int bits; kmax[H] = max key norm per
// head), then keys fp16 [H][cap_rows][64] and values fp16 [H][64][cap_rows]
// (keys permuted inside aligned groups of 16, as in the workspace).
struct DescLayout {
  int64_t cap_rows;
  size_t off_k, off_v, total;
};
inline DescLayout desc_layout(int H, int64_t capacity) {
  DescLayout L;
  L.cap_rows = (capacity + kKvAlign - 1) / kKvAlign * kKvAlign;
  const size_t hdr = (scalars_bytes(H) + 255) / 256 * 256;
  const size_t arr = (size_t)H * L.cap_rows * kDh * 2;
  L.off_k = hdr;
  L.off_v = hdr + arr;
  L.total = hdr + 2 * arr;
  return L;
}
constexpr int kDescEmpty = 127;  // exponent of an empty cache: above every real one

struct Plan {
  int mode;
  int S, T, d, H, gh, gw, off;
  float base, eps;
  // attention sets: nseq sequences of L tokens, sequence s starting at
  // workspace row s * seq_stride
  int nseq;
  int L;               // query rows of a set end here (= q0 + query count)
  int q0;              // first query row (a window of the global set), else 0
  int64_t seq_stride;
  int64_t rows;        // workspace rows held by q / k (multiple of 256)
  // v^T [H][64][vt_rows]: set s's keys start at column s * vt_seq_stride.  The
  // same as rows / seq_stride except for frame sets, whose q / k rows are
  // padded to 16 per frame and whose v^T columns to 64, so that a 64-key v^T
  // tile row is one aligned 128-byte line while the projections compute
  // fewer padding rows.  A workspace row w = s * seq_stride + t has its value
  // column at s * vt_seq_stride + t (vt_column()).
  int64_t vt_rows;
  int64_t vt_seq_stride;
  RowMap map;          // workspace row -> X row
  RowMap out_map;      // workspace row -> Y row (the window's rows only, when windowed)
  bool window;         // global mode restricted to query rows [q0, L)
  int rope_npos;       // entries per axis of the RoPE table
  int attn_qb;         // 32-query blocks per wave in the attention kernel
  int attn_waves;      // waves per attention workgroup (4 or 8)
  // keys / values of the attention sets: the q rows themselves, except in
  // subsampled mode, where they are a compact gathered copy of the kept
  // tokens (Lk of them, head stride kv_rows rows)
  int sub_h, sub_w;    // subsampling windows (1, 1 outside subsampled mode)
  int Lk;              // keys per set
  int64_t kv_rows;     // rows per head of the key / value buffers
  int64_t kv_seq_stride;
  int nD;              // subsampled mode: discarded tokens (mean-filled columns)
  // Split tail of a single-set attention grid (global sets, query windows,
  // subsampled and register sets): room for split_cap key-range units of
  // partial results (unnormalised O, reference, row sum); launch_core
  // decides from the device's CU count whether the last, partly filled round
  // of workgroups runs as key ranges that a merge kernel combines.
  int split_cap;
  bool keep_status;    // see CallOpts
  bool bf16_ops;       // see CallOpts
  bool patch_copy;     // register mode, Y != X: copy the patch rows (else see CallOpts)
  // merged mode (HTTM): blocks of hf frames x hwh x hww cells, hr merges per
  // block; the merged set has M tokens per head (L = Lk = M, kv_rows rows per
  // head in the merged buffers); merged values carry an extra 2^-hshift
  int hf, hwh, hww, hr, hshift;
  int64_t hper_run;    // merged tokens of a run of hf frames
  // workspace carve-up (byte offsets)
  size_t off_scal, off_bounds, off_rope, off_wo, off_q, off_k, off_v;
  size_t off_kc, off_vc, off_sums, off_part;  // subsampled mode only (else 0)
  size_t off_qc, off_nw, off_owner;           // merged mode only (kc / vc too; else 0)
  size_t off_split;    // [split_cap][BQ][64] fp32 O, then [split_cap][BQ] float2 (m, l)
  DescLayout desc;     // descriptor mode: layout of the key / value cache
  size_t total;
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
  char* cache;  // descriptor mode: the key / value cache (read-only there)
};

// Compute units of the current device (256 when it cannot be queried),
// cached per device.
int device_cu_count();

// Tuning overrides.  The product library reads no environment: its tile,
// split and GEMM choices depend on the shape and the device only, so a call
// gives the same bits whatever the caller's environment.  A separate tuning
// build (compiled with VGGT_ATTN_TUNING, libvggtattn_tune.so) reads these
// variables on every call, for sweeps and for tests that force a choice:
//   VGGT_ATTN_QB = 1 | 2      query blocks of 32 per attention wave
//   VGGT_ATTN_WAVES = 4 | 8   waves per attention workgroup
//   VGGT_ATTN_SPLIT = P       key ranges per split-tail workgroup (1: no split)
//   VGGT_GEMM = 0 | 1 | 2     projection kernel (128x128, 256x128 DMA, 256x256 DMA)
//   VGGT_GEMM_FGROUPS = g     weight slices an XCD walks
// Returns true and sets *value when the variable is set (tuning build only).
bool tuning_knob(const char* name, int* value);

// Fills `p`; returns VGGT_ATTN_OK or the shape / range status.  `o` carries
// the subsampling windows (VGGT_ATTN_MODE_SUBSAMPLED) or the query-row
// window (VGGT_ATTN_MODE_GLOBAL); defaults mean neither.
int make_plan(int mode, const vggt_attn_shape* s, const CallOpts& o, Plan* p);

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
// keys / values the attention loop streams (compact copies in subsampled and
// merged mode)
inline bool compact_kv(const Plan& p) {
  return p.mode == VGGT_ATTN_MODE_SUBSAMPLED || p.mode == VGGT_ATTN_MODE_MERGED;
}
inline f16* ws_kloop(const Plan& p, const Ptrs& a) {
  if (p.mode == VGGT_ATTN_MODE_DESCRIPTOR) return reinterpret_cast<f16*>(a.cache + p.desc.off_k);
  return reinterpret_cast<f16*>(a.ws + (compact_kv(p) ? p.off_kc : p.off_k));
}
inline f16* ws_vloop(const Plan& p, const Ptrs& a) {
  if (p.mode == VGGT_ATTN_MODE_DESCRIPTOR) return reinterpret_cast<f16*>(a.cache + p.desc.off_v);
  return reinterpret_cast<f16*>(a.ws + (compact_kv(p) ? p.off_vc : p.off_v));
}
// merged mode: merged queries (then their outputs) [H][kv_rows][64], key
// sizes [H][kv_rows] fp16, merged token of every token [H][S*T] int32
inline f16* ws_qc(const Plan& p, const Ptrs& a) { return reinterpret_cast<f16*>(a.ws + p.off_qc); }
inline f16* ws_nw(const Plan& p, const Ptrs& a) { return reinterpret_cast<f16*>(a.ws + p.off_nw); }
inline int32_t* ws_owner(const Plan& p, const Ptrs& a) {
  return reinterpret_cast<int32_t*>(a.ws + p.off_owner);
}
inline float* ws_sums(const Plan& p, const Ptrs& a) {
  return reinterpret_cast<float*>(a.ws + p.off_sums);
}

// Residual update of a layer schedule (prep.hip).
hipError_t launch_residual(const bf16* X, const bf16* Y, bf16* Z, int64_t rows, int d,
                           const float* gamma, int period, int active, bf16* C, int64_t c_stride,
                           hipStream_t st);

// Descriptor cache (desc.hip): fill an empty cache; append m descriptor
// tokens D [m][d] at position `count` (norm bounds, rescale of the stored
// values when the bound grows, then the K / V projection); copy the cache's
// bounds into a call's scalars (prep stage of the descriptor mode).
hipError_t launch_desc_init(char* cache, const DescLayout& L, int H, hipStream_t st);
hipError_t launch_desc_append(char* cache, const DescLayout& L, int H, int d, float eps,
                              int64_t count, const bf16* D, int64_t m, const bf16* Wqkv,
                              const float* kg, const float* kb, hipStream_t st);
hipError_t launch_desc_load(const Plan& p, const Ptrs& a, hipStream_t st);
// K / V projection of descriptor rows into the cache (gemm.hip).
hipError_t launch_desc_kv(char* cache, const DescLayout& L, int H, int d, float eps,
                          int64_t count, const bf16* D, int64_t m, const bf16* Wqkv,
                          const float* kg, const float* kb, hipStream_t st);
// Max row norm of `rows` rows of X (through `map`) into *out (atomic max; prep.hip).
hipError_t launch_rownorm_max(const bf16* X, int64_t rows, int d, RowMap map, float* out,
                              hipStream_t st);

// Subsampled mode: gather the kept tokens' keys / values and sum the
// discarded ones (first half of the CORE stage).
hipError_t launch_subsample(const Plan& p, const Ptrs& a, hipStream_t st);

// Merged mode (merge.hip): merge every head's tokens into the merged
// queries, keys and values (before the attention kernel), and give every
// token its merged token's output (after it).
hipError_t launch_merge(const Plan& p, const Ptrs& a, hipStream_t st);
hipError_t launch_unmerge(const Plan& p, const Ptrs& a, hipStream_t st);

// Merged mode: merged tokens of one block of nf frames and nd cells per
// frame with r merges (a block has (nf - 1) nd sources), and of the blocks of
// the first `wrows` window rows of a frame run of nf frames.  The same
// arithmetic on the host (the set's size) and on the device (where a strip's
// merged tokens start).
__host__ __device__ inline int64_t merged_block_count(int nf, int nd, int r) {
  const int64_t ns = (int64_t)(nf - 1) * nd;
  return (int64_t)nf * nd - (ns < r ? ns : (int64_t)r);
}
__host__ __device__ inline int64_t merged_run_count(int nf, int gh, int gw, int wh, int ww, int r,
                                                     int wrows) {
  int64_t c = 0;
  for (int wr = 0; wr < wrows; ++wr) {
    const int rh = gh - wr * wh < wh ? gh - wr * wh : wh;
    for (int c0 = 0; c0 < gw; c0 += ww) c += merged_block_count(nf, rh * (gw - c0 < ww ? gw - c0 : ww), r);
  }
  return c;
}
// A strip (one frame run x one window row, every window column) is merged by
// one workgroup holding the strip's keys in LDS: at most this many tokens.
constexpr int kMergeStripMax = 400;

}  // namespace vggt
