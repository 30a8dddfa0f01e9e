// The Aggregator's layer schedule over the attention blocks: every layer runs
// a frame block and then an inter-frame block, each as a residual branch with
// a per-channel LayerScale ("VGGT-Omega Aggregator explainer", section 三); the
// inter-frame block is in register mode at the chosen layers and global
// elsewhere, optionally frame attention in early layers and subsampled global
// attention in the rest (AVGGT summary, technical summary 2B) or global
// attention with HTTM token merging (HTTM article, section 02); the token
// states after both blocks of the cached layers are kept side by side
// (section 四).
//
// Everything is checked on the host before the first launch, so a rejected
// call enqueues nothing.  The whole forward is then 2 * n_layers block calls
// and residual updates on one stream; the block workspace that every call
// reuses starts the workspace (so its range status word is the schedule's:
// every block after the first ORs its bits in), the block output Y follows.
#include "entry.h"

namespace vggt {
namespace {

constexpr int kMaxLayers = 64;

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool bit(uint64_t m, int l) { return (m >> l) & 1u; }

// Mode of layer l's inter-frame block.
int inter_mode(const vggt_attn_schedule& sc, int l) {
  if (bit(sc.register_layers, l)) return VGGT_ATTN_MODE_REGISTER;
  if (l < sc.early_frame) return VGGT_ATTN_MODE_FRAME;
  if (sc.merge_frames > 0) return VGGT_ATTN_MODE_MERGED;
  if (sc.sub_h > 1 || sc.sub_w > 1) return VGGT_ATTN_MODE_SUBSAMPLED;
  return VGGT_ATTN_MODE_GLOBAL;
}

int check_schedule(const vggt_attn_schedule* sc) {
  if (!sc) return VGGT_ATTN_EINVAL;
  if (sc->n_layers < 1 || sc->n_layers > kMaxLayers) return VGGT_ATTN_ESHAPE;
  const uint64_t valid = sc->n_layers == 64 ? ~0ull : ((1ull << sc->n_layers) - 1);
  if ((sc->register_layers & ~valid) || (sc->cached_layers & ~valid)) return VGGT_ATTN_ERANGE;
  if (sc->early_frame < 0 || sc->early_frame > sc->n_layers) return VGGT_ATTN_ERANGE;
  if (sc->sub_h < 1 || sc->sub_w < 1) return VGGT_ATTN_ERANGE;
  if (sc->merge_frames < 0) return VGGT_ATTN_ERANGE;
  if (sc->merge_frames > 0 && (sc->sub_h > 1 || sc->sub_w > 1 || sc->merge_win_h < 1 ||
                               sc->merge_win_w < 1 || sc->merge_r < 0))
    return VGGT_ATTN_ERANGE;
  return VGGT_ATTN_OK;
}

// Call options of a block of the schedule in `mode`.
CallOpts block_opts(const vggt_attn_schedule& sc, int mode) {
  CallOpts o;
  if (mode == VGGT_ATTN_MODE_SUBSAMPLED) {
    o.sub_h = sc.sub_h;
    o.sub_w = sc.sub_w;
  }
  if (mode == VGGT_ATTN_MODE_MERGED) {
    o.httm_frames = sc.merge_frames;
    o.httm_wh = sc.merge_win_h;
    o.httm_ww = sc.merge_win_w;
    o.httm_r = sc.merge_r;
  }
  return o;
}

// Block workspace: the largest need over the modes the schedule uses.
size_t block_ws_bytes(const vggt_attn_shape* s, const vggt_attn_schedule& sc) {
  size_t need = vggt_attn_workspace_bytes(VGGT_ATTN_MODE_FRAME, s);
  if (need == 0) return 0;
  for (int l = 0; l < sc.n_layers; ++l) {
    const size_t n = vggt_attn_workspace_bytes(inter_mode(sc, l), s);
    if (n == 0) return 0;
    if (n > need) need = n;
  }
  return need;
}

size_t y_bytes(const vggt_attn_shape* s) {
  return (size_t)round_up((int64_t)s->S * s->T * s->d * 2, 256);
}

}  // namespace
}  // namespace vggt

using namespace vggt;

extern "C" {

size_t vggt_attn_schedule_workspace_bytes(const vggt_attn_shape* shape,
                                          const vggt_attn_schedule* sched) {
  if (!shape || check_schedule(sched) != VGGT_ATTN_OK) return 0;
  const size_t blk = block_ws_bytes(shape, *sched);
  return blk ? y_bytes(shape) + blk : 0;
}

int vggt_attn_schedule_run(const vggt_attn_shape* shape, const vggt_attn_schedule* sched,
                           const vggt_attn_block_weights* blocks, const void* X, void* state,
                           void* caches, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_schedule(sched);
  if (st != VGGT_ATTN_OK) return st;
  if (!shape || !blocks || !X || !state || !workspace) return VGGT_ATTN_EINVAL;
  const vggt_attn_schedule sc = *sched;
  const size_t blk = block_ws_bytes(shape, sc);
  if (blk == 0) return VGGT_ATTN_ESHAPE;
  if (!aligned(workspace, 256)) return VGGT_ATTN_EALIGN;
  if (workspace_bytes < y_bytes(shape) + blk) return VGGT_ATTN_EWORKSPACE;
  const int64_t rows = (int64_t)shape->S * shape->T;
  const int d = shape->d;
  const size_t nx = (size_t)rows * d * 2;
  char* ws = reinterpret_cast<char*>(workspace);
  void* bws = ws;
  void* Y = ws + blk;
  const int ncache = caches ? __builtin_popcountll(sc.cached_layers) : 0;
  const size_t ncb = (size_t)ncache * nx * 2;
  // state is X itself or disjoint from it; state and the caches stay clear of
  // the workspace, of each other and of every weight
  if (state != X && overlap(state, nx, X, nx)) return VGGT_ATTN_EINVAL;
  if (overlap(state, nx, workspace, workspace_bytes) || overlap(caches, ncb, workspace,
                                                                workspace_bytes) ||
      overlap(caches, ncb, state, nx) || overlap(caches, ncb, X, nx))
    return VGGT_ATTN_EINVAL;
  if (caches && !aligned(caches, 16)) return VGGT_ATTN_EALIGN;
  const size_t nw = (size_t)3 * d * d * 2, no = (size_t)d * d * 2, ng = (size_t)d * 4;
  for (int b = 0; b < 2 * sc.n_layers; ++b) {
    const vggt_attn_block_weights& w = blocks[b];
    const int mode = (b & 1) ? inter_mode(sc, b >> 1) : VGGT_ATTN_MODE_FRAME;
    const CallOpts o = block_opts(sc, mode);
    Plan plan;
    const void* in = (b == 0) ? X : state;
    st = check_call(mode, shape, o, in, w.Wqkv, w.Wo, w.q_gamma, w.q_beta, w.k_gamma, w.k_beta,
                    Y, bws, blk, &plan);
    if (st != VGGT_ATTN_OK) return st;
    st = check_residual(in, Y, state, rows, d, w.layer_scale, 1, 1, caches, 2 * (int64_t)d);
    if (st != VGGT_ATTN_OK) return st;
    const void* wp[7] = {w.Wqkv, w.Wo, w.q_gamma, w.q_beta, w.k_gamma, w.k_beta, w.layer_scale};
    const size_t wn[7] = {nw, no, ng, ng, ng, ng, ng};
    for (int i = 0; i < 7; ++i)
      if (overlap(wp[i], wn[i], state, nx) || overlap(wp[i], wn[i], caches, ncb) ||
          overlap(wp[i], wn[i], workspace, workspace_bytes))
        return VGGT_ATTN_EINVAL;
  }

  // enqueue: nothing below can fail on arguments any more
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  bf16* C = reinterpret_cast<bf16*>(caches);
  int k = 0;  // caches written so far
  for (int l = 0; l < sc.n_layers; ++l) {
    const bool keep = C && bit(sc.cached_layers, l);
    bf16* cache = keep ? C + (size_t)k * rows * 2 * d : nullptr;
    for (int half = 0; half < 2; ++half) {
      const vggt_attn_block_weights& w = blocks[2 * l + half];
      const int mode = half ? inter_mode(sc, l) : VGGT_ATTN_MODE_FRAME;
      CallOpts o = block_opts(sc, mode);
      o.keep_status = l > 0 || half > 0;
      // the residual update below reads only the special rows of a register
      // block's output: its patch rows are not copied
      o.no_patch_copy = true;
      const void* in = (l == 0 && half == 0) ? X : state;
      st = run(mode, o, VGGT_ATTN_STAGE_PREP, VGGT_ATTN_STAGE_OUT, shape, in, w.Wqkv, w.Wo,
               w.q_gamma, w.q_beta, w.k_gamma, w.k_beta, Y, bws, blk, stream);
      if (st != VGGT_ATTN_OK) return st;
      // register mode changes only the 17 special rows of every frame
      const int period = mode == VGGT_ATTN_MODE_REGISTER ? shape->T : 1;
      const int active = mode == VGGT_ATTN_MODE_REGISTER ? kSpecial : 1;
      hipError_t e = launch_residual(reinterpret_cast<const bf16*>(in),
                                     reinterpret_cast<const bf16*>(Y), reinterpret_cast<bf16*>(state),
                                     rows, d, w.layer_scale, period, active,
                                     cache ? cache + half * d : nullptr, 2 * (int64_t)d, hs);
      if (e != hipSuccess) return VGGT_ATTN_EHIP;
    }
    if (keep) ++k;
  }
  return VGGT_ATTN_OK;
}

}  // extern "C"
