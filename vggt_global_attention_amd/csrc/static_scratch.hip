// The block call without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The workspace is a fixed-size array of
// the library's own, one copy per device, that lives until the process ends.
//
// Host code never uses the array's name as an address: on the host it names
// a stand-in, not the device copy.  Each device's copy is looked up once, with
// that device current, through hipGetSymbolAddress, and that pointer is what
// the kernels receive.  Every call on a device shares its copy; the prep
// stage of a call rewrites every scratch value a later stage reads (bounds,
// cleared key norms and sums, the status word), so nothing has to be cleared
// between calls, but two calls that overlap in time on one device race.
#include <atomic>
#include <mutex>

#include "entry.h"

namespace vggt {

static_assert(VGGT_ATTN_STATIC_SCRATCH_BYTES % 256 == 0, "scratch size");

static __device__ __attribute__((aligned(256))) char scratch[VGGT_ATTN_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// This device's copy of `scratch` (looked up once per device), or nullptr.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace
}  // namespace vggt

using namespace vggt;

extern "C" int vggt_attn_block_noalloc(int mode, const vggt_attn_shape* shape, const void* X,
                                       const void* Wqkv, const void* Wo, const float* q_gamma,
                                       const float* q_beta, const float* k_gamma,
                                       const float* k_beta, void* Y, void* stream) {
  if (mode != VGGT_ATTN_MODE_FRAME && mode != VGGT_ATTN_MODE_GLOBAL &&
      mode != VGGT_ATTN_MODE_REGISTER)
    return VGGT_ATTN_EINVAL;
  // Every argument is checked before the first HIP call, first against a
  // stand-in workspace: as large as the call needs, 256-byte aligned, at the
  // top of the address space where no buffer of the caller can lie.
  Plan plan;
  const size_t need = vggt_attn_workspace_bytes(mode, shape);  // 0: bad shape (reported below)
  void* const stand_in =
      reinterpret_cast<void*>((~static_cast<uintptr_t>(0) - need - 256) & ~static_cast<uintptr_t>(255));
  int st = check_call(mode, shape, CallOpts(), X, Wqkv, Wo, q_gamma, q_beta, k_gamma, k_beta, Y,
                      stand_in, need, &plan);
  if (st != VGGT_ATTN_OK) return st;
  if (plan.total > (size_t)VGGT_ATTN_STATIC_SCRATCH_BYTES) return VGGT_ATTN_ESCRATCH;
  void* ws = scratch_ptr();
  if (!ws) return VGGT_ATTN_EHIP;
  return run(mode, CallOpts(), VGGT_ATTN_STAGE_PREP, VGGT_ATTN_STAGE_OUT, shape, X, Wqkv, Wo,
             q_gamma, q_beta, k_gamma, k_beta, Y, ws, VGGT_ATTN_STATIC_SCRATCH_BYTES, stream);
}
