// moe_dispatch_noalloc: moe_dispatch with its workspace in a fixed,
// file-scope device array instead of a caller-provided buffer, for callers
// that cannot allocate (code under stream capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array lives in the library's code object, so every GPU the library
// runs on holds its own copy from module load until the process ends.  Its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and kept; host code never passes the array's own
// name to a kernel, only that address.  Every call on a GPU shares that
// GPU's copy: calls that overlap on one GPU (different streams, no ordering
// between them) race on it.  The dispatch kernels fully overwrite what they
// read of it, so nothing needs clearing between calls.

#include <mutex>

#include "moe_internal.h"

namespace moe {
int dispatch_impl(const void* x, int act_dtype, const int32_t* idx, int T, int H,
                  int E, int k, int e_begin, int e_end, int32_t* counts,
                  int32_t* offsets, int32_t* slot_of, int32_t* row_token,
                  void* x_perm, float* x_scale, void* ws, hipStream_t s);
size_t dispatch_ws_bytes(int T, int E);
}  // namespace moe

namespace {

constexpr size_t kScratchBytes = (size_t)1 << 20;  // MOE_NOALLOC_SCRATCH_BYTES
constexpr int kMaxDevices = 64;

static_assert(kScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "header and library agree");

__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {nullptr};

// Device address of this device's copy of `scratch`, or nullptr on failure.
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

bool act_ok(int dt) {
  return dt == MOE_DTYPE_F32 || dt == MOE_DTYPE_F16 || dt == MOE_DTYPE_BF16;
}

}  // namespace

extern "C" int moe_dispatch_noalloc(const void* x, int act_dtype, const int32_t* topk_idx,
                                    int T, int H, int E, int k, int e_begin, int e_end,
                                    int32_t* counts, int32_t* offsets, int32_t* slot_of,
                                    int32_t* row_token, void* x_perm, hipStream_t stream) {
  // the same validation as moe_dispatch, then the size limit of the array
  if (!act_ok(act_dtype)) return MOE_ERR_UNSUPPORTED;
  if (T < 0 || H < 1 || E < 1 || E > 1024 || k < 1 || k > E || k > 32) return MOE_ERR_ARG;
  if ((long long)T * k >= (1ll << 31)) return MOE_ERR_ARG;
  if (e_begin < 0 || e_end < e_begin || e_end > E) return MOE_ERR_ARG;
  if ((H * (act_dtype == MOE_DTYPE_F32 ? 4 : 2)) % 16) return MOE_ERR_ARG;
  if (!counts || !offsets) return MOE_ERR_ARG;
  if (T > 0 && (!x || !topk_idx || !slot_of || !row_token)) return MOE_ERR_ARG;
  if (T > 0 && e_end > e_begin && !x_perm) return MOE_ERR_ARG;
  if (((uintptr_t)x & 15) || ((uintptr_t)x_perm & 15)) return MOE_ERR_ARG;
  if (moe::dispatch_ws_bytes(T, E) > kScratchBytes) return MOE_ERR_TOO_LARGE;
  void* ws = scratch_of_current_device();
  if (ws == nullptr) return MOE_ERR_HIP;
  return moe::dispatch_impl(x, act_dtype, topk_idx, T, H, E, k, e_begin, e_end, counts,
                            offsets, slot_of, row_token, x_perm, nullptr, ws, stream);
}
