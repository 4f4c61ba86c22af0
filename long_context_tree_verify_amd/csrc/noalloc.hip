// hsv_verify_attn_noalloc: dense verification attention whose scratch (the
// split partials, their LSEs and row scales, the validation word, wide tree
// masks) lives in a library-owned device array instead of a caller workspace,
// for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ object, so every GPU the library runs
// on holds its own copy (at its own address) until the process ends.  Its
// name is only a host-side stand-in: the device address of each GPU's copy
// is looked up once per device with hipGetSymbolAddress and kept; only that
// address is handed to the kernels.  All calls on one GPU share its copy.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hsv.h"

namespace {

constexpr size_t kScratchBytes = HSV_NOALLOC_SCRATCH_BYTES;  // per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_lock;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch copy (looked up on first use, with
// the device current).  nullptr on a HIP error.
void *scratch_on(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> hold(g_lock);
  if (g_scratch_ptr[device]) return g_scratch_ptr[device];
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return nullptr;
  if (prev != device && hipSetDevice(device) != hipSuccess) return nullptr;
  void *ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (prev != device) (void)hipSetDevice(prev);
  if (e != hipSuccess || ptr == nullptr) return nullptr;
  g_scratch_ptr[device] = ptr;
  return ptr;
}

}  // namespace

extern "C" {

hsv_status hsv_verify_attn_noalloc(const hsv_verify_desc *d, const void *q, const void *k_cache,
                                   const void *v_cache, const int32_t *ctx_lens,
                                   const int32_t *parent, const uint64_t *anc_mask, void *o,
                                   float *lse, hipStream_t stream) {
  if (!d) return HSV_ERR_NULL;
  if (d->block_size != 0 || d->n_sel != 0) return HSV_ERR_SHAPE;
  size_t need = 0;
  const hsv_status st = hsv_verify_workspace_bytes(d, &need);
  if (st != HSV_OK) return st;
  if (need > kScratchBytes) return HSV_ERR_WORKSPACE;
  // Argument errors come before any runtime call, as in hsv_verify_attn:
  // the tree part needs exactly one of parent and anc_mask.
  if (!q || !k_cache || !v_cache || !ctx_lens || !o || !lse) return HSV_ERR_NULL;
  if (!(d->flags & HSV_FLAG_NO_TREE) && ((parent == nullptr) == (anc_mask == nullptr)))
    return HSV_ERR_NULL;
  int device = -1;
  if (hipStreamGetDevice(stream, &device) != hipSuccess) return HSV_ERR_HIP;
  void *ws = scratch_on(device);
  if (!ws) return HSV_ERR_HIP;
  // Nothing in the scratch needs to start at zero: the partial kernels write
  // every partial row (empty key ranges as lse = -inf) before the merge reads
  // it, and HSV_FLAG_VALIDATE clears its error word itself.
  return hsv_verify_attn(d, q, k_cache, v_cache, ctx_lens, parent, anc_mask, o, lse, ws,
                         kScratchBytes, stream);
}

}  // extern "C"
