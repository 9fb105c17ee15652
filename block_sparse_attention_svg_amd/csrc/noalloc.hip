// svg_block_sparse_attn_noalloc: the attention call for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its only scratch buffer, the work plan of
// the 128-token-block kernels (split points, per-XCD work lists and queue
// heads), lives in a file-scope device array of fixed size; V^T comes from the
// caller (svg_prepare_kv).  The kernels are the ones svg_block_sparse_attn
// launches, so both calls give the same bits.
#include <mutex>

#include "svg_internal.h"

namespace svg {
namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;

// One copy per GPU the library runs on, held until the process ends.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array, looked up once per device with
// that device current (the array's host-side name is not a device address).
svg_status scratch_ptr(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SVG_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SVG_ERR_UNSUPPORTED, "%s: device %d beyond the %d supported", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SVG_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return SVG_OK;
}

}  // namespace
}  // namespace svg

using namespace svg;

extern "C" {

size_t svg_noalloc_scratch_bytes(void) { return kScratchBytes; }

svg_status svg_block_sparse_attn_noalloc(const void* q, const void* k, const void* v, const void* vt,
                                         void* o, const void* qp, const void* kp, const void* vp,
                                         void* op, svg_shape s, float scale, const svg_mask* masks,
                                         const int32_t* head_mask, const int32_t* head_layout,
                                         float* lse, void* stream) {
  const char* fn = "svg_block_sparse_attn_noalloc";
  AttnArgs a;
  if (svg_status st = attn_setup(fn, q, k, v, vt, o, qp, kp, vp, op, s, scale, masks, head_mask,
                                 head_layout, lse, &a))
    return st;
  if (s.block == 128) {
    if (!vt)
      return fail(SVG_ERR_INVALID_ARG, "%s: 128-token blocks need the caller's V^T (svg_prepare_kv)", fn);
    const size_t need = attn_workspace_bytes(a.BH, s.N, s.D, s.block, true);
    if (need > kScratchBytes)
      return fail(SVG_ERR_CAPACITY, "%s: the work plan needs %zu bytes, the scratch holds %zu", fn, need,
                  kScratchBytes);
    void* p = nullptr;
    if (svg_status st = scratch_ptr(fn, &p)) return st;
    a.plan = static_cast<int32_t*>(p);
  }
  launch_attn(a, reinterpret_cast<hipStream_t>(stream));
  return check_launch(fn);
}

}  // extern "C"
