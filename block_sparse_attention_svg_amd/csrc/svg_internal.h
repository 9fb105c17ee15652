// Internal declarations shared by the HIP sources of libsvg (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/svg.h"

namespace svg {

// ---- error reporting (abi.hip) -------------------------------------------
svg_status fail(svg_status st, const char* fmt, ...);
svg_status check_launch(const char* what);

// ---- small helpers ---------------------------------------------------------
__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Division of non-negative int32 values by a run-time constant divisor with a
// multiply-high and a shift (Granlund & Montgomery, "Division by invariant
// integers using multiplication", 1994): q = (umulhi(n, magic) + n) >> shift,
// exact for 0 <= n < 2^31 and 1 <= d < 2^31.
struct FastDiv {
  uint32_t d, magic, shift;
  FastDiv() : d(1), magic(1), shift(0) {}
  explicit FastDiv(uint32_t divisor) : d(divisor) {
    shift = 0;
    while (shift < 32 && (1u << shift) < divisor) ++shift;
    uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << shift) - divisor)) / divisor + 1;
    magic = uint32_t(m);
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    uint32_t t = __umulhi(n, magic);
    return (t + n) >> shift;
  }
};

// ---- launchers (one per source file) ----------------------------------------
void launch_build_masks(const svg_shape& s, int band_w, uint8_t* masks, hipStream_t st);
void launch_restrict_anchor_rows(uint8_t* masks, int n_masks, const svg_shape& s,
                                 const int32_t* mask_sel, int k, hipStream_t st);
void launch_block_energy(const void* q, const void* k, const svg_shape& s, float scale, double* E,
                         hipStream_t st);
void launch_aggregate(const uint8_t* masks, int n_sets, int64_t elems, double rho, uint8_t* out,
                      hipStream_t st);
size_t row_similarity_workspace_bytes(const svg_shape& s);
void launch_row_similarity(const void* q, const void* k, const svg_shape& s, float scale, double* score,
                           void* ws, hipStream_t st);
void launch_calibrate(const double* E, int n_masks, int n_qb, int n_kb, double eps,
                      uint8_t* out, hipStream_t st);
void launch_encode(const uint8_t* dense, int n_masks, int n_qb, int n_kb, uint32_t* bitmap,
                   int32_t* row_ptr, int32_t* iv, hipStream_t st);
void launch_permute(const void* x, void* y, int elem_bytes, const svg_shape& s,
                    const int32_t* head_sel, int inverse, hipStream_t st);
void launch_norm_rope(const void* x, void* y, const svg_shape& s, int norm_span, const float* gamma,
                      float eps, const svg_rope* rope, const int32_t* head_layout, hipStream_t st);
void launch_row_broadcast(void* o, const svg_shape& s, const int32_t* head_sel, int k,
                          hipStream_t st);

struct AttnArgs {
  const void *q, *k, *v;
  void* o;
  const void *qp, *kp, *vp;
  void* op;
  const int32_t* row_ptr;
  const int32_t* iv;
  int n_masks, n_qb, n_kb;
  const int32_t* head_mask;
  const int32_t* head_layout;
  float* lse;
  int BH, N, D, block;
  float scale_log2;  // softmax scale times log2(e)
  void* vt;          // V of every head, block-transposed (128-key blocks)
  bool vt_given;     // vt holds the caller's prepared V^T (else the call fills it)
  int32_t* plan;     // workspace: per head, 9 pair indices splitting its pairs over the XCDs
  const uint32_t* bitmap;  // [n_masks][n_qb][ceil(n_kb/32)]
  // token-major index t < Nv is frame-major (t % F) * S + t / F (text tokens
  // keep their index): used for layout-1 heads whose twin qp / vp / op is NULL
  int F, S, Nv;
  FastDiv divF;
  // FP8 calls: dequantization factors, [3][BH] (q, k, v); q, k and vt then
  // hold E4M3 codes
  const float* f8_scales;
};
// frame-major index of token-major index t
__device__ __forceinline__ int frame_major_of(int t, const AttnArgs& a) {
  if (t >= a.Nv) return t;
  const int s = int(a.divF.div(uint32_t(t)));
  return (t - s * a.F) * a.S + s;
}
size_t attn_vt_bytes(int BH, int N, int D, int block);
size_t attn_workspace_bytes(int BH, int N, int D, int block, bool vt_given);
// V^T blocks of every head into a.vt (a.v, a.vp, a.head_layout, a.N, a.n_kb,
// a.BH, a.D, the permutation fields) and, when kp is given, the token-major K
// rows of the layout-1 heads
void launch_prepare_kv(const AttnArgs& a, const void* k, void* kp, hipStream_t st);
// Longest range of query-block pairs one XCD may take of a head: 1.5x the
// even split (edge rows of banded masks carry less work), at least the even
// split itself.
__host__ __device__ inline int plan_range_cap(int pairs) {
  const int a = (3 * pairs + 15) / 16, b = (pairs + 7) / 8;
  return a > b ? a : b;
}
// Bytes of the work plan at the end of the attention workspace: 9 split
// points per head, 8 list lengths, 8 queue heads, 8 work lists of (head,
// pair) int32 pairs,
// each of capacity BH * plan_range_cap(pairs), then the work of every
// (head, pair) as int32.
// int32 offset of the work lists in the plan (8-byte aligned)
__host__ __device__ inline size_t attn_plan_list_offset(int BH) { return (size_t(BH) * 9 + 16 + 1) & ~size_t(1); }
// int32 offset of the per-pair work in the plan
__host__ __device__ inline size_t attn_plan_work_offset(int BH, int pairs) {
  return attn_plan_list_offset(BH) + size_t(8) * BH * plan_range_cap(pairs) * 2;
}
inline size_t attn_plan_bytes(int BH, int pairs) {
  return (attn_plan_work_offset(BH, pairs) + size_t(BH) * pairs) * 4;
}
void launch_attn(const AttnArgs& a, hipStream_t st);
// FP8 attention (128-token blocks): a.q E4M3 codes frame-major, a.k each head
// in its layout, a.vt the V^T blocks of svg_quantize_fp8, a.f8_scales set
void launch_attn_fp8(const AttnArgs& a, hipStream_t st);
// E4M3 codes of q, k, v in the FP8 attention's layouts and the [3][BH]
// dequantization factors (a.N, a.D, a.BH, a.n_kb, a.head_layout and the
// permutation fields set)
void launch_quantize_fp8(const AttnArgs& a, const void* q, const void* k, const void* v, uint8_t* q8,
                         uint8_t* k8, uint8_t* vt8, float* scales, hipStream_t st);
// Host-side checks of an attention call and its AttnArgs (workspace, vt and
// plan pointers left to the caller): SVG_OK or the failing status.
svg_status attn_setup(const char* fn, const void* q, const void* k, const void* v, const void* vt,
                      void* o, const void* qp, const void* kp, const void* vp, void* op,
                      const svg_shape& s, float scale, const svg_mask* masks,
                      const int32_t* head_mask, const int32_t* head_layout, float* lse,
                      AttnArgs* out);

struct ProfileArgs {
  const void *q, *k, *v;
  const int32_t* idx;
  int n_samples;
  const uint32_t* bitmap;  // [2][nB][W]
  int nB, W;
  int32_t* choice;
  float* err;
  float* ws;
  int BH, N, D, block, F, Hs, Ws;
  int chunk_keys, n_chunks;
  float scale_log2;
};
size_t profile_workspace_bytes(int BH, int N, int D, int block, int n_samples,
                               int* chunk_keys, int* n_chunks);
void launch_profile(const ProfileArgs& a, hipStream_t st);

}  // namespace svg
