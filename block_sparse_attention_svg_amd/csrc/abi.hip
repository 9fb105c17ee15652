// C ABI of libsvg: host-side argument validation, then kernel launches.
// Validation happens before any HIP call, so every error path can be checked
// without a GPU.  The library allocates nothing and keeps no state besides a
// thread-local error message.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>

#include "svg_internal.h"

namespace svg {

static thread_local char g_err[512] = "";

svg_status fail(svg_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

svg_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SVG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return SVG_OK;
}

namespace {

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int n_blocks(const svg_shape& s) { return ceil_div(s.N, s.block); }

svg_status check_shape(const svg_shape& s, const char* fn) {
  if (s.B < 1 || s.H < 1 || s.N < 1 || s.D < 1)
    return fail(SVG_ERR_INVALID_ARG, "%s: B, H, N, D must be positive (got %d, %d, %d, %d)", fn,
                s.B, s.H, s.N, s.D);
  if (s.F < 1 || s.Hs < 1 || s.Ws < 1)
    return fail(SVG_ERR_INVALID_ARG, "%s: F, Hs, Ws must be positive", fn);
  if (int64_t(s.F) * s.Hs * s.Ws > s.N)
    return fail(SVG_ERR_INVALID_ARG, "%s: F*Hs*Ws = %lld exceeds N = %d", fn,
                (long long)(int64_t(s.F) * s.Hs * s.Ws), s.N);
  if (s.block != 64 && s.block != 128)
    return fail(SVG_ERR_UNSUPPORTED, "%s: block must be 64 or 128 (got %d)", fn, s.block);
  if (int64_t(s.B) * s.H > 65535)
    return fail(SVG_ERR_UNSUPPORTED, "%s: B*H = %lld exceeds 65535", fn, (long long)(int64_t(s.B) * s.H));
  if (s.N > (1 << 30)) return fail(SVG_ERR_UNSUPPORTED, "%s: N = %d exceeds 2^30", fn, s.N);
  return SVG_OK;
}

svg_status check_head_dim(const svg_shape& s, const char* fn) {
  if (s.D != 64 && s.D != 128)
    return fail(SVG_ERR_UNSUPPORTED, "%s: head dim must be 64 or 128 (got %d)", fn, s.D);
  return SVG_OK;
}

svg_status check_mask(const svg_mask* m, const svg_shape& s, const char* fn, int want_masks) {
  if (!m) return fail(SVG_ERR_INVALID_ARG, "%s: mask struct is NULL", fn);
  if (!m->bitmap || !m->row_ptr || !m->iv)
    return fail(SVG_ERR_INVALID_ARG, "%s: mask bitmap / row_ptr / iv is NULL", fn);
  if (m->n_masks < 1) return fail(SVG_ERR_INVALID_ARG, "%s: n_masks must be >= 1", fn);
  if (want_masks > 0 && m->n_masks != want_masks)
    return fail(SVG_ERR_INVALID_ARG, "%s: expected %d masks, got %d", fn, want_masks, m->n_masks);
  int nB = n_blocks(s);
  if (m->n_qb != nB || m->n_kb != nB)
    return fail(SVG_ERR_INVALID_ARG, "%s: mask is %d x %d blocks, shape needs %d x %d", fn,
                m->n_qb, m->n_kb, nB, nB);
  return SVG_OK;
}

bool overlaps(const void* a, const void* b, size_t bytes) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + bytes && y < x + bytes;
}

// [a, a + a_bytes) and [b, b + b_bytes) share a byte
bool overlaps(const void* a, size_t a_bytes, const void* b, size_t b_bytes) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + b_bytes && y < x + a_bytes;
}

}  // namespace

svg_status attn_setup(const char* fn, const void* q, const void* k, const void* v, const void* vt,
                      void* o, const void* qp, const void* kp, const void* vp, void* op,
                      const svg_shape& s, float scale, const svg_mask* masks,
                      const int32_t* head_mask, const int32_t* head_layout, float* lse,
                      AttnArgs* out) {
  if (svg_status st = check_shape(s, fn)) return st;
  if (svg_status st = check_head_dim(s, fn)) return st;
  if (vt && s.block != 128)
    return fail(SVG_ERR_INVALID_ARG, "%s: vt is for 128-token blocks only", fn);
  if (!q || !k || !o || (!v && !vt)) return fail(SVG_ERR_INVALID_ARG, "%s: NULL q / k / v / o", fn);
  if (head_layout && !kp)
    return fail(SVG_ERR_INVALID_ARG, "%s: head_layout given but kp is NULL", fn);
  if (head_layout && s.block != 128 && (!qp || !vp || !op))
    return fail(SVG_ERR_INVALID_ARG, "%s: 64-token blocks need all token-major twins with head_layout", fn);
  if (!(scale > 0.f)) return fail(SVG_ERR_INVALID_ARG, "%s: scale must be positive", fn);
  if (svg_status st = check_mask(masks, s, fn, 0)) return st;
  const size_t bytes = size_t(s.B) * s.H * s.N * s.D * 2;
  if (overlaps(o, q, bytes) || overlaps(o, k, bytes) || (v && overlaps(o, v, bytes)) ||
      (vt && overlaps(o, bytes, vt, attn_vt_bytes(s.B * s.H, s.N, s.D, s.block))))
    return fail(SVG_ERR_INVALID_ARG, "%s: o overlaps an input", fn);
  if (vt && (reinterpret_cast<uintptr_t>(vt) & 15))
    return fail(SVG_ERR_INVALID_ARG, "%s: vt must be 16-byte aligned", fn);
  if (s.block == 128 && ((n_blocks(s) + 1) / 2 > 65535 || masks->n_masks > 32768))
    return fail(SVG_ERR_UNSUPPORTED, "%s: 128-token blocks support up to 131070 blocks and 32768 masks",
                fn);
  AttnArgs& a = *out;
  a = AttnArgs{};
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.qp = qp; a.kp = kp; a.vp = vp; a.op = op;
  a.row_ptr = masks->row_ptr;
  a.iv = masks->iv;
  a.n_masks = masks->n_masks;
  a.n_qb = masks->n_qb;
  a.n_kb = masks->n_kb;
  a.head_mask = head_mask;
  a.head_layout = head_layout;
  a.lse = lse;
  a.BH = s.B * s.H;
  a.N = s.N; a.D = s.D; a.block = s.block;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.vt = const_cast<void*>(vt);
  a.vt_given = vt != nullptr;
  a.plan = nullptr;
  a.bitmap = masks->bitmap;
  a.F = s.F;
  a.S = s.Hs * s.Ws;
  a.Nv = s.F * s.Hs * s.Ws;
  a.divF = FastDiv(uint32_t(s.F > 0 ? s.F : 1));
  return SVG_OK;
}

}  // namespace svg

using namespace svg;

extern "C" {

const char* svg_status_string(svg_status st) {
  switch (st) {
    case SVG_OK: return "SVG_OK";
    case SVG_ERR_INVALID_ARG: return "SVG_ERR_INVALID_ARG";
    case SVG_ERR_UNSUPPORTED: return "SVG_ERR_UNSUPPORTED";
    case SVG_ERR_CAPACITY: return "SVG_ERR_CAPACITY";
    case SVG_ERR_HIP: return "SVG_ERR_HIP";
  }
  return "SVG_ERR_UNKNOWN";
}

const char* svg_last_error(void) { return g_err; }

const char* svg_version(void) { return "svg-mi355x 0.1 gfx950"; }

svg_status svg_build_masks(svg_shape s, int band_w, uint8_t* masks, void* stream) {
  const char* fn = "svg_build_masks";
  if (svg_status st = check_shape(s, fn)) return st;
  if (!masks) return fail(SVG_ERR_INVALID_ARG, "%s: masks is NULL", fn);
  if (band_w < 0) return fail(SVG_ERR_INVALID_ARG, "%s: band_w must be >= 0", fn);
  launch_build_masks(s, band_w, masks, as_stream(stream));
  return check_launch(fn);
}

int64_t svg_encode_iv_capacity(int n_masks, int n_qb, int n_kb) {
  if (n_masks < 1 || n_qb < 1 || n_kb < 1) return 0;
  return int64_t(n_masks) * n_qb * ((n_kb + 1) / 2);
}

svg_status svg_encode_mask(const uint8_t* dense, int n_masks, int n_qb, int n_kb, uint32_t* bitmap,
                           int32_t* row_ptr, int32_t* iv, int64_t iv_capacity, void* stream) {
  const char* fn = "svg_encode_mask";
  if (!dense || !bitmap || !row_ptr || !iv)
    return fail(SVG_ERR_INVALID_ARG, "%s: NULL buffer", fn);
  if (n_masks < 1 || n_qb < 1 || n_kb < 1)
    return fail(SVG_ERR_INVALID_ARG, "%s: n_masks, n_qb, n_kb must be positive", fn);
  if (int64_t(n_masks) * n_qb > (1 << 28))
    return fail(SVG_ERR_UNSUPPORTED, "%s: too many rows", fn);
  int64_t need = svg_encode_iv_capacity(n_masks, n_qb, n_kb);
  if (iv_capacity < need)
    return fail(SVG_ERR_CAPACITY, "%s: iv_capacity %lld below worst case %lld", fn,
                (long long)iv_capacity, (long long)need);
  if (need > (int64_t(1) << 31) - 1)
    return fail(SVG_ERR_UNSUPPORTED, "%s: interval count exceeds int32", fn);
  launch_encode(dense, n_masks, n_qb, n_kb, bitmap, row_ptr, iv, as_stream(stream));
  return check_launch(fn);
}

svg_status svg_permute(const void* x, void* y, svg_dtype dt, svg_shape s, const int32_t* head_sel,
                       int inverse, void* stream) {
  const char* fn = "svg_permute";
  if (svg_status st = check_shape(s, fn)) return st;
  if (!x || !y) return fail(SVG_ERR_INVALID_ARG, "%s: x or y is NULL", fn);
  if (dt != SVG_BF16 && dt != SVG_F32) return fail(SVG_ERR_INVALID_ARG, "%s: unknown dtype", fn);
  int esz = dt == SVG_BF16 ? 2 : 4;
  if (s.D != 64 && s.D != 128)
    return fail(SVG_ERR_UNSUPPORTED, "%s: head dim must be 64 or 128 (got %d)", fn, s.D);
  size_t bytes = size_t(s.B) * s.H * s.N * s.D * esz;
  if (overlaps(x, y, bytes)) return fail(SVG_ERR_INVALID_ARG, "%s: x and y overlap", fn);
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15)
    return fail(SVG_ERR_INVALID_ARG, "%s: x and y must be 16-byte aligned", fn);
  launch_permute(x, y, esz, s, head_sel, inverse, as_stream(stream));
  return check_launch(fn);
}

svg_status svg_qk_norm_rope(const void* x, void* y, svg_shape s, int norm_span, const float* gamma,
                            float eps, const svg_rope* rope, const int32_t* head_layout,
                            void* stream) {
  const char* fn = "svg_qk_norm_rope";
  if (svg_status st = check_shape(s, fn)) return st;
  if (svg_status st = check_head_dim(s, fn)) return st;
  if (!x || !y) return fail(SVG_ERR_INVALID_ARG, "%s: x or y is NULL", fn);
  if (s.H * s.D > 8192)
    return fail(SVG_ERR_UNSUPPORTED, "%s: H*D = %d exceeds 8192", fn, s.H * s.D);
  size_t bytes = size_t(s.B) * s.H * s.N * s.D * 2;
  if (overlaps(x, y, bytes)) return fail(SVG_ERR_INVALID_ARG, "%s: x and y overlap", fn);
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15)
    return fail(SVG_ERR_INVALID_ARG, "%s: x and y must be 16-byte aligned", fn);
  if (norm_span < 0 || norm_span > 2)
    return fail(SVG_ERR_INVALID_ARG, "%s: norm_span must be 0, 1 or 2 (got %d)", fn, norm_span);
  if (!(eps >= 0.f) || !std::isfinite(eps))
    return fail(SVG_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
  if (gamma && (reinterpret_cast<uintptr_t>(gamma) & 15))
    return fail(SVG_ERR_INVALID_ARG, "%s: gamma must be 16-byte aligned", fn);
  if (rope) {
    const int d[3] = {rope->d_f, rope->d_y, rope->d_x};
    for (int i = 0; i < 3; ++i)
      if (d[i] < 0 || (d[i] & 1))
        return fail(SVG_ERR_INVALID_ARG, "%s: rope runs must be even and >= 0", fn);
    if (d[0] + d[1] + d[2] != s.D)
      return fail(SVG_ERR_INVALID_ARG, "%s: rope runs sum to %d, not D = %d", fn, d[0] + d[1] + d[2],
                  s.D);
    if (!(rope->theta > 0.f) || !std::isfinite(rope->theta))
      return fail(SVG_ERR_INVALID_ARG, "%s: rope theta must be finite and > 0", fn);
  }
  launch_norm_rope(x, y, s, norm_span, gamma, eps, rope, head_layout, as_stream(stream));
  return check_launch(fn);
}

size_t svg_profile_workspace_bytes(svg_shape s, int n_samples) {
  if (check_shape(s, "svg_profile_workspace_bytes") != SVG_OK) return 0;
  return profile_workspace_bytes(s.B * s.H, s.N, s.D, s.block, n_samples, nullptr, nullptr);
}

svg_status svg_profile_heads(const void* q, const void* k, const void* v, svg_shape s, float scale,
                             const int32_t* idx, int n_samples, const svg_mask* cand,
                             int32_t* choice, float* err, void* workspace, size_t workspace_bytes,
                             void* stream) {
  const char* fn = "svg_profile_heads";
  if (svg_status st = check_shape(s, fn)) return st;
  if (svg_status st = check_head_dim(s, fn)) return st;
  if (!q || !k || !v || !idx || !choice)
    return fail(SVG_ERR_INVALID_ARG, "%s: NULL q / k / v / idx / choice", fn);
  if (n_samples < 1 || n_samples > 64)
    return fail(SVG_ERR_UNSUPPORTED, "%s: n_samples must be in [1, 64] (got %d)", fn, n_samples);
  if (!(scale > 0.f)) return fail(SVG_ERR_INVALID_ARG, "%s: scale must be positive", fn);
  if (svg_status st = check_mask(cand, s, fn, 2)) return st;
  int nB = n_blocks(s);
  int W = ceil_div(nB, 32);
  if (W > 32) return fail(SVG_ERR_UNSUPPORTED, "%s: more than 1024 blocks per row", fn);
  int chunk_keys = 0, n_chunks = 0;
  size_t need = profile_workspace_bytes(s.B * s.H, s.N, s.D, s.block, n_samples, &chunk_keys, &n_chunks);
  if (!workspace || workspace_bytes < need)
    return fail(SVG_ERR_CAPACITY, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, need);
  ProfileArgs a;
  a.q = q; a.k = k; a.v = v;
  a.idx = idx;
  a.n_samples = n_samples;
  a.bitmap = cand->bitmap;
  a.nB = nB;
  a.W = W;
  a.choice = choice;
  a.err = err;
  a.ws = static_cast<float*>(workspace);
  a.BH = s.B * s.H;
  a.N = s.N; a.D = s.D; a.block = s.block;
  a.F = s.F; a.Hs = s.Hs; a.Ws = s.Ws;
  a.chunk_keys = chunk_keys;
  a.n_chunks = n_chunks;
  a.scale_log2 = scale * 1.4426950408889634f;
  launch_profile(a, as_stream(stream));
  return check_launch(fn);
}

svg_status svg_block_sparse_attn(const void* q, const void* k, const void* v, const void* vt, void* o,
                                 const void* qp, const void* kp, const void* vp, void* op,
                                 svg_shape s, float scale, const svg_mask* masks,
                                 const int32_t* head_mask, const int32_t* head_layout, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "svg_block_sparse_attn";
  AttnArgs a;
  if (svg_status st = attn_setup(fn, q, k, v, vt, o, qp, kp, vp, op, s, scale, masks, head_mask,
                                 head_layout, lse, &a))
    return st;
  const size_t need = attn_workspace_bytes(a.BH, s.N, s.D, s.block, a.vt_given);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SVG_ERR_CAPACITY, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, need);
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 15))
    return fail(SVG_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
  if (need > 0) {
    if (!a.vt_given) a.vt = workspace;
    a.plan = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                        (need - attn_plan_bytes(a.BH, (a.n_qb + 1) / 2)));
  }
  launch_attn(a, as_stream(stream));
  return check_launch(fn);
}

size_t svg_attn_workspace_bytes(svg_shape s, int vt_given) {
  if (check_shape(s, "svg_attn_workspace_bytes") != SVG_OK) return 0;
  return attn_workspace_bytes(s.B * s.H, s.N, s.D, s.block, vt_given != 0);
}

size_t svg_vt_bytes(svg_shape s) {
  if (check_shape(s, "svg_vt_bytes") != SVG_OK) return 0;
  return attn_vt_bytes(s.B * s.H, s.N, s.D, s.block);
}

svg_status svg_prepare_kv(const void* k, const void* v, void* kp, void* vt, svg_shape s,
                          const int32_t* head_layout, void* stream) {
  const char* fn = "svg_prepare_kv";
  if (svg_status st = check_shape(s, fn)) return st;
  if (svg_status st = check_head_dim(s, fn)) return st;
  if (s.block != 128)
    return fail(SVG_ERR_UNSUPPORTED, "%s: V^T blocks exist for 128-token blocks only (block %d)", fn,
                s.block);
  if (!v || !vt) return fail(SVG_ERR_INVALID_ARG, "%s: v or vt is NULL", fn);
  if (kp && !k) return fail(SVG_ERR_INVALID_ARG, "%s: kp given but k is NULL", fn);
  const size_t bytes = size_t(s.B) * s.H * s.N * s.D * 2;
  const size_t vt_bytes = attn_vt_bytes(s.B * s.H, s.N, s.D, s.block);
  if (overlaps(vt, vt_bytes, v, bytes) || (k && overlaps(vt, vt_bytes, k, bytes)))
    return fail(SVG_ERR_INVALID_ARG, "%s: vt overlaps an input", fn);
  if (kp && (overlaps(kp, k, bytes) || overlaps(kp, v, bytes) || overlaps(kp, bytes, vt, vt_bytes)))
    return fail(SVG_ERR_INVALID_ARG, "%s: kp overlaps another buffer", fn);
  if ((reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(vt) |
       reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(kp)) & 15)
    return fail(SVG_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", fn);
  if ((n_blocks(s) + 1) / 2 > 65535 || int64_t(s.B) * s.H > 65535)
    return fail(SVG_ERR_UNSUPPORTED, "%s: up to 131070 blocks and 65535 heads", fn);
  AttnArgs a = {};
  a.v = v;
  a.vp = nullptr;
  a.head_layout = head_layout;
  a.vt = vt;
  a.BH = s.B * s.H;
  a.N = s.N; a.D = s.D; a.block = s.block;
  a.n_kb = n_blocks(s);
  a.F = s.F;
  a.S = s.Hs * s.Ws;
  a.Nv = s.F * s.Hs * s.Ws;
  a.divF = FastDiv(uint32_t(s.F));
  launch_prepare_kv(a, k, kp, as_stream(stream));
  return check_launch(fn);
}

size_t svg_fp8_vt_bytes(svg_shape s) {
  if (check_shape(s, "svg_fp8_vt_bytes") != SVG_OK || s.block != 128) return 0;
  return attn_vt_bytes(s.B * s.H, s.N, s.D, s.block) / 2;
}

svg_status svg_quantize_fp8(const void* q, const void* k, const void* v, uint8_t* q8, uint8_t* k8,
                            uint8_t* vt8, float* scales, svg_shape s, const int32_t* head_layout,
                            void* stream) {
  const char* fn = "svg_quantize_fp8";
  if (svg_status st = check_shape(s, fn)) return st;
  if (svg_status st = check_head_dim(s, fn)) return st;
  if (s.block != 128)
    return fail(SVG_ERR_UNSUPPORTED, "%s: the FP8 attention takes 128-token blocks (block %d)", fn, s.block);
  if (!q || !k || !v || !q8 || !k8 || !vt8 || !scales)
    return fail(SVG_ERR_INVALID_ARG, "%s: NULL buffer", fn);
  const size_t in_bytes = size_t(s.B) * s.H * s.N * s.D * 2, codes = in_bytes / 2;
  const size_t vt_bytes = attn_vt_bytes(s.B * s.H, s.N, s.D, s.block) / 2, sc_bytes = size_t(3) * s.B * s.H * 4;
  const void* ins[3] = {q, k, v};
  const void* outs[4] = {q8, k8, vt8, scales};
  const size_t out_sz[4] = {codes, codes, vt_bytes, sc_bytes};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 3; ++i)
      if (overlaps(outs[o], out_sz[o], ins[i], in_bytes))
        return fail(SVG_ERR_INVALID_ARG, "%s: an output overlaps an input", fn);
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (overlaps(outs[o], out_sz[o], outs[o2], out_sz[o2]))
        return fail(SVG_ERR_INVALID_ARG, "%s: outputs overlap", fn);
  }
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
       reinterpret_cast<uintptr_t>(q8) | reinterpret_cast<uintptr_t>(k8) | reinterpret_cast<uintptr_t>(vt8) |
       reinterpret_cast<uintptr_t>(scales)) & 15)
    return fail(SVG_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", fn);
  AttnArgs a = {};
  a.head_layout = head_layout;
  a.BH = s.B * s.H;
  a.N = s.N; a.D = s.D; a.block = s.block;
  a.n_kb = n_blocks(s);
  a.F = s.F;
  a.S = s.Hs * s.Ws;
  a.Nv = s.F * s.Hs * s.Ws;
  a.divF = FastDiv(uint32_t(s.F));
  launch_quantize_fp8(a, q, k, v, q8, k8, vt8, scales, as_stream(stream));
  return check_launch(fn);
}

svg_status svg_block_sparse_attn_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8,
                                     const float* scales, void* o, svg_shape s, float scale,
                                     const svg_mask* masks, const int32_t* head_mask,
                                     const int32_t* head_layout, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  const char* fn = "svg_block_sparse_attn_fp8";
  if (svg_status st = check_shape(s, fn)) return st;
  if (svg_status st = check_head_dim(s, fn)) return st;
  if (s.block != 128)
    return fail(SVG_ERR_UNSUPPORTED, "%s: 128-token blocks only (block %d)", fn, s.block);
  if (!q8 || !k8 || !vt8 || !scales || !o) return fail(SVG_ERR_INVALID_ARG, "%s: NULL buffer", fn);
  if (!(scale > 0.f)) return fail(SVG_ERR_INVALID_ARG, "%s: scale must be positive", fn);
  if (svg_status st = check_mask(masks, s, fn, 0)) return st;
  if ((n_blocks(s) + 1) / 2 > 65535 || masks->n_masks > 32768)
    return fail(SVG_ERR_UNSUPPORTED, "%s: up to 131070 blocks and 32768 masks", fn);
  const size_t o_bytes = size_t(s.B) * s.H * s.N * s.D * 2, codes = o_bytes / 2;
  if (overlaps(o, o_bytes, q8, codes) || overlaps(o, o_bytes, k8, codes) ||
      overlaps(o, o_bytes, vt8, attn_vt_bytes(s.B * s.H, s.N, s.D, s.block) / 2))
    return fail(SVG_ERR_INVALID_ARG, "%s: o overlaps an input", fn);
  if ((reinterpret_cast<uintptr_t>(q8) | reinterpret_cast<uintptr_t>(k8) | reinterpret_cast<uintptr_t>(vt8) |
       reinterpret_cast<uintptr_t>(o)) & 15)
    return fail(SVG_ERR_INVALID_ARG, "%s: buffers must be 16-byte aligned", fn);
  const size_t need = attn_workspace_bytes(s.B * s.H, s.N, s.D, s.block, true);
  if (!workspace || workspace_bytes < need)
    return fail(SVG_ERR_CAPACITY, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 15)
    return fail(SVG_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", fn);
  AttnArgs a = {};
  a.q = q8; a.k = k8; a.v = nullptr; a.o = o;
  a.row_ptr = masks->row_ptr;
  a.iv = masks->iv;
  a.n_masks = masks->n_masks;
  a.n_qb = masks->n_qb;
  a.n_kb = masks->n_kb;
  a.head_mask = head_mask;
  a.head_layout = head_layout;
  a.lse = lse;
  a.BH = s.B * s.H;
  a.N = s.N; a.D = s.D; a.block = s.block;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.vt = const_cast<uint8_t*>(vt8);
  a.vt_given = true;
  a.plan = static_cast<int32_t*>(workspace);
  a.bitmap = masks->bitmap;
  a.F = s.F;
  a.S = s.Hs * s.Ws;
  a.Nv = s.F * s.Hs * s.Ws;
  a.divF = FastDiv(uint32_t(s.F));
  a.f8_scales = scales;
  launch_attn_fp8(a, as_stream(stream));
  return check_launch(fn);
}

svg_status svg_row_broadcast(void* o, svg_shape s, const int32_t* head_sel, int k_anchors,
                             void* stream) {
  const char* fn = "svg_row_broadcast";
  if (svg_status st = check_shape(s, fn)) return st;
  if (svg_status st = check_head_dim(s, fn)) return st;
  if (!o) return fail(SVG_ERR_INVALID_ARG, "%s: o is NULL", fn);
  if (k_anchors < 1 || k_anchors > s.Hs)
    return fail(SVG_ERR_INVALID_ARG, "%s: k_anchors must be in [1, Hs]", fn);
  if (reinterpret_cast<uintptr_t>(o) & 15)
    return fail(SVG_ERR_INVALID_ARG, "%s: o must be 16-byte aligned", fn);
  launch_row_broadcast(o, s, head_sel, k_anchors, as_stream(stream));
  return check_launch(fn);
}

svg_status svg_restrict_anchor_rows(uint8_t* masks, int n_masks, svg_shape s, const int32_t* mask_sel,
                                    int k_anchors, void* stream) {
  const char* fn = "svg_restrict_anchor_rows";
  if (svg_status st = check_shape(s, fn)) return st;
  if (!masks) return fail(SVG_ERR_INVALID_ARG, "%s: masks is NULL", fn);
  if (n_masks < 1 || n_masks > 65535) return fail(SVG_ERR_INVALID_ARG, "%s: bad n_masks", fn);
  if (k_anchors < 1 || k_anchors > s.Hs)
    return fail(SVG_ERR_INVALID_ARG, "%s: k_anchors must be in [1, Hs]", fn);
  launch_restrict_anchor_rows(masks, n_masks, s, mask_sel, k_anchors, as_stream(stream));
  return check_launch(fn);
}

svg_status svg_calibrate_masks(const double* energy, int n_masks, int n_qb, int n_kb, double eps,
                               uint8_t* out, void* stream) {
  const char* fn = "svg_calibrate_masks";
  if (!energy || !out) return fail(SVG_ERR_INVALID_ARG, "%s: NULL buffer", fn);
  if (n_masks < 1 || n_qb < 1 || n_kb < 1)
    return fail(SVG_ERR_INVALID_ARG, "%s: sizes must be positive", fn);
  if (n_kb > 4096) return fail(SVG_ERR_UNSUPPORTED, "%s: n_kb above 4096", fn);
  if (int64_t(n_masks) * n_qb > 0x7fffffff) return fail(SVG_ERR_UNSUPPORTED, "%s: too many rows", fn);
  if (!(eps > 0.0 && eps <= 1.0)) return fail(SVG_ERR_INVALID_ARG, "%s: eps must be in (0, 1]", fn);
  launch_calibrate(energy, n_masks, n_qb, n_kb, eps, out, as_stream(stream));
  return check_launch(fn);
}

svg_status svg_block_energy(const void* q, const void* k, svg_shape s, float scale, double* energy,
                            void* stream) {
  const char* fn = "svg_block_energy";
  if (svg_status st = check_shape(s, fn)) return st;
  if (svg_status st = check_head_dim(s, fn)) return st;
  if (!q || !k || !energy) return fail(SVG_ERR_INVALID_ARG, "%s: NULL q / k / energy", fn);
  if (!(scale > 0.f)) return fail(SVG_ERR_INVALID_ARG, "%s: scale must be positive", fn);
  if (int64_t(s.B) * s.H > 65535) return fail(SVG_ERR_UNSUPPORTED, "%s: more than 65535 heads", fn);
  launch_block_energy(q, k, s, scale, energy, as_stream(stream));
  return check_launch(fn);
}

svg_status svg_aggregate_masks(const uint8_t* masks, int n_sets, int64_t mask_elems, double rho,
                               uint8_t* out, void* stream) {
  const char* fn = "svg_aggregate_masks";
  if (!masks || !out) return fail(SVG_ERR_INVALID_ARG, "%s: NULL buffer", fn);
  if (n_sets < 1 || mask_elems < 1) return fail(SVG_ERR_INVALID_ARG, "%s: sizes must be positive", fn);
  if (!(rho > 0.0 && rho <= 1.0)) return fail(SVG_ERR_INVALID_ARG, "%s: rho must be in (0, 1]", fn);
  if (overlaps(out, masks, size_t(n_sets) * size_t(mask_elems)))
    return fail(SVG_ERR_INVALID_ARG, "%s: out overlaps the candidate masks", fn);
  launch_aggregate(masks, n_sets, mask_elems, rho, out, as_stream(stream));
  return check_launch(fn);
}

size_t svg_row_similarity_workspace_bytes(svg_shape s) {
  if (check_shape(s, "svg_row_similarity_workspace_bytes") != SVG_OK) return 0;
  return row_similarity_workspace_bytes(s);
}

svg_status svg_row_similarity(const void* q, const void* k, svg_shape s, float scale, double* score,
                              void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "svg_row_similarity";
  if (svg_status st = check_shape(s, fn)) return st;
  if (svg_status st = check_head_dim(s, fn)) return st;
  if (!q || !k || !score) return fail(SVG_ERR_INVALID_ARG, "%s: NULL q / k / score", fn);
  if (!(scale > 0.f)) return fail(SVG_ERR_INVALID_ARG, "%s: scale must be positive", fn);
  if (s.Ws > 128 || s.Hs < 2 || s.Hs > 64)
    return fail(SVG_ERR_UNSUPPORTED, "%s: needs Ws <= 128 and 2 <= Hs <= 64", fn);
  if (int64_t(s.Hs) * s.N * 4 >= (int64_t(1) << 31))
    return fail(SVG_ERR_UNSUPPORTED, "%s: a frame's row patterns (Hs * N * 4 bytes) must stay under 2 GiB", fn);
  if (int64_t(s.B) * s.H > 65535) return fail(SVG_ERR_UNSUPPORTED, "%s: more than 65535 heads", fn);
  const size_t need = row_similarity_workspace_bytes(s);
  if (!workspace || workspace_bytes < need)
    return fail(SVG_ERR_CAPACITY, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(SVG_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  launch_row_similarity(q, k, s, scale, score, workspace, as_stream(stream));
  return check_launch(fn);
}

svg_status svg_eps_schedule(int t, int T, double eps_first, double eps_last, double* eps) {
  const char* fn = "svg_eps_schedule";
  if (!eps) return fail(SVG_ERR_INVALID_ARG, "%s: NULL eps", fn);
  if (T < 1 || t < 0 || t >= T) return fail(SVG_ERR_INVALID_ARG, "%s: need 0 <= t < T", fn);
  if (!(eps_first > 0.0 && eps_first <= 1.0 && eps_last > 0.0 && eps_last <= 1.0))
    return fail(SVG_ERR_INVALID_ARG, "%s: thresholds must be in (0, 1]", fn);
  *eps = T == 1 ? eps_first : eps_first * std::pow(eps_last / eps_first, double(t) / double(T - 1));
  return SVG_OK;
}

}  // extern "C"
