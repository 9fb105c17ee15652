// Frame-major <-> token-major layout transpose ([SVG], "Layout Transformation
// + Kernel"): video token i = f*S + s moves to p = s*F + f; text tokens stay.
//
// Pure data movement, bound by HBM bandwidth.  Each thread moves 16-byte
// pieces; a token row (D elements) is 128-512 B, so every row is read and
// written as whole 16-byte-aligned segments.  Threads walk the OUTPUT in order,
// so writes are fully contiguous; reads are contiguous within each row.
#include "svg_internal.h"

namespace svg {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte pieces in flight per thread

struct PermuteGeom {
  int N, Nv;            // tokens, video tokens
  int lanes_log2;       // log2(16-byte pieces per row)
  FastDiv divF, divS;   // by frames, by positions per frame
  int F, S;
};

// Source row of output row `out` (frame->token: out is token-major p;
// token->frame: out is frame-major i).
__device__ __forceinline__ int source_row(int out, const PermuteGeom& g, int inverse) {
  if (out >= g.Nv) return out;
  if (!inverse) {  // out = p = s*F + f  ->  i = f*S + s
    int s = int(g.divF.div(uint32_t(out)));
    int f = out - s * g.F;
    return f * g.S + s;
  }
  // out = i = f*S + s  ->  p = s*F + f
  int f = int(g.divS.div(uint32_t(out)));
  int s = out - f * g.S;
  return s * g.F + f;
}

__global__ __launch_bounds__(kThreads) void permute_kernel(const u32x4* __restrict__ x,
                                                           u32x4* __restrict__ y, PermuteGeom g,
                                                           const int32_t* __restrict__ head_sel,
                                                           int inverse) {
  const int bh = blockIdx.y;
  if (head_sel && head_sel[bh] == 0) return;
  const int64_t per_head = int64_t(g.N) << g.lanes_log2;
  const u32x4* xs = x + bh * per_head;
  u32x4* ys = y + bh * per_head;
  const int lane_mask = (1 << g.lanes_log2) - 1;
  int64_t base = int64_t(blockIdx.x) * (kThreads * kUnroll) + threadIdx.x;
  u32x4 buf[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    int64_t piece = base + u * kThreads;
    if (piece < per_head) {
      int out = int(piece >> g.lanes_log2);
      int src = source_row(out, g, inverse);
      buf[u] = __builtin_nontemporal_load(xs + ((int64_t(src) << g.lanes_log2) | (piece & lane_mask)));
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    int64_t piece = base + u * kThreads;
    if (piece < per_head) __builtin_nontemporal_store(buf[u], ys + piece);
  }
}

}  // namespace

void launch_permute(const void* x, void* y, int elem_bytes, const svg_shape& s,
                    const int32_t* head_sel, int inverse, hipStream_t st) {
  PermuteGeom g;
  g.N = s.N;
  g.F = s.F;
  g.S = s.Hs * s.Ws;
  g.Nv = s.F * g.S;
  int row_pieces = s.D * elem_bytes / 16;
  g.lanes_log2 = 0;
  while ((1 << g.lanes_log2) < row_pieces) ++g.lanes_log2;
  g.divF = FastDiv(uint32_t(s.F));
  g.divS = FastDiv(uint32_t(g.S));
  int64_t per_head = int64_t(s.N) * row_pieces;
  int blocks = int((per_head + kThreads * kUnroll - 1) / (kThreads * kUnroll));
  hipLaunchKernelGGL(permute_kernel, dim3(blocks, s.B * s.H), dim3(kThreads), 0, st,
                     static_cast<const u32x4*>(x), static_cast<u32x4*>(y), g, head_sel, inverse);
}

}  // namespace svg
