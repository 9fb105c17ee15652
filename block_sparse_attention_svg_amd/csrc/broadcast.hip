// Anchor-row broadcast of row-repetitive heads ([CalibAtt] section 3.2): each
// latent row y of a frame takes the output of its anchor row
// a(y) = floor((2j+1)*Hs/(2k)), j = floor(y*k/Hs).  Anchor rows map to
// themselves and are never written, so the in-place copy has no overlap.
// A latent row is Ws contiguous tokens, i.e. one contiguous Ws*D*2-byte span.
#include "svg_internal.h"

namespace svg {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void row_broadcast_kernel(uint4* __restrict__ o, int N,
                                                                 int S, int Ws, int Hs, int k,
                                                                 int row_pieces,
                                                                 const int32_t* __restrict__ sel) {
  const int bh = blockIdx.z;
  if (sel && sel[bh] == 0) return;
  const int f = blockIdx.y / Hs;
  const int y = blockIdx.y % Hs;
  const int j = (y * k) / Hs;
  const int a = ((2 * j + 1) * Hs) / (2 * k);
  if (a == y) return;
  uint4* head = o + int64_t(bh) * N * row_pieces;
  const int64_t span = int64_t(Ws) * row_pieces;  // 16-byte pieces per latent row
  const uint4* src = head + (int64_t(f) * S + int64_t(a) * Ws) * row_pieces;
  uint4* dst = head + (int64_t(f) * S + int64_t(y) * Ws) * row_pieces;
  for (int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x; t < span;
       t += int64_t(gridDim.x) * kThreads)
    dst[t] = src[t];
}

}  // namespace

void launch_row_broadcast(void* o, const svg_shape& s, const int32_t* head_sel, int k,
                          hipStream_t st) {
  int row_pieces = s.D * 2 / 16;
  int span = s.Ws * row_pieces;
  int gx = ceil_div(span, kThreads);
  hipLaunchKernelGGL(row_broadcast_kernel, dim3(gx, s.F * s.Hs, s.B * s.H), dim3(kThreads), 0, st,
                     static_cast<uint4*>(o), s.N, s.Hs * s.Ws, s.Ws, s.Hs, k, row_pieces, head_sel);
}

}  // namespace svg
