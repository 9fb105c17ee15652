// Per-shape candidate masks, anchor-row restriction and energy-threshold
// calibration of static masks.
#include "svg_internal.h"

namespace svg {
namespace {

struct BlockSpan {
  int has_video, has_text, fmin, fmax;
};

// Frames spanned by the video tokens of a block, and whether it holds text.
// A block's tokens are consecutive, so its frames form one contiguous range.
__device__ __forceinline__ BlockSpan block_span(int b, int B, int N, int Nv, int S) {
  BlockSpan r;
  int lo = b * B;
  int hi = min(N, lo + B);
  int vhi = min(hi, Nv);
  r.has_video = lo < vhi;
  r.has_text = hi > Nv;
  r.fmin = r.has_video ? lo / S : 0;
  r.fmax = r.has_video ? (vhi - 1) / S : 0;
  return r;
}

// [SVG] "Spatial Head" / "Temporal Head": one thread per block pair writes
// both candidate masks.
__global__ void build_masks_kernel(int nB, int B, int N, int Nv, int S, int band_w,
                                   uint8_t* __restrict__ masks) {
  int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= int64_t(nB) * nB) return;
  int r = int(t / nB), c = int(t % nB);
  BlockSpan q = block_span(r, B, N, Nv, S);
  BlockSpan k = block_span(c, B, N, Nv, S);
  bool text = q.has_text || k.has_text;
  bool spatial = q.has_video && k.has_video && k.fmin <= q.fmax + 1 && k.fmax + 1 >= q.fmin;
  int d = r > c ? r - c : c - r;
  masks[t] = uint8_t(text || spatial);
  masks[int64_t(nB) * nB + t] = uint8_t(text || d <= band_w);
}

// [CalibAtt] 3.2: rows of masks whose query block holds no anchor-row token
// are emptied.  One workgroup per (mask, query block).
__global__ void restrict_anchor_kernel(uint8_t* __restrict__ masks, int nB, int B, int Nv,
                                       int S, int Ws, int Hs, int k,
                                       const int32_t* __restrict__ mask_sel) {
  int m = blockIdx.y, r = blockIdx.x;
  if (mask_sel && mask_sel[m] == 0) return;
  int lo = r * B, hi = min(Nv, lo + B);
  int found = 0;
  for (int i = lo + threadIdx.x; i < hi; i += blockDim.x) {
    int y = (i % S) / Ws;
    int j = (y * k) / Hs;
    int a = ((2 * j + 1) * Hs) / (2 * k);
    found |= (a == y);
  }
  found = __syncthreads_or(found);
  if (found) return;
  uint8_t* row = masks + (int64_t(m) * nB + r) * nB;
  for (int c = threadIdx.x; c < nB; c += blockDim.x) row[c] = 0;
}

// [CalibAtt] 3.1: per row, sort key blocks by energy (descending, ties by
// index), then keep the shortest prefix whose float64 running sum reaches
// eps * total.  One workgroup of 1024 threads per row; bitonic sort in LDS.
constexpr int kCalibMax = 4096;

__global__ __launch_bounds__(1024) void calibrate_kernel(const double* __restrict__ E, int n_kb,
                                                         double eps, uint8_t* __restrict__ out) {
  __shared__ double key[kCalibMax];
  __shared__ int idx[kCalibMax];
  __shared__ int count;
  const int64_t row = blockIdx.x;
  const double* e = E + row * n_kb;
  int n = 1;
  while (n < n_kb) n <<= 1;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    key[i] = i < n_kb ? e[i] : -1.0;  // padding sorts last (energies are >= 0)
    idx[i] = i;
  }
  __syncthreads();
  // "a before b" when a has more energy, or equal energy and a smaller index
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        int j = i ^ stride;
        if (j > i) {
          bool asc = (i & size) == 0;
          double ki = key[i], kj = key[j];
          int ii = idx[i], ij = idx[j];
          bool i_first = ki > kj || (ki == kj && ii < ij);
          if (i_first != asc) {
            key[i] = kj; key[j] = ki;
            idx[i] = ij; idx[j] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    double acc = 0.0;
    for (int t = 0; t < n_kb; ++t) acc = acc + key[t];
    double threshold = eps * acc;
    double run = 0.0;
    int c = n_kb;
    for (int t = 0; t < n_kb; ++t) {
      run = run + key[t];
      if (run >= threshold) { c = t + 1; break; }
    }
    count = c;
  }
  __syncthreads();
  uint8_t* o = out + row * n_kb;
  for (int t = threadIdx.x; t < n_kb; t += blockDim.x) o[idx[t]] = uint8_t(t < count);
}

}  // namespace

void launch_build_masks(const svg_shape& s, int band_w, uint8_t* masks, hipStream_t st) {
  int nB = ceil_div(s.N, s.block);
  int64_t total = int64_t(nB) * nB;
  int threads = 256;
  int blocks = int((total + threads - 1) / threads);
  hipLaunchKernelGGL(build_masks_kernel, dim3(blocks), dim3(threads), 0, st, nB, s.block, s.N,
                     s.F * s.Hs * s.Ws, s.Hs * s.Ws, band_w, masks);
}

void launch_restrict_anchor_rows(uint8_t* masks, int n_masks, const svg_shape& s,
                                 const int32_t* mask_sel, int k, hipStream_t st) {
  int nB = ceil_div(s.N, s.block);
  hipLaunchKernelGGL(restrict_anchor_kernel, dim3(nB, n_masks), dim3(128), 0, st, masks, nB,
                     s.block, s.F * s.Hs * s.Ws, s.Hs * s.Ws, s.Ws, s.Hs, k, mask_sel);
}

void launch_calibrate(const double* E, int n_masks, int n_qb, int n_kb, double eps, uint8_t* out,
                      hipStream_t st) {
  hipLaunchKernelGGL(calibrate_kernel, dim3(n_masks * n_qb), dim3(1024), 0, st, E, n_kb, eps, out);
}

}  // namespace svg
