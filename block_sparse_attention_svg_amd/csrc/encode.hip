// Bitmap + skip-list encoding of dense block masks ([CalibAtt] section 3.3).
//
// Three passes, all deterministic:
//   1. one wavefront per mask row: 64 key blocks per ballot; writes the bitmap
//      words and the row's interval count (runs of kept blocks) into
//      row_ptr[row + 1];
//   2. one workgroup: in-place inclusive scan of row_ptr[1..rows];
//   3. one wavefront per row: each lane that starts (ends) a run writes that
//      interval's start (end) at its rank among the row's starts (ends).
#include "svg_internal.h"

namespace svg {
namespace {

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ uint64_t row_ballot(const uint8_t* row, int c0, int n_kb, int lane) {
  int c = c0 + lane;
  bool kept = c < n_kb && row[c] != 0;
  return __ballot(kept);
}

__global__ __launch_bounds__(256) void encode_count_kernel(const uint8_t* __restrict__ dense,
                                                           int rows, int n_kb, int W,
                                                           uint32_t* __restrict__ bitmap,
                                                           int32_t* __restrict__ row_ptr) {
  int lane = threadIdx.x & 63;
  int row = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint8_t* d = dense + int64_t(row) * n_kb;
  uint32_t* bm = bitmap + int64_t(row) * W;
  int runs = 0;
  uint64_t prev_top = 0;  // was the block just before this chunk kept?
  for (int c0 = 0; c0 < n_kb; c0 += 64) {
    uint64_t bits = row_ballot(d, c0, n_kb, lane);
    uint64_t starts = bits & ~((bits << 1) | prev_top);
    runs += __popcll(starts);
    prev_top = bits >> 63;
    int w = c0 >> 5;
    if (lane == 0 && w < W) bm[w] = uint32_t(bits);
    if (lane == 1 && w + 1 < W) bm[w + 1] = uint32_t(bits >> 32);
  }
  if (lane == 0) row_ptr[row + 1] = runs;
  if (row == 0 && lane == 0) row_ptr[0] = 0;
}

__global__ __launch_bounds__(1024) void encode_scan_kernel(int32_t* __restrict__ row_ptr, int rows) {
  __shared__ int32_t buf[1024];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < rows; base += 1024) {
    int i = base + threadIdx.x;
    int32_t x = i < rows ? row_ptr[i + 1] : 0;
    buf[threadIdx.x] = x;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scan
      int32_t y = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
      __syncthreads();
      buf[threadIdx.x] += y;
      __syncthreads();
    }
    if (i < rows) row_ptr[i + 1] = carry + buf[threadIdx.x];
    __syncthreads();
    if (threadIdx.x == 1023) carry += buf[1023];
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void encode_intervals_kernel(const uint8_t* __restrict__ dense,
                                                               int rows, int n_kb,
                                                               const int32_t* __restrict__ row_ptr,
                                                               int32_t* __restrict__ iv) {
  int lane = threadIdx.x & 63;
  int row = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint8_t* d = dense + int64_t(row) * n_kb;
  int32_t* out = iv + 2 * int64_t(row_ptr[row]);
  uint64_t below = (lane == 0) ? 0 : (~uint64_t(0) >> (64 - lane));
  int n_start = 0, n_end = 0;
  uint64_t prev_top = 0;
  uint64_t bits = row_ballot(d, 0, n_kb, lane);
  for (int c0 = 0; c0 < n_kb; c0 += 64) {
    uint64_t next = (c0 + 64 < n_kb) ? row_ballot(d, c0 + 64, n_kb, lane) : 0;
    uint64_t starts = bits & ~((bits << 1) | prev_top);
    uint64_t ends = bits & ~((bits >> 1) | ((next & 1) << 63));  // last kept block of a run
    if ((starts >> lane) & 1) out[2 * (n_start + __popcll(starts & below))] = c0 + lane;
    if ((ends >> lane) & 1) out[2 * (n_end + __popcll(ends & below)) + 1] = c0 + lane + 1;
    n_start += __popcll(starts);
    n_end += __popcll(ends);
    prev_top = bits >> 63;
    bits = next;
  }
}

}  // namespace

void launch_encode(const uint8_t* dense, int n_masks, int n_qb, int n_kb, uint32_t* bitmap,
                   int32_t* row_ptr, int32_t* iv, hipStream_t st) {
  int rows = n_masks * n_qb;
  int W = ceil_div(n_kb, 32);
  int blocks = ceil_div(rows, kWavesPerBlock);
  hipLaunchKernelGGL(encode_count_kernel, dim3(blocks), dim3(64 * kWavesPerBlock), 0, st, dense,
                     rows, n_kb, W, bitmap, row_ptr);
  hipLaunchKernelGGL(encode_scan_kernel, dim3(1), dim3(1024), 0, st, row_ptr, rows);
  hipLaunchKernelGGL(encode_intervals_kernel, dim3(blocks), dim3(64 * kWavesPerBlock), 0, st,
                     dense, rows, n_kb, row_ptr, iv);
}

}  // namespace svg
