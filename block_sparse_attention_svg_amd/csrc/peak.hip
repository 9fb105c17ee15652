// Dense MFMA rate that the GPU sustains right now, for the measurement that
// puts the attention kernel's rate beside it (not part of the attention path).
//
// Every wavefront issues back-to-back v_mfma_f32_32x32x16_bf16 (or the FP8
// v_mfma_f32_32x32x64_f8f6f4) on four independent accumulators, its operands
// in registers: no memory traffic, no LDS reads, no other VALU work.  Four
// operand pairs with different values rotate so that consecutive products
// see different inputs (the power drawn depends on the operand bits).  The
// rate this reaches is bounded by the engine clock the board's power limit
// allows for dense matrix work, the ceiling of any kernel that also spends
// power on LDS, VALU and memory.
#include <hip/hip_runtime.h>

#include "mfma_common.h"
#include "svg_internal.h"

namespace svg {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kPeakWaves = 8;     // two per SIMD
constexpr int kPeakLds = 96 * 1024;

template <bool F8>
__global__ __launch_bounds__(kPeakWaves * 64) void mfma_peak_kernel(float* __restrict__ sink, int rounds) {
  // 96 KB of LDS per workgroup: one workgroup per CU (160 KB per CU)
  __shared__ float pad[kPeakLds / 4];
  const int tid = threadIdx.x;
  if (tid == 0) pad[blockIdx.x & 1023] = 1.f;
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  if constexpr (F8) {
    // E4M3 bytes with magnitude field below 0x78: finite codes only
    i32x8 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t x = (uint32_t(tid) * 2654435761u) ^ (uint32_t(i + 8 * j) * 40503u);
        a[j][i] = int(x & 0x77777777u);
        b[j][i] = int((x >> 3) & 0x77777777u);
      }
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j], b[(j + r) & 3], acc[j], 0, 0, 0, 0,
                                                                   0, 0);
    }
  } else {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t x = (uint32_t(tid) * 2654435761u) ^ (uint32_t(i + 8 * j) * 40503u);
        a[j][i] = (__bf16)(float(int(x & 0xffffu) - 32768) * 3e-5f);
        b[j][i] = (__bf16)(float(int(x >> 16) - 32768) * 3e-5f);
      }
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + r) & 3], acc[j], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][15];
  sink[int64_t(blockIdx.x) * blockDim.x + tid] = s + pad[(blockIdx.x + 1) & 1023] * 0.f;
}

}  // namespace
}  // namespace svg

using namespace svg;

extern "C" {

svg_status svg_mfma_peak_probe(int fp8, int rounds, float* sink, int64_t sink_floats, double* flop,
                               void* stream) {
  const char* fn = "svg_mfma_peak_probe";
  if (fp8 != 0 && fp8 != 1) return fail(SVG_ERR_INVALID_ARG, "%s: fp8 must be 0 or 1", fn);
  if (rounds < 1 || rounds > (1 << 20)) return fail(SVG_ERR_INVALID_ARG, "%s: rounds must be in [1, 2^20]", fn);
  if (!sink || !flop) return fail(SVG_ERR_INVALID_ARG, "%s: null pointer", fn);
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
    return fail(SVG_ERR_HIP, "%s: no device", fn);
  const int64_t need = int64_t(n_cu) * kPeakWaves * 64;
  if (sink_floats < need)
    return fail(SVG_ERR_CAPACITY, "%s: sink holds %lld floats, needs %lld", fn, (long long)sink_floats,
                (long long)need);
  // per wave: rounds x 16 products of 32 x 32 x K (K = 16 bf16, 64 FP8)
  *flop = double(n_cu) * kPeakWaves * rounds * 16 * (2.0 * 32 * 32 * (fp8 ? 64 : 16));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (fp8)
    hipLaunchKernelGGL(mfma_peak_kernel<true>, dim3(n_cu), dim3(kPeakWaves * 64), 0, st, sink, rounds);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<false>, dim3(n_cu), dim3(kPeakWaves * 64), 0, st, sink, rounds);
  return check_launch(fn);
}

}  // extern "C"
