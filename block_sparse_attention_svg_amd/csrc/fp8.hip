// FP8 (E4M3) operands for the FP8 attention variant ([CalibAtt] section 3.3:
// mixed precision with FP8 on the critical path).  One scale per (tensor,
// head): amax = max |x| over the head, every element multiplied by
// 448 / amax in fp32 and rounded to E4M3 (nearest even, v_cvt_pk_fp8_f32),
// the dequantization factor amax / 448 kept for the attention.  The codes go
// straight into the layouts the FP8 attention reads: Q rows frame-major, K
// rows in each head's layout, V block-transposed per 128 keys in each head's
// layout with the keys of every 64-key group ordered for the 64-deep FP8
// product (keys 8a + 4h + i at byte 32h + 4a + i).
#include "svg_internal.h"

namespace svg {
namespace {

__global__ void fp8_zero_kernel(uint32_t* amax, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax[i] = 0u;
}

// 16-byte load that does not keep the line in the caches: the inputs here
// are read once per pass and would only evict other data
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

constexpr int kAmaxChunks = 4096;   // 16-byte chunks per amax step of a workgroup (64 KB)

// max |x| of one (tensor, head): blockIdx.y = head, blockIdx.z = tensor.
// Workgroup x reads its contiguous share of the head in steps of 64 KB (16
// loads per thread in flight); its maximum goes to the result with one
// unsigned atomic max (the float bits of non-negative values order like the
// values), so that few atomics meet on one address.
__global__ __launch_bounds__(256) void fp8_amax_kernel(const uint4* __restrict__ q, const uint4* __restrict__ k,
                                                       const uint4* __restrict__ v, int64_t chunks_per_head,
                                                       uint32_t* __restrict__ amax, int BH) {
  const int bh = blockIdx.y, t = blockIdx.z;
  const uint4* x = (t == 0 ? q : t == 1 ? k : v) + int64_t(bh) * chunks_per_head;
  const int64_t span = (chunks_per_head + gridDim.x - 1) / gridDim.x;
  const int64_t begin = int64_t(blockIdx.x) * span, end = min(chunks_per_head, begin + span);
  uint32_t m = 0u;
  for (int64_t c0 = begin + threadIdx.x; c0 < end; c0 += kAmaxChunks) {
    // indices past the share re-read its last chunk, which leaves the maximum unchanged
    uint4 u[kAmaxChunks / 256];
#pragma unroll
    for (int r = 0; r < kAmaxChunks / 256; ++r) u[r] = ld_stream(x + min(c0 + r * 256, end - 1));
#pragma unroll
    for (int r = 0; r < kAmaxChunks / 256; ++r) {
      const uint32_t w[4] = {u[r].x, u[r].y, u[r].z, u[r].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // |bf16| bits widened to fp32 bits: the order of the values is kept
        m = max(m, (w[j] & 0x7fffu) << 16);
        m = max(m, w[j] & 0x7fff0000u);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, uint32_t(__shfl_xor(int(m), off, 64)));
  __shared__ uint32_t wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    if (m) atomicMax(amax + t * BH + bh, m);
  }
}

__device__ __forceinline__ float inv_scale(uint32_t amax_bits) {
  const float a = __uint_as_float(amax_bits);
  return a > 0.f ? __fdiv_rn(448.f, a) : 1.f;
}

// 8 bf16 (a 16-byte chunk) times inv, rounded to E4M3: 8 bytes
__device__ __forceinline__ uint2 to_e4m3(uint4 u, float inv) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __fmul_rn(__uint_as_float(w[j] << 16), inv);
    f[2 * j + 1] = __fmul_rn(__uint_as_float(w[j] & 0xffff0000u), inv);
  }
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
  return make_uint2(uint32_t(lo), uint32_t(hi));
}

// One workgroup per (128-token block, head): Q rows, K rows (in the head's
// layout) and the V^T block (in the head's layout) of that block.
template <int D>
__global__ __launch_bounds__(256) void fp8_quant_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                        const __bf16* __restrict__ v, uint8_t* __restrict__ q8,
                                                        uint8_t* __restrict__ k8, uint8_t* __restrict__ vt8,
                                                        const uint32_t* __restrict__ amax,
                                                        const int32_t* __restrict__ head_layout, AttnArgs a) {
  constexpr int BLK = 128, CPR = D / 8;
  const int kb = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int N = a.N, BH = a.BH;
  const bool tm = head_layout && head_layout[bh] != 0;
  const float iq = inv_scale(amax[bh]), ik = inv_scale(amax[BH + bh]), iv = inv_scale(amax[2 * BH + bh]);
  const int64_t off = int64_t(bh) * N * D;
  const uint4* qs = reinterpret_cast<const uint4*>(q + off);
  const uint4* ks = reinterpret_cast<const uint4*>(k + off);
  const uint4* vs = reinterpret_cast<const uint4*>(v + off);
  uint2* qd = reinterpret_cast<uint2*>(q8 + off);
  uint2* kd = reinterpret_cast<uint2*>(k8 + off);
  // Q rows (frame-major) and K rows (row r of the head's layout <- k[fm(r)]):
  // every load is issued before the first store (rows past N read row N-1
  // and are not stored)
  constexpr int U = BLK * CPR / 256;
  uint4 qv[U], kv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = t + u * 256;
    const int r = min(kb * BLK + c / CPR, N - 1), col = c % CPR;
    const int src = tm ? frame_major_of(r, a) : r;
    qv[u] = ld_stream(qs + int64_t(r) * CPR + col);
    kv[u] = ld_stream(ks + int64_t(src) * CPR + col);
  }
  // V^T: thread (kg, dc) takes keys 8 kg .. 8 kg + 7 and dims 8 dc .. 8 dc + 7
  // (loaded here, before the Q and K stores) and places them in an LDS tile
  // of the block's V^T rows (one padding word per row); the tile then leaves
  // as whole 128-byte rows
  constexpr int TASKS = (BLK / 8) * CPR;
  const int dc = t % CPR, kg = t / CPR;
  uint4 vv[8];
  if (t < TASKS) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = min(kb * BLK + 8 * kg + i, N - 1);
      const int src = tm ? frame_major_of(key, a) : key;
      vv[i] = ld_stream(vs + int64_t(src) * CPR + dc);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = t + u * 256;
    const int r = kb * BLK + c / CPR, col = c % CPR;
    if (r < N) {
      qd[int64_t(r) * CPR + col] = to_e4m3(qv[u], iq);
      kd[int64_t(r) * CPR + col] = to_e4m3(kv[u], ik);
    }
  }
  __shared__ uint32_t tile[D][BLK / 4 + 1];
  if (t < TASKS) {
    uint2 rows[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rows[i] = kb * BLK + 8 * kg + i < N ? to_e4m3(vv[i], iv) : make_uint2(0u, 0u);
    // byte j of rows[i] is (key 8 kg + i, dim 8 dc + j); keys i = 0..3 go to
    // bytes 64 g + 4 (kg % 8) + i of the V^T row, keys 4..7 32 bytes further
    const int w0 = 16 * (kg / 8) + (kg % 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t lo = 0u, hi = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t b0 = ((j < 4 ? rows[i].x : rows[i].y) >> (8 * (j & 3))) & 0xffu;
        const uint32_t b1 = ((j < 4 ? rows[i + 4].x : rows[i + 4].y) >> (8 * (j & 3))) & 0xffu;
        lo |= b0 << (8 * i);
        hi |= b1 << (8 * i);
      }
      tile[8 * dc + j][w0] = lo;
      tile[8 * dc + j][w0 + 8] = hi;
    }
  }
  __syncthreads();
  uint8_t* blk = vt8 + (int64_t(bh) * a.n_kb + kb) * BLK * D;
#pragma unroll
  for (int u = 0; u < D * 8 / 256; ++u) {
    const int e = t + u * 256, r = e / 8, c = e % 8;
    const uint4 w = make_uint4(tile[r][4 * c], tile[r][4 * c + 1], tile[r][4 * c + 2], tile[r][4 * c + 3]);
    *reinterpret_cast<uint4*>(blk + r * BLK + 16 * c) = w;
  }
}

__global__ void fp8_finalize_kernel(uint32_t* scales, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const float a = __uint_as_float(scales[i]);
    scales[i] = __float_as_uint(a > 0.f ? __fdiv_rn(a, 448.f) : 1.f);
  }
}

}  // namespace

void launch_quantize_fp8(const AttnArgs& a, const void* q, const void* k, const void* v, uint8_t* q8,
                         uint8_t* k8, uint8_t* vt8, float* scales, hipStream_t st) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(scales);
  const int n = 3 * a.BH;
  hipLaunchKernelGGL(fp8_zero_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, st, bits, n);
  const int64_t chunks = int64_t(a.N) * a.D / 8;
  // workgroups per (tensor, head): about 1024 in all, at least 8 each (fewer,
  // longer streams read faster than many short ones), at most one per step
  const int groups = int(std::min<int64_t>(64, std::max<int64_t>(8, (1024 + 3 * a.BH - 1) / (3 * a.BH))));
  const int per_head = int(std::min<int64_t>(groups, (chunks + kAmaxChunks - 1) / kAmaxChunks));
  hipLaunchKernelGGL(fp8_amax_kernel, dim3(per_head, a.BH, 3), dim3(256), 0, st,
                     static_cast<const uint4*>(q), static_cast<const uint4*>(k), static_cast<const uint4*>(v),
                     chunks, bits, a.BH);
  if (a.D == 128)
    hipLaunchKernelGGL(fp8_quant_kernel<128>, dim3(a.n_kb, a.BH), dim3(256), 0, st,
                       static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                       static_cast<const __bf16*>(v), q8, k8, vt8, bits, a.head_layout, a);
  else
    hipLaunchKernelGGL(fp8_quant_kernel<64>, dim3(a.n_kb, a.BH), dim3(256), 0, st,
                       static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                       static_cast<const __bf16*>(v), q8, k8, vt8, bits, a.head_layout, a);
  hipLaunchKernelGGL(fp8_finalize_kernel, dim3(ceil_div(n, 256)), dim3(256), 0, st, bits, n);
}

}  // namespace svg
