// Shared device helpers of the attention and profiling kernels: MFMA operand
// types, 16-byte LDS tiles with an XOR swizzle, 8x8 bf16 transposes and
// 16-byte global->LDS copies through buffer resources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace svg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 as_u4(bf16x8 b) { return __builtin_bit_cast(uint4, b); }

// A row-major tile of ROWS x COLS bf16 in LDS, stored as 16-byte chunks
// (8 elements).  Chunk c of row r lives at chunk position c ^ swz(r), where
// swz spreads the 16 rows read by one MFMA operand fetch over all 64 banks.
template <int ROWS, int COLS>
struct LdsTile {
  static constexpr int CPR = COLS / 8;                    // chunks per row
  static constexpr int RPC = (16 / CPR) > 0 ? 16 / CPR : 1;  // rows per 256-byte bank sweep
  static constexpr int CHUNKS = ROWS * CPR;
  __device__ static __forceinline__ int slot(int r, int c) {
    return r * CPR + (c ^ ((r / RPC) % CPR));
  }
};

// Transpose an 8x8 block of bf16: in[i] holds row i (8 elements, element e in
// 16-bit half e%2 of word e/2); out[j] receives column j.
__device__ __forceinline__ void transpose8x8(const uint4 in[8], uint4 out[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t a = (&in[2 * p].x)[j >> 1];
      uint32_t b = (&in[2 * p + 1].x)[j >> 1];
      w[p] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    out[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Workgroup barrier that waits only for this thread's LDS operations.  Unlike
// __syncthreads() it does not drain outstanding global loads, so 16-byte
// global->LDS copies of later tiles stay in flight across it; callers wait
// for the copies they need with an explicit vmcnt first.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }

#define LDS_AS __attribute__((address_space(3)))

// A byte range of global memory as a buffer resource, for 16-byte
// global->LDS copies (buffer_load_dwordx4 ... lds): lane offsets are 32-bit
// VGPRs, a wave-uniform offset goes in an SGPR, the range check drops reads
// past the end (nothing is fetched for them), and the LDS destination of the
// wavefront instruction is the M0 base (lane l writes 16 bytes at base + 16 l).
struct LdsCopySrc {
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t r;
#endif
  __device__ __forceinline__ LdsCopySrc(const void* base, int bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
    r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
#endif
  }
  __device__ __forceinline__ void copy16(uint32_t lane_off, uint32_t uniform_off, uint32_t lds_addr) const {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)(uintptr_t)lds_addr, 16, lane_off,
                                             uniform_off, 0, 0);
#endif
  }
};

// Scalar add of a compile-time constant, kept at its point of use: the
// per-copy offsets are loop-invariant, and hoisted out of the loop all
// together they would exceed the scalar registers and be spilled.
template <int C>
__device__ __forceinline__ uint32_t sadd(uint32_t a) {
  uint32_t r;
  asm volatile("s_add_u32 %0, %1, %2" : "=s"(r) : "s"(a), "i"(C) : "scc");
  return r;
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(LDS_AS const void*)p;
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_from(F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_from<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_from<0, N>(f);
}

}  // namespace svg
