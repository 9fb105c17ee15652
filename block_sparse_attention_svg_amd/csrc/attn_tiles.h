// Tile geometry and building blocks shared by the 128-token-block attention
// kernels and the block-energy pass of the offline calibration: the LDS
// layout of the K and V^T tiles (1-KB segments 1040 bytes apart), the
// S^T = K Q^T product of one 128-key block on v_mfma_f32_32x32x16_bf16, and
// the maximum over the two halves of a wavefront.
#pragma once

#include "mfma_common.h"

namespace svg {
namespace {

template <int D, bool F8 = false>
struct Cfg2 {
  static constexpr int BLK = 128;
  static constexpr int WAVES = 8;
  static constexpr int ES = F8 ? 1 : 2;   // bytes per element of the K and V^T tiles
  // LDS tiles are built from 1-KB segments, one 16-byte global->LDS wavefront
  // copy each, placed 1040 bytes apart.  A tile of R rows x W bytes has
  // NI = R W / 1024 segments; row r lives in segment r % NI at position
  // r / NI, so a segment holds rows s, s+NI, s+2NI, ...  Rows whose indices
  // differ by less than 16 then start 16 bytes apart modulo 256: the rows
  // one 16-byte operand fetch reads together hit distinct banks.  A
  // segment's global source is 1024/W pieces of W contiguous bytes, and a
  // lane's source offset is a per-lane constant plus s W.
  static constexpr int SEGB = 1040;
  static constexpr int KW = D * ES, KNI = BLK * KW / 1024;   // K: 128 rows (keys) x D
  static constexpr int VW = BLK * ES, VNI = D * VW / 1024;   // V^T: D rows x 128 keys
  static constexpr int KBYTES = KNI * SEGB, VBYTES = VNI * SEGB;
  static constexpr int KT = BLK / 32, DK = D / 16, DT = D / 32, PS = BLK / 16;
  static constexpr int DK8 = D / 64, PG = BLK / 64;          // FP8: 64-deep contraction steps
  static constexpr int KPW = KNI / 4, VPW = VNI / 4;       // copies per wave of a group
  static_assert(KNI % 4 == 0 && VNI % 4 == 0, "segments split evenly over a wave group");
  // byte offset of (row, 16-byte chunk) in a tile of NI segments of W-byte rows
  template <int NI, int W>
  __host__ __device__ static constexpr int at(int row, int chunk) {
    return (row % NI) * SEGB + (row / NI) * W + chunk * 16;
  }
  // FP8 tiles of 128-byte rows (D = 128): the 8 rows s + 16 j of segment s
  // sit in 128-byte slots slot(j) (bits 0 and 1 of j exchanged), so that the
  // 32 rows one half-wave reads together (32 t + n, n < 32) fall on 32
  // distinct 16-byte bank positions modulo 512 bytes (slots 0 and 2 of the
  // segments 1040 bytes apart); the 16-row stagger of the plain layout gives
  // 2-way conflicts there.
  static constexpr bool SLOTS = F8 && KNI == 16 && VNI == 16 && KW == 128 && VW == 128;
  // The bf16 K tile at D = 64 has the same geometry (16 segments of 128-byte
  // rows) and takes the same slots; its V^T rows are 256 bytes and need none.
  static constexpr bool KSLOTS = KNI == 16 && KW == 128;
  __host__ __device__ static constexpr int slot(int j) { return (j & 4) | ((j & 1) << 1) | ((j & 2) >> 1); }
  // byte offset of rows 32 t + n relative to rows n (any n < 32)
  __host__ __device__ static constexpr int tile_off(int t, int plain) {
    return SLOTS ? (4 * (t >> 1) + (t & 1)) * 128 : t * plain;
  }
  __host__ __device__ static constexpr int tile_off_k(int t, int plain) {
    return KSLOTS ? (4 * (t >> 1) + (t & 1)) * 128 : t * plain;
  }
};

// S^T (128 keys x 32 queries) = K Q^T.  The scheduling barriers keep the K
// operands of contraction step kk+1 in flight while step kk computes.
template <int D>
__device__ __forceinline__ void mfma_qk(const char* kb_lds, int k_lane, const bf16x8* qreg,
                                        f32x16* sacc) {
  using C = Cfg2<D>;
  uint4 cur[C::KT], nxt[C::KT];
#pragma unroll
  for (int kt = 0; kt < C::KT; ++kt) {
    sacc[kt] = f32x16{};
    cur[kt] = *reinterpret_cast<const uint4*>(kb_lds + k_lane + C::tile_off_k(kt, 256));   // rows +32 kt
  }
#pragma unroll
  for (int kk = 0; kk < C::DK; ++kk) {
    if (kk + 1 < C::DK) {
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
        nxt[kt] = *reinterpret_cast<const uint4*>(kb_lds + k_lane + C::tile_off_k(kt, 256) + (kk + 1) * 32);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur[kt]), qreg[kk], sacc[kt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) cur[kt] = nxt[kt];
  }
}

// max of x over lanes l and l ^ 32 (one VALU swap of the wave halves, no LDS).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second: with x in both, one register ends up with the
// lower half's values in every lane and the other with the upper half's.
// Written in asm: through the compiler builtin the maximum of the two
// results was folded away (only the first result was kept, so each lane got
// the lower half's value).  The s_nops cover the VALU -> permlane and
// permlane -> VALU operand hazards.
__device__ __forceinline__ float max_cross_half(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1"
               : "+v"(a), "+v"(b));
  return a;
}

}  // namespace
}  // namespace svg
