// Offline calibration on the GPU ([CalibAtt] section 3.1): the block
// attention energy E(r, c) that the energy-threshold rule ranks, and the merge
// of candidate masks over prompts by keep frequency.
//
// E(r, c) is the dense softmax weight the queries of block r give to the keys
// of block c: sum over i in r, j in c of exp(s_ij - lse_i), s_ij = scale q_i.k_j.
// One workgroup per (batch*head, query block), BLK/32 wavefronts of 32
// queries.  Each key block is staged in LDS by the whole workgroup; S^T = K Q^T
// runs on v_mfma_f32_32x32x16_bf16 with Q in registers (the attention kernel's
// operand layout: lane l holds query l%32, dims 16*kk + 8*(l/32) + i).  The
// first sweep over the key blocks keeps each query's running max and sum (log2
// units); the second recomputes the scores, weighs them by exp2(s - lse) and
// sums each block pair: per lane, then over the wave, then over the waves in
// order, so the result is identical on every call.  fp32 arithmetic, float64
// output for the threshold rule.  With 128-token blocks, energy_pp_kernel runs
// the same arithmetic on the attention kernel's two-group schedule (two query
// blocks per workgroup, matrix-core and VALU phases overlapped).
#include "attn_tiles.h"
#include "mfma_common.h"
#include "svg_internal.h"

namespace svg {
namespace {

template <int D, int BLK>
struct ECfg {
  static constexpr int NW = BLK / 32;          // wavefronts (32 queries each)
  static constexpr int THREADS = NW * 64;
  static constexpr int KT = BLK / 32;          // 32-key tiles per block
  static constexpr int DK = D / 16;            // contraction steps
  static constexpr int RS = D * 2 + 16;        // LDS row stride: 16 consecutive rows, distinct banks
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int LOADS = BLK * CPR / THREADS;
  static_assert(BLK * CPR % THREADS == 0, "K staging divides evenly");
};

// K block kb into registers (rows past N as zero), then into an LDS tile:
// the loads of block kb+1 are in flight while block kb is computed.
template <int D, int BLK>
__device__ __forceinline__ void load_k(uint4* kr, const __bf16* __restrict__ kh, int kb, int N, int tid) {
  using C = ECfg<D, BLK>;
#pragma unroll
  for (int u = 0; u < C::LOADS; ++u) {
    const int c = tid + u * C::THREADS;
    const int row = c / C::CPR, col = c % C::CPR;
    const int key = kb * BLK + row;
    kr[u] = key < N ? *reinterpret_cast<const uint4*>(kh + int64_t(key) * D + col * 8) : make_uint4(0, 0, 0, 0);
  }
}

template <int D, int BLK>
__device__ __forceinline__ void store_k(char* ks, const uint4* kr, int tid) {
  using C = ECfg<D, BLK>;
#pragma unroll
  for (int u = 0; u < C::LOADS; ++u) {
    const int c = tid + u * C::THREADS;
    *reinterpret_cast<uint4*>(ks + (c / C::CPR) * C::RS + (c % C::CPR) * 16) = kr[u];
  }
}

// S^T of one key block: sacc[kt] register r holds key kt*32 + 8*(r/4) +
// 4*(lane/32) + r%4 of the block, query lane%32.
template <int D, int BLK>
__device__ __forceinline__ void scores(const char* ks, const bf16x8* qreg, int n, int h, f32x16* sacc) {
  using C = ECfg<D, BLK>;
#pragma unroll
  for (int kt = 0; kt < C::KT; ++kt) {
    sacc[kt] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::DK; ++kk) {
      const uint4 a = *reinterpret_cast<const uint4*>(ks + (kt * 32 + n) * C::RS + (2 * kk + h) * 16);
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qreg[kk], sacc[kt], 0, 0, 0);
    }
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2, 2) void energy_kernel(const __bf16* __restrict__ q,
                                                         const __bf16* __restrict__ k, int N, int nB,
                                                         float c2, double* __restrict__ E) {
  using C = ECfg<D, BLK>;
  // two K tiles: block kb in tile kb % 2, so one barrier per block orders both
  // the tile refill and the per-wave block sums
  __shared__ __attribute__((aligned(16))) char ks[2][BLK * C::RS];
  __shared__ float part[2][C::NW];
  const int r = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;
  const __bf16* qh = q + int64_t(bh) * N * D;
  const __bf16* kh = k + int64_t(bh) * N * D;
  const int qi = r * BLK + wave * 32 + n;
  const bool q_ok = qi < N;
  bf16x8 qreg[C::DK];
#pragma unroll
  for (int kk = 0; kk < C::DK; ++kk) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (q_ok) u = *reinterpret_cast<const uint4*>(qh + int64_t(qi) * D + 16 * kk + 8 * h);
    qreg[kk] = as_bf16x8(u);
  }
  f32x16 sacc[C::KT];
  auto key_of = [&](int kb, int kt, int i) { return kb * BLK + kt * 32 + 8 * (i >> 2) + 4 * h + (i & 3); };

  uint4 kr[C::LOADS];
  // sweep 1: running max m and this lane's share l of the sum (log2 units)
  float m = -INFINITY, l = 0.f;
  load_k<D, BLK>(kr, kh, 0, N, tid);
  for (int kb = 0; kb < nB; ++kb) {
    char* tile = ks[kb & 1];
    store_k<D, BLK>(tile, kr, tid);   // tile kb%2 was last read for block kb-2
    __syncthreads();
    if (kb + 1 < nB) load_k<D, BLK>(kr, kh, kb + 1, N, tid);
    scores<D, BLK>(tile, qreg, n, h, sacc);
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (key_of(kb, kt, i) >= N) sacc[kt][i] = -INFINITY;
        mx = fmaxf(mx, sacc[kt][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c2;
    const float m_new = fmaxf(m, mx);
    float add = 0.f;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) add += fast_exp2(__builtin_fmaf(sacc[kt][i], c2, -m_new));
    l = l * fast_exp2(m - m_new) + add;
    m = m_new;
  }
  const float lse2 = m + __log2f(l + __shfl_xor(l, 32, 64));

  // sweep 2: block sums of exp2(s - lse); block kb's per-wave sums are added
  // up (in wave order) after the next barrier
  double* row = E + (int64_t(bh) * nB + r) * nB;
  auto finish = [&](int kb) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) t += part[kb & 1][w];
    row[kb] = double(t);
  };
  __syncthreads();   // every wave is done with sweep 1's tiles
  load_k<D, BLK>(kr, kh, 0, N, tid);
  for (int kb = 0; kb < nB; ++kb) {
    char* tile = ks[kb & 1];
    store_k<D, BLK>(tile, kr, tid);
    __syncthreads();
    if (kb > 0 && tid == 0) finish(kb - 1);
    if (kb + 1 < nB) load_k<D, BLK>(kr, kh, kb + 1, N, tid);
    scores<D, BLK>(tile, qreg, n, h, sacc);
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(__builtin_fmaf(sacc[kt][i], c2, -lse2));
        sum += key_of(kb, kt, i) < N ? p : 0.f;
      }
    if (!q_ok) sum = 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane == 0) part[kb & 1][wave] = sum;   // read after the next barrier
  }
  __syncthreads();
  if (tid == 0) finish(nB - 1);
}

// Row sums of a 32 x 128 tile held in MFMA accumulator layout (lane (n, h)
// holds query n's scores of keys 32 kt + 8 (i/4) + 4 h + i%4 in v[16 kt + i]):
// a reduce-scatter over the 32 lanes of each half.  The first step swaps
// 16-lane rows between registers (v_permlane16_swap), the next four pair
// lanes by DPP (mirror of 16, mirror of 8, quad xor 2, quad xor 1); at each
// step a lane keeps one of two value sets and adds its partner's copy.  Lane
// (n, h) ends with the sums over the 32 queries of values 2n and 2n + 1, i.e.
// keys 32 (n/8) + 8 ((n%8)/2) + 4 h + 2 (n%2) + {0, 1}.
__device__ __forceinline__ void swap_rows16(float& a, float& b) {
  // the s_nops cover the VALU -> permlane and permlane -> VALU operand hazards
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int HALF, int CTRL>
__device__ __forceinline__ void fold(float* v, bool upper) {
#pragma unroll
  for (int j = 0; j < HALF; ++j) {
    const float send = upper ? v[j] : v[j + HALF];
    const float keep = upper ? v[j + HALF] : v[j];
    v[j] = keep + dpp_f<CTRL>(send);
  }
}
__device__ __forceinline__ void key_sums32(float* v, int n) {
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float a = v[j], b = v[j + 32];
    swap_rows16(a, b);
    v[j] = a + b;
  }
  fold<16, 0x140>(v, n & 8);   // row_mirror: lane ^ 15
  fold<8, 0x141>(v, n & 4);    // row_half_mirror: lane ^ 7
  fold<4, 0x4E>(v, n & 2);     // quad_perm [2, 3, 0, 1]
  fold<2, 0xB1>(v, n & 1);     // quad_perm [1, 0, 3, 2]
}

// Where sweep 2's sums go: block energies E [bh][nB][nB] (float64), or, for
// the row-repetition test, the key-level pattern A [bh][rows][N] (fp32) of
// latent rows of Ws queries.
struct PairOut {
  double* E;
  float* A;
  int Ws, rows;
};

// 128-token blocks: the attention kernel's two-phase schedule.  One
// workgroup of 8 wavefronts takes two query sets of a head (two query blocks,
// or two latent rows): group 0 (waves 0-3) computes S^T of key block j on the
// matrix cores while group 1 works on block j-1's scores on the VALU, then
// the roles swap; K tiles reach double-buffered LDS through 16-byte
// global->LDS copies issued by group 0 before its VALU phase.  Sweep 1 keeps
// each query's running max and sum; sweep 2 sums exp2(s - lse) per key block
// (energies: the same arithmetic in the same order as energy_kernel, so the
// same bits) or per key (row patterns: key_sums32 over a wave's 32 queries,
// then the four waves added in order).
template <int D, bool ROWS>
__device__ __forceinline__ void pair_sweeps(const __bf16* __restrict__ q, const __bf16* __restrict__ k, int N,
                                            int nB, float c2, PairOut out, int pair, int bh) {
  using C = Cfg2<D>;
  // separate arrays per buffer, addressed with compile-time indices (the
  // compiler then sees that copies in flight target the other buffer)
  __shared__ uint4 kbuf0[C::KBYTES / 16], kbuf1[C::KBYTES / 16];
  __shared__ float part[2][2][ROWS ? 4 * 128 : 4];   // [block parity][group][wave (x key)]
  char* const kb_lds[2] = {reinterpret_cast<char*>(kbuf0), reinterpret_cast<char*>(kbuf1)};
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = wave >> 2;
  const int w4 = __builtin_amdgcn_readfirstlane(wave & 3);
  const int n = lane & 31, h = lane >> 5;
  const int unit = 2 * pair + grp;   // query block, or latent row
  const __bf16* qh = q + int64_t(bh) * N * D;
  const char* Kh = reinterpret_cast<const char*>(k + int64_t(bh) * N * D);
  bool has_unit, q_ok;
  int qi;
  if constexpr (ROWS) {
    has_unit = unit < out.rows;
    q_ok = has_unit && w4 * 32 + n < out.Ws;
    qi = unit * out.Ws + w4 * 32 + n;
  } else {
    has_unit = unit < nB;
    qi = unit * 128 + w4 * 32 + n;
    q_ok = qi < N;
  }
  bf16x8 qreg[C::DK];
#pragma unroll
  for (int kk = 0; kk < C::DK; ++kk) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (q_ok) u = *reinterpret_cast<const uint4*>(qh + int64_t(qi) * D + 16 * kk + 8 * h);
    qreg[kk] = as_bf16x8(u);
  }
  // K rows in natural order: register r of tile kt holds key 32 kt + 8 (r/4)
  // + 4 h + r%4 for query n (the energy_kernel layout)
  const int k_lane = C::KSLOTS ? (n % 16) * C::SEGB + C::slot(n / 16) * 128 + 16 * h
                               : C::template at<C::KNI, C::KW>(n, h);
  const int k_row_of_lane = C::KSLOTS ? C::slot(lane / 8) : lane / (C::KW / 16);
  const uint32_t k_lane_src = k_row_of_lane * C::KNI * C::KW + (lane % (C::KW / 16)) * 16;
  const uint32_t k_w4_src = w4 * C::KPW * C::KW;
  auto copy_k = [&](int kb, const char* dst) {   // group 0; rows past N are not fetched
    const bool exists = kb < nB;
    const LdsCopySrc src(Kh + int64_t(exists ? kb : 0) * 128 * D * 2,
                         exists ? min(128, N - kb * 128) * D * 2 : 0);
    const uint32_t lds_w = lds_addr_of(dst) + w4 * C::KPW * C::SEGB;
    static_for<C::KPW>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      src.copy16(k_lane_src, sadd<u * C::KW>(k_w4_src), sadd<u * C::SEGB>(lds_w));
    });
  };
  f32x16 sacc[C::KT];
  auto key_of = [&](int kb, int kt, int i) { return kb * 128 + kt * 32 + 8 * (i >> 2) + 4 * h + (i & 3); };

  float m = -INFINITY, l = 0.f, lse2 = 0.f;
  // sweep 1: running max and sum; sweep 2: sums of exp2(s - lse)
  auto stats = [&](int kb) {
    if (kb * 128 + 128 > N) {   // the ragged last block: keys past N drop out
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key_of(kb, kt, i) >= N) sacc[kt][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
    mx = max_cross_half(mx) * c2;
    const float m_new = fmaxf(m, mx);
    float add = 0.f;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) add += fast_exp2(__builtin_fmaf(sacc[kt][i], c2, -m_new));
    l = l * fast_exp2(m - m_new) + add;
    m = m_new;
  };
  auto bsum = [&](int kb) {
    if constexpr (ROWS) {
      // queries outside the row have lse2 = +inf, so their weights are 0;
      // keys past N are summed but never stored
      float v[64];
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) v[16 * kt + i] = fast_exp2(__builtin_fmaf(sacc[kt][i], c2, -lse2));
      key_sums32(v, n);
      const int key0 = 32 * (n >> 3) + 8 * ((n & 7) >> 1) + 4 * h + 2 * (n & 1);
      *reinterpret_cast<float2*>(&part[kb & 1][grp][w4 * 128 + key0]) = make_float2(v[0], v[1]);
    } else {
      float sum = 0.f;
      if (kb * 128 + 128 > N) {
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(__builtin_fmaf(sacc[kt][i], c2, -lse2));
            sum += key_of(kb, kt, i) < N ? p : 0.f;
          }
      } else {
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sum += fast_exp2(__builtin_fmaf(sacc[kt][i], c2, -lse2));
      }
      if (!q_ok) sum = 0.f;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
      if (lane == 0) part[kb & 1][grp][w4] = sum;   // summed after the iteration's barrier
    }
  };
  // iteration j: K of block j in buffer j % 2; group 1 handles block j-1's
  // scores in phase 1, group 0 block j's in phase 2
  auto iteration = [&](int j, auto kbuf_c, auto second_c) {
    constexpr int kbuf = decltype(kbuf_c)::value;
    constexpr bool SECOND = decltype(second_c)::value;
    const bool cur = j < nB, prev = j > 0;
    if (grp == 0) {
      if (cur) mfma_qk<D>(kb_lds[kbuf], k_lane, qreg, sacc);
    } else if (prev) {
      if constexpr (SECOND) bsum(j - 1);
      else stats(j - 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 0) {
      copy_k(j + 1, kb_lds[kbuf ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
      if (cur) {
        if constexpr (SECOND) bsum(j);
        else stats(j);
      }
    } else if (cur) {
      mfma_qk<D>(kb_lds[kbuf], k_lane, qreg, sacc);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this wave's copies have landed
    barrier_lds();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (SECOND) {
      // group 0's block j and group 1's block j-1 are complete: four wave
      // sums each, added in wave order
      const int kbd = grp == 0 ? j : j - 1;
      if constexpr (ROWS) {
        const int key = tid & 255;
        if (key < 128 && kbd >= 0 && kbd < nB && has_unit && kbd * 128 + key < N) {
          float t = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) t += part[kbd & 1][grp][w * 128 + key];
          out.A[(int64_t(bh) * out.rows + unit) * N + kbd * 128 + key] = t;
        }
      } else if ((tid & 255) == 0) {
        if (kbd >= 0 && kbd < nB && has_unit) {
          float t = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) t += part[kbd & 1][grp][w];
          out.E[(int64_t(bh) * nB + unit) * nB + kbd] = double(t);
        }
      }
    }
  };
  auto sweep = [&](auto second_c) {
    if (grp == 0) copy_k(0, kb_lds[0]);
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0)
    barrier_lds();
    for (int j = 0; j <= nB; j += 2) {
      iteration(j, std::integral_constant<int, 0>{}, second_c);
      if (j + 1 <= nB) iteration(j + 1, std::integral_constant<int, 1>{}, second_c);
    }
  };
  sweep(std::false_type{});
  lse2 = m + __log2f(l + __shfl_xor(l, 32, 64));
  if constexpr (ROWS) {
    if (!q_ok) lse2 = INFINITY;
  }
  barrier_lds();   // every wave is done with the tiles of sweep 1
  sweep(std::true_type{});
}

template <int D>
__global__ __launch_bounds__(512) void energy_pp_kernel(const __bf16* __restrict__ q,
                                                        const __bf16* __restrict__ k, int N, int nB,
                                                        float c2, double* __restrict__ E) {
  pair_sweeps<D, false>(q, k, N, nB, c2, PairOut{E, nullptr, 0, 0}, blockIdx.x, blockIdx.y);
}

// ---- row-repetitive heads ([CalibAtt] section 3.2) --------------------------
// The attention pattern of latent row (f, y) is the sum of the softmax weights
// of its Ws queries over all N keys; a head is row-repetitive when the mean
// cosine between the patterns of the rows of a frame exceeds gamma.
//
// row_pattern_kernel: pair_sweeps with latent rows as the query sets, two
// rows of a head per workgroup (Ws <= 128; slots past Ws have zero weight).
// fp32 sums in a fixed order, identical on every call.
template <int D>
__global__ __launch_bounds__(512) void row_pattern_kernel(const __bf16* __restrict__ q,
                                                          const __bf16* __restrict__ k, int N, int Ws,
                                                          int rows, float c2, float* __restrict__ A) {
  pair_sweeps<D, true>(q, k, N, (N + 127) / 128, c2, PairOut{nullptr, A, Ws, rows}, blockIdx.x, blockIdx.y);
}

// Per (batch*head, frame): Gram matrix G = P P^T of the frame's Hs row
// patterns (P: Hs x N), a dense float64 contraction over the keys on the
// matrix cores (v_mfma_f64_16x16x4_f64), split over key chunks to fill the
// chip, then the sum of the cosines over the pairs of distinct rows, in order.
// The fp32 pattern values convert exactly to float64, so every product is
// exact and only the float64 accumulation rounds.
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kGramWaves = 4;

// Key chunks per frame: enough workgroups for the 256 compute units, chunks a
// multiple of 128 keys (4 wavefronts x 32 keys per step).
struct GramSplit {
  int chunks, chunk_keys;
};
GramSplit gram_split(const svg_shape& s) {
  const int64_t frames = int64_t(s.B) * s.H * s.F;
  const int max_chunks = (s.N + 127) / 128;
  int chunks = int(std::min<int64_t>(max_chunks, std::max<int64_t>(1, (2048 + frames - 1) / frames)));
  const int chunk_keys = ((s.N + chunks - 1) / chunks + 127) / 128 * 128;
  chunks = (s.N + chunk_keys - 1) / chunk_keys;
  return {chunks, chunk_keys};
}
constexpr int gram_tile_pairs(int rt) { return rt * (rt + 1) / 2; }

// One workgroup per (frame, key chunk, batch*head); wave w takes the keys
// k0 = chunk start + 32 w + 128 it.  Lane l carries row 16 t + l%16 of row
// tile t and, at step s of a 32-key group, key k0 + 4 s + l/16: the same
// register is the A operand (rows x keys) and the B operand (keys x rows), so
// tile pair (ti, tj) accumulates G[16 ti + i][16 tj + j] for ti <= tj.  Each
// wave writes its partial tiles, [16 x 16] row-major per pair.
template <int RT>
__global__ __launch_bounds__(256) void row_gram_part_kernel(const float* __restrict__ A, int N, int Hs, int F,
                                                            int chunks, int chunk_keys,
                                                            double* __restrict__ part) {
  constexpr int NP = gram_tile_pairs(RT);
  const int f = blockIdx.x / chunks, c = blockIdx.x % chunks, bh = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const float* base = A + (int64_t(bh) * F + f) * Hs * int64_t(N);
  const int kbeg = c * chunk_keys, kend = min(N, kbeg + chunk_keys);
  // the frame's patterns as a buffer resource: reads at offsets past its end
  // return 0, which pads the rows past Hs and the keys past the chunk
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, Hs * N * 4, 0x00020000);
#else
  (void)base;
#endif
  uint32_t row_off[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int row = 16 * t + r16;
    row_off[t] = row < Hs ? uint32_t(row) * uint32_t(N) * 4u : 0x80000000u;
  }
  f64x4 acc[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) acc[p] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int k0 = kbeg + 32 * wave; k0 < kend; k0 += 32 * kGramWaves) {
    float x[RT][8];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int key = k0 + 4 * s + g;
        const uint32_t off = key < kend ? row_off[t] + uint32_t(key) * 4u : 0x80000000u;
#if defined(__HIP_DEVICE_COMPILE__)
        x[t][s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
#else
        x[t][s] = float(off);
#endif
      }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      double a[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) a[t] = double(x[t][s]);
      int p = 0;
#pragma unroll
      for (int ti = 0; ti < RT; ++ti)
#pragma unroll
        for (int tj = ti; tj < RT; ++tj, ++p) acc[p] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[ti], a[tj], acc[p], 0, 0, 0);
    }
  }
  // accumulator layout of the float64 product (unlike the fp32 ones): register
  // r of lane l holds row l/16 + 4 r, column l%16
  double* dst = part + (((int64_t(bh) * F + f) * chunks + c) * kGramWaves + wave) * NP * 256;
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[p * 256 + (g + 4 * r) * 16 + r16] = acc[p][r];
}

// Per (frame, batch*head): the partial tiles added in (chunk, wave) order,
// then the cosine sum over the pairs y < z in order.
template <int RT>
__global__ __launch_bounds__(256) void row_gram_sum_kernel(const double* __restrict__ part, int Hs, int F,
                                                           int chunks, double* __restrict__ fsum) {
  constexpr int NP = gram_tile_pairs(RT);
  __shared__ double gram[16 * RT][16 * RT + 1];
  const int f = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int parts = chunks * kGramWaves;
  const double* src = part + (int64_t(bh) * F + f) * parts * NP * 256;
  for (int e = tid; e < NP * 256; e += 256) {
    double t = 0.0;
    for (int u = 0; u < parts; ++u) t += src[int64_t(u) * NP * 256 + e];
    int p = e / 256, ti = 0;
    while (p >= RT - ti) { p -= RT - ti; ++ti; }
    const int tj = ti + p;
    gram[16 * ti + (e % 256) / 16][16 * tj + e % 16] = t;
  }
  __syncthreads();
  if (tid == 0) {
    double total = 0.0;
    for (int y = 0; y < Hs; ++y)
      for (int z = y + 1; z < Hs; ++z) total += gram[y][z] / sqrt(gram[y][y] * gram[z][z]);
    fsum[int64_t(bh) * F + f] = total;
  }
}

// score[bh] = mean of the frame sums over F frames and Hs (Hs - 1) / 2 pairs each.
__global__ void row_score_kernel(const double* __restrict__ fsum, int F, int Hs, int heads,
                                 double* __restrict__ score) {
  const int bh = blockIdx.x * blockDim.x + threadIdx.x;
  if (bh >= heads) return;
  double t = 0.0;
  for (int f = 0; f < F; ++f) t += fsum[int64_t(bh) * F + f];
  score[bh] = t / (double(F) * double(Hs) * double(Hs - 1) / 2.0);
}

// out[e] = 1 when the fraction of the n_sets candidate masks that keep
// element e reaches rho, the fraction taken in float64.
__global__ __launch_bounds__(256) void aggregate_kernel(const uint8_t* __restrict__ masks, int n_sets,
                                                        int64_t elems, double rho,
                                                        uint8_t* __restrict__ out) {
  for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < elems;
       e += int64_t(gridDim.x) * blockDim.x) {
    int count = 0;
    for (int p = 0; p < n_sets; ++p) count += masks[int64_t(p) * elems + e] != 0;
    out[e] = double(count) / double(n_sets) >= rho ? 1 : 0;
  }
}

template <int D, int BLK>
void launch_energy_t(const __bf16* q, const __bf16* k, const svg_shape& s, float scale, double* E,
                     hipStream_t st) {
  const int nB = ceil_div(s.N, BLK);
  if constexpr (BLK == 128)
    hipLaunchKernelGGL((energy_pp_kernel<D>), dim3((nB + 1) / 2, s.B * s.H), dim3(512), 0, st, q, k, s.N, nB,
                       scale * 1.4426950408889634f, E);
  else
    hipLaunchKernelGGL((energy_kernel<D, BLK>), dim3(nB, s.B * s.H), dim3(BLK * 2), 0, st, q, k, s.N, nB,
                       scale * 1.4426950408889634f, E);
}

}  // namespace

void launch_block_energy(const void* q, const void* k, const svg_shape& s, float scale, double* E,
                         hipStream_t st) {
  const __bf16* qb = static_cast<const __bf16*>(q);
  const __bf16* kb = static_cast<const __bf16*>(k);
  if (s.block == 128) {
    if (s.D == 128) launch_energy_t<128, 128>(qb, kb, s, scale, E, st);
    else launch_energy_t<64, 128>(qb, kb, s, scale, E, st);
  } else {
    if (s.D == 128) launch_energy_t<128, 64>(qb, kb, s, scale, E, st);
    else launch_energy_t<64, 64>(qb, kb, s, scale, E, st);
  }
}

size_t row_similarity_workspace_bytes(const svg_shape& s) {
  const int64_t heads = int64_t(s.B) * s.H;
  const int64_t a_bytes = (heads * s.F * s.Hs * int64_t(s.N) * 4 + 255) / 256 * 256;
  const int64_t f_bytes = (heads * s.F * 8 + 255) / 256 * 256;
  const GramSplit sp = gram_split(s);
  const int rt = (s.Hs + 15) / 16;
  const int64_t p_bytes = heads * s.F * sp.chunks * kGramWaves * gram_tile_pairs(rt) * 256 * 8;
  return size_t(a_bytes + f_bytes + p_bytes);
}

template <int RT>
void launch_gram(const float* A, const svg_shape& s, const GramSplit& sp, double* part, double* fsum,
                 hipStream_t st) {
  const int heads = s.B * s.H;
  hipLaunchKernelGGL(row_gram_part_kernel<RT>, dim3(s.F * sp.chunks, heads), dim3(256), 0, st, A, s.N, s.Hs, s.F,
                     sp.chunks, sp.chunk_keys, part);
  hipLaunchKernelGGL(row_gram_sum_kernel<RT>, dim3(s.F, heads), dim3(256), 0, st, part, s.Hs, s.F, sp.chunks, fsum);
}

void launch_row_similarity(const void* q, const void* k, const svg_shape& s, float scale, double* score,
                           void* ws, hipStream_t st) {
  const int heads = s.B * s.H, rows = s.F * s.Hs;
  float* A = static_cast<float*>(ws);
  const int64_t a_bytes = (int64_t(heads) * rows * int64_t(s.N) * 4 + 255) / 256 * 256;
  const int64_t f_bytes = (int64_t(heads) * s.F * 8 + 255) / 256 * 256;
  double* fsum = reinterpret_cast<double*>(static_cast<char*>(ws) + a_bytes);
  double* part = reinterpret_cast<double*>(static_cast<char*>(ws) + a_bytes + f_bytes);
  const float c2 = scale * 1.4426950408889634f;
  const __bf16* qb = static_cast<const __bf16*>(q);
  const __bf16* kb = static_cast<const __bf16*>(k);
  if (s.D == 128)
    hipLaunchKernelGGL(row_pattern_kernel<128>, dim3((rows + 1) / 2, heads), dim3(512), 0, st, qb, kb, s.N, s.Ws,
                       rows, c2, A);
  else
    hipLaunchKernelGGL(row_pattern_kernel<64>, dim3((rows + 1) / 2, heads), dim3(512), 0, st, qb, kb, s.N, s.Ws,
                       rows, c2, A);
  const GramSplit sp = gram_split(s);
  switch ((s.Hs + 15) / 16) {
    case 1: launch_gram<1>(A, s, sp, part, fsum, st); break;
    case 2: launch_gram<2>(A, s, sp, part, fsum, st); break;
    case 3: launch_gram<3>(A, s, sp, part, fsum, st); break;
    default: launch_gram<4>(A, s, sp, part, fsum, st); break;
  }
  hipLaunchKernelGGL(row_score_kernel, dim3((heads + 255) / 256), dim3(256), 0, st, fsum, s.F, s.Hs, heads, score);
}

void launch_aggregate(const uint8_t* masks, int n_sets, int64_t elems, double rho, uint8_t* out,
                      hipStream_t st) {
  const int64_t blocks = std::min<int64_t>((elems + 255) / 256, 65535);
  hipLaunchKernelGGL(aggregate_kernel, dim3(unsigned(std::max<int64_t>(blocks, 1))), dim3(256), 0, st,
                     masks, n_sets, elems, rho, out);
}

}  // namespace svg
