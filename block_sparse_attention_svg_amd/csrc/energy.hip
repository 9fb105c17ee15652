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
// output for the threshold rule.
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

// ---- row-repetitive heads ([CalibAtt] section 3.2) --------------------------
// The attention pattern of latent row (f, y) is the sum of the softmax weights
// of its Ws queries over all N keys; a head is row-repetitive when the mean
// cosine between the patterns of the rows of a frame exceeds gamma.
//
// row_pattern_kernel: one workgroup per (batch*head, latent row), four
// wavefronts of 32 query slots (Ws <= 128; slots past Ws masked).  Sweep 1 is
// the energy kernel's (running max and sum per query, K tiles double-buffered
// in LDS, the second tile borrowing the weight buffer); sweep 2 writes each
// 128-key block's weights to an LDS buffer [query][key] and 128 threads sum a
// key's column over the queries in order.  fp32 sums, identical on every call.
constexpr int kPRS = 128 * 4 + 16;   // weight-buffer row stride (bytes): one query, 128 keys

template <int D>
__global__ __launch_bounds__(256) void row_pattern_kernel(const __bf16* __restrict__ q,
                                                          const __bf16* __restrict__ k, int N, int Ws,
                                                          int rows, float c2, float* __restrict__ A) {
  using C = ECfg<D, 128>;
  static_assert(C::THREADS == 256, "four wavefronts");
  __shared__ __attribute__((aligned(16))) char ktile[128 * C::RS];
  __shared__ __attribute__((aligned(16))) char pbuf[128 * kPRS];
  static_assert(128 * kPRS >= 128 * C::RS, "the weight buffer holds a K tile in sweep 1");
  const int row = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;
  const int nB = (N + 127) / 128;
  const __bf16* qh = q + int64_t(bh) * N * D;
  const __bf16* kh = k + int64_t(bh) * N * D;
  const int slot = wave * 32 + n;
  const bool q_ok = slot < Ws;
  const int qi = row * Ws + slot;
  bf16x8 qreg[C::DK];
#pragma unroll
  for (int kk = 0; kk < C::DK; ++kk) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (q_ok) u = *reinterpret_cast<const uint4*>(qh + int64_t(qi) * D + 16 * kk + 8 * h);
    qreg[kk] = as_bf16x8(u);
  }
  f32x16 sacc[C::KT];
  auto key_of = [&](int kb, int kt, int i) { return kb * 128 + kt * 32 + 8 * (i >> 2) + 4 * h + (i & 3); };
  uint4 kr[C::LOADS];

  float m = -INFINITY, l = 0.f;
  load_k<D, 128>(kr, kh, 0, N, tid);
  for (int kb = 0; kb < nB; ++kb) {
    char* tile = (kb & 1) ? pbuf : ktile;
    store_k<D, 128>(tile, kr, tid);
    __syncthreads();
    if (kb + 1 < nB) load_k<D, 128>(kr, kh, kb + 1, N, tid);
    scores<D, 128>(tile, qreg, n, h, sacc);
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

  float* arow = A + (int64_t(bh) * rows + row) * N;
  __syncthreads();   // sweep 1's tiles are no longer read
  load_k<D, 128>(kr, kh, 0, N, tid);
  for (int kb = 0; kb < nB; ++kb) {
    store_k<D, 128>(ktile, kr, tid);   // the tile and the weights of block kb-1 are no longer read
    __syncthreads();
    if (kb + 1 < nB) load_k<D, 128>(kr, kh, kb + 1, N, tid);
    scores<D, 128>(ktile, qreg, n, h, sacc);
    char* prow = pbuf + slot * kPRS;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4 w;
        float* wp = reinterpret_cast<float*>(&w);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * g4 + j;
          const float p = fast_exp2(__builtin_fmaf(sacc[kt][i], c2, -lse2));
          wp[j] = (q_ok && key_of(kb, kt, i) < N) ? p : 0.f;
        }
        // keys kt*32 + 8*g4 + 4*h + 0..3 of the block
        *reinterpret_cast<float4*>(prow + (kt * 32 + 8 * g4 + 4 * h) * 4) = w;
      }
    __syncthreads();
    if (tid < 128 && kb * 128 + tid < N) {
      float t = 0.f;
      for (int r = 0; r < 128; ++r) t += *reinterpret_cast<const float*>(pbuf + r * kPRS + tid * 4);
      arow[kb * 128 + tid] = t;
    }
    __syncthreads();
  }
}

// Per (batch*head, frame): Gram matrix of the frame's Hs row patterns (float64
// accumulation over the keys, 64 keys at a time through LDS), then the sum of
// the cosines over the pairs of distinct rows, in order.
constexpr int kMaxHs = 64;
__global__ __launch_bounds__(256) void row_gram_kernel(const float* __restrict__ A, int N, int Hs, int F,
                                                       double* __restrict__ fsum) {
  __shared__ float tile[kMaxHs][64 + 1];
  __shared__ double gram[kMaxHs * (kMaxHs + 1) / 2];
  const int f = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int pairs = Hs * (Hs + 1) / 2;   // (y <= z), packed row-major over y
  const float* base = A + (int64_t(bh) * F + f) * Hs * int64_t(N);
  constexpr int PPT = (kMaxHs * (kMaxHs + 1) / 2 + 255) / 256;
  double acc[PPT];
  int py[PPT], pz[PPT];
#pragma unroll
  for (int u = 0; u < PPT; ++u) {
    acc[u] = 0.0;
    int p = tid + u * 256, y = 0;
    while (p >= Hs - y && y < Hs) { p -= Hs - y; ++y; }
    py[u] = y;
    pz[u] = y + p;
  }
  for (int j0 = 0; j0 < N; j0 += 64) {
    __syncthreads();
    for (int e = tid; e < Hs * 64; e += 256) {
      const int y = e / 64, j = e % 64;
      tile[y][j] = j0 + j < N ? base[int64_t(y) * N + j0 + j] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      if (tid + u * 256 < pairs) {
        double s = 0.0;
        for (int j = 0; j < 64; ++j) s += double(tile[py[u]][j]) * double(tile[pz[u]][j]);
        acc[u] += s;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < PPT; ++u)
    if (tid + u * 256 < pairs) gram[tid + u * 256] = acc[u];
  __syncthreads();
  if (tid == 0) {
    auto at = [&](int y, int z) { return gram[y * Hs - y * (y - 1) / 2 + (z - y)]; };
    double total = 0.0;
    for (int y = 0; y < Hs; ++y)
      for (int z = y + 1; z < Hs; ++z) total += at(y, z) / sqrt(at(y, y) * at(z, z));
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
  const int64_t a_bytes = heads * s.F * s.Hs * int64_t(s.N) * 4;
  return size_t((a_bytes + 255) / 256 * 256 + heads * s.F * 8);
}

void launch_row_similarity(const void* q, const void* k, const svg_shape& s, float scale, double* score,
                           void* ws, hipStream_t st) {
  const int heads = s.B * s.H, rows = s.F * s.Hs;
  float* A = static_cast<float*>(ws);
  const int64_t a_bytes = int64_t(heads) * rows * int64_t(s.N) * 4;
  double* fsum = reinterpret_cast<double*>(static_cast<char*>(ws) + (a_bytes + 255) / 256 * 256);
  const float c2 = scale * 1.4426950408889634f;
  const __bf16* qb = static_cast<const __bf16*>(q);
  const __bf16* kb = static_cast<const __bf16*>(k);
  if (s.D == 128)
    hipLaunchKernelGGL(row_pattern_kernel<128>, dim3(rows, heads), dim3(256), 0, st, qb, kb, s.N, s.Ws, rows, c2, A);
  else
    hipLaunchKernelGGL(row_pattern_kernel<64>, dim3(rows, heads), dim3(256), 0, st, qb, kb, s.N, s.Ws, rows, c2, A);
  hipLaunchKernelGGL(row_gram_kernel, dim3(s.F, heads), dim3(256), 0, st, A, s.N, s.Hs, s.F, fsum);
  hipLaunchKernelGGL(row_score_kernel, dim3((heads + 255) / 256), dim3(256), 0, st, fsum, s.F, s.Hs, heads, score);
}

void launch_aggregate(const uint8_t* masks, int n_sets, int64_t elems, double rho, uint8_t* out,
                      hipStream_t st) {
  const int64_t blocks = std::min<int64_t>((elems + 255) / 256, 65535);
  hipLaunchKernelGGL(aggregate_kernel, dim3(unsigned(std::max<int64_t>(blocks, 1))), dim3(256), 0, st,
                     masks, n_sets, elems, rho, out);
}

}  // namespace svg
