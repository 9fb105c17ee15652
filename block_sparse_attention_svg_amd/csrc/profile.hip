// Online head profiling ([SVG], online profiling: about 64 sampled queries
// per step; each head keeps whichever of the spatial / temporal masks gives
// the smaller error against dense attention).
//
// The error of a mask is computed without subtracting two nearly equal
// outputs.  Every (query, key) pair falls in one of four classes: kept by both
// masks (0), spatial only (1), temporal only (2), neither (3).  With per-class
// softmax partial sums Z_c = sum exp(s - m_c) and U_c = sum exp(s - m_c) v,
// a mask with kept set "in" and complement "out" satisfies
//     o_dense - o_mask = (Z_out / Z) (U_out / Z_out - U_in / Z_in),
// all terms being sums of non-negative weights.
//
// Pass 1 (profile_partial_kernel): split-K over key chunks.  One workgroup per
//   (chunk, batch*head), four wavefronts of 16 sampled queries each.  Key
//   tiles of 64 are staged in LDS (K row-major, V transposed); S^T = K Q^T and
//   U_c^T += V^T P_c^T run on v_mfma_f32_16x16x32_bf16; each class keeps its
//   own running max.  Writes (m_c, Z_c, U_c) per (chunk, sample, class).
// Pass 2 (profile_merge_kernel): one workgroup per (batch*head, sample):
//   merges the chunks in a fixed order and evaluates both errors.
// Pass 3 (profile_choose_kernel): sums the samples in order, picks the head's
//   mask (a tie goes to spatial).  Every reduction has a fixed order, so the
//   result is identical on every call.
//
// MFMA 16x16x32 layout used here: operand element i of lane l covers
// row/column l%16 and contraction index 8*(l/16)+i; accumulator register r of
// lane l holds row 4*(l/16)+r, column l%16.  The two 16-key S^T tiles of a
// 32-key step fetch K rows in the order 8*(m/4) + 4*tile + m%4, so lane
// group g = l/16 ends up holding keys 8g..8g+7, exactly its P^T operand.
#include "mfma_common.h"
#include "svg_internal.h"

namespace svg {
namespace {

constexpr int kQ = 64;          // samples per workgroup (4 waves x 16)
constexpr int kTK = 64;         // keys staged per LDS tile
constexpr int kThreads = 256;
constexpr int kMaxWords = 32;   // bitmap words per row held in LDS (nB <= 1024)
constexpr int kChunkKeys = 4096;
constexpr float kRescaleLog2 = 8.0f;

template <int D>
struct PCfg {
  static constexpr int DK = D / 32;   // 16x16x32 steps of the QK^T contraction
  static constexpr int DT = D / 16;   // 16-row tiles of U^T
  using KTile = LdsTile<kTK, D>;
  using VTile = LdsTile<D, kTK>;
  static constexpr int K_LOADS = KTile::CHUNKS / kThreads;
  static constexpr int V_TASKS = (kTK / 8) * (D / 8);
  static constexpr int V_PER_T = (V_TASKS + kThreads - 1) / kThreads;
  static constexpr int REC = D + 4;   // floats per (sample, class) record: m, Z, pad, U[D]
};

struct Geo {
  int N, Nv, F, S, blk_log2;
  FastDiv divS;
};

// token-major position of frame-major token j
__device__ __forceinline__ int token_major(int j, const Geo& g) {
  if (j >= g.Nv) return j;
  int f = int(g.divS.div(uint32_t(j)));
  int s = j - f * g.S;
  return s * g.F + f;
}

template <int D>
__global__ __launch_bounds__(kThreads) void profile_partial_kernel(ProfileArgs a, Geo g) {
  using C = PCfg<D>;
  __shared__ uint4 Ks[C::KTile::CHUNKS];
  __shared__ uint4 Vt[C::VTile::CHUNKS];
  __shared__ uint32_t rowS[kQ][kMaxWords];
  __shared__ uint32_t rowT[kQ][kMaxWords];
  __shared__ int blkT[kTK];

  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, grp = lane >> 4;
  const int N = g.N;
  const int64_t head_off = int64_t(bh) * N * D;
  const __bf16* Qh = static_cast<const __bf16*>(a.q) + head_off;
  const uint4* Kg = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(a.k) + head_off);
  const uint4* Vg = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(a.v) + head_off);

  // bitmap rows of every sample: spatial row = frame-major block of the query,
  // temporal row = token-major block of the query
  for (int e = tid; e < kQ * a.W; e += kThreads) {
    int sidx = e / a.W, w = e % a.W;
    uint32_t ws = 0, wt = 0;
    if (sidx < a.n_samples) {
      int qi = min(max(a.idx[sidx], 0), g.Nv - 1);
      int rs = qi >> g.blk_log2;
      int rt = token_major(qi, g) >> g.blk_log2;
      ws = a.bitmap[int64_t(rs) * a.W + w];
      wt = a.bitmap[int64_t(a.nB + rt) * a.W + w];
    }
    rowS[sidx][w] = ws;
    rowT[sidx][w] = wt;
  }

  // Q operand: lane holds sample wave*16 + n, dims 32*kk + 8*grp + i
  const int sidx = wave * 16 + n;
  const bool svalid = sidx < a.n_samples;
  bf16x8 qreg[C::DK];
  {
    int qi = svalid ? min(max(a.idx[sidx], 0), g.Nv - 1) : 0;
#pragma unroll
    for (int kk = 0; kk < C::DK; ++kk) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (svalid) u = *reinterpret_cast<const uint4*>(Qh + int64_t(qi) * D + 32 * kk + 8 * grp);
      qreg[kk] = as_bf16x8(u);
    }
  }

  f32x4 uacc[4][C::DT];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) uacc[c][dt] = f32x4{};
  float mrun[4], zpart[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) { mrun[c] = -INFINITY; zpart[c] = 0.f; }

  const int k_begin = chunk * a.chunk_keys;
  const int k_end = min(N, k_begin + a.chunk_keys);
  constexpr int CPR = D / 8;

  uint4 kst[C::K_LOADS];
  uint4 vst[C::V_PER_T][8];
  auto load = [&](int key0) {
#pragma unroll
    for (int u = 0; u < C::K_LOADS; ++u) {
      int c = tid + u * kThreads;
      int key = key0 + c / CPR;
      kst[u] = key < k_end ? Kg[int64_t(key) * CPR + c % CPR] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_T; ++u) {
      int t = tid + u * kThreads;
      int kg = t % (kTK / 8), dc = t / (kTK / 8);
      if (t < C::V_TASKS) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          int key = key0 + 8 * kg + i;
          vst[u][i] = key < k_end ? Vg[int64_t(key) * CPR + dc] : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  if (k_begin < k_end) load(k_begin);
  for (int key0 = k_begin; key0 < k_end; key0 += kTK) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < C::K_LOADS; ++u) {
      int c = tid + u * kThreads;
      Ks[C::KTile::slot(c / CPR, c % CPR)] = kst[u];
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_T; ++u) {
      int t = tid + u * kThreads;
      if (t < C::V_TASKS) {
        int kg = t % (kTK / 8), dc = t / (kTK / 8);
        uint4 cols[8];
        transpose8x8(vst[u], cols);
#pragma unroll
        for (int j = 0; j < 8; ++j) Vt[C::VTile::slot(8 * dc + j, kg)] = cols[j];
      }
    }
    if (tid < kTK) {
      int key = key0 + tid;
      blkT[tid] = key < k_end ? (token_major(key, g) >> g.blk_log2) : 0;
    }
    __syncthreads();
    if (key0 + kTK < k_end) load(key0 + kTK);

#pragma unroll
    for (int half = 0; half < kTK / 32; ++half) {
      // ---- S^T for 32 keys: two 16x16 tiles ---------------------------------
      f32x4 s2[2];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        s2[tile] = f32x4{};
        const int krow = half * 32 + 8 * (n >> 2) + 4 * tile + (n & 3);
#pragma unroll
        for (int kk = 0; kk < C::DK; ++kk) {
          bf16x8 kop = as_bf16x8(Ks[C::KTile::slot(krow, 4 * kk + grp)]);
          s2[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[kk], s2[tile], 0, 0, 0);
        }
      }
      // lane (n, grp) now holds keys half*32 + 8*grp + i, i = 0..7
      const int kbase = key0 + half * 32;
      const int kblock = min(kbase >> g.blk_log2, a.nB - 1);  // one key block for all 32 keys
      const bool inS = svalid && ((rowS[sidx][kblock >> 5] >> (kblock & 31)) & 1u);
      float x[8];
      int cls[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kl = half * 32 + 8 * grp + i;
        const int key = key0 + kl;
        const int bt = blkT[kl];
        const bool inT = (rowT[sidx][bt >> 5] >> (bt & 31)) & 1u;
        cls[i] = (inS ? 0 : 2) + (inT ? 0 : 1);
        const float sv = s2[i >> 2][i & 3] * a.scale_log2;
        x[i] = (key < k_end && svalid) ? sv : -INFINITY;
      }
      // per-class block max, combined over the 4 lane groups of a sample
      float mx[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, cls[i] == c ? x[i] : -INFINITY);
        m = fmaxf(m, shfl_xor_f(m, 16));
        m = fmaxf(m, shfl_xor_f(m, 32));
        mx[c] = m;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (mx[c] > mrun[c] + kRescaleLog2) {
          const float alpha = fast_exp2(mrun[c] - mx[c]);
          zpart[c] *= alpha;
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) uacc[c][dt] *= alpha;
          mrun[c] = mx[c];
        }
      }
      bf16x8 pb[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = cls[i];
        const float mref = c == 0 ? mrun[0] : c == 1 ? mrun[1] : c == 2 ? mrun[2] : mrun[3];
        const float p = x[i] == -INFINITY ? 0.f : fast_exp2(x[i] - mref);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const float pc = c == cc ? p : 0.f;
          zpart[cc] += pc;
          pb[cc][i] = (__bf16)pc;
        }
      }
      // ---- U_c^T += V^T P_c^T -------------------------------------------------
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        bf16x8 vop = as_bf16x8(Vt[C::VTile::slot(dt * 16 + n, 4 * half + grp)]);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          uacc[c][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[c], uacc[c][dt], 0, 0, 0);
      }
    }
  }

  // ---- write this chunk's records ---------------------------------------------
  float* rec = a.ws + ((int64_t(bh) * a.n_chunks + chunk) * kQ + sidx) * 4 * C::REC;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float z = zpart[c];
    z += shfl_xor_f(z, 16);
    z += shfl_xor_f(z, 32);
    float* r = rec + c * C::REC;
    if (grp == 0) {
      r[0] = mrun[c];
      r[1] = z;
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      *reinterpret_cast<f32x4*>(r + 4 + dt * 16 + 4 * grp) = uacc[c][dt];
  }
}

// Merge the chunks of one (head, sample) and evaluate both masks' errors.
template <int D>
__global__ __launch_bounds__(256) void profile_merge_kernel(ProfileArgs a, double* __restrict__ per_sample) {
  using C = PCfg<D>;
  const int bh = blockIdx.x, sidx = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ float M[4];
  __shared__ float Z[4];
  __shared__ double red[2][256];
  const float* base = a.ws + (int64_t(bh) * a.n_chunks * kQ + sidx) * 4 * C::REC;
  const int64_t chunk_stride = int64_t(kQ) * 4 * C::REC;
  if (tid < 4) {
    float m = -INFINITY;
    for (int ch = 0; ch < a.n_chunks; ++ch) m = fmaxf(m, base[ch * chunk_stride + tid * C::REC]);
    float z = 0.f;
    if (m != -INFINITY)
      for (int ch = 0; ch < a.n_chunks; ++ch) {
        const float* r = base + ch * chunk_stride + tid * C::REC;
        if (r[0] != -INFINITY) z += r[1] * fast_exp2(r[0] - m);
      }
    M[tid] = m;
    Z[tid] = z;
  }
  __syncthreads();
  double e[2] = {0.0, 0.0};
  for (int d = tid; d < D; d += 256) {
    float U[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float u = 0.f;
      if (M[c] != -INFINITY)
        for (int ch = 0; ch < a.n_chunks; ++ch) {
          const float* r = base + ch * chunk_stride + c * C::REC;
          if (r[0] != -INFINITY) u += r[4 + d] * fast_exp2(r[0] - M[c]);
        }
      U[c] = u;
    }
#pragma unroll
    for (int mask = 0; mask < 2; ++mask) {
      // spatial keeps classes {0, 1}; temporal keeps {0, 2}
      const int i0 = 0, i1 = mask == 0 ? 1 : 2;
      const int o0 = mask == 0 ? 2 : 1, o1 = 3;
      auto group = [&](int c0, int c1, float& mg, float& zg, float& ug) {
        mg = fmaxf(M[c0], M[c1]);
        zg = 0.f; ug = 0.f;
        if (mg == -INFINITY) return;
        if (M[c0] != -INFINITY) { float w = fast_exp2(M[c0] - mg); zg += Z[c0] * w; ug += U[c0] * w; }
        if (M[c1] != -INFINITY) { float w = fast_exp2(M[c1] - mg); zg += Z[c1] * w; ug += U[c1] * w; }
      };
      float mi, zi, ui, mo, zo, uo;
      group(i0, i1, mi, zi, ui);
      group(o0, o1, mo, zo, uo);
      float diff = 0.f;
      if (zo > 0.f) {
        if (!(zi > 0.f)) {
          diff = uo / zo;  // the mask keeps nothing: o_mask = 0
        } else {
          float r;  // Z_out / Z, evaluated without overflow
          if (mo >= mi) r = zo / (zi * fast_exp2(mi - mo) + zo);
          else { float zo_s = zo * fast_exp2(mo - mi); r = zo_s / (zi + zo_s); }
          diff = r * (uo / zo - ui / zi);
        }
      }
      e[mask] += double(diff) * double(diff);
    }
  }
  red[0][tid] = e[0];
  red[1][tid] = e[1];
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) {
      red[0][tid] += red[0][tid + off];
      red[1][tid] += red[1][tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    per_sample[(int64_t(bh) * kQ + sidx) * 2 + 0] = red[0][0];
    per_sample[(int64_t(bh) * kQ + sidx) * 2 + 1] = red[1][0];
  }
}

__global__ void profile_choose_kernel(const double* __restrict__ per_sample, int BH, int n_samples,
                                      int32_t* __restrict__ choice, float* __restrict__ err) {
  const int bh = blockIdx.x * blockDim.x + threadIdx.x;
  if (bh >= BH) return;
  double es = 0.0, et = 0.0;
  for (int s = 0; s < n_samples; ++s) {
    es += per_sample[(int64_t(bh) * kQ + s) * 2 + 0];
    et += per_sample[(int64_t(bh) * kQ + s) * 2 + 1];
  }
  choice[bh] = es <= et ? 0 : 1;
  if (err) {
    err[2 * bh + 0] = float(es);
    err[2 * bh + 1] = float(et);
  }
}

size_t records_bytes(int BH, int D, int n_chunks) {
  return size_t(BH) * n_chunks * kQ * 4 * (D + 4) * sizeof(float);
}

}  // namespace

size_t profile_workspace_bytes(int BH, int N, int D, int block, int n_samples, int* chunk_keys,
                               int* n_chunks) {
  (void)block;
  (void)n_samples;
  int ck = kChunkKeys;
  int nc = ceil_div(N, ck);
  if (chunk_keys) *chunk_keys = ck;
  if (n_chunks) *n_chunks = nc;
  size_t rec = records_bytes(BH, D, nc);
  rec = (rec + 255) / 256 * 256;
  return rec + size_t(BH) * kQ * 2 * sizeof(double);
}

void launch_profile(const ProfileArgs& a, hipStream_t st) {
  Geo g;
  g.N = a.N;
  g.F = a.F;
  g.S = a.Hs * a.Ws;
  g.Nv = a.F * g.S;
  g.blk_log2 = a.block == 128 ? 7 : 6;
  g.divS = FastDiv(uint32_t(g.S));
  size_t rec = (records_bytes(a.BH, a.D, a.n_chunks) + 255) / 256 * 256;
  double* per_sample = reinterpret_cast<double*>(reinterpret_cast<char*>(a.ws) + rec);
  dim3 grid1(a.n_chunks, a.BH);
  dim3 grid2(a.BH, a.n_samples);
  if (a.D == 128) {
    hipLaunchKernelGGL(profile_partial_kernel<128>, grid1, dim3(kThreads), 0, st, a, g);
    hipLaunchKernelGGL(profile_merge_kernel<128>, grid2, dim3(256), 0, st, a, per_sample);
  } else {
    hipLaunchKernelGGL(profile_partial_kernel<64>, grid1, dim3(kThreads), 0, st, a, g);
    hipLaunchKernelGGL(profile_merge_kernel<64>, grid2, dim3(256), 0, st, a, per_sample);
  }
  hipLaunchKernelGGL(profile_choose_kernel, dim3(ceil_div(a.BH, 64)), dim3(64), 0, st, per_sample,
                     a.BH, a.n_samples, a.choice, a.err);
}

}  // namespace svg
