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
//   tiles of 64 stream through double-buffered, padded LDS by 16-byte
//   global->LDS copies; S^T = K Q^T and U_c^T += V^T P_c^T run on
//   v_mfma_f32_16x16x32_bf16, the V^T operand coming from transposing LDS
//   reads, Z_c from one more MFMA with an all-ones operand.  Each class keeps
//   its own running max; within a 32-key step the spatial admission is the
//   same for all keys of a query, so only two classes are live per lane.
//   Writes (m_c, Z_c, U_c) per (chunk, sample, class).
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
#include <type_traits>

#include "mfma_common.h"
#include "svg_internal.h"

namespace svg {
namespace {

constexpr int kQ = 64;          // samples per workgroup (4 waves x 16)
constexpr int kTK = 32;         // keys staged per LDS tile (one 32-key step)
constexpr int kThreads = 256;
constexpr int kMaxWords = 32;   // bitmap words per row held in LDS (nB <= 1024)
constexpr int kChunkKeys = 32768;
constexpr float kRescaleLog2 = 24.0f;   // weights stay below 2^24 between moves

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

template <int D>
struct PCfg {
  static constexpr int DK = D / 32;      // 16x16x32 steps of the QK^T contraction
  static constexpr int DT = D / 16;      // 16-row tiles of U^T
  static constexpr int CPR = D / 8;      // 16-byte chunks per K / V row
  static constexpr int KROW = CPR + 1;   // padded K row (D+8 elements): conflict-free b128 fetches
  static constexpr int VROW = CPR + 4;   // padded V row (D+32): conflict-free transposing fetches
  static constexpr int KCH = kTK * KROW, VCH = kTK * VROW, BUF = KCH + VCH;
  static constexpr int SEGS = (BUF + 63) / 64;
  static constexpr int SPW = (SEGS + 3) / 4;   // load instructions per wave per tile
  static constexpr int STAGES = 3;             // ring of tiles: two loads in flight
  static constexpr int STRIDE = SEGS * 64;     // chunks per stage (whole 1-KB segments)
  static constexpr int DUMMY = STAGES * STRIDE;  // 1-KB sink for surplus segments
  static constexpr int REC = D + 4;      // floats per (sample, class) record: m, Z, pad, U[D]
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void profile_partial_kernel(ProfileArgs a, Geo g) {
  using C = PCfg<D>;
  __shared__ uint4 lds[C::STAGES * C::STRIDE + 64];   // ring stages, then a 1-KB sink
  __shared__ uint32_t rowS[kQ][kMaxWords];
  __shared__ uint32_t rowT[kQ][kMaxWords];
  __shared__ int blkT[C::STAGES][kTK];

  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, grp = lane >> 4;
  const int N = g.N;
  const int64_t head_off = int64_t(bh) * N * D;
  const __bf16* Qh = static_cast<const __bf16*>(a.q) + head_off;
  const char* Kh = reinterpret_cast<const char*>(static_cast<const __bf16*>(a.k) + head_off);
  const char* Vh = reinterpret_cast<const char*>(static_cast<const __bf16*>(a.v) + head_off);

  // bitmap rows of every sample: spatial row = frame-major block of the query,
  // temporal row = token-major block of the query
  for (int e = tid; e < kQ * a.W; e += kThreads) {
    int si = e / a.W, w = e % a.W;
    uint32_t ws = 0, wt = 0;
    if (si < a.n_samples) {
      int qi = min(max(a.idx[si], 0), g.Nv - 1);
      ws = a.bitmap[int64_t(qi >> g.blk_log2) * a.W + w];
      wt = a.bitmap[int64_t(a.nB + (token_major(qi, g) >> g.blk_log2)) * a.W + w];
    }
    rowS[si][w] = ws;
    rowT[si][w] = wt;
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

  const int k_begin = chunk * a.chunk_keys;
  const int k_end = min(N, k_begin + a.chunk_keys);
  const int n_tiles = (k_end - k_begin + kTK - 1) / kTK;

  // this thread's 16-byte global->LDS copies of one tile (K chunks, then V
  // chunks; lanes on row padding idle): byte offset inside the tile's rows,
  // bit 30 marking V, -1 when idle
  int src[C::SPW];
#pragma unroll
  for (int u = 0; u < C::SPW; ++u) {
    const int p = (u * 4 + wave) * 64 + lane;
    int off = -1;
    if (p < C::KCH) {
      const int r = p / C::KROW, c = p % C::KROW;
      if (c < C::CPR) off = (r * D + c * 8) * 2;
    } else if (p < C::BUF) {
      const int r = (p - C::KCH) / C::VROW, c = (p - C::KCH) % C::VROW;
      if (c < C::CPR) off = ((r * D + c * 8) * 2) | (1 << 30);
    }
    src[u] = off;
  }
  // Every wave issues exactly SPW copies per tile, so vmcnt(SPW) waits for
  // precisely the oldest tile in flight.  The LDS destination of a copy is
  // wave-uniform: lanes on row padding fill padding of their own stage, and
  // segments past the tile go to a sink.
  char* lds_b = reinterpret_cast<char*>(lds);
  auto stage = [&](int key0, int b) {
    char* sbase = lds_b + b * C::STRIDE * 16;
    const int last = k_end - 1 - key0;   // rows past the chunk read its last row (masked later)
#pragma unroll
    for (int u = 0; u < C::SPW; ++u) {
      const int seg = u * 4 + wave;
      int off = 0;
      const char* base = Kh;
      if (src[u] >= 0) {
        off = src[u] & ~(1 << 30);
        base = (src[u] & (1 << 30)) ? Vh : Kh;
        const int r = off / (D * 2);
        if (r > last) off += (last - r) * D * 2;
      }
      char* dst = seg < C::SEGS ? sbase + seg * 64 * 16 : lds_b + C::DUMMY * 16;
      __builtin_amdgcn_global_load_lds((GLB_AS void*)(base + int64_t(key0) * D * 2 + off),
                                       (LDS_AS void*)dst, 16, 0, 0);
    }
    if (tid < kTK) {
      const int key = min(key0 + tid, k_end - 1);
      blkT[b][tid] = token_major(key, g) >> g.blk_log2;
    }
  };

  f32x4 uacc[4][C::DT];
  f32x4 zacc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    zacc[c] = f32x4{};
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) uacc[c][dt] = f32x4{};
  }
  float mrun[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) mrun[c] = -INFINITY;
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;

  const int k_lane = ((8 * (n >> 2) + (n & 3)) * C::KROW + grp) * 16;   // tile 0, kk 0
  const int v_lane = C::KCH * 16 + ((8 * grp + (n >> 2)) * C::VROW) * 16 + ((n & 3) * 4) * 2;
  const float c2 = a.scale_log2;

  // Admission of this lane's 8 keys of a tile (8 * grp + i) for its sample:
  // bit i = kept by the temporal row, bit 8 = the tile's key block kept by
  // the spatial row.  Computed one tile ahead, so the dependent LDS lookups
  // overlap the previous tile's MFMAs.
  auto admission = [&](int key0, int b) -> uint32_t {
    const int kblock = min(key0 >> g.blk_log2, a.nB - 1);   // one key block for all 32 keys
    uint32_t bits = (svalid && ((rowS[sidx][kblock >> 5] >> (kblock & 31)) & 1u)) ? 0x100u : 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int bt = blkT[b][8 * grp + i];
      bits |= ((rowT[sidx][bt >> 5] >> (bt & 31)) & 1u) << i;
    }
    return bits;
  };

  if (n_tiles > 0) stage(k_begin, 0);
  if (n_tiles > 1) stage(k_begin + kTK, 1);
  __syncthreads();   // sample rows and the first tile's key blocks are visible
  uint32_t adm_next = n_tiles > 0 ? admission(k_begin, 0) : 0u;
  for (int t = 0; t < n_tiles; ++t) {
    const int b = t % C::STAGES;
    const int key0 = k_begin + t * kTK;
    const uint32_t adm = adm_next;
    // this thread's copies of tile t have landed (tile t+1 may still fly)
    if (t + 1 < n_tiles) __builtin_amdgcn_s_waitcnt(0x3f70 | C::SPW);   // vmcnt(SPW)
    else __builtin_amdgcn_s_waitcnt(0x3f70);                            // vmcnt(0)
    barrier_lds();     // everyone's copies landed; stage (t+2)%3 is no longer read
    if (t + 2 < n_tiles) stage(key0 + 2 * kTK, (t + 2) % C::STAGES);
    if (t + 1 < n_tiles) adm_next = admission(key0 + kTK, (t + 1) % C::STAGES);
    const char* lb = lds_b + b * C::STRIDE * 16;
#pragma unroll
    for (int half = 0; half < kTK / 32; ++half) {
      // ---- S^T for 32 keys: two 16x16 tiles; lane (n, grp) gets keys 8*grp + i
      f32x4 s2[2];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        s2[tile] = f32x4{};
#pragma unroll
        for (int kk = 0; kk < C::DK; ++kk) {
          const uint4 raw = *reinterpret_cast<const uint4*>(
              lb + k_lane + ((half * 32 + 4 * tile) * C::KROW + 4 * kk) * 16);
          s2[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(raw), qreg[kk], s2[tile], 0, 0, 0);
        }
      }
      const bool inS = (adm >> 8) & 1u;
      float x[8];
      bool inT[8];
      float m_in = -INFINITY, m_out = -INFINITY;   // this lane's max over T-kept / T-skipped keys
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kl = half * 32 + 8 * grp + i;
        inT[i] = (adm >> i) & 1u;
        const bool ok = svalid && key0 + kl < k_end;
        x[i] = ok ? s2[i >> 2][i & 3] : -INFINITY;
        m_in = fmaxf(m_in, inT[i] ? x[i] : -INFINITY);
        m_out = fmaxf(m_out, inT[i] ? -INFINITY : x[i]);
      }
      m_in *= c2;
      m_out *= c2;
      // the two classes live in this step: (both, S only) if inS, else (T only, none)
      float r_in = inS ? mrun[0] : mrun[2];
      float r_out = inS ? mrun[1] : mrun[3];
      // Fast path: no lane's block max exceeds its running max by more than
      // 2^24, so the stale maxima stay valid and no cross-lane exchange is
      // needed.  Otherwise combine the maxima over the 4 lanes of each sample
      // and rescale the classes whose maximum moved.
      if (__ballot(m_in > r_in + kRescaleLog2 || m_out > r_out + kRescaleLog2)) {
        m_in = fmaxf(m_in, shfl_xor_f(m_in, 16));
        m_in = fmaxf(m_in, shfl_xor_f(m_in, 32));
        m_out = fmaxf(m_out, shfl_xor_f(m_out, 16));
        m_out = fmaxf(m_out, shfl_xor_f(m_out, 32));
        const bool up_in = m_in > r_in + kRescaleLog2;
        const bool up_out = m_out > r_out + kRescaleLog2;
        const float al_in = up_in ? fast_exp2(r_in - m_in) : 1.f;
        const float al_out = up_out ? fast_exp2(r_out - m_out) : 1.f;
        float f[4];
        f[0] = inS ? al_in : 1.f;
        f[1] = inS ? al_out : 1.f;
        f[2] = inS ? 1.f : al_in;
        f[3] = inS ? 1.f : al_out;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          zacc[c] *= f[c];
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) uacc[c][dt] *= f[c];
        }
        if (up_in) r_in = m_in;
        if (up_out) r_out = m_out;
        mrun[0] = inS ? r_in : mrun[0];
        mrun[1] = inS ? r_out : mrun[1];
        mrun[2] = inS ? mrun[2] : r_in;
        mrun[3] = inS ? mrun[3] : r_out;
      }
      bf16x8 pin, pout;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = fast_exp2(__builtin_fmaf(x[i], c2, -(inT[i] ? r_in : r_out)));
        const __bf16 pb = (__bf16)p;
        pin[i] = inT[i] ? pb : (__bf16)0.0f;
        pout[i] = inT[i] ? (__bf16)0.0f : pb;
      }
      const bf16x8 zero8 = {};
      bf16x8 pc[4];
      pc[0] = inS ? pin : zero8;
      pc[1] = inS ? pout : zero8;
      pc[2] = inS ? zero8 : pin;
      pc[3] = inS ? zero8 : pout;
      // ---- U_c^T += V^T P_c^T; Z_c from an all-ones operand ------------------
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const char* p0 = lb + v_lane + (half * 32 * C::VROW) * 16 + dt * 32;
        bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p0);
        bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p0 + 4 * C::VROW * 16));
        const bf16x8 vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          uacc[c][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pc[c], uacc[c][dt], 0, 0, 0);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        zacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pc[c], zacc[c], 0, 0, 0);
    }
  }

  // ---- write this chunk's records ---------------------------------------------
  float* rec = a.ws + ((int64_t(bh) * a.n_chunks + chunk) * kQ + sidx) * 4 * C::REC;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float* r = rec + c * C::REC;
    if (grp == 0) {
      r[0] = mrun[c];
      r[1] = zacc[c][0];
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      *reinterpret_cast<f32x4*>(r + 4 + dt * 16 + 4 * grp) = uacc[c][dt];
  }
}

// Merge the chunks of one (head, sample) and evaluate both masks' errors.
// Wave c takes class c: the max over the chunks' maxima, each chunk's weight
// 2^(m_chunk - M) (kept in LDS) and Z; then thread d sums U[d] of every
// class with those weights.  All sums have a fixed order.
constexpr int kMergeCache = 512;   // chunk weights held in LDS (more are recomputed)

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, shfl_xor_f(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += shfl_xor_f(x, off);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void profile_merge_kernel(ProfileArgs a, double* __restrict__ per_sample) {
  using C = PCfg<D>;
  const int bh = blockIdx.x, sidx = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  __shared__ float M[4];
  __shared__ float Z[4];
  __shared__ float Wc[4][kMergeCache];
  __shared__ double red[2][4];
  const float* base = a.ws + (int64_t(bh) * a.n_chunks * kQ + sidx) * 4 * C::REC;
  const int64_t chunk_stride = int64_t(kQ) * 4 * C::REC;
  const int nc = a.n_chunks;
  auto weight = [&](int c, int ch, float m) -> float {
    const float mc = base[ch * chunk_stride + c * C::REC];
    return (m == -INFINITY || mc == -INFINITY) ? 0.f : fast_exp2(mc - m);
  };
  {
    const int c = wave;
    float m = -INFINITY;
    for (int ch = lane; ch < nc; ch += 64) m = fmaxf(m, base[ch * chunk_stride + c * C::REC]);
    m = wave_max64(m);
    float z = 0.f;
    for (int ch = lane; ch < nc; ch += 64) {
      const float w = weight(c, ch, m);
      if (ch < kMergeCache) Wc[c][ch] = w;
      z += base[ch * chunk_stride + c * C::REC + 1] * w;
    }
    z = wave_sum64(z);
    if (lane == 0) {
      M[c] = m;
      Z[c] = z;
    }
  }
  __syncthreads();
  double e[2] = {0.0, 0.0};
  for (int d = tid; d < D; d += 256) {
    float U[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float u0 = 0.f, u1 = 0.f;
      const float* r = base + c * C::REC + 4 + d;
      int ch = 0;
      for (; ch + 1 < nc; ch += 2) {
        const float w0 = ch < kMergeCache ? Wc[c][ch] : weight(c, ch, M[c]);
        const float w1 = ch + 1 < kMergeCache ? Wc[c][ch + 1] : weight(c, ch + 1, M[c]);
        u0 += r[ch * chunk_stride] * w0;
        u1 += r[(ch + 1) * chunk_stride] * w1;
      }
      if (ch < nc) u0 += r[ch * chunk_stride] * (ch < kMergeCache ? Wc[c][ch] : weight(c, ch, M[c]));
      U[c] = u0 + u1;
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
  // fixed-order sum: lanes of a wave by a butterfly, then the four waves in order
#pragma unroll
  for (int k = 0; k < 2; ++k) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) e[k] += __shfl_xor(e[k], off, 64);
  }
  if (lane == 0) {
    red[0][wave] = e[0];
    red[1][wave] = e[1];
  }
  __syncthreads();
  if (tid == 0) {
    per_sample[(int64_t(bh) * kQ + sidx) * 2 + 0] = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
    per_sample[(int64_t(bh) * kQ + sidx) * 2 + 1] = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
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
  // Chunking: the partial kernel runs two workgroups per CU, 512 at a time on
  // the 256 CUs of an MI355X.  The chunk length (whole 32-key tiles, at most
  // kChunkKeys keys) minimises a cost in units of one tile's time: rounds of
  // workgroups x (tiles per workgroup + about 3 tiles of set-up), plus the
  // chunk records written and merged (about 0.031 tile per record set of a
  // head, 64 samples x 4 classes x (D + 4) floats, at HBM speed).
  constexpr int kSlots = 512;
  int ck = kTK, nc = ceil_div(N, kTK);
  long best = -1;
  for (int t = kTK; t <= kChunkKeys; t += kTK) {
    const int c = ceil_div(N, t);
    const long cost = long(ceil_div(BH * c, kSlots)) * (t / kTK + 3) * 1000 + 31L * BH * c;
    if (best < 0 || cost < best) {
      best = cost;
      ck = t;
      nc = c;
    }
    if (c == 1) break;
  }
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
