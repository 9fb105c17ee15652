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
//   reads, Z_c from one more MFMA with an all-ones operand.  Within a 32-key
//   step the spatial admission is the same for all keys of a query, so only
//   two classes are live per lane, and only their MFMAs are issued (the other
//   two are parked in registers); the live pair shares one running max per
//   query (weights relative to a common scale lose nothing in floating
//   point, and the merge weighs every record by its own max).
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


template <int D>
struct PCfg {
  static constexpr int DK = D / 32;      // 16x16x32 steps of the QK^T contraction
  static constexpr int DT = D / 16;      // 16-row tiles of U^T
  static constexpr int CPR = D / 8;      // 16-byte chunks per K / V row
  static constexpr int KROW = CPR + 1;   // padded K row (D+8 elements): conflict-free b128 fetches
  static constexpr int VROW = CPR + 4;   // padded V row (D+32): conflict-free transposing fetches
  static constexpr int KCH = kTK * KROW, VCH = kTK * VROW;
  // K rows and V rows take whole 1-KB segments of their own, so that one
  // copy instruction reads from one tensor only
  static constexpr int KSEG = (KCH + 63) / 64, VSEG = (VCH + 63) / 64;
  static constexpr int SEGS = KSEG + VSEG;
  static constexpr int KOFF = KSEG * 64;       // first chunk of the V rows in a stage
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

// 0xffff in each 16-bit half whose bit of `bits` (bit k for the low half,
// k + 1 for the high half) is set
__device__ __forceinline__ uint32_t pair_mask(uint32_t bits, int k) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_sbfe(int(bits), k, 1)) & 0xffffu;
  const uint32_t hi = uint32_t(__builtin_amdgcn_sbfe(int(bits), k + 1, 1)) << 16;
  return lo | hi;
}

// Exchange two registers of the active lanes in place (no temporary: the
// swapped values stay in their registers, so a rarely taken swap adds no
// register pressure to the loop around it).
__device__ __forceinline__ void swap_lane(float& a, float& b) {
  asm volatile("v_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_lane(f32x4& a, f32x4& b) {
  float x[4], y[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = a[r];
    y[r] = b[r];
    swap_lane(x[r], y[r]);
  }
  a = f32x4{x[0], x[1], x[2], x[3]};
  b = f32x4{y[0], y[1], y[2], y[3]};
}

// ADM8: every frame holds a multiple of 8 tokens and 7 F <= 3 * block, so
// the 8 keys of a lane (8-aligned) lie in one frame (or all in the text), and
// their token-major blocks span at most 4 consecutive blocks: the keys'
// admission then comes from one 64-bit window of the sample's temporal row
// and four key masks per lane group (admT), instead of one lookup per key.
template <int D, bool ADM8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void profile_partial_kernel(ProfileArgs a, Geo g) {
  using C = PCfg<D>;
  __shared__ uint4 lds[C::STAGES * C::STRIDE + 64];   // ring stages, then a 1-KB sink
  // rows padded to an odd word count: the 16 samples of a wave look up the
  // same word index at once, which then falls in 16 different banks
  __shared__ uint32_t rowS[kQ][kMaxWords + 1];
  __shared__ uint32_t rowT[kQ][kMaxWords + 1];
  __shared__ int blkT[C::STAGES][kTK];
  // ADM8: per stage and lane group g (keys 8 g .. 8 g + 7 of the tile): the
  // first key's token-major block bt0, and byte d of the mask word = the keys
  // whose block is bt0 + d
  __shared__ uint2 admT[C::STAGES][4];

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

  // This thread's 16-byte global->LDS copies of one tile: copy u of wave w
  // fills segment 4u + w of the stage (K segments first, then V; segments
  // past the stage go to a 1-KB sink).  off[u] = byte offset of the lane's
  // chunk within the tile's rows (row r, chunk c: (r * D + 8 c) * 2), or
  // kNoFetch for lanes on row padding.  Every wave issues exactly SPW copies
  // per tile, so vmcnt(SPW) waits for precisely the oldest tile in flight.
  constexpr uint32_t kNoFetch = 0x80000000u;   // beyond any tile's buffer range: nothing is read
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t off[C::SPW];
#pragma unroll
  for (int u = 0; u < C::SPW; ++u) {
    const int seg = u * 4 + wave;
    uint32_t o = kNoFetch;
    if (seg < C::KSEG) {
      const int p = seg * 64 + lane, r = p / C::KROW, c = p % C::KROW;
      if (p < C::KCH && c < C::CPR) o = uint32_t(r * D + c * 8) * 2;
    } else if (seg < C::SEGS) {
      const int p = (seg - C::KSEG) * 64 + lane, r = p / C::VROW, c = p % C::VROW;
      if (p < C::VCH && c < C::CPR) o = uint32_t(r * D + c * 8) * 2;
    }
    off[u] = o;
  }
  const uint32_t lds_base = lds_addr_of(lds);
  auto stage = [&](int key0, int b) {
    // buffer resources over the tile's rows that exist (rows past N are not
    // fetched; in a tile that ends past N the lanes of those rows read the
    // last row instead, so the stage holds finite values throughout)
    const int rows = min(kTK, k_end - key0);
    const LdsCopySrc ksrc(Kh + int64_t(key0) * D * 2, rows * D * 2);
    const LdsCopySrc vsrc(Vh + int64_t(key0) * D * 2, rows * D * 2);
    const uint32_t sbase = lds_base + b * C::STRIDE * 16;
    auto issue = [&](auto ragged_c) {
      constexpr bool RAGGED = decltype(ragged_c)::value;
#pragma unroll
      for (int u = 0; u < C::SPW; ++u) {
        const int seg = u * 4 + wave_u;   // wave-uniform: scalar selects, no branches
        uint32_t o = off[u];
        if constexpr (RAGGED) {
          const int r = int(o) / (D * 2);
          if (o != kNoFetch && r >= rows) o -= uint32_t(r - rows + 1) * D * 2;
        }
        const LdsCopySrc& src = seg < C::KSEG ? ksrc : vsrc;
        src.copy16(o, 0, seg < C::SEGS ? sbase + seg * 1024 : lds_base + C::DUMMY * 16);
      }
    };
    if (rows < kTK) issue(std::true_type{});   // the chunk's last tile, past N
    else issue(std::false_type{});
    if constexpr (ADM8) {
      if (tid < 4) {
        const int j0 = min(key0 + 8 * tid, k_end - 1);   // keys past the chunk: any admission
        int tm0 = j0, step = 1;
        if (j0 < g.Nv) {
          const int f = int(g.divS.div(uint32_t(j0)));
          tm0 = (j0 - f * g.S) * g.F + f;
          step = g.F;
        }
        const int t0 = tm0 & ((1 << g.blk_log2) - 1);
        uint32_t masks = 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int d = (t0 + i * step) >> g.blk_log2;
          if (d < 4) masks |= 1u << (8 * d + i);
        }
        admT[b][tid] = make_uint2(uint32_t(tm0 >> g.blk_log2), masks);
      }
    } else if (tid < kTK) {
      const int key = min(key0 + tid, k_end - 1);
      blkT[b][tid] = token_major(key, g) >> g.blk_log2;
    }
  };

  // Per lane (its sample), the two classes of the lane's current spatial
  // state are live: [0] kept by the temporal mask, [1] not.  The other
  // state's two classes are parked and swapped in when the sample's spatial
  // admission flips (at most a few key blocks per sample: its spatial band is
  // one run of frames), so every step issues MFMAs for two classes only.
  f32x4 uL[2][C::DT], uP[2][C::DT];
  f32x4 zL[2], zP[2];
  float mL = -INFINITY, mP = -INFINITY;   // running max of the live / parked pair (log2 units)
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    zL[c] = f32x4{};
    zP[c] = f32x4{};
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      uL[c][dt] = f32x4{};
      uP[c][dt] = f32x4{};
    }
  }
  bool s_live = true;   // spatial state of the live classes: S-kept (classes 0, 1) or not (2, 3)
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;

  const int k_lane = ((8 * (n >> 2) + (n & 3)) * C::KROW + grp) * 16;   // tile 0, kk 0
  const int v_lane = C::KOFF * 16 + ((8 * grp + (n >> 2)) * C::VROW) * 16 + ((n & 3) * 4) * 2;
  const float c2 = a.scale_log2;

  // Admission of this lane's 8 keys of a tile (8 * grp + i) for its sample:
  // bit i = kept by the temporal row, bit 8 = the tile's key block kept by
  // the spatial row.  Computed one tile ahead, so the dependent LDS lookups
  // overlap the previous tile's MFMAs.
  auto admission = [&](int key0, int b) -> uint32_t {
    const int kblock = min(key0 >> g.blk_log2, a.nB - 1);   // one key block for all 32 keys
    uint32_t bits = (svalid && ((rowS[sidx][kblock >> 5] >> (kblock & 31)) & 1u)) ? 0x100u : 0u;
    if constexpr (ADM8) {
      const uint2 e = admT[b][grp];
      const uint32_t w = e.x >> 5;   // w + 1 <= kMaxWords: the row's padding word at most
      // bits bt0 .. bt0 + 3 of the temporal row, spread to bytes 0 .. 3
      const uint32_t win = __builtin_amdgcn_alignbit(rowT[sidx][w + 1], rowT[sidx][w], e.x & 31) & 0xfu;
      const uint32_t sel = ((win * 0x00204081u) & 0x01010101u) * 0xffu;
      const uint32_t x = e.y & sel;
      bits |= (x | (x >> 8) | (x >> 16) | (x >> 24)) & 0xffu;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int bt = blkT[b][8 * grp + i];
        bits |= ((rowT[sidx][bt >> 5] >> (bt & 31)) & 1u) << i;
      }
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
    // 32-bit LDS address of the stage: constant parts of the operand
    // addresses then fold into the instructions' offset fields
    const uint32_t lb = lds_base + b * C::STRIDE * 16;
#pragma unroll
    for (int half = 0; half < kTK / 32; ++half) {
      // ---- S^T for 32 keys: two 16x16 tiles; lane (n, grp) gets keys 8*grp + i
      f32x4 s2[2];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        s2[tile] = f32x4{};
#pragma unroll
        for (int kk = 0; kk < C::DK; ++kk) {
          const bf16x8 kop = *(const LDS_AS bf16x8*)(uintptr_t)(
              lb + k_lane + ((half * 32 + 4 * tile) * C::KROW + 4 * kk) * 16);
          s2[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qreg[kk], s2[tile], 0, 0, 0);
        }
      }
      const bool inS = (adm >> 8) & 1u;
      // swap the parked classes in for the lanes whose spatial state flipped
      if (__ballot(inS != s_live)) {
        if (inS != s_live) {   // these lanes only (exec mask): exchange the register pairs in place
#pragma unroll
          for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) swap_lane(uL[c][dt], uP[c][dt]);
            swap_lane(zL[c], zP[c]);
          }
          swap_lane(mL, mP);
          s_live = inS;
        }
      }
      // class bits of the lane's 8 keys: T-kept / T-skipped among the keys
      // that exist (keys past the chunk belong to neither class; lanes of
      // samples past n_samples compute on zero rows, and their records are
      // never read)
      uint32_t vbits = 0xffu;
      if (key0 + kTK > k_end) {
        const int nv = k_end - (key0 + half * 32 + 8 * grp);
        vbits = nv >= 8 ? 0xffu : nv <= 0 ? 0u : (1u << nv) - 1u;
      }
      const uint32_t in_bits = adm & vbits;
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = s2[i >> 2][i & 3];
      if (vbits != 0xffu) {   // keys past the chunk: weight 0, no part in the max
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (vbits >> i) & 1u ? x[i] : -INFINITY;
      }
      // this lane's block max over its keys, for both live classes
      float m_blk = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) m_blk = fmaxf(m_blk, x[i]);
      m_blk *= c2;
      // Fast path: no lane's block max exceeds its running max by more than
      // 2^24, so the stale maximum stays valid and no cross-lane exchange is
      // needed.  Otherwise combine the maxima over the 4 lanes of each sample
      // and rescale the live pair where its maximum moved.
      if (__ballot(m_blk > mL + kRescaleLog2)) {
        m_blk = fmaxf(m_blk, shfl_xor_f(m_blk, 16));
        m_blk = fmaxf(m_blk, shfl_xor_f(m_blk, 32));
        if (m_blk > mL + kRescaleLog2) {
          const float f = fast_exp2(mL - m_blk);
          zL[0] *= f;
          zL[1] *= f;
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) {
            uL[0][dt] *= f;
            uL[1][dt] *= f;
          }
          mL = m_blk;
        }
      }
      // bf16 weights in pairs, split by the T bits with 16-bit masks (keys
      // past the chunk have weight 0).  mL is finite here: the first tile of
      // a chunk holds a valid key for every sample (its first key), and the
      // exchange above gives every lane of the sample that key's max.
      uint32_t win[4], wout[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float pa = fast_exp2(__builtin_fmaf(x[2 * k], c2, -mL));
        const float pb = fast_exp2(__builtin_fmaf(x[2 * k + 1], c2, -mL));
        const uint32_t pk = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)pa, (__bf16)pb});
        const uint32_t m = pair_mask(in_bits, 2 * k);
        win[k] = pk & m;
        wout[k] = pk & ~m;
      }
      const bf16x8 pin = __builtin_bit_cast(bf16x8, make_uint4(win[0], win[1], win[2], win[3]));
      const bf16x8 pout = __builtin_bit_cast(bf16x8, make_uint4(wout[0], wout[1], wout[2], wout[3]));
      // ---- U^T += V^T P^T for the two live classes; Z from an all-ones operand
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const uint32_t p0 = lb + v_lane + (half * 32 * C::VROW) * 16 + dt * 32;
        bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(uintptr_t)p0);
        bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(uintptr_t)(p0 + 4 * C::VROW * 16));
        const bf16x8 vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        uL[0][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pin, uL[0][dt], 0, 0, 0);
        uL[1][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pout, uL[1][dt], 0, 0, 0);
      }
      zL[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pin, zL[0], 0, 0, 0);
      zL[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pout, zL[1], 0, 0, 0);
    }
  }

  // ---- write this chunk's records ---------------------------------------------
  // classes 0, 1 (S-kept) and 2, 3 (S-skipped), each as (T-kept, T-skipped)
  float* rec = a.ws + ((int64_t(bh) * a.n_chunks + chunk) * kQ + sidx) * 4 * C::REC;
  float* rS = rec + (s_live ? 0 : 2) * C::REC;   // the live pair's records
  float* rP = rec + (s_live ? 2 : 0) * C::REC;   // the parked pair's records
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (grp == 0) {
      rS[c * C::REC] = mL;
      rS[c * C::REC + 1] = zL[c][0];
      rP[c * C::REC] = mP;
      rP[c * C::REC + 1] = zP[c][0];
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      *reinterpret_cast<f32x4*>(rS + c * C::REC + 4 + dt * 16 + 4 * grp) = uL[c][dt];
      *reinterpret_cast<f32x4*>(rP + c * C::REC + 4 + dt * 16 + 4 * grp) = uP[c][dt];
    }
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
  __shared__ float Us[4][D];
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
  // U of class c = wave, channels lane, lane + 64, ...: the chunk chain of one
  // (class, channel) per thread and step, the four classes side by side
  {
    const int c = wave;
    for (int d = lane; d < D; d += 64) {
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
      Us[c][d] = u0 + u1;
    }
  }
  __syncthreads();
  double e[2] = {0.0, 0.0};
  for (int d = tid; d < D; d += 256) {
    float U[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) U[c] = Us[c][d];
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

// One wave per head: lane s loads sample s's two errors, a butterfly sums
// them (a fixed order, so repeated calls agree bit for bit).
__global__ __launch_bounds__(64) void profile_choose_kernel(const double* __restrict__ per_sample, int BH,
                                                            int n_samples, int32_t* __restrict__ choice,
                                                            float* __restrict__ err) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  double es = 0.0, et = 0.0;
  if (lane < n_samples) {
    es = per_sample[(int64_t(bh) * kQ + lane) * 2 + 0];
    et = per_sample[(int64_t(bh) * kQ + lane) * 2 + 1];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    es += __shfl_xor(es, off, 64);
    et += __shfl_xor(et, off, 64);
  }
  if (lane != 0) return;
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
  // Chunking: the partial kernel runs two workgroups per CU at D = 128 (its
  // registers) and three at D = 64 (143 registers, 52 KB of LDS each): 512 or
  // 768 at a time on the 256 CUs of an MI355X.  The chunk length (whole 32-key
  // tiles, at most kChunkKeys keys) minimises a cost in units of one tile's
  // time: rounds of workgroups x (tiles per workgroup + about 3 tiles of
  // set-up), plus the chunk records written and merged (about 0.031 tile per
  // record set of a head, 64 samples x 4 classes x (D + 4) floats, at HBM
  // speed).
  const int kSlots = D == 64 ? 768 : 512;
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
  const bool adm8 = g.S % 8 == 0 && 7 * g.F <= 3 * (1 << g.blk_log2);
  if (a.D == 128) {
    if (adm8) hipLaunchKernelGGL((profile_partial_kernel<128, true>), grid1, dim3(kThreads), 0, st, a, g);
    else hipLaunchKernelGGL((profile_partial_kernel<128, false>), grid1, dim3(kThreads), 0, st, a, g);
    hipLaunchKernelGGL(profile_merge_kernel<128>, grid2, dim3(256), 0, st, a, per_sample);
  } else {
    if (adm8) hipLaunchKernelGGL((profile_partial_kernel<64, true>), grid1, dim3(kThreads), 0, st, a, g);
    else hipLaunchKernelGGL((profile_partial_kernel<64, false>), grid1, dim3(kThreads), 0, st, a, g);
    hipLaunchKernelGGL(profile_merge_kernel<64>, grid2, dim3(256), 0, st, a, per_sample);
  }
  hipLaunchKernelGGL(profile_choose_kernel, dim3(a.BH), dim3(64), 0, st, per_sample,
                     a.BH, a.n_samples, a.choice, a.err);
}

}  // namespace svg
