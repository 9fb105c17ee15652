// Block-sparse attention forward for gfx950 ([CalibAtt] sections 2.2 / 3.3:
// whole key blocks are kept or skipped and the kernel walks a precomputed
// skip list of kept intervals; [VDA] section 5.3: tiled attention with an
// online softmax so the N x N score matrix never reaches memory).
//
// 64-token blocks: one workgroup per (batch*head, query block); BLK/32
// wavefronts, each owning 32 queries.  Per kept key block:
//   * the whole workgroup stages K (row-major) and V (transposed to V^T) in
//     LDS; the next block's global loads are issued before the current block
//     is computed, so they overlap with the MFMA work;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (Q stays in registers as the B
//     operand), giving each lane one query and 32 keys per 128-key block;
//   * fp32 online softmax in log2 units; the running max is only moved when
//     the block max exceeds it by more than 2^8, so the O rescale is rare;
//   * O^T += V^T P^T on the same MFMA, P rounded to bf16.
// Skipped blocks are never addressed.  Keys past N are masked to -inf and
// queries past N are not stored.
//
// MFMA 32x32x16 register layout used here (gfx950): operand element i of lane
// l covers row/column l%32 and contraction index 8*(l/32)+i; accumulator
// register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
// K rows are fetched in the order swz(m) (bits 2 and 3 of m exchanged), which
// makes register r of a 32-key tile hold key 16*(r/8) + 8*(l/32) + r%8: the
// eight keys a lane needs as its P^T operand for one PV step are then its
// own registers, and the matching V^T operand is one 16-byte LDS read.
#include <type_traits>

#include "attn_tiles.h"
#include "mfma_common.h"
#include "svg_internal.h"

namespace svg {
namespace {

constexpr float kRescaleLog2 = 8.0f;

__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int D, int BLK>
struct Cfg {
  static constexpr int NW = BLK / 32;       // wavefronts (32 queries each)
  static constexpr int THREADS = NW * 64;
  static constexpr int KT = BLK / 32;       // 32-key tiles per block
  static constexpr int DK = D / 16;         // QK^T contraction steps
  static constexpr int DT = D / 32;         // 32-row tiles of O^T
  static constexpr int PS = BLK / 16;       // PV contraction steps
  using KTile = LdsTile<BLK, D>;            // K  [key][d]
  using VTile = LdsTile<D, BLK>;            // V^T [d][key]
  static constexpr int K_LOADS = KTile::CHUNKS / THREADS;          // 16-B chunks per thread
  static constexpr int V_TASKS = (BLK / 8) * (D / 8);              // 8x8 transposes
  static constexpr int V_PER_T = (V_TASKS + THREADS - 1) / THREADS;
  static_assert(KTile::CHUNKS % THREADS == 0, "K staging must divide evenly");
};

// Registers holding one K/V block between its global load and its LDS store.
template <int D, int BLK>
struct Stage {
  uint4 k[Cfg<D, BLK>::K_LOADS];
  uint4 v[Cfg<D, BLK>::V_PER_T][8];
};

template <int D, int BLK>
__device__ __forceinline__ void stage_load(Stage<D, BLK>& st, const uint4* __restrict__ Kg,
                                           const uint4* __restrict__ Vg, int kb, int N, int tid) {
  using C = Cfg<D, BLK>;
  constexpr int CPR = D / 8;
  const int key0 = kb * BLK;
#pragma unroll
  for (int u = 0; u < C::K_LOADS; ++u) {
    int c = tid + u * C::THREADS;
    int row = c / CPR, col = c % CPR;
    int key = key0 + row;
    st.k[u] = key < N ? Kg[int64_t(key) * CPR + col] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int u = 0; u < C::V_PER_T; ++u) {
    int t = tid + u * C::THREADS;
    int kg = t % (BLK / 8), dc = t / (BLK / 8);
    if (t < C::V_TASKS) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int key = key0 + 8 * kg + i;
        st.v[u][i] = key < N ? Vg[int64_t(key) * CPR + dc] : make_uint4(0, 0, 0, 0);
      }
    }
  }
}

template <int D, int BLK>
__device__ __forceinline__ void stage_store(const Stage<D, BLK>& st, uint4* Ks, uint4* Vt, int tid) {
  using C = Cfg<D, BLK>;
  constexpr int CPR = D / 8;
#pragma unroll
  for (int u = 0; u < C::K_LOADS; ++u) {
    int c = tid + u * C::THREADS;
    Ks[C::KTile::slot(c / CPR, c % CPR)] = st.k[u];
  }
#pragma unroll
  for (int u = 0; u < C::V_PER_T; ++u) {
    int t = tid + u * C::THREADS;
    if (t < C::V_TASKS) {
      int kg = t % (BLK / 8), dc = t / (BLK / 8);
      uint4 cols[8];
      transpose8x8(st.v[u], cols);
#pragma unroll
      for (int j = 0; j < 8; ++j) Vt[C::VTile::slot(8 * dc + j, kg)] = cols[j];
    }
  }
}

// Advance (t, kb, kend) to the next kept key block of the skip list; returns
// false when the row is exhausted.  Intervals are clamped to [0, nKB).
__device__ __forceinline__ bool next_block(const int32_t* __restrict__ iv, int r1, int nKB, int& t,
                                           int& kb, int& kend) {
  if (++kb < kend) return true;
  for (++t; t < r1; ++t) {
    kb = max(iv[2 * t], 0);
    kend = min(iv[2 * t + 1], nKB);
    if (kb < kend) return true;
  }
  return false;
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK / 32 * 64) void attn_fwd_kernel(AttnArgs a) {
  using C = Cfg<D, BLK>;
  __shared__ uint4 Ks[C::KTile::CHUNKS];
  __shared__ uint4 Vt[C::VTile::CHUNKS];

  const int qb = blockIdx.x;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;
  const int N = a.N;

  int mask_id = a.head_mask ? a.head_mask[bh] : bh % a.n_masks;
  mask_id = min(max(mask_id, 0), a.n_masks - 1);
  const bool tm = a.head_layout && a.head_layout[bh] != 0;
  const int64_t head_off = int64_t(bh) * N * D;
  const __bf16* Q = static_cast<const __bf16*>(tm ? a.qp : a.q) + head_off;
  const uint4* Kg = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(tm ? a.kp : a.k) + head_off);
  const uint4* Vg = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(tm ? a.vp : a.v) + head_off);
  __bf16* O = static_cast<__bf16*>(tm ? a.op : a.o) + head_off;

  // Q as the B operand of S^T = K Q^T: lane holds query n, dims 16*kk + 8*h + i.
  const int q_row = qb * BLK + wave * 32 + n;
  bf16x8 qreg[C::DK];
#pragma unroll
  for (int kk = 0; kk < C::DK; ++kk) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (q_row < N) u = *reinterpret_cast<const uint4*>(Q + int64_t(q_row) * D + 16 * kk + 8 * h);
    qreg[kk] = as_bf16x8(u);
  }

  f32x16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled logits (log2 units)
  float l_part = 0.f;       // this lane's share of the softmax denominator

  const int row = mask_id * a.n_qb + qb;
  const int r0 = a.row_ptr[row], r1 = a.row_ptr[row + 1];
  int t = r0 - 1, kb = 0, kend = 0;
  bool valid = next_block(a.iv, r1, a.n_kb, t, kb, kend);

  Stage<D, BLK> st;
  if (valid) stage_load<D, BLK>(st, Kg, Vg, kb, N, tid);

  const int srow = swap_bits23(n);
  while (valid) {
    int nt = t, nkb = kb, nkend = kend;
    const bool nvalid = next_block(a.iv, r1, a.n_kb, nt, nkb, nkend);
    __syncthreads();  // every wave is done with the previous block's tiles
    stage_store<D, BLK>(st, Ks, Vt, tid);
    __syncthreads();
    if (nvalid) stage_load<D, BLK>(st, Kg, Vg, nkb, N, tid);  // in flight during compute

    // ---- S^T = K Q^T ------------------------------------------------------
    f32x16 sacc[C::KT];
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) {
      sacc[kt] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < C::DK; ++kk) {
        bf16x8 kop = as_bf16x8(Ks[C::KTile::slot(kt * 32 + srow, 2 * kk + h)]);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[kk], sacc[kt], 0, 0, 0);
      }
    }

    // ---- online softmax (log2 units) ---------------------------------------
    const int key0 = kb * BLK;
    const bool partial = key0 + BLK > N;
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = sacc[kt][r] * a.scale_log2;
        if (partial) {
          int key = key0 + kt * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
          x = key < N ? x : -INFINITY;
        }
        sacc[kt][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    if (mx > m_run + kRescaleLog2) {
      const float alpha = fast_exp2(m_run - mx);
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) oacc[dt] *= alpha;
      m_run = mx;
    }

    bf16x8 pb[C::PS];
#pragma unroll
    for (int s = 0; s < C::PS; ++s) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float p = fast_exp2(sacc[s >> 1][8 * (s & 1) + i] - m_run);
        l_part += p;
        pb[s][i] = (__bf16)p;
      }
    }

    // ---- O^T += V^T P^T ----------------------------------------------------
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int s = 0; s < C::PS; ++s) {
        bf16x8 vop = as_bf16x8(Vt[C::VTile::slot(dt * 32 + n, 2 * s + h)]);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[s], oacc[dt], 0, 0, 0);
      }
    }

    t = nt; kb = nkb; kend = nkend; valid = nvalid;
  }

  // ---- epilogue ---------------------------------------------------------------
  const float l_tot = l_part + shfl_xor_f(l_part, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_row < N) {
    __bf16* orow = O + int64_t(q_row) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = (__bf16)(oacc[dt][4 * g + j] * inv);
        *reinterpret_cast<bf16x4*>(orow + dt * 32 + 8 * g + 4 * h) = w;
      }
    }
    if (a.lse && h == 0) {
      const float ln2 = 0.69314718055994530942f;
      a.lse[int64_t(bh) * N + q_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * ln2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// 128-key blocks: 8 wavefronts, two query blocks per workgroup.
//
// Both query blocks (rows r and r+1 of the head's mask) share every staged
// key block; the workgroup walks the union of the two rows' skip lists and a
// wavefront skips the MFMA work of blocks its own row does not keep.  Waves
// 0-3 (group 0) own the 128 queries of block r, waves 4-7 (group 1) those of
// block r+1, 32 queries per wave, two waves per SIMD.
//
// Each key block j passes through two phases.  Phase 1: group 0 runs the
// MFMAs (O += P_{j-1} V_{j-1}, S_j = Q K_j^T) while group 1 runs the softmax
// of S_{j-1}; phase 2 swaps the roles.  The two waves sharing a SIMD thus
// alternate between matrix work and VALU work; one barrier per block (at its
// end) orders the buffer refills.  K_j and V^T_j land in
// double-buffered LDS through 16-byte global->LDS copies, all issued by
// group 0 in phase 2 (K of block j+1, V^T of block j), before its softmax:
// group 1 then runs MFMAs whose operand reads no longer compete with fresh
// copies for the LDS, and the waves running MFMAs never issue one.  V^T comes
// from a per-block transposed workspace, so both operands are read with
// plain 16-byte LDS fetches.  The merged key-block sequence of the two rows
// (their union, from the mask bitmap) is built in LDS once per 2048 key
// blocks, so choosing the next block is one LDS read.
//
// Workgroups are persistent, one per CU, and take their pairs of query blocks
// from per-XCD work queues (see attn_fwd_b128_kernel).  A layout-1 head whose
// token-major Q / V / O twin is not given reads Q and V from the frame-major
// tensors and writes O to them through the layout permutation.
// ---------------------------------------------------------------------------

// The merged key-block sequence of a workgroup's two mask rows (the skip list
// of their union), built in LDS one window of 64 bitmap words (2048 key
// blocks) at a time: one wave reads the two rows' bitmap words of the window
// (a single load each, no chain of dependent loads through the interval
// list) and lists the set bits of their union in order (prefix sum of the
// word popcounts).  Entry: key block in bits 0-29, bit 30 / 31 set when row 0
// / row 1 keeps it; the window ends with kSeqRefill (more words follow) or
// kSeqEnd.
constexpr int kSeqWords = 64, kSeqCap = 32 * kSeqWords + 1;
constexpr uint32_t kSeqEnd = 0x3fffffffu, kSeqRefill = 0x3ffffffeu;

struct SeqLds {
  uint32_t seq[kSeqCap];
};

// Workgroup barrier that orders LDS accesses only: global loads in flight
// (the Q rows of a new item) stay in flight across it.
__device__ __forceinline__ void barrier_lds_only() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Builds window w from the bitmap rows bm0 (row 0) and bm0 + W (row 1, read
// only when `two`); every thread of the workgroup calls it (it synchronizes).
// The two rows' bitmap words of window w for thread tid < 64 (its word of
// the window), requested before the caller's other loads so that they return
// first.
__device__ __forceinline__ uint2 seq_words(const uint32_t* __restrict__ bm0, bool two, int W, int w) {
  const int tid = threadIdx.x;
  uint2 r = make_uint2(0u, 0u);
  if (tid < 64) {
    const int word = kSeqWords * w + tid;
    r.x = word < W ? bm0[word] : 0u;
    r.y = two && word < W ? bm0[W + word] : 0u;
  }
  return r;
}

__device__ __forceinline__ void seq_scan(SeqLds& L, uint2 words, int W, int w) {
  const int tid = threadIdx.x;
  const int kb0 = 32 * kSeqWords * w;
  barrier_lds_only();   // the previous window is no longer read
  if (tid < 64) {
    const uint32_t a = words.x, b = words.y;
    const uint32_t u = a | b;
    const int c = __builtin_popcount(u);
    int incl = c;   // inclusive prefix sum over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (tid >= off) incl += y;
    }
    int o = incl - c;
    for (uint32_t x = u; x; x &= x - 1) {
      const int bit = __builtin_ctz(x);
      L.seq[o++] = uint32_t(kb0 + 32 * tid + bit) | (((a >> bit) & 1u) << 30) | (((b >> bit) & 1u) << 31);
    }
    const int total = __shfl(incl, 63, 64);
    if (tid == 0) L.seq[total] = (w + 1) * kSeqWords < W ? kSeqRefill : kSeqEnd;
  }
  barrier_lds_only();
}

__device__ __forceinline__ void seq_build(SeqLds& L, const uint32_t* __restrict__ bm0, bool two,
                                          int W, int w) {
  seq_scan(L, seq_words(bm0, two, W, w), W, w);
}

// S^T = K Q^T as mfma_qk, the K operands through a ring of three at D = 128
// (operand i = (contraction step i / KT, key tile i % KT); i + 2 read while
// product i computes).
template <int D>
__device__ __forceinline__ void mfma_qk_r(const char* kb_lds, int k_lane, const bf16x8* qreg,
                                          f32x16* sacc) {
  using C = Cfg2<D>;
  if constexpr (D != 128) {
    mfma_qk<D>(kb_lds, k_lane, qreg, sacc);
  } else {
    constexpr int NOP = C::DK * C::KT;
    auto op_at = [&](int i) {
      return *reinterpret_cast<const uint4*>(kb_lds + k_lane + C::tile_off_k(i % C::KT, 256) + (i / C::KT) * 32);
    };
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt) sacc[kt] = f32x16{};
    uint4 ring[3];
    ring[0] = op_at(0);
    ring[1] = op_at(1);
#pragma unroll
    for (int i = 0; i < NOP; ++i) {
      if (i + 2 < NOP) ring[(i + 2) % 3] = op_at(i + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int kk = i / C::KT, kt = i % C::KT;
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ring[i % 3]), qreg[kk], sacc[kt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// O^T (D x 32 queries) += V^T P^T, the V^T operands of key step s+1 in flight
// while step s computes (at D = 128 a ring of three operands instead, which
// frees 20 registers there).  With MS (matrix-core sum) every step also adds its
// 16 keys' weights into the denominator on the matrix core: one
// v_mfma_f32_16x16x32_bf16 with the weights as the B operand and the 0/1
// selector `sel` as A (lane l: rows 4i of A take the contraction groups
// l/16 = 0, 2, which hold queries 0-15, rows 4i+1 the groups 1, 3, queries
// 16-31), so accumulator register 0 of lane l sums query l%16 and register 1
// query 16 + l%16 over every key of the block.
template <int D, bool MS = false>
__device__ __forceinline__ void mfma_pv(const char* vb_lds, int v_lane, const bf16x8* pb,
                                        f32x16* oacc, const bf16x8& sel, f32x4& lacc) {
  using C = Cfg2<D>;
  constexpr int DT_OFF = 32 / C::VNI * C::VW;   // V^T rows +32
  if constexpr (D == 128) {
    // operand i = (key step i / DT, row tile i % DT) in a ring of three:
    // operand i + 2 is read while product i computes
    constexpr int NOP = C::PS * C::DT;
    auto op_at = [&](int i) {
      return *reinterpret_cast<const uint4*>(vb_lds + v_lane + (i % C::DT) * DT_OFF + (i / C::DT) * 32);
    };
    uint4 ring[3];
    ring[0] = op_at(0);
    ring[1] = op_at(1);
#pragma unroll
    for (int i = 0; i < NOP; ++i) {
      if (i + 2 < NOP) ring[(i + 2) % 3] = op_at(i + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int s = i / C::DT, dt = i % C::DT;
      oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ring[i % 3]), pb[s], oacc[dt], 0, 0, 0);
      if constexpr (MS) {
        if (dt == C::DT - 1) lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb[s], lacc, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
  uint4 cur[C::DT], nxt[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
    cur[dt] = *reinterpret_cast<const uint4*>(vb_lds + v_lane + dt * DT_OFF);
#pragma unroll
  for (int s = 0; s < C::PS; ++s) {
    if (s + 1 < C::PS) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
        nxt[dt] = *reinterpret_cast<const uint4*>(vb_lds + v_lane + dt * DT_OFF + (s + 1) * 32);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur[dt]), pb[s], oacc[dt], 0, 0, 0);
    if constexpr (MS) lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb[s], lacc, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) cur[dt] = nxt[dt];
  }
}

// Online softmax of one 128-key block: S (raw logits) -> P (bf16), updating the
// running max m (log2 units, moved only when the block max exceeds it by more
// than 2^8), the lane's share of the denominator and, on a move, O.  With MS
// the denominator is summed from the bf16 weights on the matrix core
// (mfma_pv) and only rescaled here.
template <int D, bool MS = false>
__device__ __forceinline__ void softmax_block(f32x16* sacc, bf16x8* pb, f32x16* oacc, float& m_run,
                                              float& l_part, f32x4& lacc, int key0, int N, int h,
                                              float c2) {
  using C = Cfg2<D>;
  if (key0 + C::BLK > N) {
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + kt * 32 + 16 * (r >> 3) + 8 * h + (r & 7);
        if (key >= N) sacc[kt][r] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
  mx = max_cross_half(mx) * c2;
  if (mx > m_run + kRescaleLog2) {
    const float alpha = fast_exp2(m_run - mx);
    if constexpr (MS) lacc *= alpha;
    else l_part *= alpha;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) oacc[dt] *= alpha;
    m_run = mx;
  }
  if constexpr (MS) {
#pragma unroll
    for (int s = 0; s < C::PS; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pb[s][i] = (__bf16)fast_exp2(__builtin_fmaf(sacc[s >> 1][8 * (s & 1) + i], c2, -m_run));
    return;
  }
  // The denominator sums the fp32 weights with plain adds (two chains): a
  // bf16 dot2 would have to wait for the matrix core, which the partner wave
  // on this SIMD keeps busy during the softmax.
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int s = 0; s < C::PS; ++s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = fast_exp2(__builtin_fmaf(sacc[s >> 1][8 * (s & 1) + i], c2, -m_run));
      pb[s][i] = (__bf16)p;
      if (i & 1) l1 += p;
      else l0 += p;
    }
  }
  l_part += l0 + l1;
}

// ---- FP8 (e4m3) products on v_mfma_f32_32x32x64_f8f6f4 --------------------
// Operand element i (byte) of lane l covers row / column l%32 and contraction
// index 32*(l/32) + i; the accumulator layout is that of the 32x32x16 form.
// K rows are taken in natural order, so register r of lane l of a 32-key tile
// holds key 8*(r/4) + 4*(l/32) + r%4.  Over the two tiles of a 64-key group
// the 32 weights a lane holds are then exactly its P^T operand when the V^T
// bytes of the group store keys 8a + 4h + i at position 32h + 4a + i (the
// layout svg_quantize_fp8 writes): contraction index 32h + 16t + r is tile
// t's register r.
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // format 0 = FP8 E4M3 for both operands; no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 lds_32bytes(const char* p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
  return i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
}

// S^T (128 keys x 32 queries) = K Q^T, the operands of tile kt+1 in flight
// while tile kt computes.
template <int D>
__device__ __forceinline__ void mfma_qk8(const char* kb_lds, int k_lane, const i32x8* qreg,
                                         f32x16* sacc) {
  using C = Cfg2<D, true>;
  constexpr int KT_OFF = 32 / C::KNI * C::KW;   // K rows +32
  i32x8 cur[C::DK8], nxt[C::DK8];
#pragma unroll
  for (int kk = 0; kk < C::DK8; ++kk) cur[kk] = lds_32bytes(kb_lds + k_lane + kk * 64);
#pragma unroll
  for (int kt = 0; kt < C::KT; ++kt) {
    if (kt + 1 < C::KT) {
#pragma unroll
      for (int kk = 0; kk < C::DK8; ++kk)
        nxt[kk] = lds_32bytes(kb_lds + k_lane + C::tile_off(kt + 1, KT_OFF) + kk * 64);
    }
    __builtin_amdgcn_sched_barrier(0);
    sacc[kt] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::DK8; ++kk) sacc[kt] = mfma_f8(cur[kk], qreg[kk], sacc[kt]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < C::DK8; ++kk) cur[kk] = nxt[kk];
  }
}

// O^T (D x 32 queries) += V^T P^T over the two 64-key groups of a block.
// With MS the group's weights are also summed into the denominator on the
// matrix core, as in mfma_pv: one v_mfma_f32_16x16x128_f8f6f4 per 64-key
// group with the E4M3 weights as B and the 0/1 selector `sel` as A (bytes of
// lane l cover row l%16 and contraction 32*(l/16) + i in that form).
template <int D, bool MS = false>
__device__ __forceinline__ void mfma_pv8(const char* vb_lds, int v_lane, const i32x8* pb,
                                         f32x16* oacc, const i32x8& sel, f32x4& lacc) {
  using C = Cfg2<D, true>;
  constexpr int DT_OFF = 32 / C::VNI * C::VW;   // V^T rows +32
  // Operand i = (group i / DT, row tile i % DT) in a ring of three: operand
  // i + 2 is read while product i computes (24 registers instead of the 64
  // that a whole group's operands in flight take at D = 128).
  constexpr int NOP = C::PG * C::DT;
  auto op_at = [&](int i) {
    return lds_32bytes(vb_lds + v_lane + C::tile_off(i % C::DT, DT_OFF) + (i / C::DT) * 64);
  };
  i32x8 ring[3];
  ring[0] = op_at(0);
  if constexpr (NOP > 1) ring[1] = op_at(1);
#pragma unroll
  for (int i = 0; i < NOP; ++i) {
    if (i + 2 < NOP) ring[(i + 2) % 3] = op_at(i + 2);
    __builtin_amdgcn_sched_barrier(0);
    const int g = i / C::DT, dt = i % C::DT;
    oacc[dt] = mfma_f8(ring[i % 3], pb[g], oacc[dt]);
    if constexpr (MS) {
      if (dt == C::DT - 1) lacc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, pb[g], lacc, 0, 0, 0, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Online softmax of one 128-key block for the FP8 products: as softmax_block,
// with the weights rounded to E4M3 (nearest even) for the PV product and
// packed in contraction order.  With MS the denominator is summed from the
// E4M3 weights on the matrix core (mfma_pv8) and only rescaled here.
template <int D, bool MS = false>
__device__ __forceinline__ void softmax_block8(f32x16* sacc, i32x8* pb, f32x16* oacc, float& m_run,
                                               float& l_part, f32x4& lacc, int key0, int N, int h,
                                               float c2) {
  using C = Cfg2<D, true>;
  if (key0 + C::BLK > N) {
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + kt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (key >= N) sacc[kt][r] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
  mx = max_cross_half(mx) * c2;
  if (mx > m_run + kRescaleLog2) {
    const float alpha = fast_exp2(m_run - mx);
    if constexpr (MS) lacc *= alpha;
    else l_part *= alpha;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) oacc[dt] *= alpha;
    m_run = mx;
  }
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int g = 0; g < C::PG; ++g) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kt = 2 * g + (w >> 2), r0 = 4 * (w & 3);
      float p[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        p[b] = fast_exp2(__builtin_fmaf(sacc[kt][r0 + b], c2, -m_run));
        if constexpr (!MS) {
          if (b & 1) l1 += p[b];
          else l0 += p[b];
        }
      }
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
      pb[g][w] = word;
    }
  }
  if constexpr (!MS) l_part += l0 + l1;
}

// One work item: query blocks 2*pair and 2*pair+1 of head bh, which uses
// mask mask_id and, when tm, the token-major tensors.  Every thread of the
// workgroup calls it; it synchronizes.  In its last key-block iteration
// thread 0 takes the index of its next item from the queue head `qhead` into
// `next_idx`, so that the atomic's round trip overlaps the item's last blocks.
template <int D, bool MS>
__device__ __forceinline__ void attn_pair(const AttnArgs& a, int bh, int pair, int mask_id, bool tm,
                                          int32_t* qhead, int& next_idx) {
  using C = Cfg2<D>;
  // Separate arrays per buffer, addressed with compile-time buffer indices:
  // the compiler can then tell that copies in flight target a buffer other
  // than the one being read, and adds no wait for them before LDS reads.
  __shared__ uint4 kbuf0[C::KBYTES / 16], kbuf1[C::KBYTES / 16];
  __shared__ uint4 vbuf0[C::VBYTES / 16], vbuf1[C::VBYTES / 16];
  char* const kb_lds[2] = {reinterpret_cast<char*>(kbuf0), reinterpret_cast<char*>(kbuf1)};
  char* const vb_lds[2] = {reinterpret_cast<char*>(vbuf0), reinterpret_cast<char*>(vbuf1)};

  // lane indices derived per item rather than kept live from one item to the next
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = wave >> 2;
  const int w4 = __builtin_amdgcn_readfirstlane(wave & 3);   // wave within its group
  const int n = lane & 31, h = lane >> 5;
  const int N = a.N;
  const int qb0 = 2 * pair;
  const bool has_b = qb0 + 1 < a.n_qb;

  const int64_t head_off = int64_t(bh) * N * D;
  // a layout-1 head reads its Q rows from q and writes its O rows to o through
  // the permutation when the token-major twin is not given
  const bool gq = tm && a.qp == nullptr, so = tm && a.op == nullptr;
  const __bf16* Q = static_cast<const __bf16*>(tm && !gq ? a.qp : a.q) + head_off;
  const char* Kh = reinterpret_cast<const char*>(static_cast<const __bf16*>(tm ? a.kp : a.k) + head_off);
  __bf16* O = static_cast<__bf16*>(tm && !so ? a.op : a.o) + head_off;

  const int q_row = (qb0 + grp) * C::BLK + w4 * 32 + n;
  // the item's block list needs its mask rows first: their words are
  // requested ahead of the Q rows
  const int W = (a.n_kb + 31) >> 5;
  const uint32_t* bm0 = a.bitmap + (int64_t(mask_id) * a.n_qb + qb0) * W;
  const uint2 words0 = seq_words(bm0, has_b, W, 0);
  bf16x8 qreg[C::DK];
  {
    const int q_src = gq && q_row < N ? frame_major_of(q_row, a) : q_row;
#pragma unroll
    for (int kk = 0; kk < C::DK; ++kk) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (q_row < N) u = *reinterpret_cast<const uint4*>(Q + int64_t(q_src) * D + 16 * kk + 8 * h);
      qreg[kk] = as_bf16x8(u);
    }
  }

  // Copies of a group: wave w4 takes the tile's segments w4*PW .. w4*PW+PW-1.
  // Per lane, the global source offset is lane_src + s * W for segment s.
  // (128-byte K rows: the lane filling slot l / 8 of a segment fetches that
  // slot's row, s + 16 slot(l / 8))
  const int k_row_of_lane = C::KSLOTS ? C::slot(lane / 8) : lane / (C::KW / 16);
  const uint32_t k_lane_src = k_row_of_lane * C::KNI * C::KW + (lane % (C::KW / 16)) * 16;
  const uint32_t v_lane_src = (lane / (C::VW / 16)) * C::VNI * C::VW + (lane % (C::VW / 16)) * 16;
  const uint32_t k_w4_src = w4 * C::KPW * C::KW, v_w4_src = w4 * C::VPW * C::VW;
  // K rows past N (ragged last block) fall outside the block's buffer range
  // and are never fetched: their scores are masked to -inf.  A block that
  // does not exist gets an empty range: its copies fetch nothing.
  auto k_src = [&](int kb, bool exists) {
    return LdsCopySrc(Kh + int64_t(exists ? kb : 0) * C::BLK * D * 2,
                      exists ? min(C::BLK, N - kb * C::BLK) * D * 2 : 0);
  };
  // V^T tiles come from the block-transposed workspace: [D][128] per block,
  // keys past N already zero
  const char* Vt = static_cast<const char*>(a.vt) + int64_t(bh) * a.n_kb * C::BLK * D * 2;
  auto v_src = [&](int kb, bool exists) {
    return LdsCopySrc(Vt + int64_t(exists ? kb : 0) * C::BLK * D * 2, exists ? C::BLK * D * 2 : 0);
  };
  auto copy_k = [&](const LdsCopySrc& src, const char* dst) {
    const uint32_t lds_w = lds_addr_of(dst) + w4 * C::KPW * C::SEGB;
    static_for<C::KPW>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      src.copy16(k_lane_src, sadd<u * C::KW>(k_w4_src), sadd<u * C::SEGB>(lds_w));
    });
  };
  auto copy_v = [&](const LdsCopySrc& src, const char* dst) {
    const uint32_t lds_w = lds_addr_of(dst) + w4 * C::VPW * C::SEGB;
    static_for<C::VPW>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      src.copy16(v_lane_src, sadd<u * C::VW>(v_w4_src), sadd<u * C::SEGB>(lds_w));
    });
  };

  f32x16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;
  f32x16 sacc[C::KT];
  bf16x8 pb[C::PS];
  // MS: denominator on the matrix core (mfma_pv); selector of lane l is 1 on
  // rows 4i (contraction groups 0, 2) or 4i + 1 (groups 1, 3)
  f32x4 lacc = f32x4{};
  bf16x8 sel;
  {
    const __bf16 one = ((lane >> 4) & 1) ? __bf16((lane & 3) == 1 ? 1.f : 0.f)
                                         : __bf16((lane & 3) == 0 ? 1.f : 0.f);
#pragma unroll
    for (int i = 0; i < 8; ++i) sel[i] = one;
  }

  __shared__ SeqLds sl;
  int seq_w = 0, seq_j = 1;
  seq_scan(sl, words0, W, 0);
  uint32_t seq_v = sl.seq[0];   // next entry, read one call ahead
  // Next block of the merged sequence; `mine` = my row keeps it.  All waves
  // call this at the same points, so a window refill may synchronize.
  auto pick = [&](int& kb, bool& mine) -> bool {
    uint32_t e = __builtin_amdgcn_readfirstlane(seq_v);
    if ((e & 0x3fffffffu) == kSeqRefill) {
      seq_build(sl, bm0, has_b, W, ++seq_w);
      e = __builtin_amdgcn_readfirstlane(sl.seq[0]);
      seq_j = 1;
    }
    kb = int(e & 0x3fffffffu);
    if (kb == int(kSeqEnd)) return false;
    seq_v = sl.seq[seq_j++];
    mine = grp == 0 ? (e >> 30) & 1u : (e >> 31) & 1u;
    return true;
  };

  const int srow = swap_bits23(n);
  const float c2 = a.scale_log2;
  const int k_lane = C::KSLOTS ? (srow % 16) * C::SEGB + C::slot(srow / 16) * 128 + 16 * h
                               : C::template at<C::KNI, C::KW>(srow, h);   // K row srow (+32 kt), chunk h (+2 kk)
  const int v_lane = C::template at<C::VNI, C::VW>(n, h);      // V^T row n (+32 dt), chunk h (+2 s)

  // cur: block j (K_j staged / being used); prev: block j-1 (V_{j-1})
  int kb_cur = 0, kb_prev = 0;
  bool mine_cur = false, mine_prev = false;
  bool have_cur = pick(kb_cur, mine_cur);
  bool have_prev = false;
  if (grp == 0) copy_k(k_src(kb_cur, have_cur), kb_lds[0]);
  __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0)
  barrier_lds();

  // Iteration j uses K buffer j%2 and V buffer (j-1)%2; unrolled by two so
  // that every buffer is a compile-time object.
  auto iteration = [&](auto kbuf_c) {
    constexpr int kbuf = decltype(kbuf_c)::value;
    const char* k_cur = kb_lds[kbuf];
    const char* v_prev = vb_lds[kbuf ^ 1];
    int kb_next = 0;
    bool mine_next = false;
    const bool have_next = have_cur && pick(kb_next, mine_next);
    if (have_cur && !have_next && tid == 0) next_idx = atomicAdd(qhead, 1);

    // ---- phase 1 --------------------------------------------------------------
    if (grp == 0) {
      if (have_prev && mine_prev) mfma_pv<D, MS>(v_prev, v_lane, pb, oacc, sel, lacc);
      if (have_cur && mine_cur) mfma_qk_r<D>(k_cur, k_lane, qreg, sacc);
    } else {
      if (have_prev && mine_prev)
        softmax_block<D, MS>(sacc, pb, oacc, m_run, l_part, lacc, kb_prev * C::BLK, N, h, c2);
    }
    // No barrier between the phases: the groups share no data within an
    // iteration (each holds its own S, P and O; the copies of this iteration
    // refill buffers last read in the previous one), so a group that is done
    // early starts its next phase at once.
    __builtin_amdgcn_sched_barrier(0);
    // ---- phase 2 --------------------------------------------------------------
    if (grp == 0) {
      // K of block j+1 into the K buffer freed by block j-1, V^T of block j
      // into the V buffer freed by block j-2
      copy_k(k_src(kb_next, have_next), kb_lds[kbuf ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
      copy_v(v_src(kb_cur, have_cur), vb_lds[kbuf]);
      __builtin_amdgcn_sched_barrier(0);
      if (have_cur && mine_cur)
        softmax_block<D, MS>(sacc, pb, oacc, m_run, l_part, lacc, kb_cur * C::BLK, N, h, c2);
    } else {
      if (have_prev && mine_prev) mfma_pv<D, MS>(v_prev, v_lane, pb, oacc, sel, lacc);
      if (have_cur && mine_cur) mfma_qk_r<D>(k_cur, k_lane, qreg, sacc);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this wave's copies have landed
    barrier_lds();
    __builtin_amdgcn_sched_barrier(0);

    kb_prev = kb_cur;
    mine_prev = mine_cur;
    have_prev = have_cur;
    kb_cur = kb_next;
    mine_cur = mine_next;
    have_cur = have_next;
  };
  while (have_cur || have_prev) {
    iteration(std::integral_constant<int, 0>{});
    if (!(have_cur || have_prev)) break;
    iteration(std::integral_constant<int, 1>{});
  }

  // ---- epilogue ---------------------------------------------------------------
  const float l_tot = MS ? ((lane & 16) ? lacc[1] : lacc[0]) : l_part + shfl_xor_f(l_part, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  {
    // lane indices recomputed here rather than kept live through the loop
    int tid_e = threadIdx.x;
    asm volatile("" : "+v"(tid_e));
    const int wave = tid_e >> 6, lane = tid_e & 63, n = lane & 31, h = lane >> 5;
    // O goes out through LDS (the tiles are free after the loop's last
    // barrier): each wave writes its 32 x D block row-major into its own
    // region (rows RS bytes apart), then stores whole rows, 16 bytes per
    // lane, instead of 16-byte pieces of 32 rows per store.
    constexpr int RS = D * 2 + 16, LPR = D * 2 / 16, RPI = 64 / LPR;
    static_assert(2 * 32 * RS <= C::KBYTES && C::KBYTES == C::VBYTES, "staging fits the tiles");
    char* stage = ((wave >> 1) == 0 ? kb_lds[0] : (wave >> 1) == 1 ? kb_lds[1]
                   : (wave >> 1) == 2 ? vb_lds[0] : vb_lds[1]) + (wave & 1) * 32 * RS;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = (__bf16)(oacc[dt][4 * g + j] * inv);
        *reinterpret_cast<bf16x4*>(stage + n * RS + (dt * 32 + 8 * g + 4 * h) * 2) = w;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int qrow0 = (qb0 + grp) * C::BLK + w4 * 32;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / LPR, c = lane % LPR;
      const uint4 x = *reinterpret_cast<const uint4*>(stage + r * RS + c * 16);
      if (qrow0 + r < N) {
        const int dst = so ? frame_major_of(qrow0 + r, a) : qrow0 + r;
        *reinterpret_cast<uint4*>(O + int64_t(dst) * D + c * 8) = x;
      }
    }
  }
  if (q_row < N) {
    if (a.lse && h == 0) {
      const float ln2 = 0.69314718055994530942f;
      a.lse[int64_t(bh) * N + q_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * ln2 : -INFINITY;
    }
  }
}

// One FP8 work item: attn_pair with E4M3 operands for both products
// (mfma_qk8, softmax_block8, mfma_pv8), the per-head dequantization factors
// folded into the softmax scale (q, k) and the output scale (v).  Written as
// a function of its own so that the bf16 item keeps its register allocation.
// The code paths shared with attn_pair keep bf16 / FP8 switches.
// mask mask_id and, when tm, the token-major tensors.  Every thread of the
// workgroup calls it; it synchronizes.  In its last key-block iteration
// thread 0 takes the index of its next item from the queue head `qhead` into
// `next_idx`, so that the atomic's round trip overlaps the item's last blocks.
template <int D, bool MS>
__device__ __forceinline__ void attn_pair_f8(const AttnArgs& a, int bh, int pair, int mask_id, bool tm,
                                             int32_t* qhead, int& next_idx) {
  constexpr bool F8 = true;
  using C = Cfg2<D, F8>;
  // Separate arrays per buffer, addressed with compile-time buffer indices:
  // the compiler can then tell that copies in flight target a buffer other
  // than the one being read, and adds no wait for them before LDS reads.
  __shared__ uint4 kbuf0[C::KBYTES / 16], kbuf1[C::KBYTES / 16];
  __shared__ uint4 vbuf0[C::VBYTES / 16], vbuf1[C::VBYTES / 16];
  char* const kb_lds[2] = {reinterpret_cast<char*>(kbuf0), reinterpret_cast<char*>(kbuf1)};
  char* const vb_lds[2] = {reinterpret_cast<char*>(vbuf0), reinterpret_cast<char*>(vbuf1)};

  // lane indices derived per item rather than kept live from one item to the next
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = wave >> 2;
  const int w4 = __builtin_amdgcn_readfirstlane(wave & 3);   // wave within its group
  const int n = lane & 31, h = lane >> 5;
  const int N = a.N;
  const int qb0 = 2 * pair;
  const bool has_b = qb0 + 1 < a.n_qb;

  const int64_t head_off = int64_t(bh) * N * D;
  // a layout-1 head reads its Q rows from q and writes its O rows to o through
  // the permutation when the token-major twin is not given.  FP8: q holds
  // every head frame-major (read through the permutation), k each head in its
  // own layout, o is frame-major.
  const bool gq = tm && (F8 || a.qp == nullptr), so = tm && (F8 || a.op == nullptr);
  const char* Qb = static_cast<const char*>(tm && !gq ? a.qp : a.q) + head_off * C::ES;
  const char* Kh = static_cast<const char*>(tm && !F8 ? a.kp : a.k) + head_off * C::ES;
  __bf16* O = static_cast<__bf16*>(tm && !so ? a.op : a.o) + head_off;

  const int q_row = (qb0 + grp) * C::BLK + w4 * 32 + n;
  // the item's block list needs its mask rows first: their words are
  // requested ahead of the Q rows
  const int W = (a.n_kb + 31) >> 5;
  const uint32_t* bm0 = a.bitmap + (int64_t(mask_id) * a.n_qb + qb0) * W;
  const uint2 words0 = seq_words(bm0, has_b, W, 0);
  // Q as the B operand: bf16, lane holds dims 16 kk + 8 h + i; FP8, bytes
  // 64 kk + 32 h + i
  using QReg = std::conditional_t<F8, i32x8, bf16x8>;
  constexpr int NQ = F8 ? C::DK8 : C::DK;
  QReg qreg[NQ];
  {
    const int q_src = gq && q_row < N ? frame_major_of(q_row, a) : q_row;
    const char* qrow = Qb + int64_t(q_src) * D * C::ES;
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) {
      if constexpr (F8) {
        uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
        if (q_row < N) {
          lo = *reinterpret_cast<const uint4*>(qrow + 64 * kk + 32 * h);
          hi = *reinterpret_cast<const uint4*>(qrow + 64 * kk + 32 * h + 16);
        }
        qreg[kk] = i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      } else {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (q_row < N) u = *reinterpret_cast<const uint4*>(qrow + (16 * kk + 8 * h) * 2);
        qreg[kk] = as_bf16x8(u);
      }
    }
  }

  // Copies of a group: wave w4 takes the tile's segments w4*PW .. w4*PW+PW-1.
  // Per lane, the global source offset is lane_src + s * W for segment s.
  // (128-byte rows: the lane filling slot l / 8 of a segment fetches that
  // slot's row, s + 16 slot(l / 8))
  const int row_of_lane = C::SLOTS ? C::slot(lane / 8) : lane / (C::KW / 16);
  const uint32_t k_lane_src = row_of_lane * C::KNI * C::KW + (lane % (C::KW / 16)) * 16;
  const uint32_t v_lane_src = (C::SLOTS ? row_of_lane : lane / (C::VW / 16)) * C::VNI * C::VW +
                              (lane % (C::VW / 16)) * 16;
  const uint32_t k_w4_src = w4 * C::KPW * C::KW, v_w4_src = w4 * C::VPW * C::VW;
  // K rows past N (ragged last block) fall outside the block's buffer range
  // and are never fetched: their scores are masked to -inf.  A block that
  // does not exist gets an empty range: its copies fetch nothing.
  auto k_src = [&](int kb, bool exists) {
    return LdsCopySrc(Kh + int64_t(exists ? kb : 0) * C::BLK * D * C::ES,
                      exists ? min(C::BLK, N - kb * C::BLK) * D * C::ES : 0);
  };
  // V^T tiles come from the block-transposed workspace: [D][128] per block,
  // keys past N already zero
  const char* Vt = static_cast<const char*>(a.vt) + int64_t(bh) * a.n_kb * C::BLK * D * C::ES;
  auto v_src = [&](int kb, bool exists) {
    return LdsCopySrc(Vt + int64_t(exists ? kb : 0) * C::BLK * D * C::ES,
                      exists ? C::BLK * D * C::ES : 0);
  };
  auto copy_k = [&](const LdsCopySrc& src, const char* dst) {
    const uint32_t lds_w = lds_addr_of(dst) + w4 * C::KPW * C::SEGB;
    static_for<C::KPW>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      src.copy16(k_lane_src, sadd<u * C::KW>(k_w4_src), sadd<u * C::SEGB>(lds_w));
    });
  };
  auto copy_v = [&](const LdsCopySrc& src, const char* dst) {
    const uint32_t lds_w = lds_addr_of(dst) + w4 * C::VPW * C::SEGB;
    static_for<C::VPW>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      src.copy16(v_lane_src, sadd<u * C::VW>(v_w4_src), sadd<u * C::SEGB>(lds_w));
    });
  };

  f32x16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;
  // MS: denominator on the matrix core (mfma_pv8); selector bytes of lane l
  // are E4M3 1.0 on rows 4i (contraction groups 0, 2) or 4i + 1 (groups 1, 3)
  f32x4 lacc = f32x4{};
  i32x8 sel8;
  {
    const int one = ((lane >> 4) & 1) ? ((lane & 3) == 1 ? 0x38383838 : 0) : ((lane & 3) == 0 ? 0x38383838 : 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) sel8[i] = one;
  }
  f32x16 sacc[C::KT];
  using PReg = std::conditional_t<F8, i32x8, bf16x8>;
  PReg pb[F8 ? C::PG : C::PS];

  __shared__ SeqLds sl;
  int seq_w = 0, seq_j = 1;
  seq_scan(sl, words0, W, 0);
  uint32_t seq_v = sl.seq[0];   // next entry, read one call ahead
  // Next block of the merged sequence; `mine` = my row keeps it.  All waves
  // call this at the same points, so a window refill may synchronize.
  auto pick = [&](int& kb, bool& mine) -> bool {
    uint32_t e = __builtin_amdgcn_readfirstlane(seq_v);
    if ((e & 0x3fffffffu) == kSeqRefill) {
      seq_build(sl, bm0, has_b, W, ++seq_w);
      e = __builtin_amdgcn_readfirstlane(sl.seq[0]);
      seq_j = 1;
    }
    kb = int(e & 0x3fffffffu);
    if (kb == int(kSeqEnd)) return false;
    seq_v = sl.seq[seq_j++];
    mine = grp == 0 ? (e >> 30) & 1u : (e >> 31) & 1u;
    return true;
  };

  // bf16: K row srow (+32 kt), chunk h (+2 kk); V^T row n (+32 dt), chunk h
  // (+2 s).  FP8: K row n, chunk 2h (+4 kk); V^T row n, chunk 2h (+4 g).
  const int srow = F8 ? n : swap_bits23(n);
  const int k_lane = C::SLOTS ? (srow % 16) * C::SEGB + C::slot(srow / 16) * 128 + 32 * h
                              : C::template at<C::KNI, C::KW>(srow, F8 ? 2 * h : h);
  const int v_lane = C::SLOTS ? (n % 16) * C::SEGB + C::slot(n / 16) * 128 + 32 * h
                              : C::template at<C::VNI, C::VW>(n, F8 ? 2 * h : h);
  float c2 = a.scale_log2;
  float o_scale = 1.f;   // FP8: V's dequantization factor
  if constexpr (F8) {
    c2 *= a.f8_scales[bh] * a.f8_scales[a.BH + bh];
    o_scale = a.f8_scales[2 * a.BH + bh];
  }

  // cur: block j (K_j staged / being used); prev: block j-1 (V_{j-1})
  int kb_cur = 0, kb_prev = 0;
  bool mine_cur = false, mine_prev = false;
  bool have_cur = pick(kb_cur, mine_cur);
  bool have_prev = false;
  if (grp == 0) copy_k(k_src(kb_cur, have_cur), kb_lds[0]);
  __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0)
  barrier_lds();

  auto qk = [&](const char* k_lds) {
    if constexpr (F8) mfma_qk8<D>(k_lds, k_lane, qreg, sacc);
    else mfma_qk<D>(k_lds, k_lane, qreg, sacc);
  };
  auto pv = [&](const char* v_lds) {
    if constexpr (F8) mfma_pv8<D, MS>(v_lds, v_lane, pb, oacc, sel8, lacc);
    else mfma_pv<D>(v_lds, v_lane, pb, oacc, pb[0], lacc);
  };
  auto smax = [&](int key0) {
    if constexpr (F8) softmax_block8<D, MS>(sacc, pb, oacc, m_run, l_part, lacc, key0, N, h, c2);
    else softmax_block<D>(sacc, pb, oacc, m_run, l_part, lacc, key0, N, h, c2);
  };

  // Iteration j uses K buffer j%2 and V buffer (j-1)%2; unrolled by two so
  // that every buffer is a compile-time object.
  auto iteration = [&](auto kbuf_c) {
    constexpr int kbuf = decltype(kbuf_c)::value;
    const char* k_cur = kb_lds[kbuf];
    const char* v_prev = vb_lds[kbuf ^ 1];
    int kb_next = 0;
    bool mine_next = false;
    const bool have_next = have_cur && pick(kb_next, mine_next);
    if (have_cur && !have_next && tid == 0) next_idx = atomicAdd(qhead, 1);

    // ---- phase 1 --------------------------------------------------------------
    if (grp == 0) {
      if (have_prev && mine_prev) pv(v_prev);
      if (have_cur && mine_cur) qk(k_cur);
    } else {
      if (have_prev && mine_prev) smax(kb_prev * C::BLK);
    }
    // The groups share no data within an iteration (each holds its own S, P
    // and O; the copies of this iteration refill buffers last read in the
    // previous one).  With FP8 products the matrix-core phase is short, and
    // a group that started its softmax early would run it beside the other
    // group's (both then slower on the shared VALU): the groups meet between
    // the phases (1.4-2.2 % faster at Wan, 3 % at CogVideoX with the
    // denominator on the matrix core).
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // ---- phase 2 --------------------------------------------------------------
    if (grp == 0) {
      // K of block j+1 into the K buffer freed by block j-1, V^T of block j
      // into the V buffer freed by block j-2
      copy_k(k_src(kb_next, have_next), kb_lds[kbuf ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
      copy_v(v_src(kb_cur, have_cur), vb_lds[kbuf]);
      __builtin_amdgcn_sched_barrier(0);
      if (have_cur && mine_cur) smax(kb_cur * C::BLK);
    } else {
      if (have_prev && mine_prev) pv(v_prev);
      if (have_cur && mine_cur) qk(k_cur);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this wave's copies have landed
    barrier_lds();
    __builtin_amdgcn_sched_barrier(0);

    kb_prev = kb_cur;
    mine_prev = mine_cur;
    have_prev = have_cur;
    kb_cur = kb_next;
    mine_cur = mine_next;
    have_cur = have_next;
  };
  while (have_cur || have_prev) {
    iteration(std::integral_constant<int, 0>{});
    if (!(have_cur || have_prev)) break;
    iteration(std::integral_constant<int, 1>{});
  }

  // ---- epilogue ---------------------------------------------------------------
  const float l_tot = MS ? ((lane & 16) ? lacc[1] : lacc[0]) : l_part + shfl_xor_f(l_part, 32);
  const float inv = l_tot > 0.f ? o_scale / l_tot : 0.f;
  {
    // lane indices recomputed here rather than kept live through the loop
    int tid_e = threadIdx.x;
    asm volatile("" : "+v"(tid_e));
    const int wave = tid_e >> 6, lane = tid_e & 63, n = lane & 31, h = lane >> 5;
    // O goes out through LDS (the tiles are free after the loop's last
    // barrier): each wave writes its 32 x D block row-major into its own
    // region (rows RS bytes apart), then stores whole rows, 16 bytes per
    // lane, instead of 16-byte pieces of 32 rows per store.
    // (FP8 tiles are half as large: rows are not padded there but their
    // 16-byte chunks are rotated by the row index instead)
    constexpr int RS = F8 ? D * 2 : D * 2 + 16, LPR = D * 2 / 16, RPI = 64 / LPR;
    static_assert(2 * 32 * RS <= C::KBYTES && C::KBYTES == C::VBYTES, "staging fits the tiles");
    auto st_off = [&](int row, int byte) -> int {
      if constexpr (F8) return row * RS + (((byte >> 4) ^ (row % LPR)) << 4) + (byte & 15);
      else return row * RS + byte;
    };
    char* stage = ((wave >> 1) == 0 ? kb_lds[0] : (wave >> 1) == 1 ? kb_lds[1]
                   : (wave >> 1) == 2 ? vb_lds[0] : vb_lds[1]) + (wave & 1) * 32 * RS;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = (__bf16)(oacc[dt][4 * g + j] * inv);
        *reinterpret_cast<bf16x4*>(stage + st_off(n, (dt * 32 + 8 * g + 4 * h) * 2)) = w;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int qrow0 = (qb0 + grp) * C::BLK + w4 * 32;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / LPR, c = lane % LPR;
      const uint4 x = *reinterpret_cast<const uint4*>(stage + st_off(r, c * 16));
      if (qrow0 + r < N) {
        const int dst = so ? frame_major_of(qrow0 + r, a) : qrow0 + r;
        *reinterpret_cast<uint4*>(O + int64_t(dst) * D + c * 8) = x;
      }
    }
  }
  if (q_row < N) {
    if (a.lse && h == 0) {
      const float ln2 = 0.69314718055994530942f;
      a.lse[int64_t(bh) * N + q_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * ln2 : -INFINITY;
    }
  }
}

// Persistent workgroups, one per CU, take work items from eight queues, one
// per XCD: workgroup i runs on XCD i % 8 and takes the items of that XCD's
// work list (plan_kernel, order_kernel: the x-th of eight contiguous ranges
// of every head's query-block pairs, ranges of about equal work, heavy pairs
// first, otherwise head after head and pair after pair, so the XCD's CUs
// read the same key blocks through one L2) in list order through an atomic
// queue head.  A workgroup whose list is done takes items from the other
// XCDs' lists.  Every item is computed the same way wherever it runs, so the
// result does not depend on the schedule.
template <int D, bool F8, bool MS = false>
__device__ __forceinline__ void persistent_items(const AttnArgs& a, int cap) {
  const int xcd = blockIdx.x % 8;
  const int32_t* counts = a.plan + a.BH * 9;
  int32_t* heads = a.plan + a.BH * 9 + 8;
  const int2* lists = reinterpret_cast<const int2*>(a.plan + attn_plan_list_offset(a.BH));
  __shared__ int2 grabbed;
  int next_idx = -1;   // thread 0: index in this XCD's queue taken ahead, -1 = none
  auto take = [&]() -> int2 {
    const int i = next_idx >= 0 ? next_idx : atomicAdd(heads + xcd, 1);
    next_idx = -1;
    if (i < counts[xcd]) return lists[int64_t(xcd) * cap + i];
    for (int t = 1; t < 8; ++t) {
      const int x = (xcd + t) & 7;
      const int n = counts[x];
      if (__hip_atomic_load(heads + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n) continue;
      const int j = atomicAdd(heads + x, 1);
      if (j < n) return lists[int64_t(x) * cap + j];
    }
    return make_int2(0, -1);   // every queue is empty
  };
  for (;;) {
    if (threadIdx.x == 0) grabbed = take();
    __syncthreads();
    // item: x = head | token-major flag << 31, y = pair | mask << 16 (order_kernel)
    const int ix = __builtin_amdgcn_readfirstlane(grabbed.x);
    const int iy = __builtin_amdgcn_readfirstlane(grabbed.y);
    if (iy < 0) break;
    if constexpr (F8)
      attn_pair_f8<D, MS>(a, ix & 0x7fffffff, iy & 0xffff, int(uint32_t(iy) >> 16), ix < 0, heads + xcd, next_idx);
    else
      attn_pair<D, MS>(a, ix & 0x7fffffff, iy & 0xffff, int(uint32_t(iy) >> 16), ix < 0, heads + xcd, next_idx);
    // attn_pair ends with no barrier: the next take must not overwrite
    // `grabbed` before every wave has read it, nor the next item's copies
    // land in tiles a slow wave still reads for its output
    __syncthreads();
  }
}

// MS: the denominator summed on the matrix core from the bf16 weights (taken
// when no LSE is asked for: the LSE needs the fp32 sum).
template <int D, bool MS>
__global__ __launch_bounds__(512) void attn_fwd_b128_kernel(AttnArgs a, int cap) {
  persistent_items<D, false, MS>(a, cap);
}

// The same schedule with FP8 (E4M3) operands for both products.  MS as in
// attn_fwd_b128_kernel.
template <int D, bool MS>
__global__ __launch_bounds__(512) void attn_fwd_fp8_kernel(AttnArgs a, int cap) {
  persistent_items<D, true, MS>(a, cap);
}

// Work of query-block pair p of a mask: key blocks in the union of its two
// rows (bitmap popcount) plus two blocks of set-up.
__device__ __forceinline__ int pair_work(const uint32_t* __restrict__ bm, int p, int n_qb, int W) {
  const uint32_t* r0 = bm + int64_t(2 * p) * W;
  const bool two = 2 * p + 1 < n_qb;
  int c = 2;
  for (int w = 0; w < W; ++w) c += __builtin_popcount(r0[w] | (two ? r0[W + w] : 0u));
  return c;
}

// Inclusive scan of one value per thread over a 256-thread workgroup; every
// thread also gets the workgroup total.
__device__ __forceinline__ long long block_scan256(long long v, long long* tmp, long long& total) {
  const int tid = threadIdx.x;
  tmp[tid] = v;
  __syncthreads();
#pragma unroll
  for (int off = 1; off < 256; off <<= 1) {
    const long long add = tid >= off ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  const long long r = tmp[tid];
  total = tmp[255];
  __syncthreads();
  return r;
}

// Work-balanced split of each head's query-block pairs over the 8 XCDs: split
// x (1..7) is the first pair whose preceding work reaches x/8 of the head's
// total, then clamped so that no range exceeds max_len and the ranges always
// cover all pairs.  One workgroup per head; pairs in chunks of 256, each
// thread checks whether a split point falls on its pair.
__global__ __launch_bounds__(256) void plan_kernel(const uint32_t* __restrict__ bitmap,
                                                   const int32_t* __restrict__ head_mask, int n_masks,
                                                   int n_qb, int W, int pairs, int max_len,
                                                   int32_t* __restrict__ plan) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  int mask_id = head_mask ? head_mask[bh] : bh % n_masks;
  mask_id = min(max(mask_id, 0), n_masks - 1);
  const uint32_t* bm = bitmap + int64_t(mask_id) * n_qb * W;
  __shared__ long long tmp[256];
  __shared__ int split[9];
  if (tid < 9) split[tid] = tid == 0 ? 0 : pairs;
  // pass 1: work of every pair (kept for order_kernel) and the total
  int32_t* work = plan + attn_plan_work_offset(gridDim.x, pairs) + int64_t(bh) * pairs;
  long long mine = 0;
  for (int p = tid; p < pairs; p += 256) {
    const int w = pair_work(bm, p, n_qb, W);
    work[p] = w;
    mine += w;
  }
  long long T = 0;
  block_scan256(mine, tmp, T);   // its barriers also publish work[]
  // pass 2: split points (excl = work of the pairs before p)
  long long carry = 0;
  for (int base = 0; base < pairs; base += 256) {
    const int p = base + tid;
    const long long w = p < pairs ? work[p] : 0;
    long long chunk = 0;
    const long long excl = carry + block_scan256(w, tmp, chunk) - w;
    if (p < pairs) {
      // p is split x iff excl(p) >= x T / 8 > excl(p - 1) = excl(p) - work(p - 1)
      const long long wprev = p == 0 ? 0 : work[p - 1];
      for (int x = 1; x < 8; ++x)
        if (excl * 8 >= T * x && (p == 0 || (excl - wprev) * 8 < T * x)) split[x] = p;
    }
    carry += chunk;
    __syncthreads();
  }
  __syncthreads();
  if (tid == 0) {
    for (int x = 1; x < 8; ++x) {
      const int lo = max(split[x - 1], pairs - (8 - x) * max_len);
      const int hi = min(split[x - 1] + max_len, pairs);
      split[x] = min(max(split[x], lo), hi);
    }
    split[8] = pairs;
    for (int x = 0; x < 9; ++x) plan[bh * 9 + x] = split[x];
  }
}

// Work list of each XCD: the ranges plan_kernel gave it, head after head,
// stably partitioned so that heavy pairs (more than half of all key blocks in
// the union of their two rows, e.g. the dense rows of text queries) come
// first and start early.  One workgroup per XCD.  Each head's range and list
// entry fields are read once into LDS (up to kOrderLdsHeads heads; beyond
// that they are read from global memory at each use).
constexpr int kOrderLdsHeads = 2048;
__global__ __launch_bounds__(256) void order_kernel(const int32_t* __restrict__ head_mask,
                                                    const int32_t* __restrict__ head_layout, int n_masks,
                                                    int n_kb, int BH, int pairs, int cap,
                                                    int32_t* __restrict__ plan) {
  const int x = blockIdx.x, tid = threadIdx.x;
  const int32_t* split = plan;
  int32_t* counts = plan + BH * 9;
  int2* list = reinterpret_cast<int2*>(plan + attn_plan_list_offset(BH)) + int64_t(x) * cap;
  __shared__ long long tmp[256];
  __shared__ int4 head_s[kOrderLdsHeads];
  const bool in_lds = BH <= kOrderLdsHeads;
  // head h: first pair and length of its range on this XCD, and the list
  // entry's fields: x = h | token-major << 31, y = mask << 16 (pair added)
  auto head_info = [&](int h) -> int4 {
    int m = head_mask ? head_mask[h] : h % n_masks;
    m = min(max(m, 0), n_masks - 1);
    const bool tm = head_layout && head_layout[h] != 0;
    return make_int4(split[h * 9 + x], split[h * 9 + x + 1] - split[h * 9 + x],
                     h | (tm ? int(0x80000000u) : 0), m << 16);
  };
  auto info = [&](int h) -> int4 { return in_lds ? head_s[h] : head_info(h); };
  // items of this XCD, head-major: item g of head h is pair start(h) + g - base(h)
  long long len_sum = 0;
  for (int h = tid; h < BH; h += 256) {
    const int4 hi = head_info(h);
    if (in_lds) head_s[h] = hi;
    len_sum += hi.y;
  }
  long long total_ll = 0;
  block_scan256(len_sum, tmp, total_ll);   // its barriers also publish head_s
  const int total = int(total_ll);
  const int chunk = (total + 255) / 256;
  const int g0 = min(tid * chunk, total), g1 = min(g0 + chunk, total);
  auto walk = [&](auto f) {
    int h = 0, base = 0;
    int4 hi = BH > 0 ? info(0) : make_int4(0, 0, 0, 0);
    while (h < BH && base + hi.y <= g0) {
      base += hi.y;
      if (++h < BH) hi = info(h);
    }
    for (int g = g0; g < g1; ++g) {
      while (g - base >= hi.y) {
        base += hi.y;
        hi = info(++h);
      }
      f(hi, h, hi.x + (g - base));
    }
  };
  const int32_t* work = plan + attn_plan_work_offset(BH, pairs);
  auto heavy = [&](int h, int p) -> bool { return 2 * (work[int64_t(h) * pairs + p] - 2) > n_kb; };
  uint64_t flags = 0;   // heavy flags of this thread's items (chunk <= 64), else recomputed
  int mine = 0, i = 0;
  walk([&](const int4&, int h, int p) {
    const bool hv = heavy(h, p);
    if (i < 64 && hv) flags |= uint64_t(1) << i;
    mine += hv;
    ++i;
  });
  long long heavy_total = 0;
  const int hp0 = int(block_scan256(mine, tmp, heavy_total)) - mine;
  int hp = hp0;                                   // next heavy slot
  int np = int(heavy_total) + (g0 - hp0);         // next normal slot
  i = 0;
  // item (h, p) as x = h | token-major << 31, y = p | mask << 16, so that the
  // attention kernel needs no further load to address its operands
  walk([&](const int4& hi, int h, int p) {
    const bool hv = i < 64 ? ((flags >> i) & 1) != 0 : heavy(h, p);
    const int2 e = make_int2(hi.z, p | hi.w);
    if (hv) list[hp++] = e;
    else list[np++] = e;
    ++i;
  });
  if (tid == 0) {
    counts[x] = total;
    counts[8 + x] = 0;   // queue head of the attention kernel
  }
}

// The layout pass of a 128-token-block attention call, one workgroup per
// (key block, head): V of the head, transposed per 128-key block
// ([bh][kb][d][128], keys past N zero), so the attention kernel can stage
// V^T tiles with plain 16-byte copies and read the PV operand with
// ds_read_b128; for a head with layout 1 the keys of a block are its
// token-major keys (read from the token-major twin vp when given, else from v
// through the permutation), and when kp is given the block's token-major K
// rows are written there too ([SVG], layout transformation: the temporal
// heads' keys made contiguous), so K and V cross HBM in one pass.  Each
// thread transposes 8 keys x 8 dims in registers; the block's V^T goes
// through LDS and leaves as whole 256-byte rows.
template <int D>
__global__ __launch_bounds__(256) void vt_prep_kernel(const __bf16* __restrict__ v,
                                                      const __bf16* __restrict__ vp,
                                                      const int32_t* __restrict__ head_layout,
                                                      __bf16* __restrict__ vt, const __bf16* __restrict__ k,
                                                      __bf16* __restrict__ kp, int N, int nKB,
                                                      AttnArgs a) {
  constexpr int BLK = 128, CPR = D / 8, TASKS = (BLK / 8) * CPR;
  constexpr int KC = BLK / 8;          // 16-byte chunks per V^T row (8 keys each)
  // V^T block staged in LDS: row d holds 16 chunks of 8 keys; chunk c of row
  // d sits at position c ^ ((d / 8) % 16), so that the 16 lanes writing the
  // rows 8 dc + j of one chunk column hit 16 different bank groups
  __shared__ uint4 tile[D * KC];
  const int kb = blockIdx.x, bh = blockIdx.y;
  const int t = threadIdx.x;
  const bool tm = head_layout && head_layout[bh] != 0;
  if (tm && kp) {
    // token-major K rows of this block: row r <- frame-major row fm(r)
    const uint4* ksrc = reinterpret_cast<const uint4*>(k + int64_t(bh) * N * D);
    uint4* kdst = reinterpret_cast<uint4*>(kp + int64_t(bh) * N * D);
    constexpr int PER = BLK * CPR / 256;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int c = t + u * 256;
      const int r = kb * BLK + c / CPR;
      if (r < N) kdst[int64_t(r) * CPR + c % CPR] = ksrc[int64_t(frame_major_of(r, a)) * CPR + c % CPR];
    }
  }
  if (t < TASKS) {
    // thread (dc, kg): keys 8 kg .. 8 kg + 7, dims 8 dc .. 8 dc + 7; a
    // wavefront reads whole 2D-byte rows
    const bool gather = tm && vp == nullptr;   // token-major keys read from v through the permutation
    const uint4* src = reinterpret_cast<const uint4*>((tm && !gather ? vp : v) + int64_t(bh) * N * D);
    const int dc = t % CPR, kg = t / CPR;
    uint4 rows[8], cols[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = kb * BLK + 8 * kg + i;
      const int row = gather && key < N ? frame_major_of(key, a) : key;
      rows[i] = key < N ? src[int64_t(row) * CPR + dc] : make_uint4(0, 0, 0, 0);
    }
    transpose8x8(rows, cols);
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[(8 * dc + j) * KC + (kg ^ (dc % KC))] = cols[j];
  }
  __syncthreads();
  // the V^T block leaves as whole 256-byte rows: lane (c, r) stores chunk c
  // of row r
  uint4* dst = reinterpret_cast<uint4*>(vt + (int64_t(bh) * nKB + kb) * BLK * D);
#pragma unroll
  for (int u = 0; u < D * KC / 256; ++u) {
    const int e = t + u * 256;
    const int r = e / KC, c = e % KC;
    dst[e] = tile[r * KC + (c ^ ((r / 8) % KC))];
  }
}

template <int D, int BLK>
void launch_t(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.n_qb, a.BH);
  hipLaunchKernelGGL((attn_fwd_kernel<D, BLK>), grid, dim3(Cfg<D, BLK>::THREADS), 0, st, a);
}

// One workgroup per CU of the current device (the 128-block kernel's LDS
// allows one per CU), a multiple of 8 so that every XCD gets as many, and no
// more than there are items.
int persistent_grid(int64_t items) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
    cus = 256;
  const int64_t g = std::min<int64_t>(cus / 8 * 8, (items + 7) / 8 * 8);
  return int(std::max<int64_t>(8, g));
}

template <int D>
void launch_vt_prep(const AttnArgs& a, const void* k, void* kp, hipStream_t st) {
  hipLaunchKernelGGL((vt_prep_kernel<D>), dim3(a.n_kb, a.BH), dim3(256), 0, st,
                     static_cast<const __bf16*>(a.v), static_cast<const __bf16*>(a.vp),
                     a.head_layout, static_cast<__bf16*>(a.vt), static_cast<const __bf16*>(k),
                     static_cast<__bf16*>(kp), a.N, a.n_kb, a);
}

template <int D, bool F8>
void launch_b128(const AttnArgs& a, hipStream_t st) {
  if (!F8 && !a.vt_given) launch_vt_prep<D>(a, nullptr, nullptr, st);
  const int pairs = (a.n_qb + 1) / 2;
  const int per_xcd = plan_range_cap(pairs);
  const int W = (a.n_kb + 31) / 32;
  hipLaunchKernelGGL(plan_kernel, dim3(a.BH), dim3(256), 0, st, a.bitmap, a.head_mask, a.n_masks,
                     a.n_qb, W, pairs, per_xcd, a.plan);
  hipLaunchKernelGGL(order_kernel, dim3(8), dim3(256), 0, st, a.head_mask, a.head_layout, a.n_masks,
                     a.n_kb, a.BH, pairs, a.BH * per_xcd, a.plan);
  const dim3 grid(persistent_grid(int64_t(a.BH) * pairs));
  // The denominators move to the matrix core unless the LSE is asked for:
  // the softmax's VALU work bounds the FP8 kernels and the bf16 one at
  // D = 64; the bf16 one at D = 128, held by the board's power limit, gains
  // less (0.6 %).
  if constexpr (F8) {
    if (a.lse == nullptr)
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, true>), grid, dim3(512), 0, st, a, a.BH * per_xcd);
    else
      hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, false>), grid, dim3(512), 0, st, a, a.BH * per_xcd);
  } else {
    if (a.lse == nullptr)
      hipLaunchKernelGGL((attn_fwd_b128_kernel<D, true>), grid, dim3(512), 0, st, a, a.BH * per_xcd);
    else
      hipLaunchKernelGGL((attn_fwd_b128_kernel<D, false>), grid, dim3(512), 0, st, a, a.BH * per_xcd);
  }
}

}  // namespace

size_t attn_vt_bytes(int BH, int N, int D, int block) {
  return block == 128 ? size_t(BH) * ceil_div(N, 128) * 128 * D * 2 : 0;
}

size_t attn_workspace_bytes(int BH, int N, int D, int block, bool vt_given) {
  if (block != 128) return 0;
  const int pairs = (ceil_div(N, 128) + 1) / 2;
  return (vt_given ? 0 : attn_vt_bytes(BH, N, D, block)) + attn_plan_bytes(BH, pairs);
}

void launch_prepare_kv(const AttnArgs& a, const void* k, void* kp, hipStream_t st) {
  if (a.D == 128) launch_vt_prep<128>(a, k, kp, st);
  else launch_vt_prep<64>(a, k, kp, st);
}

void launch_attn(const AttnArgs& a, hipStream_t st) {
  if (a.block == 128) {
    if (a.D == 128) launch_b128<128, false>(a, st);
    else launch_b128<64, false>(a, st);
  } else {
    if (a.D == 128) launch_t<128, 64>(a, st);
    else launch_t<64, 64>(a, st);
  }
}

void launch_attn_fp8(const AttnArgs& a, hipStream_t st) {
  if (a.D == 128) launch_b128<128, true>(a, st);
  else launch_b128<64, true>(a, st);
}

}  // namespace svg
