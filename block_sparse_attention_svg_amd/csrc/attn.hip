// Block-sparse attention forward for gfx950 ([CalibAtt] sections 2.2 / 3.3:
// whole key blocks are kept or skipped and the kernel walks a precomputed
// skip list of kept intervals; [VDA] section 5.3: tiled attention with an
// online softmax so the N x N score matrix never reaches memory).
//
// One workgroup per (batch*head, query block); BLK/32 wavefronts, each owning
// 32 queries.  Per kept key block:
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
// wavefront skips the MFMA work of blocks its own row does not keep.  K and V
// land in double-buffered LDS through 16-byte global->LDS loads
// (global_load_lds_dwordx4): block j+1 streams in while block j is computed,
// and no registers hold staged data, so two wavefronts fit per SIMD and one's
// softmax overlaps the other's MFMA.  V stays row-major in LDS; the V^T
// operand of the PV product comes from ds_read_b64_tr_b16, which hands each
// lane one column of a 4-row x 16-column tile.
//
// LDS rows are padded so that every operand fetch is bank-conflict free and
// every per-lane LDS address is a fixed base plus a compile-time offset:
// K rows take D+8 elements (16 rows of one 16-byte fetch land on distinct
// banks), V rows D+32 (4 rows x 64 bytes of a transposing fetch do).  The
// global->LDS loads write 1 KB per wavefront instruction; lanes that fall on
// padding stay idle.
// ---------------------------------------------------------------------------
#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

template <int D>
struct Cfg2 {
  static constexpr int BLK = 128;
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int CPR = D / 8;                  // 16-byte data chunks per row
  static constexpr int KROW = CPR + 1;               // chunks per padded K row
  static constexpr int VROW = CPR + 4;               // chunks per padded V row
  static constexpr int KCH = BLK * KROW;             // chunks of the K tile
  static constexpr int VCH = BLK * VROW;             // chunks of the V tile
  static constexpr int BUF_CH = KCH + VCH;           // chunks per buffer
  static constexpr int SEGS = (BUF_CH + 63) / 64;    // 1-KB load segments per buffer
  static constexpr int SEG_PER_WAVE = (SEGS + WAVES - 1) / WAVES;
  static constexpr int KT = BLK / 32, DK = D / 16, DT = D / 32, PS = BLK / 16;
};

struct RowCursor {
  int t, r1, kb, kend;
  bool valid;
};

__device__ __forceinline__ void cursor_start(RowCursor& c, const int32_t* __restrict__ row_ptr,
                                             const int32_t* __restrict__ iv, int row, bool exists,
                                             int nKB) {
  c.kb = 0;
  c.kend = 0;
  c.valid = false;
  if (!exists) return;
  c.t = row_ptr[row] - 1;
  c.r1 = row_ptr[row + 1];
  c.valid = next_block(iv, c.r1, nKB, c.t, c.kb, c.kend);
}

// Byte offset, inside one key block of K (or V) in global memory, of the chunk
// this lane fills in load segment u; -1 for padding / past the buffer.  Bit 30
// marks a V chunk.
template <int D>
__device__ __forceinline__ int seg_source(int u, int wave, int lane) {
  using C = Cfg2<D>;
  const int seg = u * C::WAVES + wave;
  const int p = seg * 64 + lane;
  if (seg >= C::SEGS || p >= C::BUF_CH) return -1;
  if (p < C::KCH) {
    const int r = p / C::KROW, c = p % C::KROW;
    return c < C::CPR ? (r * D + c * 8) * 2 : -1;
  }
  const int q = p - C::KCH;
  const int r = q / C::VROW, c = q % C::VROW;
  return c < C::CPR ? ((r * D + c * 8) * 2) | (1 << 30) : -1;
}

template <int D>
__global__ __launch_bounds__(512) void attn_fwd_b128_kernel(AttnArgs a, int pairs, int pairs_per_xcd) {
  using C = Cfg2<D>;
  __shared__ uint4 lds[2][C::SEGS * 64];   // [buffer][K tile | V tile], padded rows

  // XCD-aware order: workgroup i runs on XCD i % 8; XCD x takes, head after
  // head, the x-th contiguous eighth of that head's query-block pairs.
  const int xcd = blockIdx.x % 8;
  const int local = blockIdx.x / 8;
  const int bh = local / pairs_per_xcd;
  const int pair = xcd * pairs_per_xcd + local % pairs_per_xcd;
  if (bh >= a.BH || pair >= pairs) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, h = lane >> 5;
  const int N = a.N;
  const int qb0 = 2 * pair;
  const int my_qb = qb0 + (wave >> 2);
  const bool has_b = qb0 + 1 < a.n_qb;

  int mask_id = a.head_mask ? a.head_mask[bh] : bh % a.n_masks;
  mask_id = min(max(mask_id, 0), a.n_masks - 1);
  const bool tm = a.head_layout && a.head_layout[bh] != 0;
  const int64_t head_off = int64_t(bh) * N * D;
  const __bf16* Q = static_cast<const __bf16*>(tm ? a.qp : a.q) + head_off;
  const char* Kh = reinterpret_cast<const char*>(static_cast<const __bf16*>(tm ? a.kp : a.k) + head_off);
  const char* Vh = reinterpret_cast<const char*>(static_cast<const __bf16*>(tm ? a.vp : a.v) + head_off);
  __bf16* O = static_cast<__bf16*>(tm ? a.op : a.o) + head_off;

  const int q_row = my_qb * C::BLK + (wave & 3) * 32 + n;
  bf16x8 qreg[C::DK];
#pragma unroll
  for (int kk = 0; kk < C::DK; ++kk) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (q_row < N) u = *reinterpret_cast<const uint4*>(Q + int64_t(q_row) * D + 16 * kk + 8 * h);
    qreg[kk] = as_bf16x8(u);
  }

  int src[C::SEG_PER_WAVE];
#pragma unroll
  for (int u = 0; u < C::SEG_PER_WAVE; ++u) src[u] = seg_source<D>(u, wave, lane);

  // Stage key block kb into buffer b.  Keys past N (ragged last block) read
  // row N-1 instead: finite values whose scores are masked to -inf.
  auto stage = [&](int kb, int b) {
    const int64_t blk_off = int64_t(kb) * C::BLK * D * 2;
    const bool ragged = (kb + 1) * C::BLK > N;
#pragma unroll
    for (int u = 0; u < C::SEG_PER_WAVE; ++u) {
      const int seg = u * C::WAVES + wave;
      if (seg < C::SEGS && src[u] >= 0) {
        int off = src[u] & ~(1 << 30);
        const char* base = (src[u] & (1 << 30)) ? Vh : Kh;
        if (ragged) {
          const int r = off / (D * 2);
          const int last = N - 1 - kb * C::BLK;
          if (r > last) off += (last - r) * D * 2;
        }
        __builtin_amdgcn_global_load_lds((GLB_AS void*)(base + blk_off + off),
                                         (LDS_AS void*)(&lds[b][seg * 64]), 16, 0, 0);
      }
    }
  };

  f32x16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled logits (log2 units), possibly stale by < 2^8
  float l_part = 0.f;

  RowCursor ca, cb;
  cursor_start(ca, a.row_ptr, a.iv, mask_id * a.n_qb + qb0, true, a.n_kb);
  cursor_start(cb, a.row_ptr, a.iv, mask_id * a.n_qb + qb0 + 1, has_b, a.n_kb);
  auto pick = [&](int& kb, bool& in_a, bool& in_b) -> bool {
    if (!ca.valid && !cb.valid) return false;
    kb = min(ca.valid ? ca.kb : INT_MAX, cb.valid ? cb.kb : INT_MAX);
    in_a = ca.valid && ca.kb == kb;
    in_b = cb.valid && cb.kb == kb;
    if (in_a) ca.valid = next_block(a.iv, ca.r1, a.n_kb, ca.t, ca.kb, ca.kend);
    if (in_b) cb.valid = next_block(a.iv, cb.r1, a.n_kb, cb.t, cb.kb, cb.kend);
    return true;
  };

  int kb = 0;
  bool in_a = false, in_b = false;
  bool valid = pick(kb, in_a, in_b);
  if (valid) stage(kb, 0);

  const int srow = swap_bits23(n);
  const float c2 = a.scale_log2;
  // per-lane LDS byte offsets inside a buffer; everything else is immediate
  const int k_lane = (srow * C::KROW + h) * 16;
  const int v_lane = C::KCH * 16 + ((8 * h + ((lane >> 2) & 3)) * C::VROW) * 16 +
                     (((lane >> 4) & 1) * 16 + (lane & 3) * 4) * 2;
  int buf = 0;
  while (valid) {
    int nkb = 0;
    bool nin_a = false, nin_b = false;
    const bool nvalid = pick(nkb, nin_a, nin_b);
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this thread's tile loads have landed
    __syncthreads();                      // everyone's have, and buffer buf^1 is free
    if (nvalid) stage(nkb, buf ^ 1);

    const bool mine = (wave < 4) ? in_a : in_b;
    if (mine) {
      const char* lb = reinterpret_cast<const char*>(lds[buf]);
      // ---- S^T = K Q^T ----------------------------------------------------
      f32x16 sacc[C::KT];
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt) {
        sacc[kt] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < C::DK; ++kk) {
          const uint4 raw = *reinterpret_cast<const uint4*>(lb + k_lane + (kt * 32 * C::KROW + 2 * kk) * 16);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(raw), qreg[kk], sacc[kt], 0, 0, 0);
        }
      }
      // ---- online softmax on raw logits; scale folded into the exponent ----
      const int key0 = kb * C::BLK;
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
      mx = fmaxf(mx, shfl_xor_f(mx, 32)) * c2;
      if (mx > m_run + kRescaleLog2) {
        const float alpha = fast_exp2(m_run - mx);
        l_part *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) oacc[dt] *= alpha;
        m_run = mx;
      }
      bf16x8 pb[C::PS];
#pragma unroll
      for (int s = 0; s < C::PS; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = fast_exp2(__builtin_fmaf(sacc[s >> 1][8 * (s & 1) + i], c2, -m_run));
          l_part += p;
          pb[s][i] = (__bf16)p;
        }
      // ---- O^T += V^T P^T; V^T operand by transposing LDS reads -------------
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
        for (int s = 0; s < C::PS; ++s) {
          const char* p0 = lb + v_lane + (16 * s * C::VROW) * 16 + dt * 64;
          bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p0);
          bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p0 + 4 * C::VROW * 16));
          bf16x8 vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[s], oacc[dt], 0, 0, 0);
        }
      }
    }
    kb = nkb;
    in_a = nin_a;
    in_b = nin_b;
    valid = nvalid;
    buf ^= 1;
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

template <int D, int BLK>
void launch_t(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.n_qb, a.BH);
  hipLaunchKernelGGL((attn_fwd_kernel<D, BLK>), grid, dim3(Cfg<D, BLK>::THREADS), 0, st, a);
}

template <int D>
void launch_b128(const AttnArgs& a, hipStream_t st) {
  const int pairs = (a.n_qb + 1) / 2;
  const int per_xcd = (pairs + 7) / 8;
  dim3 grid(8 * per_xcd * a.BH);
  hipLaunchKernelGGL((attn_fwd_b128_kernel<D>), grid, dim3(512), 0, st, a, pairs, per_xcd);
}

}  // namespace

void launch_attn(const AttnArgs& a, hipStream_t st) {
  if (a.block == 128) {
    if (a.D == 128) launch_b128<128>(a, st);
    else launch_b128<64>(a, st);
  } else {
    if (a.D == 128) launch_t<128, 64>(a, st);
    else launch_t<64, 64>(a, st);
  }
}

}  // namespace svg
