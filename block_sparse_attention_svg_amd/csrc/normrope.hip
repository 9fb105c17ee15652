// QK-Norm + 3D rotary position embedding of query / key rows, fused with the
// move from the projection's [B, N, H, D] rows to the attention's [B, H, N, D]
// in each head's layout ([SVG], "Layout Transformation + Kernel": the custom
// QK-Norm and RoPE kernels that precede the sparse attention).
//
// Normalisation is RMS normalisation (Zhang & Sennrich, 2019) over one head's
// D channels or over the whole H*D row; the rotation is RoFormer's (Su et al.,
// 2021) with the channels cut into frame / row / column runs.  Text tokens
// after the video grid are normalised but not rotated.
//
// Bound by HBM: every input byte is read once and every output byte written
// once (2 * B*N*H*D*2 bytes).  A workgroup takes kTok consecutive tokens of one
// batch row; thread t owns 16 bytes (8 channels) of head t / (D/8) in every
// one of them, so a token's row of H*D channels is one contiguous read and
// each head's 8- or 16-lane group writes one contiguous D*2-byte output row.
// All kTok loads are issued before any arithmetic to keep enough bytes in
// flight per CU.  The D/2 rotation angles of a token are shared by its H
// heads: they are computed once per token (sincosf in fp32 of pos times the
// run's frequency, which the host computes in double) and kept in LDS.
// Arithmetic is fp32 from the exact bf16 inputs with one rounding to bf16
// (to nearest even) at the end.
#include "svg_internal.h"

#include <cmath>

namespace svg {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTok = 4;  // tokens per workgroup

struct NormRopeArgs {
  const u32x4* x;       // [B, N, H, D] bf16
  u32x4* y;             // [B, H, N, D] bf16
  const float* gamma;   // [D] (per head) or [H*D] (whole row), or NULL
  const int32_t* head_layout;  // [B*H] or NULL
  int H, N, F, S, Ws, Nv;
  int norm_span;        // 0 none, 1 one head, 2 whole row
  float eps;
  int rope;             // 0 / 1
  int pairs_f, pairs_fy;  // pair index where the row run and the column run start
  FastDiv divS, divWs;
  float inv_freq[64];   // frequency of every channel pair's run
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// two floats -> two bf16 (round to nearest even), lo in the low half
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  a += 0x7fffu + ((a >> 16) & 1u);
  b += 0x7fffu + ((b >> 16) & 1u);
  return (a >> 16) | (b & 0xffff0000u);
}

template <int D>
__global__ __launch_bounds__(1024) void norm_rope_kernel(NormRopeArgs a) {
  constexpr int LPH = D / 8;  // lanes per head
  constexpr int NP = D / 2;   // channel pairs per head
  __shared__ float2 cs[kTok][NP];
  __shared__ float red[kTok][16];
  const int tid = threadIdx.x;
  const int h = tid / LPH, c = tid - h * LPH;
  const bool act = h < a.H;
  const int b = blockIdx.y;
  const int n0 = blockIdx.x * kTok;
  const int HD8 = a.H * LPH;  // 16-byte pieces per input row

  u32x4 raw[kTok];
#pragma unroll
  for (int t = 0; t < kTok; ++t) {
    const int n = n0 + t;
    raw[t] = u32x4{0, 0, 0, 0};
    if (act && n < a.N) raw[t] = a.x[(int64_t(b) * a.N + n) * HD8 + tid];
  }

  if (a.rope) {
    for (int j = tid; j < kTok * NP; j += blockDim.x) {
      const int t = j / NP, p = j - t * NP;
      const int n = n0 + t;
      float ang = 0.f;
      if (n < a.Nv) {
        const int f = int(a.divS.div(uint32_t(n)));
        const int s = n - f * a.S;
        const int yy = int(a.divWs.div(uint32_t(s)));
        const int pos = p < a.pairs_f ? f : (p < a.pairs_fy ? yy : s - yy * a.Ws);
        ang = float(pos) * a.inv_freq[p];
      }
      float sn, cn;
      sincosf(ang, &sn, &cn);
      cs[t][p] = make_float2(cn, sn);
    }
  }

  float v[kTok][8];
#pragma unroll
  for (int t = 0; t < kTok; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[t][2 * i] = bf16_lo(raw[t][i]);
      v[t][2 * i + 1] = bf16_hi(raw[t][i]);
    }

  float r[kTok];
#pragma unroll
  for (int t = 0; t < kTok; ++t) r[t] = 1.f;
  if (a.norm_span != 0) {
    float ss[kTok];
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fmaf(v[t][i], v[t][i], acc);
      ss[t] = acc;
    }
    if (a.norm_span == 1) {
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
#pragma unroll
        for (int m = 1; m < LPH; m <<= 1) ss[t] += __shfl_xor(ss[t], m);
        r[t] = rsqrtf(ss[t] * (1.f / D) + a.eps);
      }
    } else {
      const int wave = tid >> 6, nw = blockDim.x >> 6;
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) ss[t] += __shfl_xor(ss[t], m);
        if ((tid & 63) == 0) red[t][wave] = ss[t];
      }
      __syncthreads();
      const float inv_len = 1.f / float(a.H * D);
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
        float tot = 0.f;
        for (int w = 0; w < nw; ++w) tot += red[t][w];
        r[t] = rsqrtf(tot * inv_len + a.eps);
      }
    }
  }
  if (a.rope) __syncthreads();
  if (!act) return;

  float g[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) g[i] = 1.f;
  if (a.norm_span != 0 && a.gamma) {
    const float4* gp = reinterpret_cast<const float4*>(a.gamma + (a.norm_span == 2 ? h * D : 0) + c * 8);
    const float4 g0 = gp[0], g1 = gp[1];
    g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
    g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
  }
  const int bh = b * a.H + h;
  const bool tm = a.head_layout && a.head_layout[bh] != 0;
  u32x4* yh = a.y + int64_t(bh) * a.N * LPH;

#pragma unroll
  for (int t = 0; t < kTok; ++t) {
    const int n = n0 + t;
    if (n >= a.N) break;
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = v[t][i] * r[t] * g[i];
    if (a.rope) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2 e = cs[t][c * 4 + k];
        const float x0 = w[2 * k], x1 = w[2 * k + 1];
        w[2 * k] = x0 * e.x - x1 * e.y;
        w[2 * k + 1] = x0 * e.y + x1 * e.x;
      }
    }
    int row = n;
    if (tm && n < a.Nv) {
      const int f = int(a.divS.div(uint32_t(n)));
      row = (n - f * a.S) * a.F + f;
    }
    u32x4 o;
    o[0] = pack_bf16(w[0], w[1]);
    o[1] = pack_bf16(w[2], w[3]);
    o[2] = pack_bf16(w[4], w[5]);
    o[3] = pack_bf16(w[6], w[7]);
    __builtin_nontemporal_store(o, yh + int64_t(row) * LPH + c);
  }
}

}  // namespace

void launch_norm_rope(const void* x, void* y, const svg_shape& s, int norm_span, const float* gamma,
                      float eps, const svg_rope* rope, const int32_t* head_layout, hipStream_t st) {
  NormRopeArgs a;
  a.x = static_cast<const u32x4*>(x);
  a.y = static_cast<u32x4*>(y);
  a.gamma = gamma;
  a.head_layout = head_layout;
  a.H = s.H;
  a.N = s.N;
  a.F = s.F;
  a.S = s.Hs * s.Ws;
  a.Ws = s.Ws;
  a.Nv = s.F * a.S;
  a.norm_span = norm_span;
  a.eps = eps;
  a.rope = rope != nullptr;
  a.divS = FastDiv(uint32_t(a.S));
  a.divWs = FastDiv(uint32_t(s.Ws));
  a.pairs_f = a.pairs_fy = 0;
  for (int p = 0; p < 64; ++p) a.inv_freq[p] = 0.f;
  if (rope) {
    a.pairs_f = rope->d_f / 2;
    a.pairs_fy = (rope->d_f + rope->d_y) / 2;
    const int runs[3] = {rope->d_f, rope->d_y, rope->d_x};
    int p = 0;
    for (int r = 0; r < 3; ++r)
      for (int i = 0; i < runs[r] / 2; ++i, ++p)
        a.inv_freq[p] = float(std::pow(double(rope->theta), -2.0 * i / runs[r]));
  }
  const int threads = (s.H * s.D / 8 + 63) / 64 * 64;
  const dim3 grid((s.N + kTok - 1) / kTok, s.B);
  if (s.D == 128)
    hipLaunchKernelGGL(norm_rope_kernel<128>, grid, dim3(threads), 0, st, a);
  else
    hipLaunchKernelGGL(norm_rope_kernel<64>, grid, dim3(threads), 0, st, a);
}

}  // namespace svg
