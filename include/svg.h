/*
 * svg.h - C ABI of block-sparse 3D attention for video diffusion transformers
 *         (spatial / temporal heads, online head profiling, token-major layout,
 *         calibrated static block masks), MI355X / gfx950.
 *
 * Sources named in the comments:
 *   [SVG]      Sparse VideoGen article (m.jxzklqfsx.com/article/815093)
 *   [CalibAtt] calibrated sparse attention article (lpnh.cn/news/568491)
 *   [VDA]      video-diffusion acceleration survey (wmrh.cn/news/48564)
 *   [SparsePR] SparsePR tutorial (lqnn.cn/news/72918)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Array pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors)
 *   unless a comment says "host".  The caller owns every buffer; the library
 *   never allocates, frees or keeps a pointer after the call returns.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *   call only enqueues work on `stream`; none synchronises with the host.
 * - Activations are [B, H, N, D] row-major contiguous tensors ([SparsePR]
 *   section 2.1 uses this layout; the output has the shape of dense attention
 *   so it drops in for it).  Tokens are a video latent of F frames of Hs x Ws
 *   positions stored frame-major (token f*Hs*Ws + y*Ws + x), followed by
 *   N - F*Hs*Ws appended text tokens.
 * - Return value: SVG_OK or an error code.  Arguments are validated on the host
 *   before anything is enqueued; an invalid call enqueues nothing.  On error,
 *   svg_last_error() returns a description (thread-local, valid until the next
 *   call on the same thread).  SVG_ERR_HIP means a launch failed; its HIP
 *   error string is in svg_last_error().
 * - Device contents that violate a documented precondition (an out-of-range
 *   mask index, a skip-list interval outside [0, n_kb)) are clamped or skipped
 *   by the kernels, never dereferenced out of bounds, but give unspecified
 *   numbers.
 */
#ifndef SVG_H
#define SVG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVG_OK = 0,
  SVG_ERR_INVALID_ARG = 1,  /* null pointer, bad size, aliasing, ...          */
  SVG_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. head dim 96)    */
  SVG_ERR_CAPACITY = 3,     /* an output or workspace buffer is too small      */
  SVG_ERR_HIP = 4           /* a HIP launch or query failed                    */
} svg_status;

typedef enum { SVG_BF16 = 0, SVG_F32 = 1 } svg_dtype;

/* Shape of one attention layer. */
typedef struct {
  int B, H, N, D;   /* batch, heads, tokens (video + text), head dim (64 or 128) */
  int F, Hs, Ws;    /* latent frames and rows x columns per frame; F*Hs*Ws <= N */
  int block;        /* query and key block edge: 64 or 128                      */
} svg_shape;

/* Encoded block masks ([CalibAtt] section 3.3: bitmap + skip list).
 * bitmap : uint32 [n_masks][n_qb][ceil(n_kb/32)]; key block c of row r is bit
 *          c%32 of word c/32 (LSB first); padding bits are 0.
 * row_ptr: int32 [n_masks*n_qb + 1]; the intervals of row r of mask m are
 *          iv[row_ptr[m*n_qb + r] .. row_ptr[m*n_qb + r + 1]).
 * iv     : int32 pairs [start, end) of kept key blocks, ascending, disjoint,
 *          maximal; empty rows have none. */
typedef struct {
  int n_masks, n_qb, n_kb;
  const uint32_t* bitmap;
  const int32_t* row_ptr;
  const int32_t* iv;
} svg_mask;

/* ---- a1: per-shape candidate masks ------------------------------------- */
/* Writes the dense uint8 masks [2][nB][nB] (nB = ceil(N/block)) of the two
 * head types ([SVG], "Spatial Head" and "Temporal Head"):
 *   [0] spatial, on frame-major blocks: a block pair is kept when some video
 *       token of the query block and some video token of the key block are at
 *       most one frame apart;
 *   [1] temporal, on token-major blocks: kept when |r - c| <= band_w.
 * On both, every key block holding a text token is kept in every row and every
 * query block holding a text token keeps all key blocks.  Only s.N, s.F, s.Hs,
 * s.Ws and s.block are read.  masks: device uint8, 2*nB*nB bytes. */
svg_status svg_build_masks(svg_shape s, int band_w, uint8_t* masks, void* stream);

/* ---- a2: mask encoding -------------------------------------------------- */
/* Worst-case interval count of n_masks masks (rows alternate kept / skipped):
 * n_masks * n_qb * ceil(n_kb/2).  Host function, no device work. */
int64_t svg_encode_iv_capacity(int n_masks, int n_qb, int n_kb);

/* Encodes dense uint8 masks [n_masks][n_qb][n_kb] (nonzero = keep) into the
 * bitmap and skip list of svg_mask ([CalibAtt] section 3.3).  bitmap must hold
 * n_masks*n_qb*ceil(n_kb/32) words, row_ptr n_masks*n_qb+1 entries and iv
 * iv_capacity pairs; iv_capacity below svg_encode_iv_capacity(...) gives
 * SVG_ERR_CAPACITY (the actual count is row_ptr[n_masks*n_qb], known on the
 * device only).  Output is deterministic and identical on every call. */
svg_status svg_encode_mask(const uint8_t* dense, int n_masks, int n_qb, int n_kb,
                           uint32_t* bitmap, int32_t* row_ptr, int32_t* iv,
                           int64_t iv_capacity, void* stream);

/* ---- a4 / a6: layout permutation ---------------------------------------- */
/* Frame-major <-> token-major transpose of selected heads ([SVG], "Layout
 * Transformation + Kernel"): video token i = f*S + s (S = Hs*Ws) moves to
 * p = s*F + f; text tokens keep their index.  inverse = 0: y[p(i)] = x[i]
 * (frame -> token major); inverse = 1: y[i] = x[p(i)].  x, y: [B,H,N,D] of
 * dtype dt, must not overlap.  head_sel: device int32 [B*H]; only heads with
 * a nonzero entry are written, the rest of y is left untouched.  NULL selects
 * every head.  Bit-exact data movement. */
svg_status svg_permute(const void* x, void* y, svg_dtype dt, svg_shape s,
                       const int32_t* head_sel, int inverse, void* stream);

/* ---- step before the attention: QK-Norm + 3D RoPE ------------------------ */
/* Rotary embedding split over the video grid: channel pairs [0, d_f/2) turn
 * with the frame index, the next d_y/2 with the row, the last d_x/2 with the
 * column; pair i of a run of d channels turns by pos * theta^(-2i/d) rad
 * (RoFormer, Su et al. 2021).  d_f, d_y, d_x even and >= 0, summing to D. */
typedef struct {
  int d_f, d_y, d_x;
  float theta;      /* frequency base, > 0 (10000 in most video DiTs) */
} svg_rope;

/* QK-Norm and RoPE of query or key rows, written straight into the attention
 * input in each head's layout ([SVG], "Layout Transformation + Kernel": the
 * custom QK-Norm and RoPE kernels that precede the sparse attention).
 *   x          : bf16 [B,N,H,D], the projection output, frame-major tokens.
 *   y          : bf16 [B,H,N,D] out; must not overlap x.
 *   norm_span  : 0 no normalisation, 1 RMS over each head's D channels, 2 RMS
 *                over the whole H*D row (Zhang & Sennrich 2019, no centring):
 *                x / sqrt(mean(x^2) + eps) * gamma.
 *   gamma      : device float [D] (norm_span 1) or [H*D] (norm_span 2),
 *                16-byte aligned, or NULL for all ones.  eps >= 0.
 *   rope       : host struct, or NULL for no rotation.  Video token
 *                n = f*Hs*Ws + yy*Ws + xx sits at (f, yy, xx); text tokens
 *                (n >= F*Hs*Ws) are not rotated.
 *   head_layout: device int32 [B*H], or NULL for all 0: heads with a
 *                nonzero entry are written token-major (video token f*S + s
 *                at row s*F + f, S = Hs*Ws), the rest frame-major (the same
 *                convention as svg_block_sparse_attn's head_layout).
 * fp32 arithmetic from the exact inputs, one rounding to bf16 (nearest even).
 * With norm_span 0 and rope NULL the call is an exact transpose / layout move
 * (V of a layer).  s.block is not read but must be valid.  x, y 16-byte
 * aligned; D in {64, 128}; H*D <= 8192 (SVG_ERR_UNSUPPORTED otherwise). */
svg_status svg_qk_norm_rope(const void* x, void* y, svg_shape s, int norm_span, const float* gamma,
                            float eps, const svg_rope* rope, const int32_t* head_layout,
                            void* stream);

/* ---- a3: online head profiling ------------------------------------------ */
/* Workspace size in bytes for svg_profile_heads (host function). */
size_t svg_profile_workspace_bytes(svg_shape s, int n_samples);

/* Picks each head's mask by sampled-query error ([SVG], online profiling:
 * sample about 64 queries, compute their attention under the spatial and the
 * temporal mask, compare each with dense attention, keep the smaller error).
 *   q, k, v : bf16 [B,H,N,D] frame-major.
 *   idx     : device int32 [n_samples], distinct frame-major video-token
 *             indices (< F*Hs*Ws), shared by every head; 1 <= n_samples <= 64.
 *   cand    : host struct, n_masks == 2, n_qb == n_kb == ceil(N/block):
 *             [0] spatial on frame-major blocks, [1] temporal on token-major
 *             blocks (only the bitmap is read).
 *   choice  : device int32 [B*H] out: 0 spatial, 1 temporal (a tie -> 0).
 *   err     : device float [B*H][2] out, or NULL: squared L2 error of the
 *             spatial / temporal output against dense attention, summed over
 *             the samples and the head dim (fp32, from the decomposition
 *             o_dense - o_m = (Z_out/Z) (U_out/Z_out - U_in/Z_in)).
 *   workspace: device, >= svg_profile_workspace_bytes(s, n_samples) bytes.
 * Deterministic: fixed reduction order, identical results on every call. */
svg_status svg_profile_heads(const void* q, const void* k, const void* v, svg_shape s,
                             float scale, const int32_t* idx, int n_samples,
                             const svg_mask* cand, int32_t* choice, float* err,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---- a4 / a6 fused: the layout pass of a 128-token-block layer ------------ */
/* Bytes of the block-transposed V buffer of shape s (host function):
 * B*H*ceil(N/128)*128*D*2 for 128-token blocks, 0 otherwise. */
size_t svg_vt_bytes(svg_shape s);

/* One pass over K and V after the head choice ([SVG], "Layout Transformation
 * + Kernel": the temporal heads' tokens made contiguous in token-major
 * order).  For every head (b, h):
 *   vt[bh][kb][d][j] = V'[kb*128 + j][d]  (keys past N zero), where V' is the
 *                      head's V in its layout: frame-major when
 *                      head_layout[bh] == 0, token-major otherwise (token-major
 *                      row t is frame-major row (t % F)*Hs*Ws + t / F, text
 *                      rows in place);
 *   kp[bh][t][:]     = k[bh][fm(t)][:] for heads with head_layout[bh] != 0,
 *                      when kp is given (other heads' kp rows untouched).
 *   k, v   : bf16 [B,H,N,D] frame-major (k may be NULL when kp is NULL).
 *   kp     : bf16 [B,H,N,D] or NULL.
 *   vt     : bf16, svg_vt_bytes(s) bytes, the V operand svg_block_sparse_attn
 *            takes as `vt`.
 *   head_layout: device int32 [B*H] or NULL (all frame-major).
 * A pure data move: bit-exact.  128-token blocks only (SVG_ERR_UNSUPPORTED
 * otherwise); 16-byte aligned, non-overlapping buffers. */
svg_status svg_prepare_kv(const void* k, const void* v, void* kp, void* vt, svg_shape s,
                          const int32_t* head_layout, void* stream);

/* ---- a5: block-sparse attention ----------------------------------------- */
/* Softmax attention restricted, per query block, to the key blocks of the
 * head's mask row ([CalibAtt] sections 2.2 and 3.3; [VDA] section 2.1 for the
 * attention itself, section 5.3 for tiled online softmax).  Only the kept
 * key blocks are read.  Not causal.
 *   q, k, v, o     : bf16 [B,H,N,D] frame-major.
 *   vt             : the heads' V blocks as svg_prepare_kv writes them (each
 *                    head in the layout head_layout gives it), or NULL.  With
 *                    128-token blocks and vt given, v, vp are not read (v may
 *                    be NULL) and the workspace holds the work plan only;
 *                    with vt NULL the call lays V out itself, in the
 *                    workspace.  Must be NULL for 64-token blocks.
 *   qp, kp, vp, op : bf16 [B,H,N,D] token-major twins; may be NULL when no
 *                    head uses layout 1.  With 128-token blocks only kp is
 *                    required: a layout-1 head whose qp / vp / op is NULL
 *                    reads its Q / V rows from q / v and writes its O rows
 *                    to o through the permutation (token-major row t is
 *                    frame-major row (t % F)*Hs*Ws + t / F, text rows in
 *                    place), so those tensors need no separate svg_permute
 *                    and o holds every head frame-major.
 *   masks          : host struct; n_qb == n_kb == ceil(N/block); with
 *                    128-token blocks at most 131070 blocks and 32768 masks
 *                    (SVG_ERR_UNSUPPORTED beyond).
 *   head_mask      : device int32 [B*H]: mask index of each head (clamped to
 *                    [0, n_masks)); NULL means mask h % n_masks for head h.
 *   head_layout    : device int32 [B*H]: 0 = attend q,k,v -> o; nonzero =
 *                    attend qp,kp,vp -> op (mask blocks are then token-major
 *                    blocks); NULL means all 0.
 *   lse            : device float [B,H,N] out (natural-log log-sum-exp of the
 *                    scaled logits, in the layout the head attends in), or NULL.
 *   workspace      : device scratch of >= svg_attn_workspace_bytes(s, vt != NULL)
 *                    bytes (V re-laid out per key block unless vt is given,
 *                    then a plan that splits every head's query-block pairs
 *                    over the 8 XCDs into ranges of equal work, from the mask
 *                    bitmap, and the heads of the 8 work queues the kernel's
 *                    workgroups take those ranges from); 16-byte aligned; may
 *                    be NULL when the size is 0.  Its contents need no
 *                    initialisation and are overwritten by every call; calls
 *                    in flight at the same time need separate workspaces.
 * The masks' bitmap and skip list must describe the same mask (as
 * svg_encode_mask writes them): with 128-token blocks the kernel lists each
 * pair of query blocks' kept key blocks from the bitmap (and balances work
 * with it), with 64-token blocks it walks the skip list.  A query block whose mask row is empty gets o = 0
 * and lse = -inf.  bf16 inputs, fp32 accumulation and softmax, bf16 output
 * (P rounded to bf16 for the PV product; the softmax denominator sums the
 * fp32 weights, except for 128-token blocks with lse == NULL, where it is
 * the matrix core's fp32 sum of the bf16-rounded weights the PV product
 * used).  The result does not depend on whether vt is given. */
svg_status svg_block_sparse_attn(const void* q, const void* k, const void* v, const void* vt, void* o,
                                 const void* qp, const void* kp, const void* vp, void* op,
                                 svg_shape s, float scale, const svg_mask* masks,
                                 const int32_t* head_mask, const int32_t* head_layout,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Workspace bytes svg_block_sparse_attn needs for shape s (host function).
 * 128-token blocks: B*H*ceil(N/128)*128*D*2 (V transposed per key block; none
 * when vt_given != 0), then a work plan of (9*B*H + 16 rounded up to
 * even)*4 + 8*B*H*cap*8 + B*H*pairs*4 bytes with pairs = ceil(ceil(N/128)/2)
 * and cap = max(ceil(3*pairs/16), ceil(pairs/8)).  64-token blocks: 0. */
size_t svg_attn_workspace_bytes(svg_shape s, int vt_given);

/* ---- FP8 variant ([CalibAtt] section 3.3: FP8 on the critical path) -------- */
/* Bytes of the FP8 V^T block buffer: B*H*ceil(N/128)*128*D for 128-token
 * blocks, 0 otherwise (host function). */
size_t svg_fp8_vt_bytes(svg_shape s);

/* E4M3 operands of the FP8 attention, one scale per (tensor, head).  For
 * x in {q, k, v} of head (b, h): amax = max |x|, inv = 448 / amax in fp32 (1
 * when amax = 0); every element is multiplied by inv in fp32 and rounded to
 * OCP E4M3 (nearest, ties to even; largest finite value 448).
 *   q, k, v : bf16 [B,H,N,D] frame-major.
 *   q8      : uint8 [B,H,N,D], every head frame-major.
 *   k8      : uint8 [B,H,N,D], each head in its layout (head_layout != 0:
 *             token-major rows, token-major row t = frame-major row
 *             (t % F)*Hs*Ws + t / F, text rows in place).
 *   vt8     : uint8, svg_fp8_vt_bytes(s): per head and 128-key block (keys
 *             in the head's layout) a [D][128] byte tile whose keys
 *             8a + 4h + i of each 64-key group sit at byte 32h + 4a + i;
 *             keys past N are 0.
 *   scales  : device float [3][B*H] out: the dequantization factors
 *             amax / 448 (1 when amax = 0) of q, k and v.
 *   head_layout: device int32 [B*H] or NULL (all frame-major).
 * 128-token blocks, D in {64, 128}; 16-byte aligned, non-overlapping. */
svg_status svg_quantize_fp8(const void* q, const void* k, const void* v, uint8_t* q8, uint8_t* k8,
                            uint8_t* vt8, float* scales, svg_shape s, const int32_t* head_layout,
                            void* stream);

/* Block-sparse attention with both products on FP8 (E4M3) operands
 * (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulation): S = scale * d_q * d_k *
 * (q8 . k8), the online softmax in fp32, P rounded to E4M3 for the PV
 * product, O = d_v * sum(P v8) / sum(P) with the denominator summed from the
 * fp32 weights (from the E4M3 weights on the matrix core when lse == NULL),
 * output
 * bf16 [B,H,N,D] frame-major for every head (layout-1 heads read their Q rows
 * and write their O rows through the permutation).  q8, k8, vt8, scales as
 * svg_quantize_fp8 writes them for the same head_layout; masks, head_mask,
 * head_layout, lse as for svg_block_sparse_attn.  workspace: the work plan,
 * >= svg_attn_workspace_bytes(s, 1) bytes.  128-token blocks only. */
svg_status svg_block_sparse_attn_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8,
                                     const float* scales, void* o, svg_shape s, float scale,
                                     const svg_mask* masks, const int32_t* head_mask,
                                     const int32_t* head_layout, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call and the same kernels as svg_block_sparse_attn, with the work plan of
 * the 128-token-block kernels kept in a fixed device array of the library
 * (svg_noalloc_scratch_bytes() = 8 MiB, one copy per GPU, held until the
 * process ends) instead of a workspace.  With 128-token blocks vt is required
 * (svg_prepare_kv); 64-token blocks need no scratch.  SVG_ERR_CAPACITY when
 * the plan (svg_attn_workspace_bytes(s, 1)) exceeds the array.  No
 * allocation of any kind.  Every call on a GPU shares that GPU's array and
 * rewrites all of the plan it reads, so calls that overlap on one GPU (other
 * streams, other threads) race; calls in order on one stream do not.  The
 * results equal svg_block_sparse_attn's bit for bit. */
size_t svg_noalloc_scratch_bytes(void);
svg_status svg_block_sparse_attn_noalloc(const void* q, const void* k, const void* v, const void* vt,
                                         void* o, const void* qp, const void* kp, const void* vp,
                                         void* op, svg_shape s, float scale, const svg_mask* masks,
                                         const int32_t* head_mask, const int32_t* head_layout,
                                         float* lse, void* stream);

/* ---- offline calibration ([CalibAtt] section 3.1) --------------------------- */
/* Block attention energy: energy[bh][r][c] = sum over the queries i of block r
 * and the keys j of block c of the dense softmax weight exp(s_ij - lse_i),
 * s_ij = scale * q_i.k_j, lse_i over all N keys: the E(r, c) that the
 * energy-threshold rule (svg_calibrate_masks) ranks.  Each row sums to the
 * number of queries in block r.
 *   q, k   : bf16 [B,H,N,D], blocks taken in this layout (block = s.block).
 *   energy : device double [B*H, nB, nB] out, nB = ceil(N/block).
 * Two sweeps over the keys per query block (running max and sum, then block
 * sums); fp32 arithmetic, sums in a fixed order (identical on every call).
 * Errors: SVG_ERR_INVALID_ARG for NULL pointers or scale <= 0,
 * SVG_ERR_UNSUPPORTED for D or block outside {64, 128} or B*H > 65535. */
svg_status svg_block_energy(const void* q, const void* k, svg_shape s, float scale, double* energy,
                            void* stream);

/* Merge of candidate masks over prompts: out[e] = 1 when the fraction of the
 * n_sets masks that keep element e reaches rho (count / n_sets >= rho in
 * double), else 0.
 *   masks : device uint8 [n_sets][mask_elems] (nonzero = kept); out: device
 *           uint8 [mask_elems], not overlapping masks.  0 < rho <= 1. */
svg_status svg_aggregate_masks(const uint8_t* masks, int n_sets, int64_t mask_elems, double rho,
                               uint8_t* out, void* stream);

/* Row-repetitive head test ([CalibAtt] section 3.2): for every head, the mean
 * over frames and over pairs of distinct latent rows of a frame of the cosine
 * similarity of the two rows' attention patterns, a row's pattern being the
 * sum of the dense softmax weights of its Ws queries over all N keys.  A head
 * whose score exceeds gamma (0.87 on the pages) is row-repetitive
 * (svg_restrict_anchor_rows, svg_row_broadcast).
 *   q, k      : bf16 [B,H,N,D] frame-major (rows are Ws consecutive tokens).
 *   score     : device double [B*H] out.
 *   workspace : device, >= svg_row_similarity_workspace_bytes(s) bytes,
 *               256-byte aligned: the row patterns, float [B*H][F*Hs][N],
 *               then per-frame sums and partial Gram tiles (Wan 720p: 289 MB
 *               per head).
 * fp32 weights and pattern sums, float64 Gram sums (exact products), fixed
 * order (identical on every call).  SVG_ERR_UNSUPPORTED for Ws > 128, Hs
 * outside [2, 64], Hs * N * 4 >= 2^31, D outside {64, 128} or B*H > 65535;
 * SVG_ERR_CAPACITY for a short workspace. */
size_t svg_row_similarity_workspace_bytes(svg_shape s);
svg_status svg_row_similarity(const void* q, const void* k, svg_shape s, float scale, double* score,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Energy threshold of denoising step t of T (host function): an exponential
 * decay from eps_first at t = 0 to eps_last at t = T-1,
 * eps_first * (eps_last / eps_first)^(t / (T-1)); eps_first when T == 1.
 * The pages give about 0.99 early and 0.84 late.  Needs 0 <= t < T and both
 * thresholds in (0, 1]. */
svg_status svg_eps_schedule(int t, int T, double eps_first, double eps_last, double* eps);

/* ---- a7: row-repetitive heads ------------------------------------------- */
/* Anchor-row broadcast ([CalibAtt] section 3.2): in every frame, latent row y
 * takes the output of its anchor row a(y) = floor((2j+1)*Hs/(2k)) with
 * j = floor(y*k/Hs) (k equally spaced band centres).  o: bf16 [B,H,N,D]
 * frame-major, rewritten in place for heads with head_sel != 0 (device int32
 * [B*H]); text tokens untouched.  1 <= k_anchors <= Hs. */
svg_status svg_row_broadcast(void* o, svg_shape s, const int32_t* head_sel, int k_anchors,
                             void* stream);

/* Empties, in place, the rows of dense uint8 masks [n_masks][nB][nB] whose
 * frame-major query block holds no anchor-row video token, for masks with
 * mask_sel != 0 (device int32 [n_masks]).  Attention then computes only the
 * anchor-holding query blocks of a row-repetitive head ([CalibAtt] 3.2). */
svg_status svg_restrict_anchor_rows(uint8_t* masks, int n_masks, svg_shape s,
                                    const int32_t* mask_sel, int k_anchors, void* stream);

/* ---- calibrated static masks -------------------------------------------- */
/* Energy-threshold selection ([CalibAtt] section 3.1): for each row r of
 * energies E [n_masks][n_qb][n_kb] (float64, >= 0), rank key blocks by energy
 * (descending, ties by smaller index) and keep the shortest prefix whose
 * running sum reaches eps * total; sums are taken in that order in float64,
 * term by term, total being the last running sum.  out: uint8 masks of the
 * same shape.  n_kb <= 4096; 0 < eps <= 1. */
svg_status svg_calibrate_masks(const double* energy, int n_masks, int n_qb, int n_kb,
                               double eps, uint8_t* out, void* stream);

/* ---- measurement aid (not part of the attention path) ---------------------- */
/* Dense matrix-core rate this GPU sustains under its power limit: one
 * workgroup of 8 wavefronts per CU, each issuing `rounds` x 16 back-to-back
 * 32x32 MFMAs (v_mfma_f32_32x32x16_bf16, or v_mfma_f32_32x32x64_f8f6f4 when
 * fp8 = 1) on operands held in registers: no memory or LDS traffic.  The
 * rate (FLOP / kernel time) bounds what any kernel with the same products
 * reaches on this board at this moment; the attention's rate is reported
 * beside it.  sink: device float [sink_floats] written with junk (one float
 * per thread, >= n_CU * 512 floats); flop (host out): FLOP of the launch,
 * n_CU * 8 * rounds * 16 * 2 * 32 * 32 * K (K = 16 bf16, 64 FP8).
 * Errors: SVG_ERR_INVALID_ARG for fp8 outside {0, 1}, rounds outside
 * [1, 2^20] or NULL pointers; SVG_ERR_HIP without a device;
 * SVG_ERR_CAPACITY for a short sink. */
svg_status svg_mfma_peak_probe(int fp8, int rounds, float* sink, int64_t sink_floats, double* flop,
                               void* stream);

/* ---- errors -------------------------------------------------------------- */
const char* svg_status_string(svg_status st);
const char* svg_last_error(void);
/* Library version string, e.g. "svg-mi355x 0.1 gfx950". */
const char* svg_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SVG_H */
