"""GPU parity of block-sparse attention against the float64 oracle.

Tolerance per head (bf16 in, fp32 accumulate, bf16 out): max-abs <= 2e-2 and
relative L2 <= 5e-3; log-sum-exp within LSE_ABS.  Small workloads are compared
on every row; the full-size layers are in test_gpu_full_size.py.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_svg_amd as svg
import oracle as O
import synth as S
from parity_utils import banner, assert_attn_close, to_np, LSE_ABS, sample_qblocks, fp8_bound

pytestmark = pytest.mark.gpu
DEV = "cuda"


def shape_of(w, H=None, block=None):
    return svg.Shape(w.B, H or w.H, w.N, w.D, w.F, w.Hs, w.Ws, block or w.block)


def _run_heads(w, q, k, v, masks_np, layout, block=None, lse=False):
    """GPU attention where head h uses mask masks_np[h] in layout[h]."""
    s = shape_of(w, q.shape[1], block)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    enc = svg.svg_encode_mask(torch.from_numpy(np.ascontiguousarray(masks_np)).to(DEV))
    lay = torch.tensor(layout, dtype=torch.int32, device=DEV)
    hm = torch.arange(len(layout), dtype=torch.int32, device=DEV)
    qp, kp, vp = (svg.svg_permute(t, s, lay) for t in (qd, kd, vd))
    o, op, lse_t = svg.svg_block_sparse_attn(qd, kd, vd, s, 1.0 / np.sqrt(w.D), enc, head_mask=hm,
                                             head_layout=lay, qp=qp, kp=kp, vp=vp,
                                             op=torch.empty_like(qd), lse=lse)
    torch.cuda.synchronize()
    return o, op, lse_t


def test_tiny_all_rows_and_lse(workload_inputs):
    w, q32, k32, v32, cls = workload_inputs("tiny", dtype="f32")
    banner("attn tiny")
    q, k, v = (t.to(torch.bfloat16) for t in (q32, k32, v32))   # bf16 copy, oracle on the same bits
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    o, op, lse = _run_heads(w, q, k, v, cand, [0, 1], lse=True)
    p = O.token_major_index(w.F, w.Hs, w.Ws, w.N)
    for h in range(2):
        ref_o, ref_lse = O.head_attention(q[0, h].float().numpy(), k[0, h].float().numpy(),
                                          v[0, h].float().numpy(), cand[h], h, w.F, w.Hs, w.Ws,
                                          w.block, w.scale)
        got = to_np(o[0, h]) if h == 0 else to_np(op[0, h])[p]
        assert_attn_close(got, ref_o, f"tiny head {h}")
        lse_h = lse[0, h].cpu().numpy()
        lse_fm = lse_h if h == 0 else lse_h[p]       # LSE is stored in the attended layout
        assert np.max(np.abs(lse_fm - ref_lse)) < LSE_ABS


@pytest.mark.parametrize("block", [64, 128])
def test_dense_mask_equals_dense_attention(block, workload_inputs):
    w, q32, k32, v32, _ = workload_inputs("tiny", dtype="f32")
    banner("attn dense", block)
    q, k, v = (t.to(torch.bfloat16) for t in (q32, k32, v32))
    nb = -(-w.N // block)
    masks = np.ones((2, nb, nb), np.uint8)
    o, _, _ = _run_heads(w, q, k, v, masks, [0, 0], block=block)
    for h in range(2):
        ref, _ = O.dense_attention(q[0, h].float().numpy(), k[0, h].float().numpy(),
                                   v[0, h].float().numpy(), w.scale)
        assert_attn_close(to_np(o[0, h]), ref, f"dense h{h} block {block}")


def test_ragged_partial_blocks_and_empty_rows():
    """N not a multiple of the block; some mask rows empty (o = 0, lse = -inf)."""
    banner("attn ragged/empty")
    w = S.get_workload("tiny", F=3, Hs=10, Ws=10, text=37, H=3, D=128)   # N = 337, 3 blocks of 128
    q, k, v, _ = S.gen_qkv(w, dtype="bf16")
    s = shape_of(w, block=128)
    rng = np.random.default_rng(2)
    masks = (rng.random((3, 3, 3)) < 0.6).astype(np.uint8)
    masks[:, :, 2] = 1
    masks[1, 1] = 0                     # empty row
    o, _, lse = _run_heads(w, q, k, v, masks, [0, 0, 0], block=128, lse=True)
    o2, _, _ = _run_heads(w, q, k, v, masks, [0, 0, 0], block=128)     # denominator on the matrix core
    for h in range(3):
        ref, ref_lse = O.block_masked_attention(q[0, h].float().numpy(), k[0, h].float().numpy(),
                                                v[0, h].float().numpy(), masks[h], 128, w.scale)
        assert_attn_close(to_np(o[0, h]), ref, f"ragged head {h}")
        assert_attn_close(to_np(o2[0, h]), ref, f"ragged head {h} (no LSE)")
        g = lse[0, h].cpu().numpy()
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isneginf(g), ~fin)
        assert np.max(np.abs(g[fin] - ref_lse[fin])) < LSE_ABS
    assert torch.all(o[0, 1, 128:256] == 0) and torch.all(o2[0, 1, 128:256] == 0)


@pytest.mark.parametrize("D,block", [(64, 64), (128, 64), (64, 128)])
def test_head_dims_and_blocks(D, block):
    banner("attn dims", D, block)
    w = S.get_workload("cogvideox", H=4, D=D, F=3, n_spatial=2)       # N = 4050: 32 blocks of 128, ragged
    q, k, v, cls = S.gen_qkv(w, dtype="bf16")
    s_masks = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, block, 3)
    masks = np.stack([s_masks[c] for c in cls])
    o, op, _ = _run_heads(w, q, k, v, masks, cls.tolist(), block=block)
    p = O.token_major_index(w.F, w.Hs, w.Ws, w.N)
    for h in range(4):
        ref, _ = O.head_attention(q[0, h].float().numpy(), k[0, h].float().numpy(),
                                  v[0, h].float().numpy(), masks[h], int(cls[h]), w.F, w.Hs, w.Ws,
                                  block, w.scale)
        got = to_np(o[0, h]) if cls[h] == 0 else to_np(op[0, h])[p]
        assert_attn_close(got, ref, f"D{D} B{block} head {h}")


def _layer_outputs(name, workload_inputs, t=0):
    w, q, k, v, cls = workload_inputs(name)
    s = shape_of(w)
    layer = svg.OnlineSparseAttention(s, w.band_w)
    idx = torch.from_numpy(S.sample_query_idx(w, t)).to(DEV)
    o, _ = layer(q.to(DEV), k.to(DEV), v.to(DEV), idx)
    torch.cuda.synchronize()
    return w, q, k, v, cls, layer.choice.cpu().numpy(), o


def test_online_layer_cogvideox_every_head(workload_inputs):
    """Every head: eight of them on all rows, the others on 32 query blocks."""
    banner("layer cogvideox")
    w, q, k, v, cls, choice, o = _layer_outputs("cogvideox", workload_inputs)
    assert np.array_equal(choice, cls)
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    every_row = [0, 1, 2, 3, 21, 22, 46, 47]
    for h in range(w.H):
        qbs = None if h in every_row else sample_qblocks(w.n_blocks, seed=w.seed * 100 + h)
        ref, _ = O.head_attention(q[0, h].float().numpy(), k[0, h].float().numpy(),
                                  v[0, h].float().numpy(), cand[choice[h]], int(choice[h]),
                                  w.F, w.Hs, w.Ws, w.block, w.scale, qblocks=qbs)
        rows = ~np.isnan(ref[:, 0])
        assert_attn_close(to_np(o[0, h])[rows], ref[rows], f"cog head {h}")


def test_attention_is_deterministic(workload_inputs):
    banner("attn determinism")
    w, q32, k32, v32, _ = workload_inputs("tiny", dtype="f32")
    q, k, v = (t.to(torch.bfloat16) for t in (q32, k32, v32))
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    o1, op1, _ = _run_heads(w, q, k, v, cand, [0, 1])
    o2, op2, _ = _run_heads(w, q, k, v, cand, [0, 1])
    assert torch.equal(o1[0, 0], o2[0, 0]) and torch.equal(op1[0, 1], op2[0, 1])


def test_batch2_heavy_and_empty_rows_over_many_pairs():
    """B = 2, odd head count, 21 query blocks (11 pairs spread over the XCD work
    lists): random masks with dense rows (heavy pairs, scheduled first), empty
    rows and a ragged last block; every row against the oracle."""
    banner("attn batch2 plan")
    w = S.get_workload("tiny", F=5, Hs=16, Ws=32, text=100, H=3, D=128)   # N = 2660: 21 blocks of 128
    qa, ka, va, _ = S.gen_qkv(w, dtype="bf16")
    qb, kb, vb, _ = S.gen_qkv(S.get_workload("tiny", F=5, Hs=16, Ws=32, text=100, H=3, D=128,
                                             seed=w.seed + 1), dtype="bf16")
    q, k, v = (torch.cat([x, y], 0).contiguous() for x, y in ((qa, qb), (ka, kb), (va, vb)))
    s = svg.Shape(2, w.H, w.N, w.D, w.F, w.Hs, w.Ws, 128)
    nB = -(-w.N // 128)
    rng = np.random.default_rng(11)
    masks = (rng.random((6, nB, nB)) < 0.25).astype(np.uint8)
    for m in range(6):
        masks[m, rng.integers(nB, size=2)] = 1          # two dense rows per head
        masks[m, rng.integers(nB)] = 0                  # one empty row
    enc = svg.svg_encode_mask(torch.from_numpy(masks).to(DEV))
    hm = torch.arange(6, dtype=torch.int32, device=DEV)
    o, _, _ = svg.svg_block_sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), s, w.scale, enc, head_mask=hm)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(w.H):
            ref, _ = O.block_masked_attention(q[b, h].float().numpy(), k[b, h].float().numpy(),
                                              v[b, h].float().numpy(), masks[b * w.H + h], 128, w.scale)
            assert_attn_close(to_np(o[b, h]), ref, f"batch {b} head {h}")


def test_long_rows_cross_block_list_windows():
    """More than 2048 key blocks: the kernel lists a pair's kept blocks in
    windows of 2048.  Rows whose kept blocks straddle, precede or follow the
    window boundary (also within one pair), a dense ragged last row and
    random sparse rows, sampled against the oracle."""
    banner("attn long rows")
    w = S.get_workload("tiny", F=7, Hs=160, Ws=240, text=5, H=2, D=64)   # N = 268805: 2101 blocks
    q, k, v, _ = S.gen_qkv(w, dtype="bf16")
    nB = -(-w.N // 128)
    rng = np.random.default_rng(13)
    masks = (rng.random((2, nB, nB)) < 0.02).astype(np.uint8)
    masks[0, 10, 2000:2100] = 1                    # a run across the boundary
    masks[0, 11] = 0
    masks[0, 11, 2049:] = 1                        # its pair partner: only after it
    masks[1, 20] = 0
    masks[1, 20, :2048] = 1                        # pair (20, 21): before / after
    masks[1, 21] = 0
    masks[1, 21, 2048:] = 1
    masks[:, nB - 1] = 1                           # dense ragged last row
    s = svg.Shape(1, 2, w.N, w.D, w.F, w.Hs, w.Ws, 128)
    enc = svg.svg_encode_mask(torch.from_numpy(masks).to(DEV))
    hm = torch.arange(2, dtype=torch.int32, device=DEV)
    o, _, lse = svg.svg_block_sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), s, w.scale, enc,
                                          head_mask=hm, lse=True)
    o2, _, _ = svg.svg_block_sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), s, w.scale, enc, head_mask=hm)
    torch.cuda.synchronize()
    qbs = [0, 10, 11, 20, 21, 1024, nB - 2, nB - 1]
    for h in range(2):
        ref, ref_lse = O.block_masked_attention(q[0, h].float().numpy(), k[0, h].float().numpy(),
                                                v[0, h].float().numpy(), masks[h], 128, w.scale,
                                                qblocks=qbs)
        rows = ~np.isnan(ref[:, 0])
        assert_attn_close(to_np(o[0, h])[rows], ref[rows], f"long rows head {h}")
        assert_attn_close(to_np(o2[0, h])[rows], ref[rows], f"long rows head {h} (no LSE)")
        g = lse[0, h].cpu().numpy()[rows]
        assert np.max(np.abs(g - ref_lse[rows])) < LSE_ABS


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("order", ["rising", "falling", "one_spike"])
def test_softmax_reference_moves(order, D):
    """Scores that rise by ~36 (D = 64) or ~51 (D = 128) log2 units per key block move the running
    max at every block (O and the denominator rescaled each time); falling
    scores never move it (later weights underflow towards 0); one far larger
    block moves it once.  All rows, O and LSE, against the oracle; the call
    without LSE (denominator on the matrix core) and the FP8 variant with and
    without LSE as well, FP8 against its derived bounds."""
    banner("attn reference", order, D)
    N, nB = 1000, 8                                         # ragged last block
    rng = np.random.default_rng(17)
    u = np.full(D, 0.5)                                     # |u|^2 = D / 4
    blk = np.arange(N) // 128
    c = {"rising": 25.0 * blk, "falling": 25.0 * (nB - 1 - blk),
         "one_spike": np.where(blk == 5, 60.0, 0.0)}[order]
    qn = (u[None, :] + 0.05 * rng.standard_normal((N, D)))
    kn = c[:, None] * u[None, :] / 16.0 * 8.0 + 0.05 * rng.standard_normal((N, D))   # s = c sqrt(D) / 8
    vn = rng.standard_normal((N, D))
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).reshape(1, 1, N, D).contiguous() for x in (qn, kn, vn))
    scale = 1.0 / np.sqrt(D)
    masks = np.ones((1, nB, nB), dtype=np.uint8)
    s = svg.Shape(1, 1, N, D, 1, 1, 1, 128)
    enc = svg.svg_encode_mask(torch.from_numpy(masks).to(DEV))
    hm = torch.zeros(1, dtype=torch.int32, device=DEV)
    o, _, lse = svg.svg_block_sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), s, scale, enc,
                                          head_mask=hm, lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = O.block_masked_attention(q[0, 0].float().numpy(), k[0, 0].float().numpy(),
                                            v[0, 0].float().numpy(), masks[0], 128, scale)
    assert np.all(np.isfinite(to_np(o[0, 0])))
    assert_attn_close(to_np(o[0, 0]), ref, f"reference {order}")
    assert np.max(np.abs(lse[0, 0].cpu().numpy() - ref_lse)) < LSE_ABS * max(1.0, float(np.max(np.abs(ref_lse))) / 64)
    # without the LSE: the denominator summed on the matrix core, rescaled
    # with O at every move of the running max
    o2, _, _ = svg.svg_block_sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), s, scale, enc, head_mask=hm)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(to_np(o2[0, 0])))
    assert_attn_close(to_np(o2[0, 0]), ref, f"reference {order} (no LSE)")
    # FP8, with and without the LSE, against the bounds derived from E4M3
    ops8 = svg.svg_quantize_fp8(q.to(DEV), k.to(DEV), v.to(DEV), s)
    o8, l8 = svg.svg_block_sparse_attn_fp8(ops8, s, scale, enc, head_mask=hm, lse=True)
    o8n, _ = svg.svg_block_sparse_attn_fp8(ops8, s, scale, enc, head_mask=hm)
    torch.cuda.synchronize()
    deq = [O.quantize_head(x[0, 0].float().numpy())[3] for x in (q, k, v)]
    ref8, ref8_lse = O.block_masked_attention(deq[0], deq[1], deq[2], masks[0], 128, scale)
    for got, self_norm, what in ((o8, False, "fp8"), (o8n, True, "fp8 no LSE")):
        bnd, e_lse = fp8_bound(deq[0], deq[1], deq[2], masks[0], 128, scale, list(range(nB)), self_norm=self_norm)
        g = to_np(got[0, 0])
        assert np.all(np.isfinite(g)), what
        worst = float(np.max(np.abs(g - ref8) / bnd))
        assert worst <= 1.0, f"reference {order} ({what}): error reaches {worst:.3f} of the bound"
    assert np.all(np.abs(l8[0, 0].cpu().numpy() - ref8_lse) <= e_lse), f"reference {order}: fp8 lse"


def test_fused_layout_equals_permuted_twins():
    """Layout-1 heads reading Q / V and writing O through the permutation give
    the same bits as the separate svg_permute moves (same arithmetic, only the
    addressing differs); a text tail keeps its rows; LSE stays token-major."""
    banner("attn fused layout")
    F, Hs, Ws, text, D, H = 3, 5, 40, 70, 128, 4
    N = F * Hs * Ws + text
    g = torch.Generator().manual_seed(77)
    q, k, v = (torch.randn(1, H, N, D, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    s = svg.Shape(1, H, N, D, F, Hs, Ws, 128)
    nB = s.n_blocks
    rng = np.random.default_rng(78)
    M = (rng.random((H, nB, nB)) < 0.5).astype(np.uint8)
    M[np.arange(H), :, nB - 1] = 1
    enc = svg.svg_encode_mask(torch.from_numpy(M).to(DEV))
    lay = torch.tensor([0, 1, 1, 0], dtype=torch.int32, device=DEV)
    hm = torch.arange(H, dtype=torch.int32, device=DEV)
    qp, kp, vp = (svg.svg_permute(t, s, lay) for t in (q, k, v))
    o_t, op, lse_t = svg.svg_block_sparse_attn(q, k, v, s, 0.09, enc, head_mask=hm, head_layout=lay,
                                               qp=qp, kp=kp, vp=vp, op=torch.empty_like(q), lse=True)
    svg.svg_permute(op, s, lay, inverse=True, out=o_t)
    o_f, op_f, lse_f = svg.svg_block_sparse_attn(q, k, v, s, 0.09, enc, head_mask=hm, head_layout=lay,
                                                 kp=kp, lse=True)
    torch.cuda.synchronize()
    assert op_f is None
    assert torch.equal(o_t, o_f)
    assert torch.equal(lse_t, lse_f)


def test_many_small_heads_through_the_work_queues():
    """300 heads of 700 tokens (3 pairs of query blocks each, 900 work items
    for 256 persistent workgroups): every XCD's queue drains and the
    workgroups take items from the other queues; sampled heads against the
    oracle, and a second call gives the same bits."""
    banner("attn many small heads")
    H, N, D = 300, 700, 64
    g = torch.Generator().manual_seed(91)
    q, k, v = (torch.randn(1, H, N, D, generator=g).to(torch.bfloat16) for _ in range(3))
    s = svg.Shape(1, H, N, D, 1, 1, N, 128)
    nB = s.n_blocks
    rng = np.random.default_rng(92)
    M = (rng.random((7, nB, nB)) < 0.6).astype(np.uint8)
    M[:, :, 0] = 1
    enc = svg.svg_encode_mask(torch.from_numpy(M).to(DEV))
    hm = torch.from_numpy(rng.integers(0, 7, H).astype(np.int32)).to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, _, lse1 = svg.svg_block_sparse_attn(qd, kd, vd, s, 0.125, enc, head_mask=hm, lse=True)
    o2, _, lse2 = svg.svg_block_sparse_attn(qd, kd, vd, s, 0.125, enc, head_mask=hm, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2)
    hmn = hm.cpu().numpy()
    for h in [0, 1, 150, 257, 299]:
        ref, ref_lse = O.block_masked_attention(q[0, h].float().numpy(), k[0, h].float().numpy(),
                                                v[0, h].float().numpy(), M[hmn[h]], 128, 0.125)
        assert_attn_close(to_np(o1[0, h]), ref, f"small head {h}")
        assert np.max(np.abs(lse1[0, h].cpu().numpy() - ref_lse)) < LSE_ABS


def test_more_heads_than_the_order_kernels_lds_table():
    """B x H = 2 x 1100 heads (more than the 2048 head ranges the work-list
    kernel keeps in LDS, so it reads them from global memory) of 300 tokens
    in mixed layouts through the fused path: the same bits as the two batch
    rows run as separate calls (1100 heads each, ranges in LDS), and sampled
    heads against the oracle."""
    banner("attn heads past the LDS table")
    B, H, F, Hs, Ws, D = 2, 1100, 3, 10, 10, 64
    N = F * Hs * Ws
    g = torch.Generator().manual_seed(95)
    q, k, v = (torch.randn(B, H, N, D, generator=g).to(torch.bfloat16) for _ in range(3))
    s = svg.Shape(B, H, N, D, F, Hs, Ws, 128)
    s1 = svg.Shape(1, H, N, D, F, Hs, Ws, 128)
    nB = s.n_blocks
    rng = np.random.default_rng(96)
    M = (rng.random((5, nB, nB)) < 0.6).astype(np.uint8)
    M[:, :, 0] = 1
    enc = svg.svg_encode_mask(torch.from_numpy(M).to(DEV))
    hm_np = rng.integers(0, 5, B * H).astype(np.int32)
    lay_np = rng.integers(0, 2, B * H).astype(np.int32)
    hm, lay = torch.from_numpy(hm_np).to(DEV), torch.from_numpy(lay_np).to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    kp = svg.svg_permute(kd, s, lay)
    o, _, lse = svg.svg_block_sparse_attn(qd, kd, vd, s, 0.125, enc, head_mask=hm, head_layout=lay,
                                          kp=kp, lse=True)
    torch.cuda.synchronize()
    for b in range(B):
        sl = slice(b * H, (b + 1) * H)
        ob, _, lseb = svg.svg_block_sparse_attn(qd[b:b + 1], kd[b:b + 1], vd[b:b + 1], s1, 0.125, enc,
                                                head_mask=hm[sl].contiguous(),
                                                head_layout=lay[sl].contiguous(),
                                                kp=kp[b:b + 1].contiguous(), lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o[b], ob[0]), f"batch row {b}"
        assert torch.equal(lse[b], lseb[0]), f"batch row {b} lse"
    perm = O.token_major_index(F, Hs, Ws, N)
    sample = []   # per batch row and layout, the first and the last such head
    for b in range(B):
        for layout in (0, 1):
            hs = np.flatnonzero(lay_np[b * H:(b + 1) * H] == layout)
            sample += [(b, int(hs[0])), (b, int(hs[-1]))]
    for b, h in sample:
        i = b * H + h
        ref, ref_lse = O.head_attention(q[b, h].float().numpy(), k[b, h].float().numpy(),
                                        v[b, h].float().numpy(), M[hm_np[i]], int(lay_np[i]), F, Hs, Ws,
                                        128, 0.125)
        assert_attn_close(to_np(o[b, h]), ref, f"head ({b}, {h}) layout {lay_np[i]}")
        got_lse = lse[b, h].cpu().numpy()          # in the layout the head attends in
        if lay_np[i]:
            got_lse = got_lse[perm]
        assert np.max(np.abs(got_lse - ref_lse)) < LSE_ABS


def test_fused_layout_batch2_mixed_layouts():
    """B = 2 with a text tail and per-(batch, head) layouts: the fused layout
    gives the bits of the separate permutation moves."""
    banner("attn fused layout batch2")
    B, H, F, Hs, Ws, text, D = 2, 3, 4, 6, 24, 33, 128
    N = F * Hs * Ws + text
    g = torch.Generator().manual_seed(93)
    q, k, v = (torch.randn(B, H, N, D, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    s = svg.Shape(B, H, N, D, F, Hs, Ws, 128)
    nB = s.n_blocks
    rng = np.random.default_rng(94)
    M = (rng.random((2, nB, nB)) < 0.5).astype(np.uint8)
    M[:, :, nB - 1] = 1
    enc = svg.svg_encode_mask(torch.from_numpy(M).to(DEV))
    lay = torch.tensor([1, 0, 1, 1, 1, 0], dtype=torch.int32, device=DEV)
    qp, kp, vp = (svg.svg_permute(t, s, lay) for t in (q, k, v))
    o_t, op, lse_t = svg.svg_block_sparse_attn(q, k, v, s, 0.09, enc, head_mask=lay, head_layout=lay,
                                               qp=qp, kp=kp, vp=vp, op=torch.empty_like(q), lse=True)
    svg.svg_permute(op, s, lay, inverse=True, out=o_t)
    o_f, _, lse_f = svg.svg_block_sparse_attn(q, k, v, s, 0.09, enc, head_mask=lay, head_layout=lay,
                                              kp=kp, lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_t, o_f)
    assert torch.equal(lse_t, lse_f)


@pytest.mark.parametrize("D", [128, 64])
def test_prepare_kv_bit_exact(D):
    """svg_prepare_kv: every head's V block-transposed in its layout (keys past
    N zero) and the layout-1 heads' K token-major, against the oracle's
    permutation; K rows of layout-0 heads are left untouched."""
    banner("prepare kv", D)
    B, H, F, Hs, Ws, text = 2, 3, 5, 6, 22, 41
    N = F * Hs * Ws + text
    g = torch.Generator().manual_seed(95)
    k, v = (torch.randn(B, H, N, D, generator=g).to(torch.bfloat16) for _ in range(2))
    s = svg.Shape(B, H, N, D, F, Hs, Ws, 128)
    nB = s.n_blocks
    lay = torch.tensor([1, 0, 1, 0, 0, 1], dtype=torch.int32)
    kp = torch.full((B, H, N, D), 7.0, dtype=torch.bfloat16, device=DEV)
    kp_out, vt = svg.svg_prepare_kv(k.to(DEV), v.to(DEV), s, head_layout=lay.to(DEV), kp=kp)
    torch.cuda.synchronize()
    assert kp_out is kp
    vt = vt.view(B * H, nB, D, 128).cpu()
    for b in range(B):
        for h in range(H):
            bh = b * H + h
            kn, vn = k[b, h].float().numpy(), v[b, h].float().numpy()
            if lay[bh]:
                kn, vn = O.to_token_major(kn, F, Hs, Ws), O.to_token_major(vn, F, Hs, Ws)
                assert np.array_equal(kp[b, h].float().cpu().numpy(), kn)
            else:
                assert torch.all(kp[b, h] == 7.0)
            pad = np.zeros((nB * 128, D), np.float32)
            pad[:N] = vn
            want = pad.reshape(nB, 128, D).transpose(0, 2, 1)
            assert np.array_equal(vt[bh].float().numpy(), want), f"vt of head {bh}"


@pytest.mark.parametrize("layouts", [(0, 0, 0), (1, 0, 1)])
def test_given_vt_equals_internal_layout(layouts):
    """The attention on the caller's V^T (svg_prepare_kv) gives the bits of the
    call that lays V out itself; v is not needed then."""
    banner("attn vt given", layouts)
    H, F, Hs, Ws, text, D = 3, 4, 8, 30, 19, 128
    N = F * Hs * Ws + text
    g = torch.Generator().manual_seed(96)
    q, k, v = (torch.randn(1, H, N, D, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    s = svg.Shape(1, H, N, D, F, Hs, Ws, 128)
    nB = s.n_blocks
    rng = np.random.default_rng(97)
    M = (rng.random((H, nB, nB)) < 0.4).astype(np.uint8)
    M[:, :, 0] = 1
    enc = svg.svg_encode_mask(torch.from_numpy(M).to(DEV))
    hm = torch.arange(H, dtype=torch.int32, device=DEV)
    lay = torch.tensor(layouts, dtype=torch.int32, device=DEV)
    kp, vt = svg.svg_prepare_kv(k, v, s, head_layout=lay)
    o1, _, l1 = svg.svg_block_sparse_attn(q, k, v, s, 0.1, enc, head_mask=hm, head_layout=lay, kp=kp,
                                          lse=True)
    o2, _, l2 = svg.svg_block_sparse_attn(q, k, None, s, 0.1, enc, head_mask=hm, head_layout=lay, kp=kp,
                                          lse=True, vt=vt)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
