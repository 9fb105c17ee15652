"""GPU parity of the FP8 (E4M3) variant ([CalibAtt] section 3.3: FP8 on the
critical path).

svg_quantize_fp8: the codes of q, k, v in their layouts and the per-head
dequantization factors are bit-exact against oracle.fp8 (an integer decided
in fp32 on both sides).  svg_block_sparse_attn_fp8: every element within the
bound fp8_bound derives from the format (E4M3 weights, the FP8 product's
accumulation, bf16 output) against the unchanged oracle attention on the
oracle's dequantized inputs; its distance from the bf16 result is printed.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_svg_amd as svg
import oracle as O
import synth as S
from parity_utils import banner, fp8_bound, attn_errors, to_np, sample_qblocks

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _head_codes(x, layout, F, Hs, Ws):
    """oracle: codes, inv, d, dequantized values of one head [N, D], and the
    same in the head's layout (token-major rows for layout 1)."""
    codes, inv, d, val = O.quantize_head(x)
    if layout:
        return codes, inv, d, O.to_token_major(codes, F, Hs, Ws), O.to_token_major(val, F, Hs, Ws), val
    return codes, inv, d, codes, val, val


def _inputs(B, H, F, Hs, Ws, text, D, seed, spread=1.0):
    N = F * Hs * Ws + text
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn(B, H, N, D, generator=g) * spread for _ in range(3))
    q[:, :, :, :8] *= 4.0                      # a few large channels: amax well above the bulk
    return svg.Shape(B, H, N, D, F, Hs, Ws, 128), q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


@pytest.mark.parametrize("D", [128, 64])
def test_quantize_fp8_bit_exact(D):
    banner("fp8 quantize", D)
    B, H, F, Hs, Ws, text = 2, 3, 5, 6, 22, 41
    s, q, k, v = _inputs(B, H, F, Hs, Ws, text, D, 201)
    k[1, 2] = 0                                # an all-zero head: factor 1, codes 0
    lay = torch.tensor([1, 0, 1, 0, 0, 1], dtype=torch.int32)
    ops8 = svg.svg_quantize_fp8(q.to(DEV), k.to(DEV), v.to(DEV), s, head_layout=lay.to(DEV))
    torch.cuda.synchronize()
    q8, k8 = ops8.q8.cpu().numpy(), ops8.k8.cpu().numpy()
    vt8 = ops8.vt8.cpu().numpy().reshape(B * H, s.n_blocks, D, 128)
    sc = ops8.scales.cpu().numpy()
    for b in range(B):
        for h in range(H):
            bh = b * H + h
            for t, (x, got) in enumerate(((q, q8[b, h]), (k, k8[b, h]), (v, None))):
                xs = x[b, h].float().numpy()
                codes, inv, d = O.quantize_head(xs)[:3]
                assert sc[t, bh].view(np.uint32) == np.float32(d).view(np.uint32), (t, bh)
                lay_codes = O.to_token_major(codes, F, Hs, Ws) if (lay[bh] and t > 0) else codes
                if t < 2:
                    assert np.array_equal(got, lay_codes), f"tensor {t} head {bh}"
                else:
                    assert np.array_equal(vt8[bh], O.vt8_blocks(lay_codes)), f"vt8 head {bh}"


def _run_fp8(s, q, k, v, M, lay, hm, lse=True):
    enc = svg.svg_encode_mask(torch.from_numpy(M).to(DEV))
    layd = torch.from_numpy(lay).to(DEV)
    hmd = torch.from_numpy(hm).to(DEV)
    ops8 = svg.svg_quantize_fp8(q.to(DEV), k.to(DEV), v.to(DEV), s, head_layout=layd)
    o8, l8 = svg.svg_block_sparse_attn_fp8(ops8, s, 1.0 / np.sqrt(s.D), enc, head_mask=hmd, head_layout=layd,
                                           lse=lse)
    # without the LSE (the denominator is then the matrix core's sum of the
    # E4M3 weights)
    o8n, _ = svg.svg_block_sparse_attn_fp8(ops8, s, 1.0 / np.sqrt(s.D), enc, head_mask=hmd, head_layout=layd)
    # the bf16 path on the same inputs, for the reported distance
    kp, vt = svg.svg_prepare_kv(k.to(DEV), v.to(DEV), s, head_layout=layd)
    o16, _, _ = svg.svg_block_sparse_attn(q.to(DEV), k.to(DEV), None, s, 1.0 / np.sqrt(s.D), enc,
                                          head_mask=hmd, head_layout=layd, kp=kp, vt=vt)
    torch.cuda.synchronize()
    return o8.cpu(), None if l8 is None else l8.cpu(), o16.cpu(), o8n.cpu()


def _check_head(s, q, k, v, M, lay, o8, l8, o16, b, h, qblocks=None, what="", o8n=None):
    F, Hs, Ws = s.F, s.Hs, s.Ws
    bh = b * s.H + h
    scale = 1.0 / np.sqrt(s.D)
    deq = [O.quantize_head(x[b, h].float().numpy())[3] for x in (q, k, v)]
    if lay[bh]:
        deq = [O.to_token_major(x, F, Hs, Ws) for x in deq]
    qbs = range(s.n_blocks) if qblocks is None else qblocks
    ref, ref_lse = O.block_masked_attention(deq[0], deq[1], deq[2], M, 128, scale, list(qbs))
    bnd, e_lse = fp8_bound(deq[0], deq[1], deq[2], M, 128, scale, list(qbs))
    p = O.token_major_index(F, Hs, Ws, s.N)
    got = to_np(o8[b, h])
    g_lse = l8[b, h].numpy()
    if lay[bh]:                       # o is frame-major, lse in the attended layout
        got = got[np.argsort(p)]
    rows = ~np.isnan(ref[:, 0])
    err = np.abs(got[rows] - ref[rows])
    worst = float(np.max(err / bnd[rows]))
    fin = np.isfinite(ref_lse[rows])
    le = float(np.max(np.abs(g_lse[rows][fin] - ref_lse[rows][fin]) / e_lse[rows][fin])) if fin.any() else 0.0
    mx16, rl16 = attn_errors(to_np(o8[b, h]), to_np(o16[b, h]).astype(np.float64))
    print(f"[fp8] {what} head {bh} (layout {lay[bh]}): worst error / bound {worst:.3f}, lse / bound {le:.3f}; "
          f"vs bf16 path max-abs {mx16:.3e} rel-L2 {rl16:.3e}")
    assert worst <= 1.0, f"{what} head {bh}: error reaches {worst:.3f} of the bound"
    assert le <= 1.0, f"{what} head {bh}: lse error reaches {le:.3f} of the bound"
    assert np.array_equal(np.isneginf(g_lse[rows]), np.isneginf(ref_lse[rows]))
    if o8n is not None:
        got_n = to_np(o8n[b, h])
        bnd_n, _ = fp8_bound(deq[0], deq[1], deq[2], M, 128, scale, list(qbs), self_norm=True)
        if lay[bh]:
            got_n = got_n[np.argsort(p)]
        worst_n = float(np.max(np.abs(got_n[rows] - ref[rows]) / bnd_n[rows]))
        print(f"[fp8] {what} head {bh}: no-LSE call (E4M3-weight denominator) worst error / bound {worst_n:.3f}")
        assert worst_n <= 1.0, f"{what} head {bh} (no LSE): error reaches {worst_n:.3f} of the bound"


@pytest.mark.parametrize("D", [128, 64])
def test_fp8_attention_within_derived_bound(D):
    """Random masks with an empty row and a dense row, ragged last block, text
    tail, mixed layouts, B = 2; every row of every head."""
    banner("fp8 attention", D)
    B, H, F, Hs, Ws, text = 2, 3, 4, 8, 30, 37
    s, q, k, v = _inputs(B, H, F, Hs, Ws, text, D, 202)
    nB = s.n_blocks
    rng = np.random.default_rng(203)
    M = (rng.random((B * H, nB, nB)) < 0.4).astype(np.uint8)
    M[:, :, nB - 1] = 1
    M[1, 3] = 0
    M[2, 5] = 1
    lay = np.array([0, 1, 1, 0, 1, 0], np.int32)
    hm = np.arange(B * H, dtype=np.int32)
    o8, l8, o16, o8n = _run_fp8(s, q, k, v, M, lay, hm)
    for b in range(B):
        for h in range(H):
            _check_head(s, q, k, v, M[b * H + h], lay, o8, l8, o16, b, h, what=f"D{D}", o8n=o8n)


def test_fp8_generator_heads_wan_shape_sampled():
    """Spatial and temporal heads of the synthetic generator at the Wan 720p
    token count (4 heads), through the FP8 path with their online masks;
    32 query blocks per head against the bound."""
    banner("fp8 wan heads")
    w = S.get_workload("wan720p", H=4, n_spatial=2)
    q, k, v, cls = S.gen_qkv(w, dtype="bf16")
    s = svg.Shape(w.B, w.H, w.N, w.D, w.F, w.Hs, w.Ws, w.block)
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    lay = cls.astype(np.int32)
    o8, l8, o16, o8n = _run_fp8(s, q, k, v, cand, lay, lay.copy())
    for h in range(w.H):
        qbs = sample_qblocks(w.n_blocks, seed=300 + h)
        _check_head(s, q, k, v, cand[lay[h]], lay, o8, l8, o16, 0, h, qblocks=qbs, what="wan", o8n=o8n)


def test_fp8_generator_heads_cogvideox_shape_sampled():
    """Spatial and temporal heads of the synthetic generator at the CogVideoX
    shape (D = 64, 4 heads) through the FP8 path with their online masks, with
    and without the LSE; 32 query blocks per head against the bounds."""
    banner("fp8 cogvideox heads")
    w = S.get_workload("cogvideox", H=4, n_spatial=2)
    q, k, v, cls = S.gen_qkv(w, dtype="bf16")
    s = svg.Shape(w.B, w.H, w.N, w.D, w.F, w.Hs, w.Ws, w.block)
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    lay = cls.astype(np.int32)
    o8, l8, o16, o8n = _run_fp8(s, q, k, v, cand, lay, lay.copy())
    for h in range(w.H):
        qbs = sample_qblocks(w.n_blocks, seed=310 + h)
        _check_head(s, q, k, v, cand[lay[h]], lay, o8, l8, o16, 0, h, qblocks=qbs, what="cogvideox", o8n=o8n)
