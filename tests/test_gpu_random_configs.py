"""Seeded random configurations through the attention call, every row
against the float64 oracle: batch 1-2, 1-4 heads, D 64 / 128, blocks of 64
and 128 tokens, latent grids from a single token per frame to 23 x 39, one
to six frames, text tails of up to 200 tokens, random masks of any density
(with an empty row, a dense row and a dense last column), mixed layouts.
128-token blocks run the layer's fused flow (svg_prepare_kv, Q and O through
the permutation inside the call), with and without the LSE, and, for D = 128 and 64, the FP8 variant
against its derived bound; 64-token blocks run the token-major twins.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_svg_amd as svg
import oracle as O
from parity_utils import banner, assert_attn_close, to_np, LSE_ABS, fp8_bound

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _config(seed):
    rng = np.random.default_rng(4100 + seed)
    block = (64, 128)[seed % 2]
    D = (64, 128)[(seed // 2) % 2]
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 5))
    F, Hs, Ws = int(rng.integers(1, 7)), int(rng.integers(1, 24)), int(rng.integers(1, 40))
    text = int(rng.integers(1, 201)) if rng.random() < 0.5 else 0
    N = F * Hs * Ws + text
    nB = -(-N // block)
    masks = (rng.random((B * H, nB, nB)) < rng.uniform(0.05, 0.9)).astype(np.uint8)
    if nB > 1:
        masks[:, int(rng.integers(0, nB))] = 0          # an empty row
        masks[:, int(rng.integers(0, nB))] = 1          # a dense row
    masks[:, :, nB - 1] = 1                             # the ragged last key block
    lay = rng.integers(0, 2, B * H).astype(np.int32)
    g = torch.Generator().manual_seed(4200 + seed)
    q, k, v = (torch.randn(B, H, N, D, generator=g).to(torch.bfloat16) for _ in range(3))
    return svg.Shape(B, H, N, D, F, Hs, Ws, block), masks, lay, q, k, v


def _oracle_head(s, q, k, v, M, tm, b, h, deq=None):
    """Oracle attention of one head in its layout, returned frame-major (o)
    and in the attended layout (lse)."""
    xs = deq if deq is not None else [x[b, h].float().numpy() for x in (q, k, v)]
    if tm:
        xs = [O.to_token_major(x, s.F, s.Hs, s.Ws) for x in xs]
    ref, ref_lse = O.block_masked_attention(xs[0], xs[1], xs[2], M, s.block, 1.0 / np.sqrt(s.D))
    if tm:
        ref = ref[O.token_major_index(s.F, s.Hs, s.Ws, s.N)]
    return ref, ref_lse


@pytest.mark.parametrize("seed", range(12))
def test_random_config_matches_oracle(seed):
    s, masks, lay, q, k, v = _config(seed)
    banner("random config", seed, f"B{s.B} H{s.H} N{s.N} D{s.D} block {s.block} F{s.F} {s.Hs}x{s.Ws}")
    enc = svg.svg_encode_mask(torch.from_numpy(masks).to(DEV))
    layd = torch.from_numpy(lay).to(DEV)
    hm = torch.arange(s.B * s.H, dtype=torch.int32, device=DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = 1.0 / np.sqrt(s.D)
    if s.block == 128:
        kp, vt = svg.svg_prepare_kv(kd, vd, s, head_layout=layd)
        o, _, lse = svg.svg_block_sparse_attn(qd, kd, None, s, scale, enc, head_mask=hm, head_layout=layd,
                                              kp=kp, vt=vt, lse=True)
        # without the LSE (the denominator is then summed on the matrix core
        # from the bf16 weights)
        o2, _, _ = svg.svg_block_sparse_attn(qd, kd, None, s, scale, enc, head_mask=hm, head_layout=layd,
                                             kp=kp, vt=vt)
        outs = [o, o2]
    else:
        qp, kp, vp = (svg.svg_permute(t, s, layd) for t in (qd, kd, vd))
        o, op, lse = svg.svg_block_sparse_attn(qd, kd, vd, s, scale, enc, head_mask=hm, head_layout=layd,
                                               qp=qp, kp=kp, vp=vp, op=torch.empty_like(qd), lse=True)
        outs = [o, op]
    torch.cuda.synchronize()
    p = O.token_major_index(s.F, s.Hs, s.Ws, s.N)
    for b in range(s.B):
        for h in range(s.H):
            bh = b * s.H + h
            ref, ref_lse = _oracle_head(s, q, k, v, masks[bh], lay[bh], b, h)
            if s.block == 128 or not lay[bh]:
                got = to_np(outs[0][b, h])
            else:
                got = to_np(outs[1][b, h])[p]
            assert_attn_close(got, ref, f"seed {seed} head {bh}")
            if s.block == 128:
                got2 = to_np(outs[1][b, h])
                assert_attn_close(got2, ref, f"seed {seed} head {bh} (no LSE)")
            g = lse[b, h].cpu().numpy()
            fin = np.isfinite(ref_lse)
            assert np.array_equal(np.isneginf(g), ~fin), f"seed {seed} head {bh}: empty rows"
            if fin.any():
                assert np.max(np.abs(g[fin] - ref_lse[fin])) < LSE_ABS, f"seed {seed} head {bh}: lse"


@pytest.mark.parametrize("seed", [1, 3, 5, 7, 9, 11])
def test_random_config_fp8_within_bound(seed):
    s, masks, lay, q, k, v = _config(seed)
    assert s.block == 128
    banner("random config fp8", seed, f"B{s.B} H{s.H} N{s.N} D{s.D} F{s.F} {s.Hs}x{s.Ws}")
    enc = svg.svg_encode_mask(torch.from_numpy(masks).to(DEV))
    layd = torch.from_numpy(lay).to(DEV)
    hm = torch.arange(s.B * s.H, dtype=torch.int32, device=DEV)
    ops8 = svg.svg_quantize_fp8(q.to(DEV), k.to(DEV), v.to(DEV), s, head_layout=layd)
    o8, l8 = svg.svg_block_sparse_attn_fp8(ops8, s, 1.0 / np.sqrt(s.D), enc, head_mask=hm, head_layout=layd,
                                           lse=True)
    # without the LSE: the denominator is the matrix core's sum of the E4M3
    # weights (its own bound)
    o8n, _ = svg.svg_block_sparse_attn_fp8(ops8, s, 1.0 / np.sqrt(s.D), enc, head_mask=hm, head_layout=layd)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(s.D)
    for b in range(s.B):
        for h in range(s.H):
            bh = b * s.H + h
            deq = [O.quantize_head(x[b, h].float().numpy())[3] for x in (q, k, v)]
            xs = [O.to_token_major(x, s.F, s.Hs, s.Ws) for x in deq] if lay[bh] else deq
            ref, ref_lse = _oracle_head(s, q, k, v, masks[bh], lay[bh], b, h, deq=deq)
            bnd, e_lse = fp8_bound(xs[0], xs[1], xs[2], masks[bh], 128, scale, list(range(s.n_blocks)))
            if lay[bh]:
                bnd = bnd[O.token_major_index(s.F, s.Hs, s.Ws, s.N)]
            got = to_np(o8[b, h])
            rows = ~np.isnan(ref[:, 0])
            worst = float(np.max(np.abs(got[rows] - ref[rows]) / bnd[rows])) if rows.any() else 0.0
            assert worst <= 1.0, f"seed {seed} head {bh}: error reaches {worst:.3f} of the bound"
            got_n = to_np(o8n[b, h])
            bnd_n, _ = fp8_bound(xs[0], xs[1], xs[2], masks[bh], 128, scale, list(range(s.n_blocks)),
                                 self_norm=True)
            if lay[bh]:
                bnd_n = bnd_n[O.token_major_index(s.F, s.Hs, s.Ws, s.N)]
            worst_n = float(np.max(np.abs(got_n[rows] - ref[rows]) / bnd_n[rows])) if rows.any() else 0.0
            assert worst_n <= 1.0, f"seed {seed} head {bh} (no LSE): error reaches {worst_n:.3f} of the bound"
            g = l8[b, h].cpu().numpy()
            fin = np.isfinite(ref_lse)
            assert np.array_equal(np.isneginf(g), ~fin)
            if fin.any():
                assert np.all(np.abs(g[fin] - ref_lse[fin]) <= e_lse[fin]), f"seed {seed} head {bh}: lse"
