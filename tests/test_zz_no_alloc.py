"""GPU: the allocation-free attention entry point (svg_block_sparse_attn_noalloc,
work plan in the library's fixed device array) against svg_block_sparse_attn
with a workspace, called through the C ABI.  Two calls in a row on the same
GPU, the second with a smaller input (the array still holds the first call's
plan, which the second must rewrite): outputs and log-sum-exp equal bit for
bit, with and without the LSE.  The caller passes every output, nothing is allocated by the call."""
import numpy as np
import pytest
import torch

import block_sparse_attention_svg_amd as svg
from parity_utils import banner

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, H, F, Hs, Ws, text, D, seed):
    N = F * Hs * Ws + text
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn(B, H, N, D, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    return svg.Shape(B, H, N, D, F, Hs, Ws, 128), q, k, v


def test_noalloc_equals_workspace_call_twice():
    cases = [(2, 5, 7, 16, 40, 53, 128, 101), (1, 3, 3, 8, 20, 7, 64, 102)]   # second call smaller
    for B, H, F, Hs, Ws, text, D, seed in cases:
        banner("noalloc", B, H, F, Hs, Ws, text, D)
        s, q, k, v = _inputs(B, H, F, Hs, Ws, text, D, seed)
        nB = s.n_blocks
        rng = np.random.default_rng(seed)
        M = (rng.random((3, nB, nB)) < 0.35).astype(np.uint8)
        M[:, :, nB - 1] = 1
        M[1, 2] = 0                                   # an empty row
        enc = svg.svg_encode_mask(torch.from_numpy(M).to(DEV))
        hm = torch.from_numpy(rng.integers(0, 3, B * H).astype(np.int32)).to(DEV)
        lay = torch.from_numpy((rng.random(B * H) < 0.5).astype(np.int32)).to(DEV)
        kp, vt = svg.svg_prepare_kv(k, v, s, head_layout=lay)
        o_ref, _, l_ref = svg.svg_block_sparse_attn(q, k, None, s, 0.1, enc, head_mask=hm, head_layout=lay,
                                                    kp=kp, lse=True, vt=vt)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, s.N), dtype=torch.float32, device=DEV)
        svg.svg_block_sparse_attn_noalloc(q, k, None, s, 0.1, enc, head_mask=hm, head_layout=lay, kp=kp,
                                          out=o, lse=lse, vt=vt)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"case {seed}: o differs"
        assert torch.equal(lse, l_ref), f"case {seed}: lse differs"
        # without the LSE (the denominator is then summed on the matrix
        # core): the same kernels behind both entry points
        o2_ref, _, _ = svg.svg_block_sparse_attn(q, k, None, s, 0.1, enc, head_mask=hm, head_layout=lay,
                                                 kp=kp, vt=vt)
        o2 = torch.empty_like(q)
        svg.svg_block_sparse_attn_noalloc(q, k, None, s, 0.1, enc, head_mask=hm, head_layout=lay, kp=kp,
                                          out=o2, vt=vt)
        torch.cuda.synchronize()
        assert torch.equal(o2, o2_ref), f"case {seed}: o without the LSE differs"


def test_noalloc_64_token_blocks():
    """64-token blocks use no scratch; the entry point runs the same kernel."""
    banner("noalloc block 64")
    B, H, F, Hs, Ws, D = 1, 2, 4, 16, 16, 64
    N = F * Hs * Ws
    g = torch.Generator().manual_seed(103)
    q, k, v = (torch.randn(B, H, N, D, generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    s = svg.Shape(B, H, N, D, F, Hs, Ws, 64)
    M = (np.random.default_rng(104).random((2, 16, 16)) < 0.5).astype(np.uint8)
    M[:, :, 0] = 1
    enc = svg.svg_encode_mask(torch.from_numpy(M).to(DEV))
    o_ref, _, l_ref = svg.svg_block_sparse_attn(q, k, v, s, 0.125, enc, lse=True)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    svg.svg_block_sparse_attn_noalloc(q, k, v, s, 0.125, enc, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
