"""GPU parity of the static calibrated-mask layer's masks (Wan 720p shape, 40
heads, eps = 0.9 energy-threshold masks, 5 row-repetitive heads with 5 anchor
rows): the calibrated masks against the oracle's, the anchor restriction.  The
layer's outputs on every head are in test_gpu_full_size.py."""
import numpy as np
import pytest
import torch

import block_sparse_attention_svg_amd as svg
import oracle as O
import synth as S
from parity_utils import banner

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_static_layer_masks(workload_inputs):
    banner("static layer masks")
    w = S.get_workload("static_wan720p")
    s = svg.Shape(w.B, w.H, w.N, w.D, w.F, w.Hs, w.Ws, w.block)
    E = np.stack([S.energy_matrix(w, h) for h in range(w.H)])
    dense = svg.svg_calibrate_masks(torch.from_numpy(E).to(DEV), w.eps)
    rep = S.repetitive_heads(w)
    sel = np.zeros(w.H, np.int32)
    sel[rep] = 1
    layer = svg.StaticSparseAttention(s, dense, torch.from_numpy(sel).to(DEV), w.k_anchors)
    torch.cuda.synchronize()
    masks = dense.cpu().numpy()
    # the calibrated masks themselves are bit-exact with the oracle, every head
    for h in range(w.H):
        assert np.array_equal(masks[h], O.calibrate_mask(E[h], w.eps))
    # the restricted masks keep exactly the 158 anchor-holding query blocks
    kept_rows = (layer.masks.row_ptr[1:] - layer.masks.row_ptr[:-1]).cpu().numpy().reshape(w.H, -1) > 0
    assert kept_rows[rep].sum(axis=1).tolist() == [158] * len(rep)
