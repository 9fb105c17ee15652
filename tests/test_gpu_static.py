"""GPU parity of the static calibrated-mask layer (Wan 720p shape, 40 heads,
eps = 0.9 energy-threshold masks, 5 row-repetitive heads with 5 anchor rows).
Sampled outputs against the float64 oracle; repetitive heads on whole frames."""
import numpy as np
import pytest
import torch

import block_sparse_attention_svg_amd as svg
import oracle as O
import synth as S
from parity_utils import banner, assert_attn_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_static_layer_sampled(workload_inputs):
    banner("static layer")
    w, q, k, v, _ = workload_inputs("static_wan720p")
    s = svg.Shape(w.B, w.H, w.N, w.D, w.F, w.Hs, w.Ws, w.block)
    E = np.stack([S.energy_matrix(w, h) for h in range(w.H)])
    dense = svg.svg_calibrate_masks(torch.from_numpy(E).to(DEV), w.eps)
    rep = S.repetitive_heads(w)
    sel = np.zeros(w.H, np.int32)
    sel[rep] = 1
    layer = svg.StaticSparseAttention(s, dense, torch.from_numpy(sel).to(DEV), w.k_anchors)
    o, _ = layer(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    masks = dense.cpu().numpy()
    # the calibrated masks themselves are bit-exact with the oracle
    for h in (0, int(rep[0])):
        assert np.array_equal(masks[h], O.calibrate_mask(E[h], w.eps))
    # the restricted masks keep exactly the 158 anchor-holding query blocks
    kept_rows = (layer.masks.row_ptr[1:] - layer.masks.row_ptr[:-1]).cpu().numpy().reshape(w.H, -1) > 0
    assert kept_rows[rep].sum(axis=1).tolist() == [158] * len(rep)

    rng = np.random.default_rng(11)
    nB = w.n_blocks
    plain = [h for h in range(w.H) if not sel[h]]
    for h in [plain[0], plain[-1]]:
        qbs = sorted(set([0, nB - 1] + rng.integers(0, nB, 3).tolist()))
        ref, _ = O.block_masked_attention(q[0, h].float().numpy(), k[0, h].float().numpy(),
                                          v[0, h].float().numpy(), masks[h], w.block, w.scale, qbs)
        rows = ~np.isnan(ref[:, 0])
        assert_attn_close(to_np(o[0, h])[rows], ref[rows], f"static head {h}")

    S_ = w.Hs * w.Ws
    anchors = np.unique(O.anchor_rows(w.Hs, w.k_anchors))
    for h in rep[:2]:
        f = int(rng.integers(w.F))
        tok = np.array([f * S_ + a * w.Ws + x for a in anchors for x in range(w.Ws)])
        qbs = np.unique(tok // w.block).tolist()
        ref, _ = O.block_masked_attention(q[0, h].float().numpy(), k[0, h].float().numpy(),
                                          v[0, h].float().numpy(), masks[h], w.block, w.scale, qbs)
        frame = slice(f * S_, (f + 1) * S_)
        full = np.nan_to_num(ref)
        want = O.row_broadcast(full, w.F, w.Hs, w.Ws, w.k_anchors)[frame]
        assert_attn_close(to_np(o[0, h])[frame], want, f"repetitive head {h} frame {f}")
