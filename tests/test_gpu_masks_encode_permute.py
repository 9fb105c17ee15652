"""GPU parity, bit-exact: candidate masks, mask encoding, layout permutation,
calibrated masks, anchor-row restriction and row broadcast."""
import numpy as np
import pytest
import torch

import block_sparse_attention_svg_amd as svg
import oracle as O
import synth as S
from parity_utils import banner

pytestmark = pytest.mark.gpu
DEV = "cuda"
ONLINE = ["tiny", "cogvideox", "wan720p", "hunyuan720p"]


def shape_of(w, H=None):
    return svg.Shape(w.B, H or w.H, w.N, w.D, w.F, w.Hs, w.Ws, w.block)


@pytest.mark.parametrize("name", ONLINE)
def test_build_masks_bit_exact(name):
    w = S.get_workload(name)
    banner("build_masks", name)
    gpu = svg.svg_build_masks(shape_of(w), w.band_w).cpu().numpy()
    ref = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    assert np.array_equal(gpu, ref)


def _check_encoded(enc, ref_masks):
    bm, rp, iv = O.encode_masks(ref_masks)
    torch.cuda.synchronize()
    g_bm = enc.bitmap.cpu().numpy().view(np.uint32)
    g_rp = enc.row_ptr.cpu().numpy()
    assert np.array_equal(g_bm, bm)
    assert np.array_equal(g_rp, rp)
    n = int(g_rp[-1])
    assert np.array_equal(enc.iv[:n].cpu().numpy(), iv)


@pytest.mark.parametrize("name", ONLINE)
def test_encode_online_masks(name):
    w = S.get_workload(name)
    banner("encode online", name)
    dense = svg.svg_build_masks(shape_of(w), w.band_w)
    enc = svg.svg_encode_mask(dense)
    _check_encoded(enc, O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w))


@pytest.mark.parametrize("shape,p", [((3, 17, 70), 0.5), ((2, 5, 64), 0.1), ((1, 40, 33), 0.9),
                                     ((2, 9, 32), 0.0), ((1, 3, 1), 1.0), ((1, 7, 129), 0.97),
                                     ((40, 591, 591), 0.3)])
def test_encode_random(shape, p):
    banner("encode random", shape, p)
    M = (np.random.default_rng(sum(shape)).random(shape) < p).astype(np.uint8)
    enc = svg.svg_encode_mask(torch.from_numpy(M).to(DEV))
    _check_encoded(enc, M)


def test_encode_alternating_worst_case():
    banner("encode alternating")
    M = np.zeros((2, 3, 71), np.uint8)
    M[..., ::2] = 1
    enc = svg.svg_encode_mask(torch.from_numpy(M).to(DEV))
    _check_encoded(enc, M)
    assert enc.n_intervals() == svg.svg_encode_iv_capacity(2, 3, 71)


@pytest.mark.parametrize("name,dtype", [("tiny", "f32"), ("tiny", "bf16"), ("cogvideox", "bf16"),
                                        ("hunyuan720p", "bf16")])
def test_permute_bit_exact(name, dtype, workload_inputs):
    banner("permute", name, dtype)
    w, q, _, _, _ = workload_inputs(name, dtype=dtype)
    s = shape_of(w)
    x = q.to(DEV)
    H = w.H
    sel = torch.tensor([(h % 3) != 1 for h in range(H)], dtype=torch.int32, device=DEV)
    sentinel = torch.full_like(x, 7.0)
    y = svg.svg_permute(x, s, sel, inverse=False, out=sentinel.clone())
    xr = q.float().numpy() if dtype == "bf16" else q.numpy()
    ref_y = O.to_token_major(xr, w.F, w.Hs, w.Ws)
    yn = y.float().cpu().numpy()
    for h in range(H):
        if sel[h]:
            assert np.array_equal(yn[0, h], ref_y[0, h]), h
        else:
            assert np.all(yn[0, h] == 7.0), h
    back = svg.svg_permute(y, s, sel, inverse=True, out=sentinel.clone())
    bn = back.float().cpu().numpy()
    for h in range(H):
        if sel[h]:
            assert np.array_equal(bn[0, h], xr[0, h]), h
    # no selection array: every head
    y_all = svg.svg_permute(x, s, None)
    assert torch.equal(y_all.cpu(), torch.from_numpy(ref_y).to(q.dtype))


def test_permute_full_wan_bit_exact(workload_inputs):
    banner("permute wan720p full")
    w, q, _, _, cls = workload_inputs("wan720p")
    s = shape_of(w)
    sel = torch.from_numpy(cls.astype(np.int32)).to(DEV)
    y = svg.svg_permute(q.to(DEV), s, sel)
    p = O.token_major_index(w.F, w.Hs, w.Ws, w.N)
    yc = y.cpu()
    for h in np.nonzero(cls)[0][:4]:
        assert torch.equal(yc[0, h][torch.from_numpy(p)], q[0, h])


def test_calibrate_static_bit_exact():
    w = S.get_workload("static_wan720p")
    banner("calibrate", w.name)
    E = np.stack([S.energy_matrix(w, h) for h in range(w.H)])
    gpu = svg.svg_calibrate_masks(torch.from_numpy(E).to(DEV), w.eps).cpu().numpy()
    for h in range(w.H):
        assert np.array_equal(gpu[h], O.calibrate_mask(E[h], w.eps)), h
    assert abs(gpu.mean() - 0.32) < 0.01


def test_calibrate_edge_cases():
    banner("calibrate edges")
    rng = np.random.default_rng(9)
    E = rng.random((3, 5, 37))
    E[0, 0] = 1.0                       # all ties: smaller index first
    E[1, 1] = 0.0
    E[1, 1, 3] = 2.0                    # single positive block
    for eps in (1e-9, 0.5, 0.9, 1.0):
        gpu = svg.svg_calibrate_masks(torch.from_numpy(E).to(DEV), eps).cpu().numpy()
        for m in range(3):
            assert np.array_equal(gpu[m], O.calibrate_mask(E[m], eps)), (eps, m)


def test_restrict_anchor_rows_bit_exact():
    w = S.get_workload("static_wan720p")
    banner("restrict anchors", w.name)
    s = shape_of(w)
    rng = np.random.default_rng(3)
    M = (rng.random((4, w.n_blocks, w.n_blocks)) < 0.3).astype(np.uint8)
    sel = np.array([1, 0, 1, 0], np.int32)
    g = torch.from_numpy(M).to(DEV)
    svg.svg_restrict_anchor_rows(g, s, torch.from_numpy(sel).to(DEV), w.k_anchors)
    gn = g.cpu().numpy()
    for m in range(4):
        ref = O.restrict_to_anchor_blocks(M[m], w.F, w.Hs, w.Ws, w.N, w.block, w.k_anchors) if sel[m] else M[m]
        assert np.array_equal(gn[m], ref), m


@pytest.mark.parametrize("k", [5, 1, 45])
def test_row_broadcast_bit_exact(k):
    w = S.get_workload("static_wan720p")
    banner("row broadcast", k)
    H = 3
    s = shape_of(w, H)
    o = torch.randn((1, H, w.N, w.D), generator=torch.Generator().manual_seed(k)).to(torch.bfloat16)
    sel = torch.tensor([1, 0, 1], dtype=torch.int32)
    g = o.to(DEV)
    svg.svg_row_broadcast(g, s, sel.to(DEV), k)
    gn = g.float().cpu().numpy()
    on = o.float().numpy()
    for h in range(H):
        ref = O.row_broadcast(on[0, h], w.F, w.Hs, w.Ws, k) if sel[h] else on[0, h]
        assert np.array_equal(gn[0, h], ref), h
