"""GPU parity of svg_qk_norm_rope (QK-Norm + 3D RoPE into per-head layouts)
against the fp64 oracle, through the C ABI.

Tolerance, from the arithmetic: the kernel works in fp32 from the exact bf16
inputs and rounds once to bf16 (half an ulp, 2^-9 relative).  Its fp32
errors — the sum of squares over at most 8192 terms, rsqrt, the angle
pos * freq (<= 80 rad, relative 2^-24) and sincosf — stay below 1e-5 of a
pair's magnitude, which can move the final rounding across one boundary:
|y_gpu - y| <= 2^-8 |y| + 1e-4 * max(1, max |gamma|) for values of RMS about
max |gamma|.  With neither norm nor rotation the call is a move: bit-exact."""
import numpy as np
import pytest
import torch

import block_sparse_attention_svg_amd as svg
import oracle as O
import synth as S

pytestmark = pytest.mark.gpu

RTOL = 2.0 ** -8


def _check(got, want, gmax):
    got = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - want)
    lim = RTOL * np.abs(want) + 1e-4 * max(1.0, gmax)
    bad = err > lim
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} outside the bound; worst excess "
                           f"{float((err - lim).max()):.3g} at {np.unravel_index(np.argmax(err - lim), err.shape)}")


def _case(B, H, D, F, Hs, Ws, text, norm, use_gamma, rope, layout, seed):
    N = F * Hs * Ws + text
    s = svg.Shape(B=B, H=H, N=N, D=D, F=F, Hs=Hs, Ws=Ws, block=64)
    x = S.gen_projection_rows(B, N, H, D, seed=seed).cuda()
    gamma = None
    if norm is not None and use_gamma:
        gamma = S.gen_norm_weight(D if norm == "head" else H * D, seed + 1)
    lay = None
    if layout == "mixed":
        lay = (np.arange(B * H) % 3 == 1).astype(np.int32)
    elif layout == "tm":
        lay = np.ones(B * H, np.int32)
    y = svg.svg_qk_norm_rope(
        x, s, norm=norm, gamma=None if gamma is None else torch.from_numpy(gamma).cuda(), eps=1e-6,
        rope=rope, head_layout=None if lay is None else torch.from_numpy(lay).cuda())
    torch.cuda.synchronize()
    want = O.qk_norm_rope(x.float().cpu().numpy(), F, Hs, Ws, norm, gamma, 1e-6, rope, lay)
    return y, want, 1.0 if gamma is None else float(np.max(np.abs(gamma)))


@pytest.mark.parametrize("norm", [None, "head", "row"])
@pytest.mark.parametrize("use_gamma", [False, True])
@pytest.mark.parametrize("layout", [None, "mixed", "tm"])
def test_small_d64(norm, use_gamma, layout):
    # N = 3*5*7 + 9 = 114: the last workgroup holds 2 of its 4 tokens
    y, want, gmax = _case(2, 3, 64, 3, 5, 7, 9, norm, use_gamma, (16, 24, 24, 10000.0), layout, 11)
    _check(y, want, gmax)


@pytest.mark.parametrize("H,D,rope", [
    (40, 128, (44, 42, 42, 10000.0)),   # Wan-like head split, 10 waves per workgroup
    (24, 128, (16, 56, 56, 256.0)),     # HunyuanVideo-like split
    (48, 64, (0, 32, 32, 10000.0)),     # no frame run
    (64, 128, (128, 0, 0, 10000.0)),    # 1024 threads, frame run only
    (5, 64, (20, 22, 22, 10000.0)),     # 40 active threads in one 64-lane wave
    (128, 64, (24, 20, 20, 10000.0)),   # H*D = 8192, the largest row: 1024 threads
])
@pytest.mark.parametrize("norm", ["head", "row"])
def test_head_counts_and_splits(H, D, rope, norm):
    y, want, gmax = _case(1, H, D, 2, 3, 8, 5, norm, True, rope, "mixed", 12)
    _check(y, want, gmax)


def test_three_batch_rows_per_row_layouts():
    # B = 3: the grid's second dimension; layouts differ per (batch, head)
    y, want, gmax = _case(3, 4, 128, 2, 3, 5, 2, "row", True, (44, 42, 42, 10000.0), "mixed", 22)
    _check(y, want, gmax)


def test_no_rope_and_move_only():
    y, want, gmax = _case(1, 4, 128, 2, 4, 6, 3, "head", True, None, "mixed", 13)
    _check(y, want, gmax)
    # neither norm nor rotation: an exact transpose into the layouts
    y, want, _ = _case(2, 4, 128, 2, 4, 6, 3, None, False, None, "mixed", 14)
    assert np.array_equal(y.float().cpu().numpy().astype(np.float64), want)


def test_single_token_and_text_only_tail():
    # N = 1 video token; and a grid of one frame with a long text tail
    y, want, gmax = _case(1, 2, 64, 1, 1, 1, 0, "head", True, (0, 32, 32, 10000.0), "tm", 15)
    _check(y, want, gmax)
    y, want, gmax = _case(1, 2, 64, 1, 2, 2, 33, "row", True, (16, 24, 24, 10000.0), "mixed", 16)
    _check(y, want, gmax)


def test_deterministic_and_output_rows_covered():
    s = svg.Shape(B=1, H=8, N=2 * 4 * 6 + 7, D=128, F=2, Hs=4, Ws=6, block=64)
    x = S.gen_projection_rows(1, s.N, 8, 128, seed=17).cuda()
    lay = torch.tensor([0, 1] * 4, dtype=torch.int32, device="cuda")
    a = torch.full((1, 8, s.N, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    svg.svg_qk_norm_rope(x, s, norm="row", rope=(44, 42, 42, 10000.0), head_layout=lay, out=a)
    b = svg.svg_qk_norm_rope(x, s, norm="row", rope=(44, 42, 42, 10000.0), head_layout=lay)
    torch.cuda.synchronize()
    assert not torch.isnan(a).any(), "every output row is written"
    assert torch.equal(a, b)


def test_wan_size_sampled_rows():
    """Wan 2.1 720p: B=1, N = 21*45*80 = 75600 tokens, 40 heads of 128 with the
    whole-row norm; 16 temporal heads written token-major.  The oracle checks
    sampled tokens (every head) one by one."""
    F, Hs, Ws, H, D = 21, 45, 80, 40, 128
    N = F * Hs * Ws
    s = svg.Shape(B=1, H=H, N=N, D=D, F=F, Hs=Hs, Ws=Ws, block=128)
    x = S.gen_projection_rows(1, N, H, D, seed=18, device="cuda")
    gamma = S.gen_norm_weight(H * D, 19)
    lay = np.zeros(H, np.int32)
    lay[np.random.default_rng(20).choice(H, 16, replace=False)] = 1
    rope = (44, 42, 42, 10000.0)
    y = svg.svg_qk_norm_rope(x, s, norm="row", gamma=torch.from_numpy(gamma).cuda(), eps=1e-6, rope=rope,
                             head_layout=torch.from_numpy(lay).cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(21)
    toks = np.unique(np.concatenate([[0, 1, Ws, Hs * Ws, N - 1], rng.choice(N, 250, replace=False)]))
    xs = x[0, torch.from_numpy(toks).cuda()].float().cpu().numpy().astype(np.float64)  # [T, H, D]
    normed = O.rms_norm(xs, gamma, 1e-6, "row")
    ang = O.rope_angles(F, Hs, Ws, N, rope[:3], rope[3])[toks]
    want = O.rope_rotate(np.transpose(normed, (1, 0, 2)), ang)  # [H, T, D]
    p = O.token_major_index(F, Hs, Ws, N)
    rows = np.where(lay[:, None] == 1, p[toks][None, :], toks[None, :])  # [H, T]
    got = y[0][torch.arange(H)[:, None].cuda(), torch.from_numpy(rows).cuda()]
    _check(got, want, float(np.max(gamma)))


def test_layer_prepare_inputs_then_attention():
    """OnlineSparseAttention.prepare_inputs: q, k through norm + rotation, v
    moved bit-exactly; the layer then runs on them like on any q, k, v."""
    w = S.get_workload("tiny")
    s = svg.Shape(w.B, w.H, w.N, w.D, w.F, w.Hs, w.Ws, w.block)
    xq, xk, xv = (S.gen_projection_rows(w.B, w.N, w.H, w.D, seed=30 + i).cuda() for i in range(3))
    gq, gk = (torch.from_numpy(S.gen_norm_weight(w.H * w.D, 40 + i)).cuda() for i in range(2))
    rope = (24, 20, 20, 10000.0)
    layer = svg.OnlineSparseAttention(s, w.band_w)
    q, k, v = layer.prepare_inputs(xq, xk, xv, norm="row", gamma_q=gq, gamma_k=gk, rope=rope)
    torch.cuda.synchronize()
    for t, x_, g_ in ((q, xq, gq), (k, xk, gk)):
        want = O.qk_norm_rope(x_.float().cpu().numpy(), w.F, w.Hs, w.Ws, "row", g_.cpu().numpy(), 1e-6, rope)
        _check(t, want, float(g_.max()))
    assert torch.equal(v, xv.transpose(1, 2).contiguous())
    idx = torch.from_numpy(S.sample_query_idx(w)).cuda()
    o, _ = layer(q, k, v, idx)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()


def test_any_nonzero_layout_is_token_major():
    """head_layout follows the attention's convention: any nonzero entry means
    token-major, so a layout array holding 2 or -1 gives the bits of 1."""
    B, H, D, F, Hs, Ws, text = 1, 4, 128, 3, 6, 10, 5
    N = F * Hs * Ws + text
    s = svg.Shape(B=B, H=H, N=N, D=D, F=F, Hs=Hs, Ws=Ws, block=128)
    x = S.gen_projection_rows(B, N, H, D, seed=23).cuda()
    rope = (44, 42, 42, 10000.0)
    odd = torch.tensor([0, 2, -1, 1], dtype=torch.int32, device="cuda")
    ones = torch.tensor([0, 1, 1, 1], dtype=torch.int32, device="cuda")
    y_odd = svg.svg_qk_norm_rope(x, s, norm="head", rope=rope, head_layout=odd)
    y_one = svg.svg_qk_norm_rope(x, s, norm="head", rope=rope, head_layout=ones)
    torch.cuda.synchronize()
    assert torch.equal(y_odd, y_one)
    want = O.qk_norm_rope(x.float().cpu().numpy(), F, Hs, Ws, "head", None, 1e-6, rope,
                          odd.cpu().numpy())
    _check(y_odd, want, 1.0)
