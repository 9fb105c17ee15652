"""The C ABI loads, exports every declared symbol and rejects bad arguments
on the host, before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_svg_amd as svg
from block_sparse_attention_svg_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svg.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libsvg.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svg_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 13
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L._SIGS), "binding signatures must cover the header exactly"


def test_version_and_status_strings():
    lib = L.lib()
    assert lib.svg_version().decode().startswith("svg-mi355x")
    assert lib.svg_status_string(L.SVG_ERR_CAPACITY) == b"SVG_ERR_CAPACITY"


def _shape(**kw):
    d = dict(B=1, H=2, N=1024, D=64, F=4, Hs=16, Ws=16, block=64)
    d.update(kw)
    return L.SvgShape(*[d[k] for k in ("B", "H", "N", "D", "F", "Hs", "Ws", "block")])


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x20000000)


def _err():
    return L.lib().svg_last_error().decode()


def test_build_masks_validation():
    lib = L.lib()
    assert lib.svg_build_masks(_shape(block=96), 1, FAKE, None) == L.SVG_ERR_UNSUPPORTED
    assert lib.svg_build_masks(_shape(N=1000), 1, FAKE, None) == L.SVG_ERR_INVALID_ARG
    assert "exceeds N" in _err()
    assert lib.svg_build_masks(_shape(), 1, None, None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_build_masks(_shape(), -1, FAKE, None) == L.SVG_ERR_INVALID_ARG


def test_encode_capacity():
    lib = L.lib()
    assert lib.svg_encode_iv_capacity(2, 591, 591) == 2 * 591 * 296
    need = lib.svg_encode_iv_capacity(1, 3, 5)
    st = lib.svg_encode_mask(FAKE, 1, 3, 5, FAKE, FAKE, FAKE, need - 1, None)
    assert st == L.SVG_ERR_CAPACITY and "below worst case" in _err()
    assert lib.svg_encode_mask(None, 1, 3, 5, FAKE, FAKE, FAKE, need, None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_encode_mask(FAKE, 0, 3, 5, FAKE, FAKE, FAKE, need, None) == L.SVG_ERR_INVALID_ARG


def test_permute_validation():
    lib = L.lib()
    assert lib.svg_permute(FAKE, FAKE, L.SVG_BF16, _shape(), None, 0, None) == L.SVG_ERR_INVALID_ARG
    assert "overlap" in _err()
    assert lib.svg_permute(FAKE, FAKE2, L.SVG_BF16, _shape(D=96), None, 0, None) == L.SVG_ERR_UNSUPPORTED
    assert lib.svg_permute(FAKE, FAKE2, 7, _shape(), None, 0, None) == L.SVG_ERR_INVALID_ARG
    odd = ctypes.c_void_p(0x20000008)
    assert lib.svg_permute(FAKE, odd, L.SVG_BF16, _shape(), None, 0, None) == L.SVG_ERR_INVALID_ARG


def _mask(n_masks=2, n=16):
    return L.SvgMask(n_masks, n, n, FAKE.value, FAKE.value, FAKE.value)


def test_profile_validation():
    lib = L.lib()
    s = _shape()
    ws = lib.svg_profile_workspace_bytes(s, 64)
    assert ws > 0
    m = _mask()
    args = lambda **kw: [kw.get("q", FAKE), FAKE, FAKE, kw.get("s", s), kw.get("scale", 0.125), FAKE,
                         kw.get("ns", 64), ctypes.byref(kw.get("m", m)), FAKE, None, FAKE,
                         kw.get("ws", ws), None]
    assert lib.svg_profile_heads(*args(ns=65)) == L.SVG_ERR_UNSUPPORTED
    assert lib.svg_profile_heads(*args(ns=0)) == L.SVG_ERR_UNSUPPORTED
    assert lib.svg_profile_heads(*args(ws=ws - 1)) == L.SVG_ERR_CAPACITY
    assert lib.svg_profile_heads(*args(m=_mask(n_masks=3))) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_profile_heads(*args(m=_mask(n=17))) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_profile_heads(*args(q=None)) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_profile_heads(*args(scale=0.0)) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_profile_heads(*args(s=_shape(D=80))) == L.SVG_ERR_UNSUPPORTED


def test_attention_validation():
    lib = L.lib()
    s = _shape()
    m = _mask(n_masks=1)
    # q, k, v, vt, o, qp, kp, vp, op, s, scale, masks, head_mask, head_layout, lse, ws, ws_bytes, stream
    base = [FAKE, FAKE2, ctypes.c_void_p(0x30000000), None, ctypes.c_void_p(0x40000000),
            None, None, None, None, s, 0.125, ctypes.byref(m), None, None, None, None, 0, None]
    a = list(base); a[13] = FAKE           # head_layout without token-major twins
    assert lib.svg_block_sparse_attn(*a) == L.SVG_ERR_INVALID_ARG
    a = list(base); a[4] = FAKE            # o aliases q
    assert lib.svg_block_sparse_attn(*a) == L.SVG_ERR_INVALID_ARG
    a = list(base); a[9] = _shape(D=256)
    assert lib.svg_block_sparse_attn(*a) == L.SVG_ERR_UNSUPPORTED
    bad = _mask(n_masks=1, n=8)
    a = list(base); a[11] = ctypes.byref(bad)
    assert lib.svg_block_sparse_attn(*a) == L.SVG_ERR_INVALID_ARG
    a = list(base); a[3] = ctypes.c_void_p(0x60000000)   # vt with 64-token blocks
    assert lib.svg_block_sparse_attn(*a) == L.SVG_ERR_INVALID_ARG
    a = list(base); a[2] = None                           # neither v nor vt
    assert lib.svg_block_sparse_attn(*a) == L.SVG_ERR_INVALID_ARG
    # 128-token blocks: work items hold the pair index in 16 bits and the mask
    # index in 15, so longer rows or more masks are refused before any launch
    big = _shape(block=128, N=128 * 131072)
    a = list(base); a[4] = ctypes.c_void_p(1 << 40); a[9] = big
    a[11] = ctypes.byref(_mask(n_masks=1, n=131072))
    assert lib.svg_block_sparse_attn(*a) == L.SVG_ERR_UNSUPPORTED
    a = list(base); a[9] = _shape(block=128)
    a[11] = ctypes.byref(_mask(n_masks=32769, n=8))
    assert lib.svg_block_sparse_attn(*a) == L.SVG_ERR_UNSUPPORTED
    # 128-token blocks: V^T blocks B*H*ceil(N/128)*128*D*2 bytes (none when the
    # caller gives vt), then the work plan: (9*B*H + 16 int32, rounded to
    # even) + 8 lists of B*H*cap int32 pairs + B*H*pairs int32,
    # cap = max(ceil(3*pairs/16), ceil(pairs/8)), pairs = ceil(ceil(N/128)/2)
    s128 = _shape(block=128)
    need = lib.svg_attn_workspace_bytes(s128, 0)
    BH, pairs = 2, 4
    cap = max((3 * pairs + 15) // 16, (pairs + 7) // 8)
    plan = ((9 * BH + 16 + 1) // 2 * 2) * 4 + 8 * BH * cap * 8 + BH * pairs * 4
    vt_bytes = 1 * 2 * 8 * 128 * 64 * 2
    assert lib.svg_vt_bytes(s128) == vt_bytes and lib.svg_vt_bytes(_shape()) == 0
    assert need == vt_bytes + plan
    assert lib.svg_attn_workspace_bytes(s128, 1) == plan
    assert lib.svg_attn_workspace_bytes(_shape(), 0) == 0
    m128 = L.SvgMask(1, 8, 8, FAKE.value, FAKE.value, FAKE.value)
    a = list(base); a[9] = s128; a[11] = ctypes.byref(m128); a[15] = ctypes.c_void_p(0x50000000); a[16] = need - 1
    assert lib.svg_block_sparse_attn(*a) == L.SVG_ERR_CAPACITY
    a[3] = ctypes.c_void_p(0x60000000); a[16] = plan - 1   # vt given: the plan alone
    assert lib.svg_block_sparse_attn(*a) == L.SVG_ERR_CAPACITY


def test_prepare_kv_validation():
    lib = L.lib()
    s128 = _shape(block=128)
    K, V, KP, VT = (ctypes.c_void_p(x) for x in (0x10000000, 0x20000000, 0x30000000, 0x40000000))
    ok = [K, V, KP, VT, s128, None, None]
    a = list(ok); a[4] = _shape()                 # 64-token blocks have no V^T blocks
    assert lib.svg_prepare_kv(*a) == L.SVG_ERR_UNSUPPORTED
    a = list(ok); a[1] = None
    assert lib.svg_prepare_kv(*a) == L.SVG_ERR_INVALID_ARG
    a = list(ok); a[3] = None
    assert lib.svg_prepare_kv(*a) == L.SVG_ERR_INVALID_ARG
    a = list(ok); a[0] = None                     # kp without k
    assert lib.svg_prepare_kv(*a) == L.SVG_ERR_INVALID_ARG
    a = list(ok); a[3] = V                        # vt aliases v
    assert lib.svg_prepare_kv(*a) == L.SVG_ERR_INVALID_ARG
    a = list(ok); a[2] = K                        # kp aliases k
    assert lib.svg_prepare_kv(*a) == L.SVG_ERR_INVALID_ARG
    a = list(ok); a[3] = ctypes.c_void_p(0x40000008)
    assert lib.svg_prepare_kv(*a) == L.SVG_ERR_INVALID_ARG
    a = list(ok); a[4] = _shape(block=128, D=96)
    assert lib.svg_prepare_kv(*a) == L.SVG_ERR_UNSUPPORTED


def test_broadcast_calibrate_validation():
    lib = L.lib()
    assert lib.svg_row_broadcast(FAKE, _shape(), None, 0, None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_row_broadcast(FAKE, _shape(), None, 17, None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_restrict_anchor_rows(FAKE, 1, _shape(), None, 0, None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_calibrate_masks(FAKE, 1, 4, 5000, 0.9, FAKE2, None) == L.SVG_ERR_UNSUPPORTED
    assert lib.svg_calibrate_masks(FAKE, 1, 4, 8, 0.0, FAKE2, None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_calibrate_masks(FAKE, 1, 4, 8, 1.5, FAKE2, None) == L.SVG_ERR_INVALID_ARG


def test_python_binding_raises_on_error():
    with pytest.raises(svg.SvgError) as e:
        L.check("svg_build_masks", L.lib().svg_build_masks(_shape(block=96), 1, FAKE, None))
    assert e.value.status == L.SVG_ERR_UNSUPPORTED


def test_flop_count_from_skip_list():
    """Host-side FLOP count of the bench from an encoded mask (CPU tensors)."""
    import torch
    from block_sparse_attention_svg_amd.layer import kept_pairs_per_mask
    N, B = 150, 64   # 3 blocks, the last one 22 tokens
    # mask 0 keeps (0,0) and (2,2); mask 1 keeps everything
    rp = torch.tensor([0, 1, 1, 2, 3, 4, 5], dtype=torch.int32)
    iv = torch.tensor([[0, 1], [2, 3], [0, 3], [0, 3], [0, 3]], dtype=torch.int32)
    m = svg.EncodedMasks(2, 3, 3, torch.zeros(1), rp, iv)
    pairs = kept_pairs_per_mask(m, N, B)
    assert pairs.tolist() == [64 * 64 + 22 * 22, N * N]


def test_calibration_validation():
    lib = L.lib()
    s = _shape()
    m = ctypes.c_void_p(0x30000000)
    assert lib.svg_block_energy(None, FAKE, s, 0.1, FAKE2, None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_block_energy(FAKE, FAKE, s, 0.0, FAKE2, None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_block_energy(FAKE, FAKE, _shape(D=80), 0.1, FAKE2, None) == L.SVG_ERR_UNSUPPORTED
    assert lib.svg_aggregate_masks(FAKE, 0, 10, 0.5, FAKE2, None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_aggregate_masks(FAKE, 2, 10, 0.0, FAKE2, None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_aggregate_masks(FAKE, 2, 10, 1.5, FAKE2, None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_aggregate_masks(FAKE, 2, 10, 0.5, ctypes.c_void_p(FAKE.value + 5), None) == L.SVG_ERR_INVALID_ARG
    v = ctypes.c_double()
    assert lib.svg_eps_schedule(3, 3, 0.99, 0.84, ctypes.byref(v)) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_eps_schedule(0, 1, 0.99, 1.5, ctypes.byref(v)) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_eps_schedule(2, 5, 0.99, 0.84, ctypes.byref(v)) == L.SVG_OK
    assert abs(v.value - (0.99 * 0.84) ** 0.5) < 1e-15
    ws = lib.svg_row_similarity_workspace_bytes(s)
    assert ws >= 1 * 2 * 4 * 16 * 1024 * 4
    big = ctypes.c_void_p(1 << 40)
    assert lib.svg_row_similarity(FAKE, FAKE, s, 0.1, FAKE2, big, ws - 1, None) == L.SVG_ERR_CAPACITY
    assert lib.svg_row_similarity(FAKE, FAKE, s, 0.1, FAKE2, ctypes.c_void_p((1 << 40) + 16), ws, None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_row_similarity(FAKE, FAKE, _shape(Ws=256, N=4 * 16 * 256), 0.1, FAKE2, big, 1 << 40, None) == L.SVG_ERR_UNSUPPORTED
    assert lib.svg_row_similarity(FAKE, FAKE, _shape(Hs=1, Ws=256, N=1024), 0.1, FAKE2, big, 1 << 40, None) == L.SVG_ERR_UNSUPPORTED
    assert lib.svg_row_similarity(FAKE, FAKE, _shape(Hs=65, Ws=4, N=1040), 0.1, FAKE2, big, 1 << 40, None) == L.SVG_ERR_UNSUPPORTED
    assert lib.svg_row_similarity(FAKE, FAKE, _shape(Hs=64, Ws=1, N=1 << 23), 0.1, FAKE2, big, 1 << 40, None) == L.SVG_ERR_UNSUPPORTED


def test_qk_norm_rope_validation():
    lib = L.lib()
    s = _shape()
    y = ctypes.c_void_p(1 << 40)
    ok_rope = L.SvgRope(s.D - 64, 32, 32, 10000.0)
    call = lambda x=FAKE, y=y, s=s, span=1, g=None, eps=1e-6, r=ctypes.byref(ok_rope), lay=None: \
        lib.svg_qk_norm_rope(x, y, s, span, g, eps, r, lay, None)
    assert call(x=None) == L.SVG_ERR_INVALID_ARG
    assert call(y=FAKE) == L.SVG_ERR_INVALID_ARG                       # x and y overlap
    assert call(y=ctypes.c_void_p((1 << 40) + 8)) == L.SVG_ERR_INVALID_ARG
    assert call(span=3) == L.SVG_ERR_INVALID_ARG
    assert call(eps=-1.0) == L.SVG_ERR_INVALID_ARG
    assert call(eps=float("inf")) == L.SVG_ERR_INVALID_ARG
    assert call(g=ctypes.c_void_p(FAKE2.value + 4)) == L.SVG_ERR_INVALID_ARG
    assert call(s=_shape(D=80)) == L.SVG_ERR_UNSUPPORTED
    assert call(s=_shape(H=65, D=128)) == L.SVG_ERR_UNSUPPORTED        # H*D > 8192
    for bad in ((s.D - 62, 31, 31), (s.D, 2, 0), (-2, s.D, 2)):
        r = L.SvgRope(*bad, 10000.0)
        assert call(r=ctypes.byref(r)) == L.SVG_ERR_INVALID_ARG, bad
    r = L.SvgRope(s.D - 64, 32, 32, 0.0)
    assert call(r=ctypes.byref(r)) == L.SVG_ERR_INVALID_ARG


def test_static_layer_rejects_flags_that_differ_across_batch_rows():
    """The static layer's masks are per head, shared by the batch rows: row-
    repetitive flags that differ between batch rows are refused on the host
    before any device call."""
    import torch
    from block_sparse_attention_svg_amd.layer import StaticSparseAttention
    from block_sparse_attention_svg_amd.ops import Shape
    s = Shape(B=2, H=3, N=256, D=64, F=1, Hs=16, Ws=16, block=128)
    masks = torch.ones((3, 2, 2), dtype=torch.uint8)
    flags = torch.tensor([1, 0, 0, 0, 0, 0], dtype=torch.int32)
    with pytest.raises(ValueError, match="same in every batch row"):
        StaticSparseAttention(s, masks, flags)
    with pytest.raises(ValueError, match="must hold 3 or 6 flags"):
        StaticSparseAttention(s, masks, torch.zeros(4, dtype=torch.int32))


def test_noalloc_validation():
    """The allocation-free attention call refuses, on the host, 128-token
    blocks without V^T and shapes whose work plan exceeds its fixed array."""
    lib = L.lib()
    assert lib.svg_noalloc_scratch_bytes() == 8 << 20
    s128 = _shape(block=128)
    m128 = L.SvgMask(1, 8, 8, FAKE.value, FAKE.value, FAKE.value)
    base = [FAKE, FAKE2, ctypes.c_void_p(0x30000000), None, ctypes.c_void_p(0x40000000),
            None, None, None, None, s128, 0.125, ctypes.byref(m128), None, None, None, None]
    assert lib.svg_block_sparse_attn_noalloc(*base) == L.SVG_ERR_INVALID_ARG
    assert "need the caller's V^T" in _err()
    # plan of B*H = 4096 heads x 512 pairs: about 33 MB > 8 MiB
    big = _shape(block=128, H=4096, N=128 * 1024, F=1, Hs=1, Ws=1)
    nb = 1024
    mbig = L.SvgMask(1, nb, nb, FAKE.value, FAKE.value, FAKE.value)
    a = list(base); a[3] = ctypes.c_void_p(1 << 44); a[4] = ctypes.c_void_p(1 << 45); a[9] = big
    a[11] = ctypes.byref(mbig)
    assert lib.svg_attn_workspace_bytes(big, 1) > lib.svg_noalloc_scratch_bytes()
    assert lib.svg_block_sparse_attn_noalloc(*a) == L.SVG_ERR_CAPACITY


def test_fp8_validation():
    lib = L.lib()
    s128 = _shape(block=128)
    assert lib.svg_fp8_vt_bytes(s128) == 1 * 2 * 8 * 128 * 64 and lib.svg_fp8_vt_bytes(_shape()) == 0
    bufs = [ctypes.c_void_p(x << 24) for x in range(1, 8)]
    q, k, v, q8, k8, vt8, sc = bufs
    ok = [q, k, v, q8, k8, vt8, sc, s128, None, None]
    a = list(ok); a[7] = _shape()
    assert lib.svg_quantize_fp8(*a) == L.SVG_ERR_UNSUPPORTED
    a = list(ok); a[3] = None
    assert lib.svg_quantize_fp8(*a) == L.SVG_ERR_INVALID_ARG
    a = list(ok); a[4] = q                      # k8 overlaps q
    assert lib.svg_quantize_fp8(*a) == L.SVG_ERR_INVALID_ARG
    a = list(ok); a[5] = ctypes.c_void_p((6 << 24) + 4)
    assert lib.svg_quantize_fp8(*a) == L.SVG_ERR_INVALID_ARG
    m128 = L.SvgMask(1, 8, 8, FAKE.value, FAKE.value, FAKE.value)
    plan = lib.svg_attn_workspace_bytes(s128, 1)
    att = [q8, k8, vt8, sc, q, s128, 0.125, ctypes.byref(m128), None, None, None,
           ctypes.c_void_p(9 << 24), plan, None]
    a = list(att); a[12] = plan - 1
    assert lib.svg_block_sparse_attn_fp8(*a) == L.SVG_ERR_CAPACITY
    a = list(att); a[5] = _shape()
    assert lib.svg_block_sparse_attn_fp8(*a) == L.SVG_ERR_UNSUPPORTED
    a = list(att); a[4] = q8                    # o overlaps q8
    assert lib.svg_block_sparse_attn_fp8(*a) == L.SVG_ERR_INVALID_ARG
    a = list(att); a[6] = 0.0
    assert lib.svg_block_sparse_attn_fp8(*a) == L.SVG_ERR_INVALID_ARG


def test_mfma_peak_probe_validation():
    """The measurement probe checks its arguments before any HIP call."""
    lib = L.lib()
    flop = ctypes.c_double(0.0)
    assert lib.svg_mfma_peak_probe(2, 10, FAKE, 1 << 20, ctypes.byref(flop), None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_mfma_peak_probe(0, 0, FAKE, 1 << 20, ctypes.byref(flop), None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_mfma_peak_probe(1, (1 << 20) + 1, FAKE, 1 << 20, ctypes.byref(flop), None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_mfma_peak_probe(0, 10, None, 1 << 20, ctypes.byref(flop), None) == L.SVG_ERR_INVALID_ARG
    assert lib.svg_mfma_peak_probe(0, 10, FAKE, 1 << 20, None, None) == L.SVG_ERR_INVALID_ARG
