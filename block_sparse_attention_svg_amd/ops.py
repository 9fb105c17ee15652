"""Python binding of the C ABI: one function per entry point, same names.

Argument marshalling only (dtype / shape / device checks, raw pointers and
torch's current stream); every step of the computation runs in libsvg's HIP
kernels.  Tensors are torch CUDA tensors; PyTorch provides device memory and
streams.
"""
import ctypes
from dataclasses import dataclass

import torch

from . import _lib as L


@dataclass(frozen=True)
class Shape:
    B: int
    H: int
    N: int
    D: int
    F: int
    Hs: int
    Ws: int
    block: int

    @property
    def n_blocks(self) -> int:
        return -(-self.N // self.block)

    @property
    def N_video(self) -> int:
        return self.F * self.Hs * self.Ws

    def c(self) -> L.SvgShape:
        return L.SvgShape(self.B, self.H, self.N, self.D, self.F, self.Hs, self.Ws, self.block)


@dataclass
class EncodedMasks:
    """Bitmap + skip list of n_masks block masks (device tensors)."""
    n_masks: int
    n_qb: int
    n_kb: int
    bitmap: torch.Tensor    # int32 view of uint32 words [n_masks, n_qb, ceil(n_kb/32)]
    row_ptr: torch.Tensor   # int32 [n_masks*n_qb + 1]
    iv: torch.Tensor        # int32 [capacity, 2]

    def c(self) -> L.SvgMask:
        return L.SvgMask(self.n_masks, self.n_qb, self.n_kb, self.bitmap.data_ptr(),
                         self.row_ptr.data_ptr(), self.iv.data_ptr())

    def n_intervals(self) -> int:
        return int(self.row_ptr[-1].item())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, device=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_act(t, name, s: Shape, dtype=torch.bfloat16):
    _need(t, name, dtype)
    if tuple(t.shape) != (s.B, s.H, s.N, s.D):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(s.B, s.H, s.N, s.D)}")


def svg_build_masks(s: Shape, band_w: int, out: torch.Tensor = None, device="cuda") -> torch.Tensor:
    """Dense uint8 candidate masks [2, nB, nB]: [0] spatial, [1] temporal."""
    nB = s.n_blocks
    if out is None:
        out = torch.empty((2, nB, nB), dtype=torch.uint8, device=device)
    _need(out, "out", torch.uint8)
    L.check("svg_build_masks", L.lib().svg_build_masks(s.c(), band_w, _ptr(out), _stream()))
    return out


def svg_encode_iv_capacity(n_masks: int, n_qb: int, n_kb: int) -> int:
    return int(L.lib().svg_encode_iv_capacity(n_masks, n_qb, n_kb))


def svg_encode_mask(dense: torch.Tensor) -> EncodedMasks:
    """Encode dense uint8 masks [n_masks, n_qb, n_kb] into bitmap + skip list."""
    _need(dense, "dense", torch.uint8)
    if dense.dim() != 3:
        raise ValueError("dense must be [n_masks, n_qb, n_kb]")
    M, nq, nk = dense.shape
    cap = svg_encode_iv_capacity(M, nq, nk)
    dev = dense.device
    bitmap = torch.empty((M, nq, -(-nk // 32)), dtype=torch.int32, device=dev)
    row_ptr = torch.empty(M * nq + 1, dtype=torch.int32, device=dev)
    iv = torch.empty((max(cap, 1), 2), dtype=torch.int32, device=dev)
    L.check("svg_encode_mask", L.lib().svg_encode_mask(
        _ptr(dense), M, nq, nk, _ptr(bitmap), _ptr(row_ptr), _ptr(iv), cap, _stream()))
    return EncodedMasks(M, nq, nk, bitmap, row_ptr, iv)


def svg_permute(x: torch.Tensor, s: Shape, head_sel: torch.Tensor = None, inverse: bool = False,
                out: torch.Tensor = None) -> torch.Tensor:
    """Frame-major -> token-major (inverse=False) or back, for heads with head_sel != 0."""
    dt = {torch.bfloat16: L.SVG_BF16, torch.float32: L.SVG_F32}.get(x.dtype)
    if dt is None:
        raise TypeError("x must be bfloat16 or float32")
    _need_act(x, "x", s, x.dtype)
    if out is None:
        out = torch.empty_like(x)
    _need_act(out, "out", s, x.dtype)
    if head_sel is not None:
        _need(head_sel, "head_sel", torch.int32)
    L.check("svg_permute", L.lib().svg_permute(_ptr(x), _ptr(out), dt, s.c(), _ptr(head_sel),
                                               int(bool(inverse)), _stream()))
    return out


_NORM_SPAN = {None: 0, "head": 1, "row": 2}


def svg_qk_norm_rope(x: torch.Tensor, s: Shape, norm: str = "head", gamma: torch.Tensor = None,
                     eps: float = 1e-6, rope=None, head_layout: torch.Tensor = None,
                     out: torch.Tensor = None) -> torch.Tensor:
    """Projection rows x [B, N, H, D] -> attention input [B, H, N, D], RMS
    normalised over each head (norm="head") or the whole row (norm="row") or
    not at all (None), turned by the 3D rotary embedding rope = (d_f, d_y, d_x,
    theta) or not (None), each head written in its layout (head_layout [B*H],
    nonzero = token-major; None = all frame-major)."""
    if norm not in _NORM_SPAN:
        raise ValueError(f"norm must be None, 'head' or 'row' (got {norm!r})")
    if tuple(x.shape) != (s.B, s.N, s.H, s.D) or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError(f"x must be contiguous bfloat16 [{s.B}, {s.N}, {s.H}, {s.D}]")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    if out is None:
        out = torch.empty((s.B, s.H, s.N, s.D), dtype=torch.bfloat16, device=x.device)
    _need_act(out, "out", s)
    if gamma is not None:
        _need(gamma, "gamma", torch.float32)
        want = s.D if norm == "head" else s.H * s.D
        if gamma.numel() != want:
            raise ValueError(f"gamma must hold {want} values for norm={norm!r}")
    if head_layout is not None:
        _need(head_layout, "head_layout", torch.int32)
    r = None
    if rope is not None:
        d_f, d_y, d_x, theta = rope
        r = ctypes.byref(L.SvgRope(int(d_f), int(d_y), int(d_x), float(theta)))
    L.check("svg_qk_norm_rope", L.lib().svg_qk_norm_rope(
        _ptr(x), _ptr(out), s.c(), _NORM_SPAN[norm], _ptr(gamma), float(eps), r, _ptr(head_layout),
        _stream()))
    return out


def svg_profile_workspace_bytes(s: Shape, n_samples: int) -> int:
    return int(L.lib().svg_profile_workspace_bytes(s.c(), n_samples))


def svg_profile_heads(q, k, v, s: Shape, scale: float, idx: torch.Tensor, cand: EncodedMasks,
                      workspace: torch.Tensor = None, choice: torch.Tensor = None,
                      err: torch.Tensor = None):
    """Per-head mask choice (0 spatial, 1 temporal) and errors [B*H, 2]."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need_act(t, n, s)
    _need(idx, "idx", torch.int32)
    ns = idx.numel()
    need = svg_profile_workspace_bytes(s, ns)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if choice is None:
        choice = torch.empty(s.B * s.H, dtype=torch.int32, device=q.device)
    if err is None:
        err = torch.empty((s.B * s.H, 2), dtype=torch.float32, device=q.device)
    cm = cand.c()
    L.check("svg_profile_heads", L.lib().svg_profile_heads(
        _ptr(q), _ptr(k), _ptr(v), s.c(), float(scale), _ptr(idx), ns, ctypes.byref(cm),
        _ptr(choice), _ptr(err), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream()))
    return choice, err


def svg_attn_workspace_bytes(s: Shape, vt_given: bool = False) -> int:
    return int(L.lib().svg_attn_workspace_bytes(s.c(), int(bool(vt_given))))


def svg_vt_bytes(s: Shape) -> int:
    return int(L.lib().svg_vt_bytes(s.c()))


def svg_prepare_kv(k, v, s: Shape, head_layout: torch.Tensor = None, kp: torch.Tensor = None,
                   vt: torch.Tensor = None, move_k: bool = True):
    """The layout pass of a 128-token-block layer: V of every head block-
    transposed in its layout (vt), and K token-major for the heads with
    head_layout != 0 (kp, when move_k).  Returns (kp or None, vt)."""
    _need_act(v, "v", s)
    if move_k:
        _need_act(k, "k", s)
        if kp is None:
            kp = torch.empty_like(k)
        _need_act(kp, "kp", s)
    else:
        kp = None
    if vt is None:
        vt = torch.empty(svg_vt_bytes(s) // 2, dtype=torch.bfloat16, device=v.device)
    _need(vt, "vt", torch.bfloat16)
    if vt.numel() * 2 < svg_vt_bytes(s):
        raise ValueError("vt is smaller than svg_vt_bytes(s)")
    if head_layout is not None:
        _need(head_layout, "head_layout", torch.int32)
    L.check("svg_prepare_kv", L.lib().svg_prepare_kv(
        _ptr(k if move_k else None), _ptr(v), _ptr(kp), _ptr(vt), s.c(), _ptr(head_layout), _stream()))
    return kp, vt


def _attn_args(q, k, v, vt, s, head_mask, head_layout, qp, kp, vp, out, op, lse):
    for t, n in ((q, "q"), (k, "k")):
        _need_act(t, n, s)
    if v is not None or vt is None:
        _need_act(v, "v", s)
    if vt is not None:
        _need(vt, "vt", torch.bfloat16)
        if vt.numel() * 2 < svg_vt_bytes(s):
            raise ValueError("vt is smaller than svg_vt_bytes(s)")
    if out is None:
        out = torch.empty_like(q)
    _need_act(out, "out", s)
    if head_layout is not None:
        _need(head_layout, "head_layout", torch.int32)
        _need_act(kp, "kp", s)
        for t, n in ((qp, "qp"), (vp, "vp"), (op, "op")):
            if t is not None:
                _need_act(t, n, s)
    if head_mask is not None:
        _need(head_mask, "head_mask", torch.int32)
    lse_t = torch.empty((s.B, s.H, s.N), dtype=torch.float32, device=q.device) if lse else None
    return out, lse_t


def svg_block_sparse_attn(q, k, v, s: Shape, scale: float, masks: EncodedMasks,
                          head_mask: torch.Tensor = None, head_layout: torch.Tensor = None,
                          qp=None, kp=None, vp=None, out=None, op=None, lse: bool = False,
                          workspace: torch.Tensor = None, vt: torch.Tensor = None):
    """Block-sparse attention; returns (o, op, lse or None).

    With head_layout, kp is required; qp, vp and op may be None (128-token
    blocks): layout-1 heads then read Q / V from q / v and write O to `out`
    through the permutation, and the returned op is None.  vt: V^T blocks
    from svg_prepare_kv (128-token blocks; v may then be None)."""
    out, lse_t = _attn_args(q, k, v, vt, s, head_mask, head_layout, qp, kp, vp, out, op, lse)
    need = svg_attn_workspace_bytes(s, vt is not None)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    mc = masks.c()
    L.check("svg_block_sparse_attn", L.lib().svg_block_sparse_attn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(vt), _ptr(out), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(op), s.c(),
        float(scale), ctypes.byref(mc), _ptr(head_mask), _ptr(head_layout), _ptr(lse_t),
        _ptr(workspace), ws_bytes, _stream()))
    return out, op, lse_t


def svg_fp8_vt_bytes(s: Shape) -> int:
    return int(L.lib().svg_fp8_vt_bytes(s.c()))


@dataclass
class Fp8Operands:
    """E4M3 codes of q, k, v in the FP8 attention's layouts and their [3, B*H]
    dequantization factors (svg_quantize_fp8)."""
    q8: torch.Tensor       # uint8 [B, H, N, D], frame-major
    k8: torch.Tensor       # uint8 [B, H, N, D], each head in its layout
    vt8: torch.Tensor      # uint8 [svg_fp8_vt_bytes]
    scales: torch.Tensor   # float32 [3, B*H]


def svg_quantize_fp8(q, k, v, s: Shape, head_layout: torch.Tensor = None, out: Fp8Operands = None):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need_act(t, n, s)
    if head_layout is not None:
        _need(head_layout, "head_layout", torch.int32)
    if out is None:
        dev = q.device
        shape = (s.B, s.H, s.N, s.D)
        out = Fp8Operands(torch.empty(shape, dtype=torch.uint8, device=dev),
                          torch.empty(shape, dtype=torch.uint8, device=dev),
                          torch.empty(svg_fp8_vt_bytes(s), dtype=torch.uint8, device=dev),
                          torch.empty((3, s.B * s.H), dtype=torch.float32, device=dev))
    for t, n in ((out.q8, "q8"), (out.k8, "k8"), (out.vt8, "vt8")):
        _need(t, n, torch.uint8)
    _need(out.scales, "scales", torch.float32)
    L.check("svg_quantize_fp8", L.lib().svg_quantize_fp8(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out.q8), _ptr(out.k8), _ptr(out.vt8), _ptr(out.scales), s.c(),
        _ptr(head_layout), _stream()))
    return out


def svg_block_sparse_attn_fp8(ops8: Fp8Operands, s: Shape, scale: float, masks: EncodedMasks,
                              head_mask: torch.Tensor = None, head_layout: torch.Tensor = None,
                              out: torch.Tensor = None, lse: bool = False, workspace: torch.Tensor = None):
    """FP8 block-sparse attention; returns (o bf16 [B,H,N,D] frame-major, lse or None)."""
    dev = ops8.q8.device
    if out is None:
        out = torch.empty((s.B, s.H, s.N, s.D), dtype=torch.bfloat16, device=dev)
    _need_act(out, "out", s)
    for t, n in ((head_mask, "head_mask"), (head_layout, "head_layout")):
        if t is not None:
            _need(t, n, torch.int32)
    lse_t = torch.empty((s.B, s.H, s.N), dtype=torch.float32, device=dev) if lse else None
    need = svg_attn_workspace_bytes(s, True)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    mc = masks.c()
    L.check("svg_block_sparse_attn_fp8", L.lib().svg_block_sparse_attn_fp8(
        _ptr(ops8.q8), _ptr(ops8.k8), _ptr(ops8.vt8), _ptr(ops8.scales), _ptr(out), s.c(), float(scale),
        ctypes.byref(mc), _ptr(head_mask), _ptr(head_layout), _ptr(lse_t), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream()))
    return out, lse_t


def svg_noalloc_scratch_bytes() -> int:
    return int(L.lib().svg_noalloc_scratch_bytes())


def svg_block_sparse_attn_noalloc(q, k, v, s: Shape, scale: float, masks: EncodedMasks,
                                  head_mask: torch.Tensor = None, head_layout: torch.Tensor = None,
                                  qp=None, kp=None, vp=None, out=None, op=None, lse: bool = False,
                                  vt: torch.Tensor = None):
    """svg_block_sparse_attn without a workspace (the library's fixed scratch
    array holds the work plan); 128-token blocks need vt.  Outputs must be
    passed in (out, and lse as a tensor) by callers that cannot allocate."""
    if isinstance(lse, torch.Tensor):
        lse_t = lse
        _need(lse_t, "lse", torch.float32)
        out, _ = _attn_args(q, k, v, vt, s, head_mask, head_layout, qp, kp, vp, out, op, False)
    else:
        out, lse_t = _attn_args(q, k, v, vt, s, head_mask, head_layout, qp, kp, vp, out, op, lse)
    mc = masks.c()
    L.check("svg_block_sparse_attn_noalloc", L.lib().svg_block_sparse_attn_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(vt), _ptr(out), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(op), s.c(),
        float(scale), ctypes.byref(mc), _ptr(head_mask), _ptr(head_layout), _ptr(lse_t), _stream()))
    return out, op, lse_t


def svg_row_broadcast(o: torch.Tensor, s: Shape, head_sel: torch.Tensor, k_anchors: int):
    _need_act(o, "o", s)
    if head_sel is not None:
        _need(head_sel, "head_sel", torch.int32)
    L.check("svg_row_broadcast", L.lib().svg_row_broadcast(_ptr(o), s.c(), _ptr(head_sel),
                                                           int(k_anchors), _stream()))
    return o


def svg_restrict_anchor_rows(masks: torch.Tensor, s: Shape, mask_sel: torch.Tensor, k_anchors: int):
    _need(masks, "masks", torch.uint8)
    if mask_sel is not None:
        _need(mask_sel, "mask_sel", torch.int32)
    L.check("svg_restrict_anchor_rows", L.lib().svg_restrict_anchor_rows(
        _ptr(masks), masks.shape[0], s.c(), _ptr(mask_sel), int(k_anchors), _stream()))
    return masks


def svg_calibrate_masks(energy: torch.Tensor, eps: float, out: torch.Tensor = None) -> torch.Tensor:
    """uint8 masks from float64 block energies [n_masks, n_qb, n_kb]."""
    _need(energy, "energy", torch.float64)
    M, nq, nk = energy.shape
    if out is None:
        out = torch.empty((M, nq, nk), dtype=torch.uint8, device=energy.device)
    _need(out, "out", torch.uint8)
    L.check("svg_calibrate_masks", L.lib().svg_calibrate_masks(
        _ptr(energy), M, nq, nk, float(eps), _ptr(out), _stream()))
    return out


def svg_block_energy(q: torch.Tensor, k: torch.Tensor, s: Shape, scale: float,
                     out: torch.Tensor = None) -> torch.Tensor:
    """float64 [B*H, nB, nB] block attention energies of every head."""
    _need_act(q, "q", s)
    _need_act(k, "k", s)
    nB = s.n_blocks
    if out is None:
        out = torch.empty((s.B * s.H, nB, nB), dtype=torch.float64, device=q.device)
    _need(out, "out", torch.float64)
    if tuple(out.shape) != (s.B * s.H, nB, nB):
        raise ValueError(f"out must be [{s.B * s.H}, {nB}, {nB}]")
    L.check("svg_block_energy", L.lib().svg_block_energy(_ptr(q), _ptr(k), s.c(), float(scale),
                                                         _ptr(out), _stream()))
    return out


def svg_aggregate_masks(masks: torch.Tensor, rho: float = 0.5, out: torch.Tensor = None) -> torch.Tensor:
    """uint8 mask of the elements kept by at least a fraction rho of the
    candidate masks stacked along dim 0."""
    _need(masks, "masks", torch.uint8)
    if out is None:
        out = torch.empty(masks.shape[1:], dtype=torch.uint8, device=masks.device)
    _need(out, "out", torch.uint8)
    if tuple(out.shape) != tuple(masks.shape[1:]):
        raise ValueError("out must have the shape of one candidate mask")
    L.check("svg_aggregate_masks", L.lib().svg_aggregate_masks(
        _ptr(masks), masks.shape[0], out.numel(), float(rho), _ptr(out), _stream()))
    return out


def svg_row_similarity_workspace_bytes(s: Shape) -> int:
    return int(L.lib().svg_row_similarity_workspace_bytes(s.c()))


def svg_row_similarity(q: torch.Tensor, k: torch.Tensor, s: Shape, scale: float,
                       workspace: torch.Tensor = None) -> torch.Tensor:
    """float64 [B*H] mean within-frame cosine of the rows' attention patterns."""
    _need_act(q, "q", s)
    _need_act(k, "k", s)
    need = svg_row_similarity_workspace_bytes(s)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    out = torch.empty(s.B * s.H, dtype=torch.float64, device=q.device)
    L.check("svg_row_similarity", L.lib().svg_row_similarity(
        _ptr(q), _ptr(k), s.c(), float(scale), _ptr(out), _ptr(workspace), workspace.numel(), _stream()))
    return out


def svg_eps_schedule(t: int, T: int, eps_first: float = 0.99, eps_last: float = 0.84) -> float:
    """Energy threshold of denoising step t of T (host)."""
    v = ctypes.c_double()
    L.check("svg_eps_schedule", L.lib().svg_eps_schedule(int(t), int(T), float(eps_first),
                                                         float(eps_last), ctypes.byref(v)))
    return v.value


def svg_version() -> str:
    return L.lib().svg_version().decode()


def svg_mfma_peak_probe(fp8: bool, rounds: int, sink: torch.Tensor) -> float:
    """Enqueue one launch of the dense-MFMA probe (a measurement aid, not part
    of the attention path); returns the launch's FLOP.  sink: float32 device
    tensor of at least n_CU * 512 elements."""
    _need(sink, "sink", torch.float32)
    flop = ctypes.c_double(0.0)
    L.check("svg_mfma_peak_probe", L.lib().svg_mfma_peak_probe(int(bool(fp8)), int(rounds), _ptr(sink),
                                                               sink.numel(), ctypes.byref(flop), _stream()))
    return float(flop.value)
