"""Seeded generators of synthetic q/k/v, profiler sample indices and block energies.

Recipe (float64 draws, then float64 -> float32 -> bfloat16 with round-to-nearest-even):

* spatial head: phi_d(f, y, x) = cos(2*pi*(a_d*f + b_d*y/Hs + c_d*x/Ws) + beta_d),
  a_d, b_d, c_d ~ N(0, 0.5^2), beta_d ~ U[0, 2*pi); q = 2*phi + sigma*eps_q,
  k = 2*phi + sigma*eps_k.  Nearby frames and positions get similar features, so
  attention concentrates in the same and adjacent frames (the spatial pattern of
  the Sparse VideoGen article, "Spatial Head").
* temporal head: one vector u_s ~ N(0, I_D) per spatial position s, rescaled to
  norm sqrt(D) and shared by every frame; q = 2*u_s + sigma*eps_q,
  k = 2*u_s + sigma*eps_k.  A token then attends to the same position in other
  frames (the article's "Temporal Head": diagonals with a constant stride).
* v ~ N(0, 1); appended text tokens have q, k, v ~ N(0, 1).

Seeds: workload seed c; head h draws from default_rng(c*1000 + h); the profiler
sample set of call t from default_rng(c*7919 + t); block energies of head h from
default_rng(c*1000 + 500 + h); head classes from default_rng(c*31); the
row-repetitive heads from default_rng(c*7 + 3).
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from .configs import Workload

SPATIAL = 0
TEMPORAL = 1


def head_classes(w: Workload) -> np.ndarray:
    """Generator class of every head (0 spatial, 1 temporal), int32 [H]."""
    if w.name == "tiny" and w.H == 2:
        return np.array([SPATIAL, TEMPORAL], dtype=np.int32)
    perm = np.random.default_rng(w.seed * 31).permutation(w.H)
    cls = np.full(w.H, TEMPORAL, dtype=np.int32)
    cls[perm[: min(w.n_spatial, w.H)]] = SPATIAL
    return cls


def _video_coords(w: Workload):
    i = np.arange(w.N_video)
    f = i // w.S
    s = i % w.S
    return f, s // w.Ws, s % w.Ws, s


def gen_head_qkv(w: Workload, h: int, cls: int):
    """float64 q, k, v of one head, each [N, D], frame-major token order."""
    rng = np.random.default_rng(w.seed * 1000 + h)
    D = w.D
    f, y, x, s = _video_coords(w)
    if cls == SPATIAL:
        a = rng.normal(0.0, 0.5, D)
        b = rng.normal(0.0, 0.5, D)
        c = rng.normal(0.0, 0.5, D)
        beta = rng.uniform(0.0, 2.0 * math.pi, D)
        phase = (np.outer(f, a) + np.outer(y / w.Hs, b) + np.outer(x / w.Ws, c))
        feat = np.cos(2.0 * math.pi * phase + beta[None, :])
    else:
        u = rng.standard_normal((w.S, D))
        u *= math.sqrt(D) / np.linalg.norm(u, axis=1, keepdims=True)
        feat = u[s]
    eq = rng.standard_normal((w.N_video, D))
    ek = rng.standard_normal((w.N_video, D))
    v = rng.standard_normal((w.N, D))
    q = np.empty((w.N, D))
    k = np.empty((w.N, D))
    q[: w.N_video] = 2.0 * feat + w.sigma * eq
    k[: w.N_video] = 2.0 * feat + w.sigma * ek
    if w.text:
        q[w.N_video:] = rng.standard_normal((w.text, D))
        k[w.N_video:] = rng.standard_normal((w.text, D))
    return q, k, v


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float64 array -> float32 -> bfloat16 tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def gen_qkv(w: Workload, dtype: str = None, heads=None):
    """Canonical q, k, v tensors [B, H, N, D] on the CPU.

    dtype: "bf16" or "f32"; defaults to the workload's stored dtype.
    heads: optional subset of head ids (the result then holds only those heads,
    in the given order); every head keeps its own seed.
    """
    dtype = dtype or w.in_dtype
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cls = head_classes(w)
    heads = list(range(w.H)) if heads is None else list(heads)
    out = [torch.empty((w.B, len(heads), w.N, w.D), dtype=tdt) for _ in range(3)]

    def one(job):
        b, j, h = job
        arrs = gen_head_qkv(w, h + b * w.H, int(cls[h]))
        for t, a in zip(out, arrs):
            a32 = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
            t[b, j] = a32.to(tdt)

    jobs = [(b, j, h) for b in range(w.B) for j, h in enumerate(heads)]
    # heads are independent and NumPy releases the GIL in the bulk draws
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1, len(jobs))) as ex:
        list(ex.map(one, jobs))
    return out[0], out[1], out[2], cls[heads]


def sample_query_idx(w: Workload, t: int = 0) -> np.ndarray:
    """n_samples distinct frame-major video-token indices, int32, for call t."""
    rng = np.random.default_rng(w.seed * 7919 + t)
    return rng.choice(w.N_video, size=w.n_samples, replace=False).astype(np.int32)


def energy_matrix(w: Workload, h: int, lam: float = None) -> np.ndarray:
    """Synthetic block-energy matrix of head h, float64 [nB, nB].

    E[r, c] = exp(-|r - c| / lam) * J[r, c], J iid LogNormal(0, 0.5^2): energy
    decays away from the diagonal with random per-block jitter.
    """
    lam = w.energy_lambda if lam is None else lam
    n = w.n_blocks
    rng = np.random.default_rng(w.seed * 1000 + 500 + h)
    J = rng.lognormal(0.0, 0.5, (n, n))
    r = np.arange(n)
    return np.exp(-np.abs(r[:, None] - r[None, :]) / lam) * J


def repetitive_heads(w: Workload) -> np.ndarray:
    """Sorted ids of the row-repetitive heads (static workload), int32."""
    if w.n_repetitive == 0:
        return np.zeros(0, dtype=np.int32)
    rng = np.random.default_rng(w.seed * 7 + 3)
    return np.sort(rng.choice(w.H, size=w.n_repetitive, replace=False)).astype(np.int32)


def gen_projection_rows(B: int, N: int, H: int, D: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """Seeded bf16 [B, N, H, D] query / key projection rows (frame-major tokens):
    standard normal entries times a per-head scale drawn log-uniformly from
    [1/4, 4] and a per-token scale from [1/2, 2], so that RMS normalisation has
    rows of different size to equalise."""
    g = torch.Generator(device=device).manual_seed(seed)
    x = torch.randn((B, N, H, D), generator=g, device=device, dtype=torch.float32)
    hs = torch.exp(torch.rand(H, generator=g, device=device) * (2 * math.log(4.0)) - math.log(4.0))
    ts = torch.exp(torch.rand((B, N), generator=g, device=device) * (2 * math.log(2.0)) - math.log(2.0))
    return (x * ts[:, :, None, None] * hs[None, None, :, None]).to(torch.bfloat16)


def gen_norm_weight(n: int, seed: int = 0) -> np.ndarray:
    """Seeded float32 norm weights, uniform in [0.5, 1.5]."""
    return np.random.default_rng(seed).uniform(0.5, 1.5, n).astype(np.float32)
