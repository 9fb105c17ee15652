"""Workload shapes of the synthetic video-DiT attention layers.

Each workload is one attention layer at batch 1.  Tokens are a video latent of
F frames x Hs x Ws positions stored frame-major (token i = f*Hs*Ws + y*Ws + x),
followed by `text` appended text tokens.  The shapes follow the models the
Sparse VideoGen article and the calibrated-attention article name (CogVideoX,
Wan 2.1 720p, HunyuanVideo 720p); the tiny case is the 4-frame 16x16 latent of
the worked example in the video-diffusion acceleration survey (section 2.1,
4 * (256/16)^2 = 1024 tokens).

`band_w` is the half-width, in token-major blocks, of the temporal block band.
It is a workload constant: the smallest width whose kept-block fraction reaches
0.30 (checked against the oracle by a CPU test).  The tiny case uses +/-1 block.

`energy_lambda` is the decay length (in blocks) of the synthetic block-energy
matrix of the static calibrated workload; with eps = 0.9 it gives about 68 %
block sparsity (checked by a CPU test).
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    H: int            # heads
    D: int            # head dim
    F: int            # latent frames
    Hs: int           # latent rows per frame
    Ws: int           # latent columns per frame
    text: int         # appended text tokens
    block: int        # query/key block edge
    band_w: int       # temporal band half-width (token-major blocks)
    sigma: float      # std-dev of the q/k noise
    n_spatial: int    # heads generated as spatial (rest temporal)
    seed: int         # workload seed
    in_dtype: str = "bf16"   # canonical stored dtype ("f32" for the tiny case)
    B: int = 1               # batch
    n_samples: int = 64      # profiler sample size (Sparse VideoGen: about 64 queries)
    mode: str = "online"     # "online" (profiled spatial/temporal) or "static"
    eps: float = 0.9         # static: cumulative-energy fraction per query row
    energy_lambda: float = 0.0   # static: energy decay length in blocks
    n_repetitive: int = 0        # static: row-repetitive heads
    k_anchors: int = 5           # static: anchor rows per frame

    @property
    def S(self) -> int:
        return self.Hs * self.Ws

    @property
    def N_video(self) -> int:
        return self.F * self.S

    @property
    def N(self) -> int:
        return self.N_video + self.text

    @property
    def n_blocks(self) -> int:
        return -(-self.N // self.block)

    @property
    def scale(self) -> float:
        return 1.0 / (self.D ** 0.5)


CONFIGS = {
    "tiny": Workload("tiny", H=2, D=64, F=4, Hs=16, Ws=16, text=0, block=64,
                     band_w=1, sigma=0.1, n_spatial=1, seed=1001, in_dtype="f32"),
    "cogvideox": Workload("cogvideox", H=48, D=64, F=13, Hs=30, Ws=45, text=0,
                          block=128, band_w=23, sigma=0.1, n_spatial=24, seed=1002),
    "wan720p": Workload("wan720p", H=40, D=128, F=21, Hs=45, Ws=80, text=0,
                        block=128, band_w=97, sigma=0.3, n_spatial=24, seed=1003),
    "hunyuan720p": Workload("hunyuan720p", H=24, D=128, F=33, Hs=45, Ws=80, text=256,
                            block=128, band_w=149, sigma=0.1, n_spatial=12, seed=1004),
    "static_wan720p": Workload("static_wan720p", H=40, D=128, F=21, Hs=45, Ws=80, text=0,
                               block=128, band_w=97, sigma=0.3, n_spatial=24, seed=1005,
                               mode="static", eps=0.9, energy_lambda=52.0,
                               n_repetitive=5, k_anchors=5),
}


def get_workload(name: str, **overrides) -> Workload:
    """Return a named workload, optionally with fields replaced (e.g. fewer heads)."""
    w = CONFIGS[name]
    if overrides:
        d = dict(w.__dict__)
        d.update(overrides)
        w = Workload(**d)
    return w
