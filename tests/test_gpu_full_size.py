"""Full-size parity: every head of the Wan 720p, HunyuanVideo 720p, CogVideoX
and static calibrated layers against the float64 oracle.

The layers run once per workload through the same drivers the bench times
(OnlineSparseAttention / StaticSparseAttention, persistent per-XCD queues,
fused layout).  Each head is then compared on at least 32 seeded query blocks
of its own mask layout, always including block 0, the ragged last block and
(HunyuanVideo) the mixed video/text block; O per head within max-abs 2e-2 and
rel-L2 5e-3, the log-sum-exp within LSE_ABS; the online layers also run
without the LSE, as the bench calls them, and that output is checked too.  The profiler's choice is compared
with the oracle's on every head, its errors within ERR_REL.  The oracle runs
one head at a time (bounded memory), so the heads are split over several tests.
Each test prints the worst errors it measured.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_svg_amd as svg
import oracle as O
import synth as S
from parity_utils import (banner, attn_errors, to_np, ATTN_MAX_ABS, ATTN_REL_L2, LSE_ABS,
                          PROFILE_ERR_REL, sample_qblocks)

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_QBLOCKS = 32

_ONLINE = {}
_STATIC = {}


def _online(name, workload_inputs):
    """Run the online layer once (call t = 0); keep its outputs on the host."""
    if name not in _ONLINE:
        w, q, k, v, cls = workload_inputs(name)
        s = svg.Shape(w.B, w.H, w.N, w.D, w.F, w.Hs, w.Ws, w.block)
        layer = svg.OnlineSparseAttention(s, w.band_w)
        idx = torch.from_numpy(S.sample_query_idx(w, 0)).to(DEV)
        o, lse = layer(q.to(DEV), k.to(DEV), v.to(DEV), idx, lse=True)
        torch.cuda.synchronize()
        choice = layer.choice.cpu().numpy()
        # the bench's call: no LSE (the denominator is then summed on the
        # matrix core from the bf16 weights)
        o2, _ = layer(q.to(DEV), k.to(DEV), v.to(DEV), idx)
        torch.cuda.synchronize()
        assert np.array_equal(layer.choice.cpu().numpy(), choice)
        _ONLINE[name] = dict(w=w, q=q, k=k, v=v, cls=cls, choice=choice,
                             err=layer.err.cpu().numpy().astype(np.float64), o=o.cpu(), lse=lse.cpu(),
                             o_nolse=o2.cpu())
        del layer, o, lse, o2
        torch.cuda.empty_cache()
    return _ONLINE[name]


def _parts(H, n):
    step = -(-H // n)
    return [list(range(i, min(H, i + step))) for i in range(0, H, step)]


ONLINE_PARTS = ([("wan720p", i, 5) for i in range(5)] + [("hunyuan720p", i, 4) for i in range(4)]
                + [("cogvideox", i, 2) for i in range(2)])


@pytest.mark.parametrize("name,part,n_parts", ONLINE_PARTS)
def test_online_layer_every_head(name, part, n_parts, workload_inputs):
    banner("full-size layer", name, "part", part)
    r = _online(name, workload_inputs)
    w = r["w"]
    heads = _parts(w.H, n_parts)[part]
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    p = O.token_major_index(w.F, w.Hs, w.Ws, w.N)
    must = [928] if name == "hunyuan720p" else []
    worst = [0.0, 0.0, 0.0]
    for h in heads:
        lay = int(r["choice"][h])
        qbs = sample_qblocks(w.n_blocks, seed=w.seed * 100 + h, n=N_QBLOCKS, must=must)
        ref, ref_lse = O.head_attention(r["q"][0, h].float().numpy(), r["k"][0, h].float().numpy(),
                                        r["v"][0, h].float().numpy(), cand[lay], lay, w.F, w.Hs,
                                        w.Ws, w.block, w.scale, qblocks=qbs)
        rows = ~np.isnan(ref[:, 0])
        got = to_np(r["o"][0, h])[rows]
        mx, rl = attn_errors(got, ref[rows])
        g_lse = r["lse"][0, h].numpy()
        g_lse = g_lse[p] if lay == 1 else g_lse          # stored in the attended layout
        le = float(np.max(np.abs(g_lse[rows] - ref_lse[rows])))
        # without the LSE: the denominator summed on the matrix core
        got2 = to_np(r["o_nolse"][0, h])[rows]
        mx2, rl2 = attn_errors(got2, ref[rows])
        print(f"[parity] {name} head {h} ({'TS'[lay]}) {len(qbs)} blocks {int(rows.sum())} rows: "
              f"max-abs {mx:.3e} rel-L2 {rl:.3e} lse {le:.3e}; no-LSE call max-abs {mx2:.3e} rel-L2 {rl2:.3e}")
        worst = [max(worst[0], mx, mx2), max(worst[1], rl, rl2), max(worst[2], le)]
        assert mx <= ATTN_MAX_ABS and rl <= ATTN_REL_L2, f"{name} head {h}: {mx:.3e} {rl:.3e}"
        assert mx2 <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2, f"{name} head {h} (no LSE): {mx2:.3e} {rl2:.3e}"
        assert le <= LSE_ABS, f"{name} head {h}: lse error {le:.3e}"
    print(f"[worst] {name} heads {heads[0]}-{heads[-1]}: max-abs {worst[0]:.3e} rel-L2 {worst[1]:.3e} "
          f"lse {worst[2]:.3e}")


PROFILE_PARTS = ([("wan720p", i, 5) for i in range(5)] + [("hunyuan720p", i, 4) for i in range(4)]
                 + [("cogvideox", i, 2) for i in range(2)])


@pytest.mark.parametrize("name,part,n_parts", PROFILE_PARTS)
def test_profiler_choice_every_head(name, part, n_parts, workload_inputs):
    """The layer's own head choice (call t = 0) against the oracle's, head by head."""
    banner("full-size profiler", name, "part", part)
    r = _online(name, workload_inputs)
    w = r["w"]
    heads = _parts(w.H, n_parts)[part]
    cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
    idx = S.sample_query_idx(w, 0)
    worst = 0.0
    for h in heads:
        ref_c, ref_e = O.profile_heads(r["q"][0, h:h + 1].float().numpy(), r["k"][0, h:h + 1].float().numpy(),
                                       r["v"][0, h:h + 1].float().numpy(), w.F, w.Hs, w.Ws, w.block,
                                       w.scale, idx, cand)
        rel = np.abs(r["err"][h] - ref_e[0]) / np.maximum(ref_e[0], 1e-300)
        ratio = ref_e[0, 0] / max(ref_e[0, 1], 1e-300)
        print(f"[profile] {name} head {h}: choice {r['choice'][h]} oracle {ref_c[0]} "
              f"err ratio S/T {ratio:.3e} rel-err {rel.max():.3e}")
        worst = max(worst, float(rel.max()))
        assert r["choice"][h] == ref_c[0], f"{name} head {h}"
        assert np.all(rel < PROFILE_ERR_REL), (h, rel, r["err"][h], ref_e[0])
    print(f"[worst] {name} profiler heads {heads[0]}-{heads[-1]}: rel-err {worst:.3e}")


def _static(workload_inputs):
    if not _STATIC:
        w, q, k, v, _ = workload_inputs("static_wan720p")
        s = svg.Shape(w.B, w.H, w.N, w.D, w.F, w.Hs, w.Ws, w.block)
        E = np.stack([S.energy_matrix(w, h) for h in range(w.H)])
        dense = svg.svg_calibrate_masks(torch.from_numpy(E).to(DEV), w.eps)
        rep = S.repetitive_heads(w)
        sel = np.zeros(w.H, np.int32)
        sel[rep] = 1
        layer = svg.StaticSparseAttention(s, dense, torch.from_numpy(sel).to(DEV), w.k_anchors)
        o, lse = layer(q.to(DEV), k.to(DEV), v.to(DEV), lse=True)
        torch.cuda.synchronize()
        _STATIC.update(w=w, q=q, k=k, v=v, E=E, rep=rep, sel=sel, masks=dense.cpu().numpy(),
                       o=o.cpu(), lse=lse.cpu())
        del layer, o, lse, dense
        torch.cuda.empty_cache()
    return _STATIC


@pytest.mark.parametrize("part", range(5))
def test_static_layer_every_head(part, workload_inputs):
    """Plain heads on >= 32 query blocks; row-repetitive heads on four whole
    frames (anchor blocks from the oracle, the other rows broadcast)."""
    banner("full-size static", part)
    r = _static(workload_inputs)
    w = r["w"]
    S_ = w.Hs * w.Ws
    anchors = np.unique(O.anchor_rows(w.Hs, w.k_anchors))
    worst = [0.0, 0.0, 0.0]
    for h in _parts(w.H, 5)[part]:
        qh, kh, vh = (r[t][0, h].float().numpy() for t in ("q", "k", "v"))
        g = to_np(r["o"][0, h])
        g_lse = r["lse"][0, h].numpy()
        if r["sel"][h]:
            rng = np.random.default_rng(w.seed * 100 + h)
            frames = sorted(set([0, w.F - 1] + rng.choice(w.F, 2, replace=False).tolist()))
            tok = np.array([f * S_ + a * w.Ws + x for f in frames for a in anchors for x in range(w.Ws)])
            qbs = np.unique(tok // w.block).tolist()
            ref, ref_lse = O.block_masked_attention(qh, kh, vh, r["masks"][h], w.block, w.scale, qbs)
            want = O.row_broadcast(np.nan_to_num(ref), w.F, w.Hs, w.Ws, w.k_anchors)
            rows = np.concatenate([np.arange(f * S_, (f + 1) * S_) for f in frames])
            mx, rl = attn_errors(g[rows], want[rows])
            le = float(np.max(np.abs(g_lse[tok] - ref_lse[tok])))
            what = f"repetitive, frames {frames}, {len(qbs)} anchor blocks"
        else:
            qbs = sample_qblocks(w.n_blocks, seed=w.seed * 100 + h, n=N_QBLOCKS)
            ref, ref_lse = O.block_masked_attention(qh, kh, vh, r["masks"][h], w.block, w.scale, qbs)
            rows = ~np.isnan(ref[:, 0])
            mx, rl = attn_errors(g[rows], ref[rows])
            le = float(np.max(np.abs(g_lse[rows] - ref_lse[rows])))
            what = f"{len(qbs)} blocks"
        print(f"[parity] static head {h} ({what}): max-abs {mx:.3e} rel-L2 {rl:.3e} lse {le:.3e}")
        worst = [max(worst[0], mx), max(worst[1], rl), max(worst[2], le)]
        assert mx <= ATTN_MAX_ABS and rl <= ATTN_REL_L2, f"static head {h}: {mx:.3e} {rl:.3e}"
        assert le <= LSE_ABS, f"static head {h}: lse error {le:.3e}"
    print(f"[worst] static part {part}: max-abs {worst[0]:.3e} rel-L2 {worst[1]:.3e} lse {worst[2]:.3e}")
