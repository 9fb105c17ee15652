#!/usr/bin/env python3
"""Benchmark of one block-sparse 3D attention layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan720p]

A step is one pass of the whole hot path over one synthetic layer input:
candidate-mask build and encoding, online head profiling on 64 sampled
queries, forward permutation of q/k/v for the temporal heads, block-sparse
attention, inverse permutation of the temporal heads' output (online
workloads); block-sparse attention plus anchor-row broadcast (the static
calibrated workload).  Inputs are resident in HBM before timing starts.

Prints one JSON line.  `value` is the effective TFLOP/s over the kept blocks
for the whole step (algorithmic FLOP of the attention / step time); the
attention kernel's own rate, per-call times and the roofline of the dominant
kernel (HIP events on the launch stream) are reported beside it, together with
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s on kept blocks + ms/attention layer, Wan-720p shape, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PMC_FILE = os.path.join(ROOT, "profiles", "attn_pmc_counters.json")
# the attention kernel's sources: its file and the two headers it includes
ATTN_SRCS = [os.path.join(ROOT, "block_sparse_attention_svg_amd", "csrc", f)
             for f in ("attn.hip", "attn_tiles.h", "mfma_common.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan720p",
                    choices=["tiny", "cogvideox", "wan720p", "hunyuan720p", "static_wan720p"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU oracle sample (0 disables it)")
    ap.add_argument("--sustained-seconds", type=float, default=2.0,
                    help="seconds of the dense-MFMA probe per data type (0 disables it)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain device copy of 1 GiB (HBM counter calibration)")
    return ap.parse_args()


def describe(w):
    return (f"{w.name}: 1 layer, B={w.B}, {w.H} heads, D={w.D}, {w.F}x{w.Hs}x{w.Ws}"
            f"{' + %d text' % w.text if w.text else ''} = {w.N} tokens, bf16, block {w.block}")


def code_hash(paths):
    """Hash of C++/HIP sources (in the given order) with their comments and
    whitespace removed: the counters recorded for the attention kernel stay
    valid across comment edits and are dropped as soon as its code changes."""
    import re
    h = hashlib.sha256()
    for path in paths:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = re.sub(r"\s+", "", text)
        h.update(os.path.basename(path).encode() + b"\0" + text.encode() + b"\0")
    return h.hexdigest()[:16]


def cpu_baseline(w, q, k, v, classes, budget_s):
    """fp64 oracle on a bounded sample: whole query blocks of one spatial and one
    temporal head, processed until the time budget is spent."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    import synth
    if w.mode == "static":
        masks = {h: O.calibrate_mask(synth.energy_matrix(w, h), w.eps) for h in (0, 1)}
        jobs = [(0, 0), (1, 0)]
    else:
        cand = O.online_candidate_masks(w.F, w.Hs, w.Ws, w.N, w.block, w.band_w)
        hs = int(np.nonzero(classes == 0)[0][0]) if (classes == 0).any() else 0
        ht = int(np.nonzero(classes == 1)[0][0]) if (classes == 1).any() else hs
        masks = {hs: cand[0], ht: cand[1]}
        jobs = [(hs, 0), (ht, 1)]
    sizes = np.array([min(w.N, (b + 1) * w.block) - b * w.block for b in range(w.n_blocks)])
    rng = np.random.default_rng(17)
    order = rng.permutation(w.n_blocks)
    flops = 0
    blocks = 0
    prepared = []
    for h, lay in jobs:
        qh, kh, vh = (t[0, h].float().numpy().astype(np.float64) for t in (q, k, v))
        if lay == 1:
            qh, kh, vh = (O.to_token_major(t, w.F, w.Hs, w.Ws) for t in (qh, kh, vh))
        prepared.append((qh, kh, vh, masks[h]))
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < budget_s and i < w.n_blocks:
        r = int(order[i])
        for qh, kh, vh, M in prepared:
            O.block_masked_attention(qh, kh, vh, M, w.block, w.scale, qblocks=[r])
            flops += 4 * w.D * int(sizes[r]) * int(sizes @ M[r].astype(np.int64))
            blocks += 1
        i += 1
    dt = time.perf_counter() - t0
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": (f"fp64 NumPy oracle, {blocks} whole query blocks ({i} per head) of one "
                      f"spatial and one temporal head, {flops / 1e9:.1f} GFLOP in {dt:.1f} s; "
                      f"host has {os.cpu_count()} cores"),
           "cpu_model": cpu_model(), "blas": blas_info(), "host_cores": os.cpu_count(),
           "attention_s_per_layer_est": round(dt / max(i, 1) * w.n_blocks * w.H / len(jobs), 1)}
    if w.mode == "online":
        # the profiler's oracle on one head (64 samples against every key), and
        # the permutation of one head's tensor, each scaled to the layer
        h = jobs[0][0]
        idx = synth.sample_query_idx(w, 0)
        qh, kh, vh = (t[0, h:h + 1].float().numpy() for t in (q, k, v))
        t1 = time.perf_counter()
        O.profile_heads(qh, kh, vh, w.F, w.Hs, w.Ws, w.block, w.scale, idx, cand)
        t_prof = time.perf_counter() - t1
        x = k[0, h].float().numpy().astype(np.float64)
        t1 = time.perf_counter()
        O.to_token_major(x, w.F, w.Hs, w.Ws)
        t_perm = time.perf_counter() - t1
        n_t = int((classes == 1).sum())
        out["profile"] = {"s_per_head": round(t_prof, 3), "s_per_layer": round(t_prof * w.H, 2),
                          "note": f"oracle profile_heads on one head x {w.H} heads"}
        out["permute"] = {"s_per_head": round(t_perm, 4), "s_per_layer": round(t_perm * n_t, 3),
                          "note": f"oracle to_token_major of one head's K (float64) x {n_t} temporal heads"}
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_info():
    try:
        from threadpoolctl import threadpool_info
        return [{"api": p.get("internal_api"), "threads": p.get("num_threads")} for p in threadpool_info()]
    except Exception:  # pragma: no cover
        return None


def norm_rope_leg(w, s, classes, dev, stream, reps=50):
    """QK-Norm + 3D RoPE of one projection tensor (query or key rows) into the
    attention input, each head in its layout, timed over `reps` calls after ten
    warm-up calls; beside it the same arithmetic as plain PyTorch eager ops (the
    pages' comparison point), its cos / sin table built outside the timing."""
    import torch
    import synth
    import block_sparse_attention_svg_amd as svg

    x = synth.gen_projection_rows(w.B, w.N, w.H, w.D, seed=w.seed + 5, device=dev)
    gamma = torch.from_numpy(synth.gen_norm_weight(w.H * w.D, w.seed + 6)).to(dev)
    third = w.D // 6
    rope = (w.D - 4 * third, 2 * third, 2 * third, 10000.0)
    lay = torch.from_numpy(np.tile(classes.astype(np.int32), w.B)).to(dev)
    y = svg.svg_qk_norm_rope(x, s, norm="row", gamma=gamma, rope=rope, head_layout=lay)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(10):
        svg.svg_qk_norm_rope(x, s, norm="row", gamma=gamma, rope=rope, head_layout=lay, out=y)
    e0.record(stream)
    for _ in range(reps):
        svg.svg_qk_norm_rope(x, s, norm="row", gamma=gamma, rope=rope, head_layout=lay, out=y)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 2 * x.numel() * x.element_size()              # read x once, write y once

    # plain PyTorch: fp32 norm, rotation by a cached table, transpose, layout gather
    S_ = w.Hs * w.Ws
    n = torch.arange(w.N, device=dev)
    f, sp = n // S_, n % S_
    pos = [f, sp // w.Ws, sp % w.Ws]
    ang = []
    for p_, d in zip(pos, rope[:3]):
        fr = rope[3] ** (-2.0 * torch.arange(d // 2, device=dev, dtype=torch.float64) / d)
        ang.append(p_[:, None].double() * fr[None, :])
    ang = torch.cat(ang, 1)
    ang[n >= w.F * S_] = 0
    cos, sin = ang.cos().float(), ang.sin().float()
    tm = torch.arange(w.N, device=dev)
    tm[: w.F * S_] = (sp * w.F + f)[: w.F * S_]
    g2 = gamma.view(w.H, w.D)

    def eager():
        xf = x.float()
        xn = xf * torch.rsqrt(xf.pow(2).mean(dim=(-2, -1), keepdim=True) + 1e-6) * g2
        a_, b_ = xn[..., 0::2], xn[..., 1::2]
        c_, s_ = cos[None, :, None, :], sin[None, :, None, :]
        r = torch.stack((a_ * c_ - b_ * s_, a_ * s_ + b_ * c_), -1).flatten(-2)
        r = r.to(torch.bfloat16).transpose(1, 2).contiguous()
        out = torch.empty_like(r)
        sel = lay.view(w.B, w.H).bool()
        out[~sel] = r[~sel]
        rs = r[sel]
        out[sel] = torch.empty_like(rs).index_copy_(1, tm, rs)
        return out

    ref = eager()
    e0.record(stream)
    for _ in range(3):
        eager()
    e1.record(stream)
    torch.cuda.synchronize()
    t_ms = e0.elapsed_time(e1) / 3
    diff = (ref.float() - y.float()).abs().max().item()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "bytes": nbytes, "torch_eager_ms": round(t_ms, 3), "speedup_vs_torch": round(t_ms / ms, 1),
            "max_abs_diff_vs_torch": round(diff, 4),
            "note": "one tensor (query or key rows) [B,N,H,D] -> [B,H,N,D]: RMS over the H*D row, "
                    f"rope runs {rope[:3]}, theta 1e4, temporal heads token-major; not part of the layer step"}


PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA


def phase(name, what):
    """Wall-clock stamp of a phase on stderr (lines up external power / clock
    samples with the work)."""
    print(f"[phase] {name} {what} {time.time():.3f}", file=sys.stderr, flush=True)


def sustained_mfma_leg(stream, seconds):
    """Dense MFMA rate the board sustains right after the timed steps, from
    svg_mfma_peak_probe (products on register operands only, one workgroup of
    8 waves per CU): bf16, then FP8, each launched back to back for `seconds`
    after one warm-up launch; rate = FLOP / event time."""
    import torch
    import block_sparse_attention_svg_amd as svg
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(n_cu * 512, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fp8, rounds in (("bf16", False, 2000), ("fp8", True, 1000)):   # about 1 ms per launch
        svg.svg_mfma_peak_probe(fp8, rounds, sink)
        torch.cuda.synchronize()
        phase(f"mfma probe {name}", "start")
        t0, flop, ms = time.time(), 0.0, 0.0
        while time.time() - t0 < seconds:
            e0.record(stream)
            for _ in range(20):
                flop += svg.svg_mfma_peak_probe(fp8, rounds, sink)
            e1.record(stream)
            torch.cuda.synchronize()
            ms += e0.elapsed_time(e1)
        phase(f"mfma probe {name}", "end")
        res[f"{name}_tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
    res["note"] = ("back-to-back 32x32 MFMAs on register operands, no memory or LDS traffic: the rate the "
                   "board's power limit allows for dense matrix work right now, on this GPU")
    return res


def fp8_leg(w, s, q, k, v, layer, flop, o_bf16, stream, reps=20):
    """The FP8 (E4M3) variant on the same layer input and head choice:
    svg_quantize_fp8 and svg_block_sparse_attn_fp8 each timed over `reps`
    calls after three warm-up calls; roofline against the FP8 dense peak;
    relative L2 distance of its output from the bf16 path's."""
    import torch
    import block_sparse_attention_svg_amd as svg
    ops8 = svg.svg_quantize_fp8(q, k, v, s, head_layout=layer.choice)
    ws = torch.empty(max(svg.svg_attn_workspace_bytes(s, True), 1), dtype=torch.uint8, device=q.device)
    o8 = torch.empty_like(q)

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    t_q = timed(lambda: svg.svg_quantize_fp8(q, k, v, s, head_layout=layer.choice, out=ops8))
    t_a = timed(lambda: svg.svg_block_sparse_attn_fp8(ops8, s, layer.scale, layer.cand, head_mask=layer.choice,
                                                       head_layout=layer.choice, out=o8, workspace=ws))
    d = (o8.float() - o_bf16.float())
    rl = float(d.norm() / o_bf16.float().norm())
    tf = flop / (t_a * 1e-3) / 1e12
    return {"attention_ms": round(t_a, 4), "attention_tflops": round(tf, 2),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_FP8_TFLOPS, 4)},
            "quantize_ms": round(t_q, 4), "rel_l2_vs_bf16": round(rl, 4),
            "note": "E4M3 q, k, v (one scale per tensor and head), E4M3 weights for PV, fp32 softmax; "
                    "same head choice and masks as the bf16 step; not part of the bf16 layer step"}


def permute_leg(w, s, x, head_sel, n_temporal, stream, reps=50):
    """svg_permute (frame-major -> token-major) of one tensor's temporal heads,
    timed alone over `reps` calls after five warm-up calls (not part of the
    fused layer step, where svg_prepare_kv moves K with V)."""
    import torch
    import block_sparse_attention_svg_amd as svg
    y = torch.empty_like(x)
    for _ in range(5):
        svg.svg_permute(x, s, head_sel, out=y)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        svg.svg_permute(x, s, head_sel, out=y)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    moved = 2 * n_temporal * w.N * w.D * 2
    gbs = moved / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "bytes": moved, "note": f"svg_permute of K, {n_temporal} temporal heads, read + write"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(heads shard with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import block_sparse_attention_svg_amd as svg

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(2)
    dev = "cuda"
    w = synth.get_workload(args.workload)
    q_c, k_c, v_c, classes = synth.gen_qkv(w, dtype="bf16")
    q, k, v = (t.to(dev) for t in (q_c, k_c, v_c))
    s = svg.Shape(w.B, w.H, w.N, w.D, w.F, w.Hs, w.Ws, w.block)
    scale = 1.0 / math.sqrt(w.D)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    if w.mode == "online":
        layer = svg.OnlineSparseAttention(s, w.band_w, scale=scale, n_samples=w.n_samples)
        n_idx = max(args.steps + args.warmup, 1)
        idx = [torch.from_numpy(synth.sample_query_idx(w, t)).to(dev) for t in range(n_idx)]
        names = ["masks", "profile", "layout", "attention", "unpermute"]
    else:
        E = torch.from_numpy(np.stack([synth.energy_matrix(w, h) for h in range(w.H)])).to(dev)
        dense = svg.svg_calibrate_masks(E, w.eps)
        del E
        sel = np.zeros(w.B * w.H, np.int32)
        sel[synth.repetitive_heads(w)] = 1
        layer = svg.StaticSparseAttention(s, dense, torch.from_numpy(sel).to(dev), w.k_anchors, scale)
        names = ["attention", "broadcast"]

    def step(t, ev):
        """One pass of the hot path; ev[i] records before call i (len(names)+1 events)."""
        if w.mode == "online":
            ev[0].record(stream)
            dm = svg.svg_build_masks(s, w.band_w, out=layer.dense_masks)
            layer.cand = svg.svg_encode_mask(dm)
            ev[1].record(stream)
            layer.profile(q, k, v, idx[t % len(idx)])
            ev[2].record(stream)
            layer.permute_inputs(q, k, v)
            ev[3].record(stream)
            layer.attend(q, k, v, out=o)
            ev[4].record(stream)
            layer.restore_output(o)
            ev[5].record(stream)
        else:
            ev[0].record(stream)
            svg.svg_block_sparse_attn(q, k, v, s, scale, layer.masks, out=o,
                                      workspace=layer.attn_workspace)
            ev[1].record(stream)
            svg.svg_row_broadcast(o, s, layer.repetitive, layer.k)
            ev[2].record(stream)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
    for t in range(args.warmup):
        step(t, mk())
    torch.cuda.synchronize()

    # algorithmic FLOP of the attention call (kept blocks of each head's mask)
    if w.mode == "online":
        head_mask = layer.choice.cpu().numpy().tolist()
        flop = svg.attention_flops(layer.cand, head_mask, w.N, w.block, w.D)
        n_temporal = int(sum(head_mask))
    else:
        flop = svg.attention_flops(layer.masks, list(range(w.H)), w.N, w.block, w.D)
        n_temporal = 0

    evs = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    phase("timed steps", "start")
    t_start.record(stream)
    for t in range(args.steps):
        step(args.warmup + t, evs[t])
    t_end.record(stream)
    torch.cuda.synchronize()
    phase("timed steps", "end")
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    per = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}
    per_med = {n: float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}
    step_med = float(np.median([e[0].elapsed_time(e[-1]) for e in evs]))

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    attn_ms = per["attention"]
    achieved = flop / (attn_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(PMC_FILE):
        try:
            pmc = json.load(open(PMC_FILE))
            key = w.name
            if pmc.get("attn_code_sha") == code_hash(ATTN_SRCS) and key in pmc.get("workloads", {}):
                traffic = pmc["workloads"][key]["hbm_bytes_per_launch"]
        except Exception:
            traffic = None

    out = {
        "metric": METRIC,
        "value": round(flop / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator; no model weights)",
        "config": {"workload": describe(w), "heads_temporal": n_temporal,
                   "heads_spatial": w.H - n_temporal, "profiler_samples": w.n_samples,
                   "attention_gflop": round(flop / 1e9, 2),
                   "layout": (("one svg_prepare_kv pass after the head choice (temporal heads' K token-major, "
                               "every head's V block-transposed in its layout); Q and O of temporal heads "
                               "through the permutation inside the attention call")
                              if w.mode == "online" and layer.fused_layout
                              else "svg_permute of q, k, v and of op" if w.mode == "online" else "frame-major")},
        "ms_per_step_median": round(step_med, 4),
        "timing": f"{args.warmup} warm-up steps, then {args.steps} timed steps; HIP events on the launch "
                  "stream around every call (mean and median over the timed steps)",
        "ms_per_call": {n: round(v, 4) for n, v in per.items()},
        "ms_per_call_median": {n: round(v, 4) for n, v in per_med.items()},
        "attention_tflops": round(achieved, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    if w.mode == "online":
        tensor_bytes = w.N * w.D * 2
        if layer.fused_layout:
            # K of the temporal heads and V of every head, each read and written once
            moved = 2 * (n_temporal + w.B * w.H) * tensor_bytes
        else:
            moved = 2 * 3 * n_temporal * tensor_bytes            # q, k, v of the temporal heads
        out["layout_gbs"] = round(moved / (per["layout"] * 1e-3) / 1e9, 1)
        out["layout_hbm_frac"] = round(out["layout_gbs"] / PEAK_HBM_GBS, 4)
        out["layout_bytes"] = moved
        out["permute"] = permute_leg(w, s, k, layer.choice, n_temporal, stream)
        if w.block == 128:
            phase("fp8 leg", "start")
            out["fp8"] = fp8_leg(w, s, q, k, v, layer, flop, o, stream)
            phase("fp8 leg", "end")
        kv_bytes = 2 * w.B * w.H * tensor_bytes
        out["profile_gbs"] = round(kv_bytes / (per["profile"] * 1e-3) / 1e9, 1)
        out["profile_share"] = round(per["profile"] / ms_step, 4)
        out["qk_norm_rope"] = norm_rope_leg(w, s, classes, dev, stream)
    if w.mode == "static":
        # offline calibration's block-energy pass over every head, timed once
        # after a warm-up call (not part of the layer step)
        e_out = svg.svg_block_energy(q, k, s, scale)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        svg.svg_block_energy(q, k, s, scale, out=e_out)
        e1.record(stream)
        torch.cuda.synchronize()
        e_ms = e0.elapsed_time(e1)
        e_flop = 2.0 * w.B * w.H * w.N * w.N * w.D            # one Q K^T per head
        out["calibration_energy"] = {"ms": round(e_ms, 3), "tflops": round(e_flop / (e_ms * 1e-3) / 1e12, 2),
                                     "note": "block attention energies of all heads; FLOP = one QK^T "
                                             "(the kernel computes it twice: max/sum, then block sums)"}
        del e_out
        # and the row-repetitive head test over every head (row patterns + Gram)
        r_ws = torch.empty(svg.svg_row_similarity_workspace_bytes(s), dtype=torch.uint8, device=dev)
        svg.svg_row_similarity(q, k, s, scale, workspace=r_ws)
        e0.record(stream)
        r_score = svg.svg_row_similarity(q, k, s, scale, workspace=r_ws)
        e1.record(stream)
        torch.cuda.synchronize()
        r_ms = e0.elapsed_time(e1)
        out["calibration_rows"] = {"ms": round(r_ms, 3),
                                   "tflops": round(e_flop / (r_ms * 1e-3) / 1e12, 2),
                                   "repetitive_heads": int((r_score > 0.87).sum().item()),
                                   "note": "row attention patterns of all heads + per-frame cosines; "
                                           "FLOP = one QK^T (computed twice)"}
        del r_ws
    if args.sustained_seconds > 0:
        sus = sustained_mfma_leg(stream, args.sustained_seconds)
        sus["attention_frac_of_bf16"] = round(achieved / sus["bf16_tflops"], 4)
        if "fp8" in out:
            sus["fp8_attention_frac_of_fp8"] = round(out["fp8"]["attention_tflops"] / sus["fp8_tflops"], 4)
        out["mfma_sustained"] = sus
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(w, q_c, k_c, v_c, classes, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
