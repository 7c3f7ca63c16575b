#!/usr/bin/env python
"""Benchmark of the PACK3D local-global attention forward on one MI355X.

One step = one ``pack3d_forward`` over the whole synthetic workload (its four
launches: the block pass building the summaries and rotating K_loc, the
per-group summary-norm maximum with the rotary table, local attention and
query->summary attention, each rotating Q in registers and adding its gated
share to the output), inputs resident in HBM.  Prints ONE JSON line with the
throughput in tokens/s, the roofline position of the dominant kernel
(k_global_attn, bf16 MFMA), per-kernel figures, and the fp64 CPU oracle timed
on a bounded sample of the same workload on this host's cores.  A second leg
("training") times the training forward plus the backward (all six input
gradients) on the same inputs with a seeded upstream gradient, and a third
("layer") the layer around the operator: LayerNorm + the five projections
with RoPE, the operator, the output projection + residual (width Hq*64), and
a fourth ("c4_1m_random") the 1 048 576-token random-packing forward beside
dense axial-RoPE attention on the same inputs.  The step time is the median
over the timed steps; a plain 1 GiB device copy reports the achievable HBM
bandwidth beside the 8 TB/s peak.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--dense]
                    [--no-backward] [--no-layer] [--no-c4] [--summary-mode MODE]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthgen as sg  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0                # MI355X HBM3E
METRIC = "PACK3D attention fwd tokens/sec at 262k tokens; % bf16 MFMA peak; HBM GB/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_global_attn_block_bf16_64x64x64_hbm_traffic.txt")
GLOBAL_SOURCES = [os.path.join(ROOT, "geometry_aware_local_amd", "csrc", f)
                  for f in ("global_attn.hip", "pack3d_device.h", "local_tiles.h")]


def source_sha(paths) -> str:
    """Hash of the compressed kernel's sources and of the compiler flags its
    file is built with (the counters belong to that build only)."""
    from geometry_aware_local_amd import build as gb
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    flags = [f for f in gb.FLAGS + gb.FILE_FLAGS.get("global_attn.hip", [])
             if f != "-I" and not os.path.isabs(f)]     # include paths vary by checkout
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per k_global_attn launch from the committed counter summary,
    or None if it is missing or the kernel source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    sha = re.search(r"^source_sha256_16:\s*(\w+)", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch:\s*([\d.eE+]+)", text, re.M)
    if not sha or not val or sha.group(1) != source_sha(GLOBAL_SOURCES):
        return None
    return float(val.group(1))


def window_pairs(grid, window) -> int:
    """Sum over all cells of the clipped box window's size.  The clipped box
    is a product of per-axis intervals, so the sum factors over the axes."""
    total = 1
    for n, wa in zip(grid, window):
        r = wa // 2
        total *= sum(min(c + r, n - 1) - max(c - r, 0) + 1 for c in range(n))
    return total


def algorithmic(w: sg.Workload) -> dict:
    """Work each step must do, per kernel (what the method moves or computes)."""
    n, hq, hkv, m = w.n_tokens, w.n_q_heads, w.n_kv_heads, w.n_blocks
    es = 2 if w.dtype == "bf16" else 4
    nbr = window_pairs(w.grid, w.window)
    return {
        # summary: read K_cmp, V_cmp, a, cell_to_pos; write K~, V~
        "summary_bytes": 2 * n * hkv * 64 * es + n * hkv * 4 + n * 4 + 2 * hkv * m * 64 * es,
        # the forward's block pass: the summaries, their norms, and K_loc read,
        # rotated and written
        "block_pass_bytes": (2 * n * hkv * 64 * es + n * hkv * 4 + n * 4 + 2 * hkv * m * 64 * es
                             + hkv * m * 4 + 2 * n * hkv * 64 * es),
        # the compressed kernel's HBM streams: Q read (unrotated) with coords,
        # the local share read and the output written, the summaries once
        "global_bytes": 3 * n * hq * 64 * es + n * 12 + 2 * hkv * m * 64 * es,
        # local: QK^T and PV over every clipped window
        "local_flops": 4 * nbr * hq * 64,
        # global: QK^T and PV against all M summaries: 256 flops per (row, summary)
        "global_flops": 4 * n * hq * m * 64,
        # backward, per (row, key) pair of either branch: recompute S = QK^T,
        # dP = dO V^T, dQ = dS K, dK = dS^T Q, dV = P^T dO: 5 products of
        # 2 * 64 flops (the usual 2.5x of the forward's two)
        "local_bwd_flops": 10 * nbr * hq * 64,
        "global_bwd_flops": 10 * n * hq * m * 64,
    }


def cpu_baseline(w: sg.Workload, inp: sg.Inputs, rows: int) -> dict:
    """The fp64 oracle on a bounded sample: rotated keys and summaries in full,
    both branches and the gate for `rows` sampled query tokens; the whole-job
    time is extrapolated linearly in the number of query tokens."""
    import threadpoolctl
    from oracle import pack3d_oracle as orc
    cores = len(os.sched_getaffinity(0))
    blas = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    threads = min(cores, blas)
    sel = np.sort(np.random.default_rng(0).choice(w.n_tokens, rows, replace=False))
    limiter = threadpoolctl.threadpool_limits(limits=threads)
    t0 = time.perf_counter()
    k_rot = orc.rotate(inp.k_loc, inp.coords, w.rope_pairs, w.rope_base)
    ks, vs = orc.block_summaries(inp.k_cmp, inp.v_cmp, inp.a, inp.coords, w.grid, w.block,
                                 w.rope_pairs, w.rope_base)
    t1 = time.perf_counter()
    q_rot = orc.rotate(inp.q[sel], inp.coords[sel], w.rope_pairs, w.rope_base)
    ol, _ = orc.local_attention(q_rot, k_rot, inp.v_loc, inp.coords, w.grid, w.window, 0.125,
                                sel, q_is_rows=True)
    oc, _ = orc.global_attention(q_rot, ks, vs, 0.125, q_is_rows=True)
    orc.gate_mix(ol, oc, inp.gate[sel])
    t2 = time.perf_counter()
    limiter.restore_original_limits()
    whole = (t1 - t0) + (t2 - t1) * w.n_tokens / rows
    return {"value": w.n_tokens / whole, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "affinity_cores": cores, "cpu_model": cpu_model(),
            "threads_note": "BLAS threads (the oracle's only parallel part), capped at the "
                            "process's CPU affinity",
            "sample": f"{rows} of {w.n_tokens} query tokens (all heads), rotated keys and "
                      f"summaries in full; {t2 - t0:.1f} s measured, whole job extrapolated "
                      f"linearly in query tokens to {whole:.0f} s"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_probe(torch) -> dict:
    """Achievable HBM bandwidth on this GPU: a plain device copy of 1 GiB
    (read + write), median of 10 timed copies."""
    x = torch.empty(256 << 20, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    ts = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        y.copy_(x)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    del x, y
    gbs = 2 * (1 << 30) / (ms * 1e-3) / 1e9
    return {"bytes": 2 * (1 << 30), "ms": ms, "gbs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}


def c4_leg(pk, torch, steps) -> dict:
    """The 1 048 576-token workload (random packing, M = 65 536): the forward,
    and dense axial-RoPE attention on the same inputs, for the speedup of
    PACK3D over dense attention.  The dense time is the same forward with
    1x1x1 blocks and a = 1 (m = N: every token its own summary, so the
    compressed branch is dense attention over all rotated keys, on the same
    kernel path; the local branch it also runs is < 0.1% of that time)."""
    w = sg.WORKLOADS["random_bf16_64x128x128"]
    print(f"[bench] C4 leg: {w.name}, generating inputs", file=sys.stderr, flush=True)
    inp = sg.make_inputs(w)
    bf = torch.bfloat16
    dev = lambda x, t=None: None if x is None else (torch.from_numpy(x).to(t) if t else
                                                    torch.from_numpy(x)).cuda()
    q, k_loc, v_loc = dev(inp.q, bf), dev(inp.k_loc, bf), dev(inp.v_loc, bf)
    k_cmp, v_cmp = dev(inp.k_cmp, bf), dev(inp.v_cmp, bf)
    a, coords, c2p, gate = dev(inp.a), dev(inp.coords), dev(inp.cell_to_pos), dev(inp.gate)
    del inp
    prob = pk.make_problem(w.grid, w.n_q_heads, w.n_kv_heads, w.window, w.block, bf,
                           w.rope_pairs, w.rope_base)
    fargs = (prob, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, c2p, gate)
    ws = pk.alloc_workspace(prob, q.device)
    out = torch.empty_like(q)
    pk.pack3d_forward(*fargs, workspace=ws, out=out)
    ts = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pk.pack3d_forward(*fargs, workspace=ws, out=out)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    f_ms = float(np.median(ts))
    del ws, out
    dprob = pk.make_problem(w.grid, w.n_q_heads, w.n_kv_heads, w.window, (1, 1, 1), bf,
                            w.rope_pairs, w.rope_base)
    dargs = (dprob, q, k_loc, v_loc, k_cmp, v_cmp, None, coords, c2p, gate)
    dws = pk.alloc_workspace(dprob, q.device)
    dout = torch.empty_like(q)
    pk.pack3d_forward(*dargs, workspace=dws, out=dout)          # warm
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    pk.pack3d_forward(*dargs, workspace=dws, out=dout)
    e1.record()
    torch.cuda.synchronize()
    d_ms = e0.elapsed_time(e1)
    del dws, dout
    n = w.n_tokens
    g_flops = 4 * n * w.n_q_heads * w.n_blocks * 64
    d_flops = 4 * n * w.n_q_heads * n * 64
    print(f"[bench] C4: forward {f_ms:.2f} ms, dense {d_ms:.1f} ms, speedup {d_ms / f_ms:.1f}x",
          file=sys.stderr, flush=True)
    return {"workload": w.name, "tokens": n, "forward_ms": f_ms, "forward_steps": steps,
            "tokens_per_s": n / (f_ms * 1e-3),
            "compressed_branch_tflop": g_flops / 1e12,
            "dense_ms": d_ms, "dense_tflops": d_flops / (d_ms * 1e-3) / 1e12,
            "speedup_pack3d_vs_dense": d_ms / f_ms}


def training_leg(pk, torch, w, inp, dev, dt, fargs, ws, out, args, work, peak_mfma) -> dict:
    """Training forward (saves both branches' outputs and log-sum-exp) and the
    backward (dq, dk_loc, dv_loc, dk_cmp, dv_cmp, dgate), timed with events on
    the launch stream around each call."""
    print("[bench] training leg: forward_train + backward", file=sys.stderr, flush=True)
    dout = dev(sg.make_upstream_grad(inp), dt)
    bws = torch.empty(pk.pack3d_backward_workspace_size(fargs[0]), dtype=torch.uint8,
                      device="cuda")
    out_t, saved = pk.pack3d_forward_train(*fargs, workspace=ws, out=out)
    grads = pk.pack3d_backward(*fargs, saved, dout, workspace=bws)
    for _ in range(max(args.warmup - 1, 0)):
        pk.pack3d_forward_train(*fargs, workspace=ws, saved=saved, out=out_t)
        pk.pack3d_backward(*fargs, saved, dout, workspace=bws, grads=grads)
    steps = max(args.steps // 2, 1)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record()
        pk.pack3d_forward_train(*fargs, workspace=ws, saved=saved, out=out_t)
        e[1].record()
        pk.pack3d_backward(*fargs, saved, dout, workspace=bws, grads=grads)
        e[2].record()
    torch.cuda.synchronize()
    f_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    b_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    bwd_flops = work["local_bwd_flops"] + work["global_bwd_flops"]
    print(f"[bench] training: forward_train {f_ms:.3f} ms, backward {b_ms:.3f} ms",
          file=sys.stderr, flush=True)
    return {"steps": steps, "forward_train_ms": f_ms, "backward_ms": b_ms,
            "tokens_per_s": w.n_tokens / ((f_ms + b_ms) * 1e-3),
            "backward_algorithmic_tflop": bwd_flops / 1e12,
            "backward_tflops": bwd_flops / (b_ms * 1e-3) / 1e12,
            "backward_frac": bwd_flops / (b_ms * 1e-3) / 1e12 / peak_mfma}


def layer_leg(pk, torch, w, inp, fargs, args, peak_mfma) -> dict:
    """The layer around the operator on the same lattice: width C = Hq*64,
    h and the weights from synthgen.make_layer_inputs; timed with events on
    the launch stream around the whole layer and around its two projections
    (the split entry points, run separately)."""
    print("[bench] layer leg", file=sys.stderr, flush=True)
    prob, coords, c2p, a, gate = fargs[0], fargs[7], fargs[8], fargs[6], fargs[9]
    L = sg.make_layer_inputs(inp)
    bf = torch.bfloat16
    h = torch.from_numpy(L.h).to(bf).cuda()
    gamma, beta = torch.from_numpy(L.gamma).cuda(), torch.from_numpy(L.beta).cuda()
    w_qkv, w_o = torch.from_numpy(L.w_qkv).to(bf).cuda(), torch.from_numpy(L.w_o).to(bf).cuda()
    n, c = w.n_tokens, L.h.shape[1]
    ws = torch.empty(pk.pack3d_layer_workspace_size(prob, c), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(h)
    run = lambda: pk.pack3d_layer_forward(prob, h, gamma, beta, w_qkv, w_o, a, coords, c2p, gate,
                                          workspace=ws, out=out)
    for _ in range(max(args.warmup, 1)):
        run()
    steps = max(args.steps // 2, 1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # the projections alone (split entry points)
    qkv = pk.pack3d_layernorm_qkv(prob, h, gamma, beta, w_qkv, coords)
    o = torch.empty((n, w.n_q_heads * 64), dtype=bf, device="cuda").normal_()
    pk.pack3d_out_proj(prob, o, w_o, h)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        qkv = pk.pack3d_layernorm_qkv(prob, h, gamma, beta, w_qkv, coords)
    e1.record()
    torch.cuda.synchronize()
    ms_qkv = e0.elapsed_time(e1) / steps
    e0.record()
    for _ in range(steps):
        pk.pack3d_out_proj(prob, o, w_o, h)
    e1.record()
    torch.cuda.synchronize()
    ms_out = e0.elapsed_time(e1) / steps
    cout = (w.n_q_heads + 4 * w.n_kv_heads) * 64
    fl_qkv, fl_out = 2 * n * c * cout, 2 * n * w.n_q_heads * 64 * c
    print(f"[bench] layer {ms:.3f} ms (layernorm+qkv {ms_qkv:.3f}, out_proj {ms_out:.3f})",
          file=sys.stderr, flush=True)
    del qkv
    return {"steps": steps, "width": c, "ms": ms, "tokens_per_s": n / (ms * 1e-3),
            "layernorm_qkv_ms": ms_qkv, "layernorm_qkv_tflops": fl_qkv / (ms_qkv * 1e-3) / 1e12,
            "out_proj_ms": ms_out, "out_proj_tflops": fl_out / (ms_out * 1e-3) / 1e12,
            "out_proj_gbs": 3 * n * c * 2 / (ms_out * 1e-3) / 1e9}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="block_bf16_64x64x64", choices=sorted(sg.WORKLOADS))
    ap.add_argument("--cpu-rows", type=int, default=16384)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dense", action="store_true",
                    help="also time dense axial-RoPE attention (1x1x1 blocks) on the same inputs")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the training leg (forward_train + backward)")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the layer leg (LayerNorm + projections, operator, output proj)")
    ap.add_argument("--no-c4", action="store_true",
                    help="skip the 1M-token leg (forward + dense axial-RoPE companion)")
    ap.add_argument("--summary-mode", default="token", choices=("token", "centre", "blind"),
                    help="compressed-branch variant (token: the exact rotate-before-sum form)")
    ap.add_argument("--profile-only", action="store_true",
                    help="for counter runs: a known-size copy probe, then 3 forwards")
    ap.add_argument("--profile-backward", action="store_true",
                    help="with --profile-only: 3 training forwards + backwards instead")
    ap.add_argument("--profile-layer", action="store_true",
                    help="with --profile-only: 3 whole layers (LayerNorm + projections, "
                         "operator, output projection) instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the operator's "
              "multi-GPU sharding is a design note, not built", file=sys.stderr)
        return 2

    import torch
    from geometry_aware_local_amd import pack3d as pk
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        return 1

    w = sg.WORKLOADS[args.workload].with_(summary_mode=args.summary_mode)
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    inp = sg.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = lambda x, t=None: None if x is None else torch.from_numpy(x).to(t).cuda() if t else \
        torch.from_numpy(x).cuda()
    q, k_loc, v_loc = dev(inp.q, dt), dev(inp.k_loc, dt), dev(inp.v_loc, dt)
    k_cmp, v_cmp = dev(inp.k_cmp, dt), dev(inp.v_cmp, dt)
    a, coords, c2p, gate = dev(inp.a), dev(inp.coords), dev(inp.cell_to_pos), dev(inp.gate)
    prob = pk.make_problem(w.grid, w.n_q_heads, w.n_kv_heads, w.window, w.block, dt,
                           w.rope_pairs, w.rope_base, summary_mode=w.summary_mode)
    ws = pk.alloc_workspace(prob, q.device)
    out = torch.empty_like(q)
    n = w.n_tokens
    fargs = (prob, q, k_loc, v_loc, k_cmp, v_cmp, a, coords, c2p, gate)

    if args.profile_only:
        x = torch.empty(64 << 20, dtype=torch.float32, device="cuda")    # 256 MiB
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)           # copy probe: reads and writes 256 MiB
        if args.profile_layer:
            L = sg.make_layer_inputs(inp)
            bf = torch.bfloat16
            lh = torch.from_numpy(L.h).to(bf).cuda()
            lg, lb = torch.from_numpy(L.gamma).cuda(), torch.from_numpy(L.beta).cuda()
            lq, lo = torch.from_numpy(L.w_qkv).to(bf).cuda(), torch.from_numpy(L.w_o).to(bf).cuda()
            for _ in range(3):
                pk.pack3d_layer_forward(prob, lh, lg, lb, lq, lo, a, coords, c2p, gate)
        elif args.profile_backward:
            dout = dev(sg.make_upstream_grad(inp), dt)
            saved, grads = None, None
            for _ in range(3):
                _, saved = pk.pack3d_forward_train(*fargs, workspace=ws, saved=saved, out=out)
                grads = pk.pack3d_backward(*fargs, saved, dout, grads=grads)
        else:
            for _ in range(3):
                pk.pack3d_forward(*fargs, workspace=ws, out=out)
        torch.cuda.synchronize()
        print("[bench] profile-only run done", file=sys.stderr, flush=True)
        return 0

    for _ in range(args.warmup):
        pk.pack3d_forward(*fargs, workspace=ws, out=out)
    # timed region: every step records an event before and after each stage,
    # on the stream the kernels run on
    nev = pk.PACK3D_FORWARD_STAGES + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)]
              for _ in range(args.steps)]
    for evs in events:
        for e in evs:
            e.record()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for evs in events:
        pk.pack3d_forward_timed(*fargs, evs, workspace=ws, out=out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    # per step: first event to last event of that step; the step time is the
    # median over the timed steps, each stage's time too
    step_ms = [evs[0].elapsed_time(evs[-1]) for evs in events]
    ms = float(np.median(step_ms))
    mean_ms = events[0][0].elapsed_time(events[-1][-1]) / args.steps
    stage_ms = [float(np.median([evs[i].elapsed_time(evs[i + 1]) for evs in events]))
                for i in range(nev - 1)]
    stages = dict(zip(pk.FORWARD_STAGE_NAMES, stage_ms))
    print(f"[bench] forward {ms:.3f} ms/step median (mean {mean_ms:.3f}, wall "
          f"{1e3 * wall / args.steps:.3f}); " +
          ", ".join(f"{k} {v:.3f}" for k, v in stages.items()), file=sys.stderr, flush=True)

    work = algorithmic(w)
    es = 2 if w.dtype == "bf16" else 4
    peak_mfma = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    gbs = lambda b, t: b / (t * 1e-3) / 1e9
    tfl = lambda f, t: f / (t * 1e-3) / 1e12
    # kernel serving each stage (see pack3d_backend_info)
    fast_local = w.dtype == "bf16" and w.n_q_heads // w.n_kv_heads in (4, 8, 16)
    local_kernel = (("k_local_zrun" if w.window[0] == 3 else "k_local_bf16") if fast_local
                    else "k_local_attn")
    kernels = {
        # one pass over the blocks: summaries with their norms + RoPE of K_loc
        "k_block_summary(+rope k_loc)": {"ms": stages["block_pass"], "bound": "hbm",
                                         "gbs": gbs(work["block_pass_bytes"],
                                                    stages["block_pass"])},
        "k_kmax(+rope table)": {"ms": stages["kmax+rope_table"], "bound": "launch"},
        # query->summary attention, RoPE of Q and the compressed gated share
        "k_global_attn(gated)": {"ms": stages["global_attn+gate"], "bound": "mfma",
                                 "tflops": tfl(work["global_flops"], stages["global_attn+gate"]),
                                 "hbm_gbs": gbs(work["global_bytes"],
                                                stages["global_attn+gate"])},
        local_kernel: {"ms": stages["local_attn"], "bound": "mfma",
                       "tflops": tfl(work["local_flops"], stages["local_attn"])},
    }
    for v in kernels.values():
        if v["bound"] == "hbm":
            v["frac"] = v["gbs"] / HBM_PEAK_GBS
        elif v["bound"] == "mfma":
            v["frac"] = v["tflops"] / peak_mfma
    g_tflops = kernels["k_global_attn(gated)"]["tflops"]

    extra = {}
    if args.dense:
        # dense axial-RoPE attention on the same inputs: the same forward
        # with 1x1x1 blocks and a = 1 (m = N), on the same kernel path
        dprob = pk.make_problem(w.grid, w.n_q_heads, w.n_kv_heads, w.window, (1, 1, 1), dt,
                                w.rope_pairs, w.rope_base)
        dargs = (dprob, q, k_loc, v_loc, k_cmp, v_cmp, None, coords, c2p, gate)
        dws = pk.alloc_workspace(dprob, q.device)
        dout = torch.empty_like(q)
        pk.pack3d_forward(*dargs, workspace=dws, out=dout)
        torch.cuda.synchronize()
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        pk.pack3d_forward(*dargs, workspace=dws, out=dout)
        b1.record()
        torch.cuda.synchronize()
        dms = b0.elapsed_time(b1)
        del dws, dout
        dfl = 4 * n * w.n_q_heads * n * 64
        extra["dense_companion"] = {
            "ms": dms, "tflops": tfl(dfl, dms), "frac": tfl(dfl, dms) / peak_mfma,
            "speedup_pack3d_vs_dense": dms / ms}

    hbm = copy_probe(torch)
    print(f"[bench] copy probe: {hbm['gbs']:.0f} GB/s", file=sys.stderr, flush=True)

    training = None
    if not args.no_backward and w.dtype == "bf16":   # the backward takes bf16
        training = training_leg(pk, torch, w, inp, dev, dt, fargs, ws, out, args, work, peak_mfma)

    layer = None
    if not args.no_layer and w.dtype == "bf16":     # the layer takes bf16
        layer = layer_leg(pk, torch, w, inp, fargs, args, peak_mfma)

    c4 = None
    if not args.no_c4 and w.name == "block_bf16_64x64x64":
        c4 = c4_leg(pk, torch, max(args.steps // 4, 2))

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, inp, min(args.cpu_rows, n))

    line = {
        "metric": METRIC,
        "value": n / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_mean": mean_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "grid": list(w.grid), "tokens": n, "packing": w.packing,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": 64,
                   "window": list(w.window), "block": list(w.block), "summaries": w.n_blocks,
                   "summary_mode": w.summary_mode, "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "kernel": "k_global_attn (gated, in the forward)",
                     "achieved": g_tflops, "peak": peak_mfma, "unit": "TFLOP/s",
                     "frac": g_tflops / peak_mfma, "traffic": measured_traffic()},
        "cpu_baseline": cpu,
        "kernels": kernels,
        "hbm_copy_probe": hbm,
        "training": training,
        "layer": layer,
        "c4_1m_random": c4,
        **extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
