#!/usr/bin/env python3
"""Benchmark: one full MuonClip optimizer step for one MoE layer on one MI355X.

Workload (synthetic, seeded, resident in HBM before timing):
  * 384 experts x {gate 2048x7168, up 2048x7168, down 7168x2048} bf16 weights
    ~N(0, 0.02) with float32 momentum and gradients ~N(0, 1e-4), plus the MLA
    attention projections W_q 12288x7168, W_kc 8192x7168, W_kr 64x7168
    (4 random heads x6 so they exceed tau);
  * Q / K of 8 x 4096 tokens through those projections (64 heads, 128 + 64
    head dim), computed before timing: the max logit is measured on them.
One step = every row of the path, on one stream, in a training step's order:
  per-head max logit on the forward's Q / K -> per shape group and chunk of
  64 matrices, one fused call: momentum, Newton-Schulz x 5 with the Muon
  scale, decoupled-decay update (--unfused: momentum over all matrices in one
  launch, then Newton-Schulz and the update as separate calls) -> QK-Clip of
  W_q / W_kc with that S_max.

Prints one JSON line on stdout (progress goes to stderr).  `value` is the
step's MFMA work divided by the step time, counting what the method needs:
per matrix and Newton-Schulz iteration 3n^2m + n^3 (X X^T and A A are
symmetric, so half of each is redundant; B'X is 2n^2m), plus 2 B H Sq Sk d
for the max logit.  The dense count 4n^2m + 2n^3 is reported beside it.  `roofline` covers the dominant kernel, timed per launch with HIP
events on the library's stream.  `cpu_baseline` times the fp64 oracle on a
bounded sample of the same workload.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MuonClip step: NS + max-logit TFLOP/s (MFMA util), rescale GB/s"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
HBM_PEAK_GBPS = 8000.0

D_MODEL, D_EXPERT, N_HEADS, D_NOPE, D_ROPE, D_V = 7168, 2048, 64, 128, 64, 128
LR, WD, MU, TAU, ALPHA = 2e-4, 0.1, 0.95, 100.0, 0.5


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "ns_gemm_kernel2_traffic_muonclip_step.md")
GEMM_SOURCE = os.path.join(ROOT, "muonclip_muon_amd", "csrc", "ns_gemm.hip")


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, or None when it is missing or the kernel source changed
    since the counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
        src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    vals = dict(line.split(":", 1) for line in text.splitlines()
                if line.startswith(("traffic_bytes_per_launch:", "kernel_source_sha256_16:")))
    if vals.get("kernel_source_sha256_16", "").strip() != src:
        return None
    return float(vals["traffic_bytes_per_launch"])


def ns_flops(rows, cols, steps):
    """Dense (nominal) Newton-Schulz flops: 4n^2m + 2n^3 per iteration."""
    n, m = min(rows, cols), max(rows, cols)
    return steps * (4 * n * n * m + 2 * n ** 3)


def ns_flops_sym(rows, cols, steps):
    """The method's Newton-Schulz work with the symmetric products counted
    once: X X^T n^2m, A A n^3, B'X 2n^2m per iteration."""
    n, m = min(rows, cols), max(rows, cols)
    return steps * (3 * n * n * m + n ** 3)


def gemm_flops_executed(rows, cols):
    """MFMA flops each GEMM of one iteration executes for one matrix: X X^T and
    A A compute the upper-triangle 256 x 256 tiles of the zero-padded matrix,
    B'X every tile."""
    n, m = min(rows, cols), max(rows, cols)
    n_pad, m_pad = -(-n // 256) * 256, -(-m // 256) * 256
    t = n_pad // 256
    tri = t * (t + 1) // 2
    return {0: tri * 2 * 256 * 256 * m_pad, 1: tri * 2 * 256 * 256 * n_pad, 2: 2 * n_pad * n_pad * m_pad}


class Workload:
    """Flat parameter buffers and the groups of equally shaped matrices."""

    def __init__(self, torch, experts, device, seed):
        import workloads
        self.groups = []  # (name, offset (elements), count, rows, cols)
        off = 0
        for name, count, rows, cols in (("expert_gate_up", 2 * experts, D_EXPERT, D_MODEL),
                                        ("expert_down", experts, D_MODEL, D_EXPERT),
                                        ("attn_q", 1, N_HEADS * (D_NOPE + D_ROPE), D_MODEL),
                                        ("attn_kc", 1, N_HEADS * D_NOPE, D_MODEL),
                                        ("attn_kr", 1, D_ROPE, D_MODEL)):
            self.groups.append((name, off, count, rows, cols))
            off += count * rows * cols
        self.numel = off
        log(f"allocating {self.numel / 1e9:.2f} G parameters: W bf16 {2 * off / 1e9:.1f} GB, "
            f"M and G float32 {8 * off / 1e9:.1f} GB")
        self.W = torch.empty(off, dtype=torch.bfloat16, device=device)
        self.M = torch.empty(off, dtype=torch.float32, device=device)
        self.G = torch.empty(off, dtype=torch.float32, device=device)
        gen = workloads.generator(seed, device)
        chunk = 1 << 28
        t0 = time.time()
        for s in range(0, off, chunk):
            e = min(off, s + chunk)
            self.W[s:e] = workloads.normal((e - s,), 0.02, gen, device, torch.bfloat16)
            self.M[s:e] = workloads.normal((e - s,), 1e-4, gen, device)
            self.G[s:e] = workloads.normal((e - s,), 1e-4, gen, device)
        torch.cuda.synchronize()
        log(f"filled in {time.time() - t0:.1f} s")
        # attention projections: the 4-hot-head MLA weights, and the forward's Q / K
        Wq, Wkc, Wkr, hot = workloads.mla_weights(seed=seed + 1, device=device)
        self.view("attn_q").copy_(Wq.view(1, *Wq.shape))
        self.view("attn_kc").copy_(Wkc.view(1, *Wkc.shape))
        self.view("attn_kr").copy_(Wkr.view(1, *Wkr.shape))
        self.hot = hot
        X = workloads.normal((8, 4096, D_MODEL), 1.0, workloads.generator(seed + 2, device), device,
                             torch.bfloat16)
        self.Q, self.Kc, self.Kr = workloads.mla_project(X, Wq, Wkc, Wkr, N_HEADS)
        del X, Wq, Wkc, Wkr
        # values for the forward that yields the max logit as a by-product
        self.V = workloads.normal((8, N_HEADS, 4096, D_V), 1.0, workloads.generator(seed + 3, device), device,
                                  torch.bfloat16)
        torch.cuda.synchronize()

    def group(self, name):
        return next(g for g in self.groups if g[0] == name)

    def view(self, name, buf=None, start=0, count=None):
        _, off, n, rows, cols = self.group(name)
        count = n - start if count is None else count
        buf = self.W if buf is None else buf
        s = off + start * rows * cols
        return buf[s:s + count * rows * cols].view(count, rows, cols)


def run(args):
    import torch

    import muonclip_muon_amd as mc

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    wl = Workload(torch, args.experts, dev, args.seed)
    steps_ns = mc.NS_STEPS

    chunk = args.chunk
    ws_bytes = max(mc.muon_ns_workspace_bytes(min(chunk, n), r, c) for _, _, n, r, c in wl.groups)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    o_elems = max(min(chunk, n) * r * c for _, _, n, r, c in wl.groups)
    O_buf = torch.empty(o_elems if args.unfused else 1, dtype=torch.bfloat16, device=dev)
    smax = torch.empty(N_HEADS, dtype=torch.float32, device=dev)
    gamma = torch.empty(N_HEADS, dtype=torch.float32, device=dev)
    clipped = torch.empty(N_HEADS, dtype=torch.int32, device=dev)
    B, H, Sq, dq = wl.Q.shape
    Sk = wl.Kc.shape[2]

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # NS calls of one step, and per-call event pairs
    ns_calls = []
    for name, off, n, rows, cols in wl.groups:
        for s in range(0, n, chunk):
            ns_calls.append((name, s, min(chunk, n - s), rows, cols))
    def new_events():
        """One step's events: per Newton-Schulz call its GEMMs' pairs, the call's
        pair (and the update's, unfused), and the max logit's and clip's pairs.
        Each timed step gets its own set, so no step waits for the host to
        read the previous one's."""
        return ([[ev() for _ in range(6 * steps_ns)] for _ in ns_calls],
                {k: (ev(), ev()) for k in ("momentum", "maxlogit", "clip")},
                [(ev(), ev()) for _ in ns_calls], [(ev(), ev()) for _ in ns_calls])

    gemm_ev, call_ev, upd_ev, ns_ev = new_events()

    def step(timed):
        # S_max^h comes from the forward pass that precedes the optimizer step
        # (measured at the weights before the update, applied after it)
        e = call_ev["maxlogit"]
        timed and e[0].record(stream)
        mc.qk_maxlogit(wl.Q, wl.Kc, wl.Kr, smax=smax)
        timed and e[1].record(stream)
        if args.unfused:
            e = call_ev["momentum"]
            timed and e[0].record(stream)
            mc.muonclip_momentum(wl.M, wl.G, MU)
            timed and e[1].record(stream)
        for k, (name, s, cnt, rows, cols) in enumerate(ns_calls):
            M = wl.view(name, wl.M, s, cnt)
            W = wl.view(name, wl.W, s, cnt)
            timed and ns_ev[k][0].record(stream)
            if not args.unfused:
                # momentum, Newton-Schulz and update of the chunk in one call
                mc.muon_momentum_ns_update_batched(M, wl.view(name, wl.G, s, cnt), W, LR, WD, MU,
                                                   workspace=workspace, gemm_events=gemm_ev[k] if timed else None)
                timed and ns_ev[k][1].record(stream)
                continue
            O = O_buf[:cnt * rows * cols].view(cnt, rows, cols)
            mc.muon_ns_orthogonalize_batched(M, O, workspace=workspace, out_scale=mc.muon_out_scale(rows, cols),
                                             gemm_events=gemm_ev[k] if timed else None)
            timed and ns_ev[k][1].record(stream)
            timed and upd_ev[k][0].record(stream)
            mc.muon_apply_update(W, O, LR, WD)
            timed and upd_ev[k][1].record(stream)
        e = call_ev["clip"]
        timed and e[0].record(stream)
        mc.qk_clip_apply(smax, wl.view("attn_q")[0], wl.view("attn_kc")[0], D_NOPE + D_ROPE, D_NOPE, D_NOPE,
                         TAU, ALPHA, gamma=gamma, clipped=clipped)
        timed and e[1].record(stream)

    log(f"{len(ns_calls)} Newton-Schulz calls per step; warmup {args.warmup}")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    # timed region: K steps bracketed by synchronisation
    acc = {"momentum": 0.0, "maxlogit": 0.0, "clip": 0.0, "ns": 0.0, "update": 0.0}
    gemm_ms = {0: [], 1: [], 2: []} if args.unfused else {0: [], 1: [], 2: [], "2u": []}
    gemm_flops = {k: [] for k in gemm_ms}       # the method's flops (symmetric products counted once)
    gemm_flops_nom = {k: [] for k in gemm_ms}   # dense 2 n^2 m / 2 n^3
    gemm_flops_exe = {k: [] for k in gemm_ms}   # what the MFMAs execute (tiles, padding)
    t_start, t_end = ev(), ev()
    step_events = [new_events() for _ in range(args.steps)]
    for g_ev, c_ev, u_ev, n_ev in step_events:  # torch creates an event at its first record
        for e in [e for pairs in g_ev for e in pairs] + [e for pair in c_ev.values() for e in pair] + \
                 [e for pair in u_ev + n_ev for e in pair]:
            e.record(stream)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        gemm_ev, call_ev, upd_ev, ns_ev = step_events[i]
        step(True)
        log(f"step {i + 1}/{args.steps} enqueued")
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    for i in range(args.steps):
        gemm_ev, call_ev, upd_ev, ns_ev = step_events[i]
        for k in ("momentum", "maxlogit", "clip") if args.unfused else ("maxlogit", "clip"):
            acc[k] += call_ev[k][0].elapsed_time(call_ev[k][1])
        for k, (name, s, cnt, rows, cols) in enumerate(ns_calls):
            acc["ns"] += ns_ev[k][0].elapsed_time(ns_ev[k][1])
            if args.unfused:
                acc["update"] += upd_ev[k][0].elapsed_time(upd_ev[k][1])
            n_, m_ = min(rows, cols), max(rows, cols)
            per = {0: n_ * n_ * m_, 1: n_ ** 3, 2: 2 * n_ * n_ * m_}
            per_nom = {0: 2 * n_ * n_ * m_, 1: 2 * n_ ** 3, 2: 2 * n_ * n_ * m_}
            per_exe = gemm_flops_executed(rows, cols)
            for st in range(steps_ns):
                for gm in range(3):
                    a, b = gemm_ev[k][2 * (3 * st + gm)], gemm_ev[k][2 * (3 * st + gm) + 1]
                    # the fused path's last B'X launch also applies the update to W
                    key = "2u" if (gm == 2 and st == steps_ns - 1 and not args.unfused) else gm
                    gemm_ms[key].append(a.elapsed_time(b))
                    gemm_flops[key].append(per[gm] * cnt)
                    gemm_flops_nom[key].append(per_nom[gm] * cnt)
                    gemm_flops_exe[key].append(per_exe[gm] * cnt)
    log(f"{args.steps} timed steps done")
    total_ms = t_start.elapsed_time(t_end)
    K = args.steps
    ms_per_step = total_ms / K

    ns_fl = sum(ns_flops_sym(r, c, steps_ns) * n for _, _, n, r, c in wl.groups)
    ns_fl_nom = sum(ns_flops(r, c, steps_ns) * n for _, _, n, r, c in wl.groups)
    ml_fl = 2.0 * B * H * Sq * Sk * dq
    value = (ns_fl + ml_fl) / (ms_per_step * 1e-3) / 1e12
    value_nominal = (ns_fl_nom + ml_fl) / (ms_per_step * 1e-3) / 1e12
    E = wl.numel
    n_clip = int((clipped == 1).sum().item())
    d_in = D_MODEL
    rescale_bytes = 2 * n_clip * ((D_NOPE + D_ROPE) + D_NOPE) * d_in * 2  # read + write, bf16

    # The attention forward that yields the same max logit as a by-product
    # (outside the step: the optimizer step reads S_max; where the forward
    # runs here, this replaces the stand-alone pass).  Timed on the step's
    # stream, 3 launches each, plain and causal.
    fwd = {}
    for causal in (False, True):
        smax_f = torch.empty(N_HEADS, dtype=torch.float32, device=dev)
        mc.attention_fwd_maxlogit(wl.Q, wl.Kc, wl.Kr, wl.V, causal=causal, smax=smax_f)
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(3):
            O_f, _ = mc.attention_fwd_maxlogit(wl.Q, wl.Kc, wl.Kr, wl.V, causal=causal, smax=smax_f)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 3
        fl = 2.0 * B * H * Sq * Sk * (dq + D_V) * ((Sq + 1) / (2.0 * Sq) if causal else 1.0)
        key = "causal" if causal else "full"
        fwd[key + "_ms"] = round(ms, 4)
        fwd[key + "_tflops"] = round(fl / (ms * 1e-3) / 1e12, 1)
        if not causal:
            fwd["smax_rel_diff_vs_standalone"] = float(((smax_f - smax).abs() / smax.abs()).max().item())
        del O_f

    # Long-context max logit (outside the step): 1 x 32768 tokens, 64 heads,
    # the same MLA projections with no hot head (S about 18, nothing clipped)
    import workloads
    L32 = workloads.mla_logits(seed=args.seed + 4, device=dev, batch=1, seq=32768, n_hot=0)
    smax_l = torch.empty(N_HEADS, dtype=torch.float32, device=dev)
    mc.qk_maxlogit(L32.Q, L32.Kc, L32.Kr, smax=smax_l)
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(3):
        mc.qk_maxlogit(L32.Q, L32.Kc, L32.Kr, smax=smax_l)
    e1.record(stream)
    torch.cuda.synchronize()
    ml_long_ms = e0.elapsed_time(e1) / 3
    ml_long = {"shape": "1 x 64 heads x 32768 x 32768, d 128 + 64", "ms": round(ml_long_ms, 3),
               "tflops": round(2.0 * 32768 * 32768 * 64 * (D_NOPE + D_ROPE) / (ml_long_ms * 1e-3) / 1e12, 1),
               "max_s": round(float(smax_l.max().item()), 2)}
    del L32

    # Newton-Schulz alone on one chunk of 64 expert matrices (2048 x 7168):
    # pre-scale (with the norm partials), 5 iterations and the bf16 output, no
    # momentum or update.
    ns_name, _, ns_n, ns_rows, ns_cols = wl.groups[0]
    ns_cnt = min(64, ns_n)
    M_ns = wl.view(ns_name, wl.M, 0, ns_cnt)
    O_ns = torch.empty((ns_cnt, ns_rows, ns_cols), dtype=torch.bfloat16, device=dev)
    mc.muon_ns_orthogonalize_batched(M_ns, O_ns, workspace=workspace, out_scale=mc.muon_out_scale(ns_rows, ns_cols))
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(3):
        mc.muon_ns_orthogonalize_batched(M_ns, O_ns, workspace=workspace,
                                         out_scale=mc.muon_out_scale(ns_rows, ns_cols))
    e1.record(stream)
    torch.cuda.synchronize()
    ns_only_ms = e0.elapsed_time(e1) / 3
    ns_only = {"shape": f"{ns_cnt} x {ns_rows} x {ns_cols}", "ms": round(ns_only_ms, 3),
               "tflops": round(ns_flops_sym(ns_rows, ns_cols, steps_ns) * ns_cnt / (ns_only_ms * 1e-3) / 1e12, 1),
               "tflops_nominal": round(ns_flops(ns_rows, ns_cols, steps_ns) * ns_cnt / (ns_only_ms * 1e-3) / 1e12, 1),
               "note": "muon_ns_orthogonalize_batched alone: pre-scale with norm partials, 5 iterations, bf16 output; "
                       "tflops counts 3n^2m + n^3 per matrix per iteration, tflops_nominal 4n^2m + 2n^3"}
    del O_ns

    # The HBM-bound steps on their own (outside the step), each a median over
    # repetitions:
    #  * momentum over all parameters in one launch (12 B per element; 205 GB,
    #    far past the 256 MB last-level cache);
    #  * the update on one 64-expert chunk (bf16 W and O: 6 B per element);
    #  * QK-Clip of the 4 hot heads (36.7 MB) and of all 64 heads (587 MB),
    #    with 1 GiB written between repetitions so the rows come from HBM;
    #  * QK-Clip of 61 attention layers (Kimi K2's count) with 4 hot heads
    #    each, one launch.
    def timed(fn, reps, flush=None):
        ts = []
        for _ in range(reps):
            if flush is not None:
                flush()
            e0, e1 = ev(), ev()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        return ts[len(ts) // 2]

    hbm = {}
    ms = timed(lambda: mc.muonclip_momentum(wl.M, wl.G, MU), 3)
    hbm["momentum"] = {"elements": E, "bytes_per_element": 12, "ms": round(ms, 3),
                       "gbps": round(12.0 * E / (ms * 1e-3) / 1e9, 1)}
    ns_name, _, ns_n, ns_rows, ns_cols = wl.groups[0]
    upd_cnt = min(64, ns_n)
    W_u = wl.view(ns_name, wl.W, 0, upd_cnt)
    O_u = torch.empty_like(W_u)
    O_u.normal_(0.0, 0.2)
    ms = timed(lambda: mc.muon_apply_update(W_u, O_u, LR, WD), 5)
    n_u = W_u.numel()
    hbm["update"] = {"elements": n_u, "bytes_per_element": 6, "ms": round(ms, 3),
                     "gbps": round(6.0 * n_u / (ms * 1e-3) / 1e9, 1)}
    del O_u
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush = lambda: flush_buf.fill_(1)  # noqa: E731  (1 GiB written: evicts the 256 MB cache)
    Wq_v, Wkc_v = wl.view("attn_q")[0], wl.view("attn_kc")[0]
    for label, s_vals in (("clip_4_hot_heads", smax), ("clip_all_64_heads", torch.full_like(smax, 1000.0))):
        Wq_c, Wkc_c = Wq_v.clone(), Wkc_v.clone()
        g_c = torch.empty_like(gamma)
        c_c = torch.empty_like(clipped)
        mc.qk_clip_apply(s_vals, Wq_c, Wkc_c, D_NOPE + D_ROPE, D_NOPE, D_NOPE, TAU, ALPHA, gamma=g_c, clipped=c_c)
        ms = timed(lambda: mc.qk_clip_apply(s_vals, Wq_c, Wkc_c, D_NOPE + D_ROPE, D_NOPE, D_NOPE, TAU, ALPHA,
                                            gamma=g_c, clipped=c_c), 20, flush)
        heads = int((c_c == 1).sum().item())
        nbytes = 2 * heads * ((D_NOPE + D_ROPE) + D_NOPE) * D_MODEL * 2
        hbm[label] = {"heads": heads, "bytes": nbytes, "ms": round(ms, 4),
                      "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1), "cache": "flushed (1 GiB written between runs)"}
        del Wq_c, Wkc_c
    n_layers = 61
    Wq_l = [Wq_v.clone() for _ in range(n_layers)]
    Wk_l = [Wkc_v.clone() for _ in range(n_layers)]
    s_l = smax.view(1, -1).repeat(n_layers, 1).contiguous()
    mc.qk_clip_apply_layers(s_l, Wq_l, Wk_l, D_NOPE + D_ROPE, D_NOPE, D_NOPE, TAU, ALPHA)
    ms = timed(lambda: mc.qk_clip_apply_layers(s_l, Wq_l, Wk_l, D_NOPE + D_ROPE, D_NOPE, D_NOPE, TAU, ALPHA), 10,
               flush)
    nbytes = n_layers * rescale_bytes
    hbm["clip_61_layers_one_launch"] = {"layers": n_layers, "heads_per_layer": n_clip, "bytes": nbytes,
                                        "ms": round(ms, 4), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    del Wq_l, Wk_l, flush_buf
    hbm["note"] = ("medians over repetitions on the step's stream; bytes are algorithmic (read + write); "
                   "peak 8000 GB/s")
    for v in hbm.values():
        if isinstance(v, dict):
            v["frac_of_peak"] = round(v["gbps"] / HBM_PEAK_GBPS, 3)

    # Self-measured ceilings on this GPU (measurement aids, outside the step):
    # the MFMA rate with register operands only (random and zero operands:
    # the clock the chip holds depends on how many bits switch), and a plain
    # device copy through the workspace (no longer needed at this point).
    probes = {}
    for zero in (False, True):
        p_out, p_fl = mc.probe_mfma_bf16(1024, 20000, zero_operands=zero, device=dev)
        e0, e1 = ev(), ev()
        e0.record(stream)
        mc.probe_mfma_bf16(1024, 20000, zero_operands=zero, out=p_out)
        e1.record(stream)
        torch.cuda.synchronize()
        probes["mfma_bf16_zero_operands_tflops" if zero else "mfma_bf16_random_operands_tflops"] = round(
            p_fl / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    half_ws = (workspace.numel() // 2) // (1 << 20) * (1 << 20)
    cp_src, cp_dst = workspace[:half_ws], workspace[half_ws:2 * half_ws]
    mc.probe_copy(cp_src, cp_dst)
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(5):
        mc.probe_copy(cp_src, cp_dst)
    e1.record(stream)
    torch.cuda.synchronize()
    probes["copy_gbps"] = round(2.0 * half_ws * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    probes["copy_bytes"] = half_ws

    # dominant kernel: the GEMM mode with the largest total time
    dom = max(gemm_ms, key=lambda g: sum(gemm_ms[g]))
    dom_launches = len(gemm_ms[dom])
    dom_avg_ms = sum(gemm_ms[dom]) / dom_launches
    dom_avg_flops = sum(gemm_flops[dom]) / dom_launches
    achieved = dom_avg_flops / (dom_avg_ms * 1e-3) / 1e12
    kernel_names = {0: "ns_gemm_kernel<0, 0, *> (A = Xh Xh^T)",
                    1: "ns_gemm_kernel<1, 0, *> (B = bA + cAA: float32 diagonal d, bf16 rest N)",
                    2: "ns_gemm_kernel<2, 0, *> (X' = aX + d Xh + N Xh)",
                    "2u": "ns_gemm_kernel<2, 1, *> (last step: X' applied as the update of bf16 W)"}

    breakdown = {
        "path": "three calls: momentum, Newton-Schulz, update" if args.unfused else
                "fused call per chunk: momentum + Newton-Schulz + update (O not stored)",
        "wall_s_timed_region": round(wall, 3),
        ("newton_schulz_ms" if args.unfused else "momentum_ns_update_ms"): round(acc["ns"] / K, 3),
        ("newton_schulz_tflops" if args.unfused else "momentum_ns_update_tflops"):
            round(ns_fl / (acc["ns"] / K * 1e-3) / 1e12, 1),
        "value_nominal_tflops": round(value_nominal, 2),
        "value_note": "value counts 3n^2m + n^3 per Newton-Schulz iteration (symmetric X X^T and A A once); "
                      "value_nominal_tflops the dense 4n^2m + 2n^3",
        "maxlogit_ms": round(acc["maxlogit"] / K, 4),
        "maxlogit_tflops": round(ml_fl / (acc["maxlogit"] / K * 1e-3) / 1e12, 1),
    }
    if args.unfused:
        breakdown.update({
            "momentum_ms": round(acc["momentum"] / K, 3),
            "momentum_gbps": round(12.0 * E / (acc["momentum"] / K * 1e-3) / 1e9, 1),
            "update_ms": round(acc["update"] / K, 3),
            "update_gbps": round(6.0 * E / (acc["update"] / K * 1e-3) / 1e9, 1),
        })
    breakdown.update({
        "rescale_ms": round(acc["clip"] / K, 4),
        "rescale_gbps": round(rescale_bytes / (acc["clip"] / K * 1e-3) / 1e9, 1),
        "clipped_heads": n_clip,
        "gemm_tflops": {str(g): round(sum(gemm_flops[g]) / (sum(gemm_ms[g]) * 1e-3) / 1e12, 1)
                        for g in gemm_ms},
        "gemm_tflops_executed": {str(g): round(sum(gemm_flops_exe[g]) / (sum(gemm_ms[g]) * 1e-3) / 1e12, 1)
                                 for g in gemm_ms},
        "gemm_frac_executed": {str(g): round(sum(gemm_flops_exe[g]) / (sum(gemm_ms[g]) * 1e-3) / 1e12
                                             / MFMA_BF16_PEAK_TFLOPS, 4) for g in gemm_ms},
        "gemm_tflops_nominal": {str(g): round(sum(gemm_flops_nom[g]) / (sum(gemm_ms[g]) * 1e-3) / 1e12, 1)
                                for g in gemm_ms},
        "gemm_note": "per GEMM (0 X X^T, 1 bA+cAA, 2 aX+BX, 2u the last aX+BX applying the update): gemm_tflops on "
                     "the method's flops (n^2m, n^3, 2n^2m), executed on the tiles the MFMAs compute, nominal dense",
        "newton_schulz_only": ns_only,
        "hbm_steps": hbm,
        "maxlogit_long_context": ml_long,
        "probes": dict(probes, dominant_gemm_frac_of_mfma_probe=round(
            achieved / probes["mfma_bf16_random_operands_tflops"], 3),
            note="self-measured ceilings: MFMA-only loop on register operands, plain 16-byte copy "
                 "(read + write bytes)"),
        "attention_forward_with_max_logit": dict(
            fwd, note="outside the step: softmax(QK^T/sqrt(d))V with d_v 128 on the same Q/K, S_max as a by-product; "
                      "flops 2 B H Sq Sk (192 + 128), causal counts the visible half"),
    })

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "full MuonClip step, one MoE layer: 384 experts x (gate, up 2048x7168; down 7168x2048) "
                        "+ W_q 12288x7168, W_kc 8192x7168, W_kr 64x7168; max logit over 8 x 4096 tokens, "
                        "64 heads, d 128+64; QK-Clip tau 100",
            "experts": args.experts,
            "matrices": sum(g[2] for g in wl.groups),
            "parameters": E,
            "ns_iterations": steps_ns,
            "ns_chunk": chunk,
            "lr": LR, "weight_decay": WD, "mu": MU, "tau": TAU, "alpha": ALPHA,
        },
        "breakdown": breakdown,
        "roofline": {
            "kernel": kernel_names[dom],
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(),
            "avg_launch_ms": round(dom_avg_ms, 4),
            "algorithmic_flops_per_launch": dom_avg_flops,
            "launches": dom_launches,
        },
    }
    return out, wl


def host_info():
    """Host cores, affinity mask and BLAS library the oracle runs on."""
    info = {"nproc": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except AttributeError:  # not on Linux
        info["affinity_cpus"] = None
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        blas = [p for p in pools if p.get("user_api") == "blas"]
        info["blas"] = ", ".join(f"{p.get('internal_api')} {p.get('version')} ({p.get('num_threads')} threads)"
                                 for p in blas) or None
        info["threads"] = max((p.get("num_threads", 1) for p in blas), default=os.cpu_count())
    except Exception:  # noqa: BLE001
        info["blas"], info["threads"] = None, os.cpu_count()
    return info


def cpu_baseline(wl, torch, n_matrices=6):
    """The fp64 oracle on a bounded sample of the same workload (about 10 s of
    CPU work): n_matrices expert matrices, alternately 2048x7168 and
    7168x2048 (momentum, Newton-Schulz x5, update), and the max logit of two
    heads over the full 8 x 4096 batch."""
    import numpy as np

    import oracle
    import workloads
    host = host_info()
    # seeded inputs of the workload's shapes and distributions, drawn on the
    # host (not the buffers the library has already stepped)
    gen = workloads.generator(77, "cpu")
    data = []
    for k in range(n_matrices):
        shape = (D_EXPERT, D_MODEL) if k % 2 == 0 else (D_MODEL, D_EXPERT)
        data.append((workloads.normal(shape, 1e-4, gen, "cpu").numpy(), workloads.normal(shape, 1e-4, gen, "cpu").numpy(),
                     workloads.normal(shape, 0.02, gen, "cpu", torch.bfloat16).double().numpy()))
    heads = [int(wl.hot[0]), (int(wl.hot[0]) + 1) % N_HEADS]
    Qh = [wl.Q[:, h:h + 1].float().cpu().numpy() for h in heads]
    Kch = [wl.Kc[:, h:h + 1].float().cpu().numpy() for h in heads]
    Kr = wl.Kr.float().cpu().numpy()
    t0 = time.perf_counter()
    flops = 0.0
    for M, G, W in data:
        Mn = oracle.momentum_update(M, G, MU)
        O = oracle.muon_orthogonalised_update(Mn.astype(np.float64))
        oracle.apply_update(W, O, LR, WD, "bf16")
        flops += ns_flops_sym(*M.shape, oracle.NS_STEPS)
    for q, k in zip(Qh, Kch):
        oracle.max_logit(q, k, Kr)
        flops += 2.0 * q.shape[0] * q.shape[2] * k.shape[2] * q.shape[3]
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": host["threads"], "kind": "oracle",
            "seconds": round(dt, 2), "host": host,
            "sample": f"fp64 oracle: momentum + Newton-Schulz x5 + update of {n_matrices} expert matrices "
                      "(2048x7168 and 7168x2048 alternately) and the max logit of 2 heads over 8 x 4096 "
                      "tokens; same flop accounting as value"}


def cpu_baseline_configs():
    """The oracle per workload, each on a bounded seeded sample, median of 3
    runs, extrapolated linearly to the whole workload (matrices and heads are
    independent) and labelled so: the tiny fp32 step (whole), Newton-Schulz
    alone (2 of 64 matrices), the max logit + QK-Clip at 8 x 4096 (2 of 64
    heads), the full step for one MoE layer (2 expert matrices of each shape
    and W_kr whole; W_q and W_kc by their flop share), and the 32K-token max
    logit (1 of 64 heads)."""
    import numpy as np
    import torch

    import oracle
    import workloads

    def med3(fn):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return sorted(ts)[1]

    out = {"host": host_info(), "configs": []}

    def done(rec):
        out["configs"].append(rec)
        log(f"cpu baseline: {rec['workload']} done")
    # tiny fp32 attention layer: one whole step
    t = workloads.tiny_attention(seed=1, device="cpu", weight_reading="variance")
    Wn = {n: w.double().numpy() for n, w in t.W.items()}
    Gn = {n: g.numpy() for n, g in t.G.items()}
    att = dict(q="q", k="k", q_rows_per_head=t.head_dim, q_c_rows=t.head_dim, k_rows_per_head=t.head_dim)

    def tiny():
        q = oracle.project_heads(t.X.double().numpy(), Wn["q"], t.n_heads)
        k = oracle.project_heads(t.X.double().numpy(), Wn["k"], t.n_heads)
        oracle.muonclip_step(Wn, Gn, {}, oracle.max_logit(q, k), att, lr=0.02, w_dtype="f32")
    s = med3(tiny)
    done({"workload": "tiny fp32 attention layer, one step", "sample": "whole", "seconds": s})
    # Newton-Schulz alone, 64 x 2048 x 7168: 2 matrices
    eb = workloads.expert_batch(seed=2, device="cpu", batch=2)
    Ms = [oracle.momentum_update(eb.M_prev[i].numpy(), eb.G[i].numpy(), MU) for i in range(2)]
    s = med3(lambda: [oracle.newton_schulz(m.astype(np.float64)) for m in Ms])
    fl = ns_flops_sym(2048, 7168, oracle.NS_STEPS) * 64
    done({"workload": "Newton-Schulz alone, 64 x 2048 x 7168", "sample": "2 of 64 matrices",
                           "seconds_sample": s, "seconds_extrapolated": s * 32,
                           "tflops": fl / (s * 32) / 1e12})
    # max logit + clip at 8 x 4096, 64 heads: 2 heads
    L = workloads.mla_logits(seed=3, device="cpu", batch=8, seq=4096)
    Kr = L.Kr.double().numpy()
    qs = [L.Q[:, h:h + 1].double().numpy() for h in (0, 1)]
    ks = [L.Kc[:, h:h + 1].double().numpy() for h in (0, 1)]
    s = med3(lambda: [oracle.max_logit(q, k, Kr) for q, k in zip(qs, ks)])
    fl = 2.0 * 8 * 64 * 4096 * 4096 * (D_NOPE + D_ROPE)
    done({"workload": "max logit, 8 x 4096 tokens, 64 heads, d 128+64", "sample": "2 of 64 heads",
                           "seconds_sample": s, "seconds_extrapolated": s * 32, "tflops": fl / (s * 32) / 1e12})
    del L, qs, ks, Kr
    # full step for one MoE layer: 2 matrices of each expert shape
    g = workloads.generator(4, "cpu")
    secs = 0.0
    for rows, cols, count in ((2048, 7168, 768), (7168, 2048, 384)):
        data = [(workloads.normal((rows, cols), 1e-4, g, "cpu").numpy(), workloads.normal((rows, cols), 1e-4, g, "cpu").numpy(),
                 workloads.normal((rows, cols), 0.02, g, "cpu", torch.bfloat16).double().numpy()) for _ in range(2)]

        def run(data=data):
            for M, G, W in data:
                Mn = oracle.momentum_update(M, G, MU)
                oracle.apply_update(W, oracle.muon_orthogonalised_update(Mn.astype(np.float64)), LR, WD, "bf16")
        secs += med3(run) * count / 2
    expert_fl = ns_flops_sym(2048, 7168, oracle.NS_STEPS) * 1152
    attn_fl = sum(ns_flops_sym(r, D_MODEL, oracle.NS_STEPS) for r in (12288, 8192, 64))
    secs_total = secs * (expert_fl + attn_fl) / expert_fl
    done({"workload": "full MuonClip step, one MoE layer (NS x5 of 1155 matrices)",
                           "sample": "2 matrices of each expert shape; the attention projections by their flop share",
                           "seconds_extrapolated": secs_total,
                           "tflops": (expert_fl + attn_fl) / secs_total / 1e12})
    # long-context max logit: 1 of 64 heads
    L = workloads.mla_logits(seed=5, device="cpu", batch=1, seq=32768, n_hot=0)
    q, k, Kr = L.Q[:, :1].double().numpy(), L.Kc[:, :1].double().numpy(), L.Kr.double().numpy()
    s = med3(lambda: oracle.max_logit(q, k, Kr, block=4096))
    fl = 2.0 * 32768 * 32768 * 64 * (D_NOPE + D_ROPE)
    done({"workload": "max logit, 1 x 32768 tokens, 64 heads", "sample": "1 of 64 heads",
                           "seconds_sample": s, "seconds_extrapolated": s * 64, "tflops": fl / (s * 64) / 1e12})
    print(json.dumps(out), flush=True)


def copy_calibration():
    """A plain 1 GiB device copy, repeated: the reference kernel for scaling
    the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": 4 * n, "launches": 5}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--experts", type=int, default=384)
    ap.add_argument("--chunk", type=int, default=64, help="matrices per Newton-Schulz call")
    ap.add_argument("--seed", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="momentum, Newton-Schulz and update as three calls (O stored in bf16)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--cpu-baseline-configs", action="store_true",
                    help="time the fp64 oracle per workload on bounded samples (CPU only, several minutes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(there is no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.cpu_baseline_configs:
        cpu_baseline_configs()
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no ROCm GPU visible", file=sys.stderr)
        sys.exit(1)
    out, wl = run(args)
    if not args.no_cpu_baseline:
        log("timing the oracle on a CPU sample")
        out["cpu_baseline"] = cpu_baseline(wl, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
