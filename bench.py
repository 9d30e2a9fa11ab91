#!/usr/bin/env python3
"""Throughput of the EAGLE-3 draft-and-verify hot path on one MI355X.

One step = one speculation round for the whole batch: feature fusion of the
seed rows, D draft passes with EAGLE-2 growth and the final rerank/flatten,
then verification against per-node target logits with the accepted-path KV
commit.  The round is replayed with identical inputs (lengths in and out are
separate arrays), so every timed step does the same work.

Prints one JSON line.  value = draft-tree steps (rounds) per second.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="8b_bs1")
    ap.add_argument("--secondary", default="8b_bs64",
                    help="second workload reported beside the main one ('' = none)")
    ap.add_argument("--secondary-steps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one plain device copy of this size (counter scaling)")
    return ap.parse_args()


def gpu_weights(cfg, seed=0):
    """Random-init drafter weights generated on the device (same shapes and
    distributions as the test generator, a different random stream)."""
    import torch
    import synth
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shapes = {
        "w_fuse": (cfg.H, 3 * cfg.H), "w_in": (cfg.H, 2 * cfg.H),
        "embed": (cfg.V, cfg.H), "wq": (cfg.n_q * cfg.hd, cfg.H),
        "wk": (cfg.n_kv * cfg.hd, cfg.H), "wv": (cfg.n_kv * cfg.hd, cfg.H),
        "wo": (cfg.H, cfg.n_q * cfg.hd), "w_gate": (cfg.F, cfg.H),
        "w_up": (cfg.F, cfg.H), "w_down": (cfg.H, cfg.F), "w_lm": (cfg.V, cfg.H)}
    w = {}
    for n, s in shapes.items():
        w[n] = (torch.randn(s, generator=gen, device="cuda") * 0.02).to(dt)
    for n in ("g_attn", "g_mlp", "g_final"):
        w[n] = (1.0 + 0.02 * torch.randn(cfg.H, generator=gen, device="cuda")).to(dt)
    del synth
    return w


class Workload:
    """Device-resident inputs of one round for a config."""

    def __init__(self, cfg, weights, seed=1):
        import torch
        import synth
        from eagle_draft_tree_amd import Drafter, DrafterShape, KVCache
        self.cfg = cfg
        B = cfg.B
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        ctx = torch.from_numpy(synth.contexts(cfg)).to(torch.int32)
        self.ctx = ctx
        cap = (int(ctx.max()) + cfg.s_max + (cfg.D - 1) * cfg.K + 64 + 7) // 8 * 8
        k = torch.zeros(B, cfg.n_kv, cap, cfg.hd, dtype=dt, device="cuda")
        v = torch.zeros(B, cfg.n_kv, cfg.hd, cap, dtype=dt, device="cuda")
        for b in range(B):
            L = int(ctx[b])
            k[b, :, :L] = torch.randn(cfg.n_kv, L, cfg.hd, generator=gen, device="cuda").to(dt)
            v[b, :, :, :L] = torch.randn(cfg.n_kv, cfg.hd, L, generator=gen, device="cuda").to(dt)
        self.kv = KVCache(k, v, ctx.cuda())
        self.d = Drafter(DrafterShape(
            hidden=cfg.H, n_q_heads=cfg.n_q, n_kv_heads=cfg.n_kv, head_dim=cfg.hd,
            ffn=cfg.F, vocab=cfg.V, dtype=cfg.dtype, rope_theta=cfg.theta,
            depth=cfg.D, topk=cfg.K, budget=cfg.N, max_batch=B,
            max_seed=cfg.s_max, rms_eps=cfg.eps), weights)
        rows = B * cfg.s_max
        self.taps = [torch.randn(rows, cfg.H, generator=gen, device="cuda").to(dt)
                     for _ in range(3)]
        self.seed_src = torch.zeros(B, cfg.s_max, cfg.H, dtype=torch.float32,
                                    device="cuda")
        tok = torch.full((B, cfg.s_max), -1, dtype=torch.int32, device="cuda")
        tok[:, 0] = torch.randint(0, cfg.V, (B,), generator=gen, device="cuda",
                                  dtype=torch.int32)
        self.tok = tok
        self.seed_len = torch.ones(B, dtype=torch.int32, device="cuda")
        self.len_out = torch.empty(B, dtype=torch.int32, device="cuda")
        self.kv_len = torch.empty(B, dtype=torch.int32, device="cuda")
        self.tree = self.d.alloc_tree(B)
        self.res = None
        # one untimed round gives the tree the target logits are built on:
        # N(0, 2^2) noise, with the drafter's highest-valued child of every
        # row raised by 20 so greedy verification follows the best path
        self.logits = torch.zeros(B, cfg.N + 1, cfg.V, device="cuda")
        self.uniforms = torch.rand(B, cfg.N + 1, cfg.K + 1, generator=gen,
                                   device="cuda") if cfg.T > 0 else None
        self.step()
        torch.cuda.synchronize()
        noise = torch.randn(B, cfg.N + 1, cfg.V, generator=gen, device="cuda") * 2.0
        t = {k: v.cpu().numpy() for k, v in self.tree.items()}
        rows_b, rows_r, toks = [], [], []
        for b in range(B):
            best = {}
            for r in range(1, int(t["n_nodes"][b]) + 1):
                p = int(t["parent"][b, r])
                if p not in best or t["score"][b, r] > t["score"][b, best[p]]:
                    best[p] = r
            for p, r in best.items():
                rows_b.append(b)
                rows_r.append(p)
                toks.append(int(t["token"][b, r]))
        if rows_b:
            noise[torch.tensor(rows_b), torch.tensor(rows_r), torch.tensor(toks)] += 20.0
        self.logits = noise.contiguous()

    def step(self):
        cfg = self.cfg
        g = self.seed_src.view(cfg.B * cfg.s_max, cfg.H)
        self.d.fuse(*self.taps, out=g)
        self.d.draft_tree(self.seed_src, self.tok, self.seed_len, self.kv,
                          len_out=self.len_out, tree=self.tree)
        self.res = self.d.verify(self.tree, self.logits, cfg.T, seed=1, round=0,
                                 kv=self.kv, kv_len_out=self.kv_len, out=self.res)

    def run(self, steps, warmup):
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            self.step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        # the same steps again with per-launch events for the kernel table
        self.d.profile(True)
        for _ in range(steps):
            self.step()
        prof = self.d.profile_read()
        self.d.profile(False)
        acc = self.res["accept_len"].cpu()
        return ms, prof, acc


def roofline(prof, kind, cfg):
    p = prof[kind]
    if p["launches"] == 0 or p["ms"] <= 0:
        return None
    if cfg.B > 16:  # M = B*K rows: a dense contraction, priced against MFMA
        ach = p["flops"] / (p["ms"] * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2),
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "skinny_gemm_kernel (draft-layer GEMMs)",
                "avg_launch_us": round(1e3 * p["ms"] / p["launches"], 2),
                "flops_per_launch": p["flops"] / p["launches"]}
    ach = p["bytes"] / (p["ms"] * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "skinny_gemm_kernel (draft-layer GEMMs)",
            "avg_launch_us": round(1e3 * p["ms"] / p["launches"], 2),
            "bytes_per_launch": p["bytes"] / p["launches"]}


def cpu_baseline(cfg):
    """The oracle (as it stands) timed on this host for one round of one
    sequence of the same shape: fuse + draft tree + greedy verify."""
    import numpy as np
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count()
    c1 = cfg.replace(B=1, ctx=(cfg.ctx[0], cfg.ctx[0]))
    W = O.Weights(c1, synth.weights(c1, 0))
    s = synth.seq_inputs(c1, 0)
    P = c1.ctx[0]
    cap = P + 2 + (c1.D - 1) * c1.K + 8
    kk, vv = synth.prefix_kv(c1, 0, P)
    k = np.zeros((c1.n_kv, cap, c1.hd))
    v = np.zeros_like(k)
    k[:, :P] = O.store(kk, c1.dtype)
    v[:, :P] = O.store(vv, c1.dtype)
    kv = O.DraftKV(k, v)
    t0 = time.perf_counter()
    g = O.fuse(W, O.store(s["low"], c1.dtype), O.store(s["mid"], c1.dtype),
               O.store(s["high"], c1.dtype))
    tree, info = O.draft_tree(W, kv, g, [s["token"]], P)
    tl = np.zeros((c1.N + 1, c1.V), dtype=np.float32)
    O.verify(c1, tree, tl, 0.0)
    dt = time.perf_counter() - t0
    return {"value": round(1.0 / dt, 5), "unit": "draft-tree steps/s",
            "cores": int(cores), "kind": "oracle",
            "sample": f"one round of one sequence at the {cfg.name} shape "
                      f"(fuse, {c1.D} draft passes, rerank, greedy verify) in "
                      f"{dt:.1f} s; batch-1 rounds/s, float64 NumPy"}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import synth
    cfg = synth.config(a.config)
    w = gpu_weights(cfg)
    wl = Workload(cfg, w)
    ms, prof, acc = wl.run(a.steps, a.warmup)
    mean_a = float(acc.float().mean())
    ver = float((acc.clamp(min=0) + 1).sum())
    out = {
        "metric": "draft-tree steps/s + verified tokens/s at bs1 & bs64; % of HBM/MFMA roofline",
        "value": round(1e3 / ms, 3),
        "unit": "draft-tree steps/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name}: H={cfg.H} FC {3*cfg.H}->{cfg.H}, "
                   f"{cfg.n_q}q/{cfg.n_kv}kv x {cfg.hd}, FFN {cfg.F}, V={cfg.V}, "
                   f"ctx {cfg.ctx[0]}-{cfg.ctx[1]}, bs={cfg.B}, depth {cfg.D} "
                   f"top-k {cfg.K} nodes {cfg.N}, "
                   + ("greedy" if cfg.T == 0 else f"T={cfg.T}") + " verify",
                   "batch": cfg.B, "depth": cfg.D, "topk": cfg.K, "nodes": cfg.N},
        "draft_passes_per_s": round(cfg.D * 1e3 / ms, 2),
        "verified_tokens_per_s": round(ver * 1e3 / ms, 2),
        "mean_accept_len": mean_a, "tau": mean_a + 1,
        "roofline": roofline(prof, "gemm", cfg),
        "kernel_ms_per_step": {k: round(v["ms"] / a.steps, 4) for k, v in prof.items()},
    }
    if a.secondary:
        c2 = synth.config(a.secondary)
        wl2 = Workload(c2, w if (c2.H, c2.F, c2.V) == (cfg.H, cfg.F, cfg.V) else gpu_weights(c2))
        ms2, prof2, acc2 = wl2.run(a.secondary_steps, 2)
        ver2 = float((acc2.clamp(min=0) + 1).sum())
        out["secondary"] = {
            "workload": c2.name, "batch": c2.B, "ms_per_step": round(ms2, 3),
            "draft_tree_steps_per_s": round(1e3 / ms2, 3),
            "draft_passes_per_s": round(c2.D * 1e3 / ms2, 2),
            "verified_tokens_per_s": round(ver2 * 1e3 / ms2, 1),
            "mean_accept_len": float(acc2.float().mean()),
            "roofline": roofline(prof2, "gemm", c2),
            "kernel_ms_per_step": {k: round(v["ms"] / a.secondary_steps, 3)
                                   for k, v in prof2.items()}}
        del wl2
    if a.calib_copy_mb:
        n = a.calib_copy_mb * (1 << 20) // 4
        x = torch.ones(n, device="cuda")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = n * 4
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
