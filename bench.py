#!/usr/bin/env python3
"""Throughput of the EAGLE-3 draft-and-verify hot path on one MI355X.

One step = one speculation round for the whole batch: fusion of the seed
rows' target taps, D draft passes with EAGLE-2 growth and the final
rerank/flatten, then verification against per-node target logits (greedy,
or seeded rejection sampling) with the accepted-path KV commit.  The round
is replayed with identical inputs (lengths in and out are separate arrays),
so every timed step does the same work.

Target logits follow the workload's statement: the drafter's own logits at
every flattened tree row plus N(0, 2^2) noise.  They are synthesised once,
untimed: the tree rows are replayed through the library's draft step (depth
by depth, each row seeing the prefix, its ancestors' draft K/V and itself)
and the LM head is applied to their draft states with torch.

Prints one JSON line.  value = draft-tree steps (rounds) per second at the
primary workload; secondary workloads are reported beside it.
    python bench.py [--gpus 1] [--steps 100] [--warmup 10]
    python bench.py --summarize-trace DIR   (rocprofv3 output -> text summary)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "draft-tree steps/s + verified tokens/s at bs1 & bs64; % of HBM/MFMA roofline"
GEMM_SRC = os.path.join(ROOT, "eagle_draft_tree_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic_8b_bs1.json")
FLUSH_MB = 512
PROFILE_PAIRS = 8000           # launches the library's event record holds (8192)
PROFILE_STRIDE = 10            # profile one timed step in ten


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="8b_bs1")
    ap.add_argument("--secondary", default="8b_bs64,8b_chain_bs16",
                    help="comma-separated workloads reported beside the main one")
    ap.add_argument("--secondary-steps", type=int, default=20)
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="cold-cache pass: MB written between steps (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true",
                    help="no per-launch events in the timed region")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run one plain 'MB'-sized device copy (counter scaling)")
    ap.add_argument("--summarize-trace", default=None,
                    help="print a per-kernel summary of a rocprofv3 csv output dir and exit")
    ap.add_argument("--traffic-from", nargs=2, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the GEMM traffic record from two --pmc runs and exit "
                         "(with --calib-copy-mb: the copy size those runs used)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# rocprofv3 output -> short text summaries (the files in profiles/)
# ---------------------------------------------------------------------------
def _short(name):
    return name.split("(")[0].replace("void ", "")


def _csv_rows(path, suffix):
    import csv
    files = sorted(glob.glob(os.path.join(path, "**", "*" + suffix), recursive=True))
    rows = []
    for f in files:
        rows.extend(csv.DictReader(open(f)))
    return rows


def _gemm_dispatch_classes(rows):
    """Dispatch id -> 'fuse' | 'draft' for stream_gemm_kernel dispatches: a
    step launches the fusion GEMM right before the tree pass's seed set-up
    kernel, every other GEMM belongs to a draft layer."""
    seq = {}
    for r in rows:
        seq[int(r["Dispatch_Id"])] = _short(r["Kernel_Name"])
    ids = sorted(seq)
    cls = {}
    for i, d in enumerate(ids):
        if "stream_gemm_kernel" in seq[d]:
            nxt = seq[ids[i + 1]] if i + 1 < len(ids) else ""
            cls[d] = "fuse" if "seed_setup_kernel" in nxt else "draft"
    return cls


def summarize_trace(path):
    """Per-kernel launches and durations of a kernel trace, or per-dispatch
    counter means of a --pmc run, from a rocprofv3 --output-format csv dir."""
    out = []
    kt = _csv_rows(path, "kernel_trace.csv")
    if kt:
        agg = {}
        for r in kt:
            agg.setdefault(_short(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        cls = _gemm_dispatch_classes(kt)
        for r in kt:
            c = cls.get(int(r["Dispatch_Id"]))
            if c:
                agg.setdefault(f"stream_gemm_kernel [all {c} GEMMs]", []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        out.append("kernel | launches | mean_us | median_us | total_ms")
        for n, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"{n} | {len(v)} | {sum(v) / len(v):.2f} | "
                       f"{statistics.median(v):.2f} | {sum(v) / 1e3:.3f}")
    pc = _csv_rows(path, "counter_collection.csv")
    if pc:
        cls = _gemm_dispatch_classes(pc)
        cnt = {}
        for r in pc:
            k = _short(r["Kernel_Name"])
            c = cls.get(int(r["Dispatch_Id"]))
            v = float(r["Counter_Value"])
            cnt.setdefault((k, r["Counter_Name"]), {})[int(r["Dispatch_Id"])] = v
            if c:
                cnt.setdefault((f"stream_gemm_kernel [all {c} GEMMs]",
                                r["Counter_Name"]), {})[int(r["Dispatch_Id"])] = v
        out.append("kernel | counter | dispatches | mean per dispatch")
        for (n, c), v in sorted(cnt.items()):
            vals = list(v.values())
            out.append(f"{n} | {c} | {len(vals)} | {sum(vals) / len(vals):.1f}")
    print("\n".join(out))


def counter_mean(path, kernel_key, counter):
    """Mean per dispatch of `counter` over the dispatches whose short name
    contains kernel_key ('draft-gemm' = draft-layer stream_gemm_kernel)."""
    pc = _csv_rows(path, "counter_collection.csv")
    cls = _gemm_dispatch_classes(pc)
    per = {}
    for r in pc:
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        if kernel_key == "draft-gemm":
            ok = cls.get(d) == "draft"
        else:
            ok = kernel_key in _short(r["Kernel_Name"])
        if ok:
            per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    if not per:
        return None, 0
    if kernel_key == "copyBuffer":  # the calibration copy: the largest one
        return max(per.values()), 1
    return sum(per.values()) / len(per), len(per)


def traffic_record(fetch_dir, write_dir, copy_bytes, out_path):
    """HBM bytes per draft-layer GEMM launch from a FETCH_SIZE run and a
    WRITE_SIZE run (KiB per dispatch), each scaled by what the counter reads
    for the plain device copy of copy_bytes in the same run."""
    f_gemm, nf = counter_mean(fetch_dir, "draft-gemm", "FETCH_SIZE")
    w_gemm, nw = counter_mean(write_dir, "draft-gemm", "WRITE_SIZE")
    f_copy, _ = counter_mean(fetch_dir, "copyBuffer", "FETCH_SIZE")
    w_copy, _ = counter_mean(write_dir, "copyBuffer", "WRITE_SIZE")
    f_scale = copy_bytes / (f_copy * 1024.0)
    w_scale = copy_bytes / (w_copy * 1024.0)
    rec = {
        "kernel": "stream_gemm_kernel, draft-layer GEMMs, 8b_bs1 workload",
        "fetch_kib_per_launch": f_gemm, "write_kib_per_launch": w_gemm,
        "launches": [nf, nw],
        "copy_bytes": copy_bytes, "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "traffic_bytes_per_launch": f_gemm * 1024.0 * f_scale + w_gemm * 1024.0 * w_scale,
        "gemm_source_sha16": hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()[:16],
    }
    json.dump(rec, open(out_path, "w"), indent=1)
    print(json.dumps(rec, indent=1))


# ---------------------------------------------------------------------------
# workload
# ---------------------------------------------------------------------------
def gpu_weights(cfg, seed=0):
    """Random-init drafter weights on the device: matrices N(0, 0.02^2), norm
    gains 1 + N(0, 0.02^2) (the workload's distributions)."""
    import torch
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
    return w


class Workload:
    """Device-resident inputs of one round for a config."""

    def __init__(self, cfg, weights, seed=1):
        import torch
        import synth
        from eagle_draft_tree_amd import Drafter, DrafterShape, KVCache
        self.cfg, self.w = cfg, weights
        B = cfg.B
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        self.gen = gen
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
        self.logits = None
        # an untimed draft builds the tree the target logits are made for
        # (before any verification: its commit rewrites the scratch rows the
        # replay reads)
        self.d.fuse(*self.taps, out=self.seed_src.view(B * cfg.s_max, cfg.H))
        self.d.draft_tree(self.seed_src, self.tok, self.seed_len, self.kv,
                          len_out=self.len_out, tree=self.tree)
        torch.cuda.synchronize()
        self.logits = self.target_logits()
        self.step()
        torch.cuda.synchronize()

    def step(self):
        cfg = self.cfg
        g = self.seed_src.view(cfg.B * cfg.s_max, cfg.H)
        self.d.fuse(*self.taps, out=g)
        self.d.draft_tree(self.seed_src, self.tok, self.seed_len, self.kv,
                          len_out=self.len_out, tree=self.tree)
        self.res = self.d.verify(self.tree, self.logits, cfg.T, seed=1, round=0,
                                 kv=self.kv, kv_len_out=self.kv_len, out=self.res)

    def target_logits(self):
        """Draft logits at every flattened row + N(0, 2^2) noise (float32).
        Each row's draft state comes from the library's draft step with the
        row's token and position, its parent's state as source, and the
        prefix, its ancestors' draft K/V and itself visible; ancestors keep
        the scratch rows the tree pass wrote, each replayed row gets a
        spare scratch row past them."""
        import numpy as np
        import torch
        cfg, d = self.cfg, self.d
        B, N, K, D, H, S = cfg.B, cfg.N, cfg.K, cfg.D, cfg.H, cfg.s_max
        t = {k: v.cpu().numpy() for k, v in self.tree.items()}
        len_out = self.len_out.cpu().numpy().astype(np.int32)
        a_node = torch.zeros(B, N + 1, H, dtype=torch.float32, device="cuda")
        self.pass_args = None

        def cu(x):
            return torch.from_numpy(np.ascontiguousarray(x)).cuda()

        # root: the seed rows again (same inputs, so the same K/V rewritten)
        len_in = self.kv.length.cpu().numpy().astype(np.int32)
        pos = (len_in[:, None] + np.arange(S, dtype=np.int32)[None, :]).ravel()
        a, _, _, _ = d.draft_step(
            B, S, self.seed_src.view(B * S, H), self.tok.view(-1), cu(pos),
            cu(pos), cu(pos + 1), cu(len_out),
            torch.zeros(B * S, dtype=torch.int64, device="cuda"), self.kv)
        sl = self.seed_len.cpu().numpy()
        for b in range(B):
            a_node[b, 0] = a[b * S + int(sl[b]) - 1]

        base_slot = max(D - 1, 0) * K

        def rows(nodes, rps):
            """draft_step arguments for rps rows per sequence; nodes[b] are
            the tree rows of sequence b (at most rps, the rest padding)."""
            tok = np.full(B * rps, -1, np.int32)
            posa = np.zeros(B * rps, np.int32)
            dest = np.zeros(B * rps, np.int32)
            mask = np.zeros(B * rps, np.uint64)
            src = torch.zeros(B * rps, H, dtype=torch.float32, device="cuda")
            which = []
            for b in range(B):
                for i, r in enumerate(nodes[b]):
                    q = b * rps + i
                    tok[q] = t["token"][b, r]
                    posa[q] = t["position"][b, r]
                    dest[q] = len_out[b] + base_slot + i
                    m = np.uint64(1) << np.uint64(base_slot + i)
                    p = int(t["parent"][b, r])
                    src[q] = a_node[b, p]
                    while p > 0:
                        slot = int(t["kv_slot"][b, p])
                        assert 0 <= slot < base_slot, (b, r, p, slot)
                        m |= np.uint64(1) << np.uint64(slot)
                        p = int(t["parent"][b, p])
                    mask[q] = m
                    which.append((b, r, q))
            args = (B, rps, src, cu(tok), cu(posa), cu(dest),
                    cu(np.repeat(len_out, rps)), cu(len_out), cu(mask.view(np.int64)))
            return args, which

        chunk = min(max(S, K), 64 - base_slot)
        if D == 0 or chunk <= 0:
            return self._noise(a_node, t)
        for depth in range(1, D + 1):
            nodes = [[r for r in range(1, int(t["n_nodes"][b]) + 1)
                      if t["depth"][b, r] == depth] for b in range(B)]
            if depth == 1 and base_slot + K <= 64 and K <= max(S, K):
                self.pass_args, _ = rows([n[:K] for n in nodes], K)
            most = max(len(n) for n in nodes)
            for c0 in range(0, most, chunk):
                args, which = rows([n[c0:c0 + chunk] for n in nodes], chunk)
                out, _, _, _ = d.draft_step(*args, self.kv)
                for b, r, q in which:
                    a_node[b, r] = out[q]
        return self._noise(a_node, t)

    def _noise(self, a_node, t):
        import torch
        cfg = self.cfg
        w = self.w
        x = a_node.view(-1, cfg.H)
        x = x * torch.rsqrt((x * x).mean(-1, keepdim=True) + cfg.eps) * w["g_final"].float()
        logits = (x @ w["w_lm"].float().t()).view(cfg.B, cfg.N + 1, cfg.V)
        logits += 2.0 * torch.randn(logits.shape, generator=self.gen, device="cuda")
        for b in range(cfg.B):
            logits[b, int(t["n_nodes"][b]) + 1:] = 0.0
        return logits.contiguous()

    def launches_per_step(self):
        import torch
        self.d.profile(True)
        self.step()
        torch.cuda.synchronize()
        prof = self.d.profile_read()
        self.d.profile(False)
        return sum(v["launches"] for v in prof.values())

    def run(self, steps, warmup, profile=True):
        """K timed steps back to back.  With profile, the library brackets
        every launch of a sample of the steps (one in PROFILE_STRIDE, spread
        over the timed region) with HIP events on the launch stream; each
        event pair costs a few microseconds of launch gap, so the rest run
        without them."""
        import torch
        prof_steps = set()
        if profile:
            per = self.launches_per_step()
            stride = PROFILE_STRIDE if steps >= PROFILE_STRIDE else 1
            prof_steps = set(range(0, steps, stride))
            while len(prof_steps) * per > PROFILE_PAIRS:
                prof_steps = set(sorted(prof_steps)[::2])
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        started = False
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(steps):
            if i in prof_steps:
                self.d.profile(True, resume=started)
                started = True
            self.step()
            if i in prof_steps:
                self.d.profile(False)
            ev[i + 1].record()
        torch.cuda.synchronize()
        prof = self.d.profile_read() if prof_steps else None
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        total = ev[0].elapsed_time(ev[steps])
        acc = self.res["accept_len"].cpu()
        return total / steps, per, prof, len(prof_steps), acc

    def run_cold(self, steps, flush_mb):
        """Steps with a flush_mb write between them (caches cold, as after
        the target model's forward): per-step events around the step only."""
        import torch
        junk = torch.empty(flush_mb << 18, dtype=torch.float32, device="cuda")
        per = []
        for i in range(steps):
            junk.fill_(float(i))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            self.step()
            e1.record()
            e1.synchronize()
            per.append(e0.elapsed_time(e1))
        del junk
        return per

    def time_draft_pass(self, iters=50):
        """One eagle_draft_step over K rows per sequence (a depth-2 pass of
        the tree: join, decoder layer, LM head, top-k) timed directly."""
        import torch
        args = self.pass_args
        if args is None:
            return None
        for _ in range(3):
            self.d.draft_step(*args, self.kv)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            self.d.draft_step(*args, self.kv)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters


def pct(xs, q):
    s = sorted(xs)
    return s[min(len(s) - 1, max(0, int(round(q * (len(s) - 1)))))]


def workload_name(cfg):
    return (f"{cfg.name}: H={cfg.H} FC {3 * cfg.H}->{cfg.H}, {cfg.n_q}q/{cfg.n_kv}kv x "
            f"{cfg.hd}, FFN {cfg.F}, V={cfg.V}, ctx {cfg.ctx[0]}-{cfg.ctx[1]}, "
            f"bs={cfg.B}, depth {cfg.D} top-k {cfg.K} nodes {cfg.N}, "
            + ("greedy" if cfg.T == 0 else f"T={cfg.T}") + " verify")


def gemm_roofline(prof, cfg):
    """Roofline of the draft-layer GEMMs (the dominant kernel) from per-launch
    events in the timed region: algorithmic bytes (weights once, activation
    rows in, results out) or flops per launch / mean launch time."""
    p = prof["gemm"]
    if p["launches"] == 0 or p["ms"] <= 0:
        return None
    avg_us = 1e3 * p["ms"] / p["launches"]
    if cfg.B > 16:  # B*K rows: a dense contraction, priced against MFMA
        ach = p["flops"] / (p["ms"] * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                "traffic": None, "kernel": "stream_gemm_kernel (draft-layer GEMMs)",
                "avg_launch_us": round(avg_us, 2),
                "flops_per_launch": p["flops"] / p["launches"]}
    ach = p["bytes"] / (p["ms"] * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
            "traffic": traffic_per_launch(), "kernel": "stream_gemm_kernel (draft-layer GEMMs)",
            "avg_launch_us": round(avg_us, 2),
            "bytes_per_launch": p["bytes"] / p["launches"]}


def traffic_per_launch():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or None if
    the GEMM source changed since they were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    h = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()[:16]
    if rec.get("gemm_source_sha16") != h:
        return None
    return rec.get("traffic_bytes_per_launch")


def run_workload(cfg, w, steps, warmup, profile, flush_mb):
    wl = Workload(cfg, w)
    ms, per, prof, n_prof, acc = wl.run(steps, warmup, profile)
    cold = wl.run_cold(min(steps, 50), flush_mb) if flush_mb else None
    pass_ms = wl.time_draft_pass()
    a = acc.clamp(min=0).float()
    out = {"ms_per_step": ms, "per_step_ms": per, "prof": prof, "n_prof": n_prof,
           "cold_ms": cold, "pass_ms": pass_ms,
           "mean_accept_len": float(a.mean()),
           "verified_tokens_per_s": float((a + 1).sum()) * 1e3 / ms}
    del wl
    return out


def timing_fields(r, cfg, nd=4):
    per = r["per_step_ms"]
    f = {"step_ms_median": round(statistics.median(per), nd),
         "step_ms_p10": round(pct(per, 0.1), nd),
         "step_ms_p90": round(pct(per, 0.9), nd),
         "verified_tokens_per_s": round(r["verified_tokens_per_s"], 2),
         "mean_accept_len": round(r["mean_accept_len"], 4),
         "tau": round(r["mean_accept_len"] + 1, 4)}
    if r["cold_ms"]:
        c = r["cold_ms"]
        f["cold_cache"] = {"steps": len(c), "flush_mb_between_steps": FLUSH_MB,
                           "step_ms_median": round(statistics.median(c), nd),
                           "step_ms_p10": round(pct(c, 0.1), nd),
                           "step_ms_p90": round(pct(c, 0.9), nd)}
    if r["pass_ms"] is not None:
        f["draft_pass_ms"] = round(r["pass_ms"], nd)
        f["draft_pass_rows_per_seq"] = cfg.K
    prof = r["prof"]
    if prof is not None:
        n = r["n_prof"]
        f["roofline"] = gemm_roofline(prof, cfg)
        f["roofline"]["steps_profiled"] = n
        f["kernel_ms_per_step"] = {k: round(v["ms"] / n, nd) for k, v in prof.items()}
        f["kernel_launches_per_step"] = {k: v["launches"] // n for k, v in prof.items()}
    return f


def cpu_baseline(cfg):
    """The oracle (as it stands: float64 NumPy) timed on this host for
    rounds of one sequence at the workload's shape: fuse, D draft passes,
    rerank/flatten, verification.  After a warm-up round, whole rounds until
    about 10 s with BLAS at all host threads, then about 5 s at one thread;
    the median round gives the rate."""
    import numpy as np
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:
        threadpool_info = threadpool_limits = None
    nproc = os.cpu_count() or 1
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    c1 = cfg.replace(B=1, ctx=(cfg.ctx[0], cfg.ctx[0]))
    W = O.Weights(c1, synth.weights(c1, 0))
    s = synth.seq_inputs(c1, 0)
    P = c1.ctx[0]
    cap = P + 2 + (c1.D - 1) * c1.K + 8
    kk, vv = synth.prefix_kv(c1, 0, P)
    tl = np.zeros((c1.N + 1, c1.V), dtype=np.float32)

    def one_round():
        k = np.zeros((c1.n_kv, cap, c1.hd))
        v = np.zeros_like(k)
        k[:, :P] = O.store(kk, c1.dtype)
        v[:, :P] = O.store(vv, c1.dtype)
        kv = O.DraftKV(k, v)
        t0 = time.perf_counter()
        g = O.fuse(W, O.store(s["low"], c1.dtype), O.store(s["mid"], c1.dtype),
                   O.store(s["high"], c1.dtype))
        tree, info = O.draft_tree(W, kv, g, [s["token"]], P)
        O.verify(c1, tree, tl, c1.T, seed=1, rnd=0, b=0)
        return time.perf_counter() - t0

    def timed(threads, budget_s):
        """Warm-up round, then whole rounds until budget_s of CPU time."""
        def go():
            one_round()
            ts = []
            while sum(ts) < budget_s or len(ts) < 3:
                ts.append(one_round())
            return ts
        if threadpool_limits is not None and threads is not None:
            with threadpool_limits(limits=threads):
                return go()
        return go()

    used = nproc
    if threadpool_info is not None:
        used = max([i.get("num_threads", 1) for i in threadpool_info()] or [nproc])
    ts_all = timed(None, 10.0)
    ts_one = timed(1, 5.0)
    t_all = statistics.median(ts_all)
    t_one = statistics.median(ts_one)
    return {"value": round(1.0 / t_all, 4), "unit": "draft-tree steps/s",
            "cores": int(used), "kind": "oracle",
            "sample": (f"rounds of one sequence at the {cfg.name} shape "
                       f"(fuse, {c1.D} draft passes, rerank, "
                       + ("greedy" if c1.T == 0 else "sampling") +
                       " verify), float64 NumPy oracle, after one warm-up round: "
                       f"{len(ts_all)} rounds, median {t_all:.3f} s, with {used} "
                       f"BLAS threads; {len(ts_one)} rounds, median {t_one:.3f} s, "
                       "with 1; value = batch-1 rounds/s at all threads"),
            "single_thread_value": round(1.0 / t_one, 4), "host_cpu": model,
            "host_nproc": nproc}


def main():
    a = parse()
    if a.summarize_trace:
        summarize_trace(a.summarize_trace)
        return
    if a.traffic_from:
        traffic_record(*a.traffic_from, a.calib_copy_mb << 20, TRAFFIC_FILE)
        return
    if a.gpus != 1:
        print("bench.py measures one GPU: there is no multi-GPU path, so --gpus "
              "must be 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    global FLUSH_MB
    FLUSH_MB = a.flush_mb
    cfg = synth.config(a.config)
    w = gpu_weights(cfg)
    r = run_workload(cfg, w, a.steps, a.warmup, not a.no_profile, a.flush_mb)
    ms = r["ms_per_step"]
    out = {
        "metric": METRIC,
        "value": round(1e3 / ms, 3),
        "unit": "draft-tree steps/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": workload_name(cfg), "batch": cfg.B, "depth": cfg.D,
                   "topk": cfg.K, "nodes": cfg.N},
        "target_logits": "draft logits at every tree row + N(0, 2^2) noise",
    }
    out.update(timing_fields(r, cfg))
    for name in [s for s in a.secondary.split(",") if s]:
        c2 = synth.config(name)
        same = (c2.H, c2.F, c2.V, c2.n_q, c2.n_kv) == (cfg.H, cfg.F, cfg.V, cfg.n_q, cfg.n_kv)
        w2 = w if same else gpu_weights(c2)
        r2 = run_workload(c2, w2, a.secondary_steps, 3, not a.no_profile, a.flush_mb)
        sec = {"workload": workload_name(c2), "batch": c2.B,
               "steps": a.secondary_steps,
               "ms_per_step": round(r2["ms_per_step"], 3),
               "draft_tree_steps_per_s": round(1e3 / r2["ms_per_step"], 3)}
        sec.update(timing_fields(r2, c2, nd=3))
        out.setdefault("secondary", []).append(sec)
        if not same:
            del w2
        torch.cuda.empty_cache()
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
