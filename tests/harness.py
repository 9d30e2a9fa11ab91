"""Parity harness: seeded inputs fed to both the oracle and the HIP library.

Inputs come from `synth`; they are rounded to the drafter's storage type by
torch and the oracle receives exactly the stored values.  A sequence whose
tree decisions have a score margin below 1e-3 (the oracle decides) is redrawn
with the next attempt index."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import synth

MARGIN = 1e-3


# Progress lines reach the terminal even while pytest captures output: the
# full-shape tests spend minutes in the oracle between results, and a run that
# prints nothing for that long looks hung.  The capture manager is set by
# those tests' fixture; elsewhere say() is a plain print.
_capman = None


def say(msg: str) -> None:
    if _capman is not None:
        with _capman.global_and_fixture_disabled():
            print(msg, flush=True)
    else:
        print(msg, flush=True)


def tol(cfg):
    return (2e-2, 2e-2) if cfg.dtype == "bf16" else (1e-4, 1e-4)


def tdtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def stored(cfg, arr) -> torch.Tensor:
    """numpy float32 -> torch tensor in the storage type (CPU)."""
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(tdtype(cfg))


def as_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def shape_of(cfg, max_batch=None, **kw):
    from eagle_draft_tree_amd import DrafterShape
    kw.setdefault("max_seed", cfg.s_max)
    return DrafterShape(hidden=cfg.H, n_q_heads=cfg.n_q, n_kv_heads=cfg.n_kv,
                        head_dim=cfg.hd, ffn=cfg.F, vocab=cfg.V, dtype=cfg.dtype,
                        rope_theta=cfg.theta, depth=cfg.D, topk=cfg.K,
                        budget=cfg.N, max_batch=max_batch or cfg.B,
                        rms_eps=cfg.eps, **kw)


class Model:
    """Weights in storage type on CPU/GPU plus the oracle's float64 copy."""

    def __init__(self, cfg, seed=0, gpu=True):
        self.cfg = cfg
        w32 = synth.weights(cfg, seed)
        self.cpu = {n: stored(cfg, a) for n, a in w32.items()}
        del w32
        self.oracle = O.Weights(cfg, {n: t.float().numpy()
                                      for n, t in self.cpu.items()})
        self.gpu = {n: t.cuda() for n, t in self.cpu.items()} if gpu else None

    def drafter(self, max_batch=None, **kw):
        from eagle_draft_tree_amd import Drafter
        return Drafter(shape_of(self.cfg, max_batch, **kw), self.gpu)


class Seq:
    """One sequence's first-round inputs, with its oracle tree."""

    def __init__(self, model: Model, b: int, ctx: int, cap: int, attempt: int,
                 run_oracle=True, record=False, d2t=None):
        cfg = model.cfg
        self.b, self.ctx, self.cap, self.attempt = b, ctx, cap, attempt
        s = synth.seq_inputs(cfg, b, attempt)
        self.low, self.mid, self.high = (stored(cfg, s[k]) for k in
                                         ("low", "mid", "high"))
        self.token = s["token"] if d2t is None else int(d2t[s["token"]])
        kk, vv = synth.prefix_kv(cfg, b, ctx, attempt)
        self.k = torch.zeros(cfg.n_kv, cap, cfg.hd, dtype=tdtype(cfg))
        self.v = torch.zeros_like(self.k)
        self.k[:, :ctx] = stored(cfg, kk)
        self.v[:, :ctx] = stored(cfg, vv)
        self.tree = self.info = self.kv = self.g = None
        if run_oracle:
            W = model.oracle
            self.g = O.fuse(W, as_np(self.low), as_np(self.mid), as_np(self.high))
            self.kv = O.DraftKV(as_np(self.k), as_np(self.v))
            self.tree, self.info = O.draft_tree(W, self.kv, self.g, [self.token],
                                                ctx, record=record, d2t=d2t)
            self.margin = O.decision_margin(cfg, self.info)


def make_seq(model, b, ctx, cap, run_oracle=True, record=False, max_attempts=50,
             d2t=None):
    for attempt in range(max_attempts):
        s = Seq(model, b, ctx, cap, attempt, run_oracle, record, d2t)
        if not run_oracle or s.margin >= MARGIN:
            return s
    raise RuntimeError("no input draw met the decision margin")


def cap_for(cfg, ctx_max, rounds=1):
    extra = cfg.s_max + (cfg.D - 1) * cfg.K + rounds * (cfg.D + 2) + 64
    return int(ctx_max + extra + 7) // 8 * 8


def upload_batch(model, seqs, cap, s_max=None):
    """KV caches, lengths and first-round seed arrays on the GPU."""
    from eagle_draft_tree_amd import KVCache
    cfg = model.cfg
    B = len(seqs)
    S = s_max or cfg.s_max
    k = torch.stack([s.k for s in seqs]).cuda()
    v = torch.stack([s.v for s in seqs]).cuda()
    kv = KVCache.from_rows(k, v, torch.tensor([s.ctx for s in seqs], dtype=torch.int32).cuda())
    low = torch.stack([s.low for s in seqs]).cuda()
    mid = torch.stack([s.mid for s in seqs]).cuda()
    high = torch.stack([s.high for s in seqs]).cuda()
    tok = torch.full((B, S), -1, dtype=torch.int32)
    tok[:, 0] = torch.tensor([s.token for s in seqs], dtype=torch.int32)
    seed_len = torch.ones(B, dtype=torch.int32)
    return kv, (low, mid, high), tok.cuda(), seed_len.cuda()


def gpu_tree_round(drafter, model, seqs, kv, feats, tok, seed_len):
    """fuse + draft_tree on the GPU for the first round."""
    cfg = model.cfg
    B = len(seqs)
    low, mid, high = feats
    g = drafter.fuse(low, mid, high)
    seed_src = torch.zeros(B, drafter.shape.max_seed, cfg.H, dtype=torch.float32,
                           device="cuda")
    seed_src[:, 0] = g
    tree, len_out = drafter.draft_tree(seed_src, tok, seed_len, kv)
    torch.cuda.synchronize()
    return g, tree, len_out


def tree_to_np(tree, b):
    return {k: v[b].cpu().numpy() for k, v in tree.items()}


def assert_tree_equal(cfg, got, want):
    """Bit-exact topology, tokens, slots, masks; scores within tolerance."""
    n = int(want["n_nodes"])
    assert int(got["n_nodes"]) == n
    for k in ("token", "parent", "depth", "position", "kv_slot", "first_child",
              "n_child"):
        assert np.array_equal(got[k], want[k]), (k, got[k], want[k])
    gm = got["mask"].astype(np.uint64)
    assert np.array_equal(gm, want["mask"]), "mask"
    atol, rtol = tol(cfg)
    np.testing.assert_allclose(got["score"], want["score"], atol=atol, rtol=rtol)


def target_logits(model, seq, rnd=0, attempt=0):
    """Oracle draft logits at every tree row + N(0, 2^2) noise (float32)."""
    cfg = model.cfg
    base = O.score_rows(model.oracle, seq.kv, seq.tree, seq.info)
    noise = synth.target_noise(cfg, seq.b, rnd, cfg.N + 1, attempt)
    out = (base.astype(np.float64) + noise).astype(np.float32)
    out[seq.tree["n_nodes"] + 1:] = 0.0
    return out


# ---------------------------------------------------------------------------
# chained rounds: verify -> commit -> fuse next seed -> draft, oracle side
# ---------------------------------------------------------------------------
SEED = 20240917        # Philox key word 0 of every verification in the tests


def target_logits_for(model, tree, info, kv, b, rnd, attempt=0, d2t=None,
                      target_vocab=None):
    """Oracle draft logits at every tree row + N(0, 2^2) noise (float32),
    spread over the target vocabulary when a reduced draft vocabulary is in
    use (rows outside the draft vocabulary get noise only)."""
    cfg = model.cfg
    base = O.score_rows(model.oracle, kv, tree, info)
    TV = target_vocab or cfg.V
    noise = synth.normal(synth.GenKey(0, "tn", b, rnd, attempt),
                         (cfg.N + 1, TV), std=2.0)
    out = noise.astype(np.float64)
    if d2t is None:
        out += base
    else:
        out[:, d2t] += base
    out = out.astype(np.float32)
    out[tree["n_nodes"] + 1:] = 0.0
    return out


class ChainSeq:
    """One sequence's oracle state across chained rounds."""

    def __init__(self, model, seq, T, mode="keep", d2t=None, target_vocab=None,
                 boost=0.0):
        self.m, self.cfg, self.b = model, model.cfg, seq.b
        self.kv, self.tree, self.info = seq.kv, seq.tree, seq.info
        self.T, self.mode, self.d2t, self.TV = T, mode, d2t, target_vocab
        self.boost = boost
        self.len_out = seq.ctx + 1

    def verify(self, rnd):
        """Target logits for this round (noise redrawn while a sampling
        decision sits within 1e-6 of its threshold) and the oracle's verify
        and commit.  Returns (logits, result, new_len, seed rows, tokens)."""
        for att in range(30):
            tl = target_logits_for(self.m, self.tree, self.info, self.kv,
                                   self.b, rnd, att, self.d2t, self.TV)
            if self.boost:
                # the target leans towards each row's best-valued child, so
                # that paths get accepted and every commit case is reached
                t = self.tree
                for v in range(t["n_nodes"] + 1):
                    if t["n_child"][v] > 0:
                        kids = range(t["first_child"][v],
                                     t["first_child"][v] + t["n_child"][v])
                        best = max(kids, key=lambda c: t["score"][c])
                        tl[v, t["token"][best]] += np.float32(self.boost)
            res = O.verify(self.cfg, self.tree, tl, self.T, seed=SEED, rnd=rnd,
                           b=self.b)
            if self.T == 0 or res["margin"] >= 1e-6:
                break
        self.kv_before_commit = self.kv.copy()
        new_len, rows, toks = O.commit(self.cfg, self.tree, res, self.kv,
                                       mode=self.mode)
        self.new_len, self.seed_rows, self.seed_toks = new_len, rows, toks
        return tl, res

    def draft(self, rnd):
        """Fuse the next seed's synthetic target taps and draft the next tree
        (taps redrawn while the tree's decision margin is below 1e-3)."""
        cfg = self.cfg
        for att in range(50):
            feats = [synth.seed_features(cfg, self.b, rnd, r, att)
                     for r in self.seed_rows]
            taps = [np.stack([as_np(stored(cfg, f[i])) for f in feats])
                    for i in range(3)]
            g = O.fuse(self.m.oracle, *taps)
            kv = self.kv.copy()
            tree, info = O.draft_tree(self.m.oracle, kv, g, self.seed_toks,
                                      self.new_len, d2t=self.d2t)
            if O.decision_margin(cfg, info) >= MARGIN:
                break
        else:
            raise RuntimeError("no input draw met the decision margin")
        self.kv, self.tree, self.info, self.g = kv, tree, info, g
        self.taps = taps
        self.len_out = self.new_len + len(self.seed_rows)
        return att


def close(cfg, got, want, what=""):
    atol, rtol = tol(cfg)
    np.testing.assert_allclose(got, want, atol=atol, rtol=rtol, err_msg=what)


def first_round(m, B, cap_rounds=1, d2t=None, s_max=None, check=None, **shape_kw):
    """Seeded sequences for m.cfg at batch B (contexts drawn as the config
    says), their oracle trees, and the library's first round checked
    against them: fuse, draft_tree, len_out and the tree arrays.  With
    `check`, only those sequences get an oracle tree and are compared."""
    cfg = m.cfg.replace(B=B)
    ctxs = synth.contexts(cfg)
    cap = cap_for(cfg, int(ctxs.max()) + (s_max or 0), rounds=cap_rounds)
    seqs = []
    for b in range(B):
        on = check is None or b in check
        seqs.append(make_seq(m, b, int(ctxs[b]), cap, run_oracle=on, d2t=d2t))
        if on:
            say(f"[oracle] sequence {b} ctx {int(ctxs[b])} tree built")
    d = m.drafter(max_batch=B, **({"max_seed": s_max} if s_max else {}), **shape_kw)
    kv, feats, tok, seed_len = upload_batch(m, seqs, cap, s_max=d.shape.max_seed)
    g, tree, len_out = gpu_tree_round(d, m, seqs, kv, feats, tok, seed_len)
    for b, s in enumerate(seqs):
        assert int(len_out[b]) == s.ctx + 1
        if s.tree is not None:
            assert_tree_equal(m.cfg, tree_to_np(tree, b), s.tree)
    return seqs, d, kv, tree


def run_chain(m, seqs, d, kv, tree, rounds, T, mode, d2t=None, TV=None):
    """`rounds` chained rounds on the GPU against the oracle's ChainSeq:
    verify (accept lengths, tokens), commit (seed rows and tokens, new
    length, committed K/V rows), then fuse the next seed rows and draft the
    next tree (tree arrays).  Sequences with odd b get the target as drawn;
    even b get a target leaning towards each row's best child."""
    from eagle_draft_tree_amd import COMMIT_KEEP, COMMIT_RESEED
    cfg = m.cfg
    B, S = len(seqs), d.shape.max_seed
    chains = [ChainSeq(m, s, T, mode, d2t, TV, boost=0.0 if s.b % 2 else 8.0)
              for s in seqs]
    kv_len = torch.empty(B, dtype=torch.int32, device="cuda")
    accepted = 0
    for rnd in range(rounds):
        outs = [c.verify(rnd) for c in chains]
        tl = np.stack([o[0] for o in outs])
        res = d.verify(tree, torch.from_numpy(tl).cuda(), T, seed=SEED,
                       round=rnd, kv=kv, kv_len_out=kv_len,
                       commit_mode=COMMIT_RESEED if mode == "reseed" else COMMIT_KEEP)
        torch.cuda.synchronize()
        for b, c in enumerate(chains):
            want = outs[b][1]
            accepted += want["accept_len"]
            assert int(res["accept_len"][b]) == want["accept_len"], (rnd, b)
            assert np.array_equal(res["tokens"][b].cpu().numpy(), want["tokens"])
            n = int(res["seed_len"][b])
            assert n == len(c.seed_rows), (rnd, b)
            assert list(res["seed_rows"][b, :n].cpu().numpy()) == c.seed_rows
            assert list(res["seed_tokens"][b, :n].cpu().numpy()) == c.seed_toks
            assert int(kv_len[b]) == c.new_len
            close(cfg, as_np(kv.k[b, :, :c.new_len].cpu()), c.kv.k[:, :c.new_len],
                   "k after commit")
            close(cfg, as_np(kv.v_rows()[b, :, :c.new_len].cpu()), c.kv.v[:, :c.new_len],
                   "v after commit")
        if rnd == rounds - 1:
            break
        atts = [c.draft(rnd) for c in chains]
        low = torch.zeros(B * S, cfg.H, dtype=kv.k.dtype)
        mid, high = low.clone(), low.clone()
        for b, c in enumerate(chains):
            for i in range(len(c.seed_rows)):
                for t, arr in zip((low, mid, high), c.taps):
                    t[b * S + i] = stored(cfg, arr[i])
        g = d.fuse(low.cuda(), mid.cuda(), high.cuda())
        seed_src = g.view(B, S, cfg.H)
        kv.length.copy_(kv_len)
        tree, len_out = d.draft_tree(seed_src, res["seed_tokens"].contiguous(),
                                     res["seed_len"], kv)
        torch.cuda.synchronize()
        for b, c in enumerate(chains):
            assert int(len_out[b]) == c.len_out
            assert_tree_equal(cfg, tree_to_np(tree, b), c.tree)
        say(f"[chain] round {rnd + 1} trees equal (attempts {atts})")
    say(f"[chain] T={T} mode={mode}: accepted {accepted} over {rounds} rounds")
