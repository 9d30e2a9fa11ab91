"""GPU parity of trees with sampled children and their verification, through
the C ABI against the oracle on the same seeded inputs:

  * eagle_draft_tree_sampled: every tree array bit-exact (tokens in draw
    order, topology, slots, masks; values within the bf16 tolerance) and the
    expanded nodes' draft logits within tolerance, at batch 3 and at batch
    23 (the dense GEMM path);
  * eagle_verify_tree_sampled: accepted lengths, tokens and the commit equal
    the oracle's Algorithm 1 with per-child draft distributions, both sides
    reading the same trees, draft logits and target logits, over several
    seeded rounds and two temperatures.

Inputs whose drafting draws come within 1e-3 of a tie are redrawn (next
attempt); target noise is redrawn while a verification decision sits within
1e-6 of its threshold."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from harness import (MARGIN, SEED, Model, Seq, as_np, assert_tree_equal, cap_for, tol,
                     tree_to_np, upload_batch)

pytestmark = pytest.mark.gpu

MID = dict(H=1024, n_q=8, n_kv=2, hd=128, F=2816, V=8000, ctx=(200, 700),
           D=3, K=3, N=21)
_models = {}
RND = 5


def _model(B):
    if B not in _models:
        print(f"[setup] model B={B}", flush=True)
        _models[B] = Model(synth.config("8b_bs1", **dict(MID, B=B)))
    return _models[B]


def _sampled_seq(m, b, ctx, cap, T):
    """Seeded inputs of sequence b with the oracle's sampled tree; redrawn
    while a drafting decision lies within MARGIN of a tie."""
    for attempt in range(40):
        s = Seq(m, b, ctx, cap, attempt, run_oracle=False)
        W = m.oracle
        s.g = O.fuse(W, as_np(s.low), as_np(s.mid), as_np(s.high))
        s.kv = O.DraftKV(as_np(s.k), as_np(s.v))
        s.tree, s.info = O.draft_tree(W, s.kv, s.g, [s.token], ctx,
                                      sample={"T": T, "seed": SEED, "rnd": RND, "b": b})
        s.margin = O.decision_margin(m.cfg, s.info)
        if s.margin >= MARGIN:
            return s
    raise RuntimeError("no input draw met the decision margin")


def _draft(B, T):
    m = _model(B)
    cfg = m.cfg
    ctxs = synth.contexts(cfg)
    cap = cap_for(cfg, int(ctxs.max()))
    seqs = [_sampled_seq(m, b, int(ctxs[b]), cap, T) for b in range(B)]
    d = m.drafter(max_batch=B)
    kv, feats, tok, seed_len = upload_batch(m, seqs, cap)
    g = d.fuse(*feats)
    seed_src = torch.zeros(B, d.shape.max_seed, cfg.H, dtype=torch.float32, device="cuda")
    seed_src[:, 0] = g
    tree, len_out, dlog = d.draft_tree_sampled(seed_src, tok, seed_len, kv, T, SEED, RND)
    torch.cuda.synchronize()
    assert d.device_status() == 0
    return m, seqs, d, kv, tree, len_out, dlog


@pytest.mark.parametrize("B,T", [(3, 1.0), (3, 0.6), (23, 1.0)])
def test_sampled_draft_matches_oracle(B, T):
    m, seqs, d, kv, tree, len_out, dlog = _draft(B, T)
    cfg = m.cfg
    atol, rtol = tol(cfg)
    for b, s in enumerate(seqs):
        assert int(len_out[b]) == s.ctx + 1
        t = tree_to_np(tree, b)
        assert int(t["n_nodes"]) == cfg.n_cand
        assert_tree_equal(cfg, t, s.tree)
        want = O.draft_rows(cfg, s.tree, s.info)
        np.testing.assert_allclose(dlog[b].cpu().numpy(), want, atol=atol, rtol=rtol,
                                   err_msg=f"draft logits seq {b}")
    print(f"[sampled] B={B} T={T}: {B} sampled trees equal", flush=True)


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_sampled_verify_matches_oracle(T):
    B = 3
    m, seqs, d, kv, tree, _, _ = _draft(B, T)
    cfg = m.cfg
    rows = np.stack([O.draft_rows(cfg, s.tree, s.info) for s in seqs])
    dlog = torch.from_numpy(rows).cuda()
    kv_len = torch.empty(B, dtype=torch.int32, device="cuda")
    accepted = 0
    for rnd in range(6):
        tl = []
        for s in seqs:
            base = O.score_rows(m.oracle, s.kv, s.tree, s.info).astype(np.float64)
            for att in range(30):
                noise = synth.normal(synth.GenKey(3, "sv", s.b, rnd, att), base.shape, std=2.0)
                # sharpened towards the drafter so children get accepted; in
                # round 0 the target of sequence 0 is the drafter itself, so
                # every visited row with children accepts its first child
                t = ((base + noise) * (3.0 if rnd % 2 else 1.0)).astype(np.float32)
                if rnd == 0 and s.b == 0:
                    t = base.astype(np.float32)
                w = O.verify_sampled(cfg, s.tree, t, rows[s.b], T, seed=SEED, rnd=rnd, b=s.b)
                if w["margin"] >= 1e-6:
                    break
            tl.append(t)
        tl = np.stack(tl)
        res = d.verify_sampled(tree, torch.from_numpy(tl).cuda(), dlog, T, seed=SEED,
                               round=rnd, kv=kv, kv_len_out=kv_len)
        torch.cuda.synchronize()
        for b, s in enumerate(seqs):
            want = O.verify_sampled(cfg, s.tree, tl[b], rows[b], T, seed=SEED, rnd=rnd, b=b)
            accepted += want["accept_len"]
            if rnd == 0 and b == 0:
                # each visited row accepts its first child until a leaf
                assert want["accept_len"] >= 1, "target = drafter accepts the first child"
            assert int(res["accept_len"][b]) == want["accept_len"], (rnd, b)
            assert np.array_equal(res["tokens"][b].cpu().numpy(), want["tokens"]), (rnd, b)
            okv = s.kv.copy()
            new_len, srows, stoks = O.commit(cfg, s.tree, want, okv)
            assert int(kv_len[b]) == new_len
            n = int(res["seed_len"][b])
            assert list(res["seed_rows"][b, :n].cpu().numpy()) == srows
            assert list(res["seed_tokens"][b, :n].cpu().numpy()) == stoks
    print(f"[sampled] verify T={T}: accepted {accepted} over 6 rounds", flush=True)
