"""GPU parity of the library's seeded draws, chain drafting (top-1, depth
2-3), the full-reseed commit, the reduced draft vocabulary and chained
verify -> commit -> fuse -> draft rounds, all through the C ABI against the
CPU oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from harness import SEED, Model, first_round, run_chain, stored, tdtype

pytestmark = pytest.mark.gpu

MID = dict(H=1024, n_q=8, n_kv=2, hd=128, F=2816, V=8000, ctx=(200, 700))


def test_philox_draws_match_oracle_on_a_million_counters():
    from eagle_draft_tree_amd import draw_uniforms
    for stream, rnd in ((O.STREAM_VERIFY, 0), (O.STREAM_DRAFT, 12345678901)):
        B, R, J = 16, 977, 64
        got = draw_uniforms(SEED, stream, rnd, B, R, J).cpu().numpy()
        want = O.uniform01(SEED, stream, rnd, np.arange(B)[:, None, None],
                           np.arange(R)[None, :, None], np.arange(J)[None, None, :])
        print(f"[rng] stream {stream}: {got.size} draws", flush=True)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


_models = {}


def _model(key, cfg, embed_rows=None):
    if key not in _models:
        print(f"[setup] model {key}", flush=True)
        m = Model(cfg)
        if embed_rows is not None:
            # a target-vocabulary embedding [TV, H]
            e = synth.normal(synth.GenKey(0, "embed-tv", embed_rows),
                             (embed_rows, cfg.H), std=0.02)
            m.cpu["embed"] = stored(cfg, e)
            m.oracle.embed = O.store(m.cpu["embed"].float().numpy(), cfg.dtype)
            m.gpu["embed"] = m.cpu["embed"].cuda()
        _models[key] = m
    return _models[key]


@pytest.mark.parametrize("B", [2, 16, 64])
def test_chain_mode_top1(B):
    """Chain drafting (K = 1, depth 3): the tree is a single path, verified
    greedily and by seeded sampling."""
    m = _model("chain", synth.config("8b_bs1", **MID, K=1, D=3, N=3))
    cfg = m.cfg
    seqs, d, kv, tree = first_round(m, B)
    print(f"[chain] B={B} trees equal", flush=True)
    for T in (0.0, 1.0):
        tl = []
        for s in seqs:
            t = O.score_rows(m.oracle, s.kv, s.tree, s.info)
            if T == 0:
                # the target agrees with the draft on every second sequence
                if s.b % 2:
                    t = t + synth.normal(synth.GenKey(2, "chain", s.b),
                                         t.shape, std=2.0)
            tl.append(np.asarray(t, dtype=np.float32))
        tl = np.stack(tl)
        res = d.verify(tree, torch.from_numpy(tl).cuda(), T, seed=SEED, round=7)
        torch.cuda.synchronize()
        total = 0
        for b, s in enumerate(seqs):
            want = O.verify(cfg, s.tree, tl[b], T, seed=SEED, rnd=7, b=b)
            if T > 0 and want["margin"] < 1e-6:
                continue
            total += want["accept_len"]
            assert int(res["accept_len"][b]) == want["accept_len"], b
            assert np.array_equal(res["tokens"][b].cpu().numpy(), want["tokens"])
        print(f"[chain] B={B} T={T} accepted {total}", flush=True)
        if T == 0:
            assert total >= (B // 2) * cfg.D


def test_reseed_commit_and_next_draft():
    """Full reseed: nothing moves in the cache, every verified row seeds the
    next round, and the next draft over those seeds matches the oracle."""
    cfg0 = synth.config("8b_bs1", **MID, K=4, D=3, N=10)
    m = _model("reseed", cfg0)
    seqs, d, kv, tree = first_round(m, 3, cap_rounds=2, s_max=cfg0.D + 1)
    run_chain(m, seqs, d, kv, tree, rounds=3, T=1.0, mode="reseed")


@pytest.mark.parametrize("T,mode", [(0.6, "keep"), (0.0, "keep"), (0.6, "reseed")])
def test_chained_rounds(T, mode):
    """Five rounds of verify -> commit -> fuse the next seed -> draft."""
    cfg0 = synth.config("8b_bs1", **MID, K=4, D=4, N=12)
    m = _model("chained", cfg0)
    s_max = cfg0.D + 1 if mode == "reseed" else 2
    seqs, d, kv, tree = first_round(m, 3, cap_rounds=6, s_max=s_max)
    run_chain(m, seqs, d, kv, tree, rounds=5, T=T, mode=mode)


def test_reduced_draft_vocabulary():
    """LM head over a 4000-token draft vocabulary mapped into a 9000-token
    target vocabulary by an increasing d2t; tree tokens, embeddings, target
    logits and verification all use target ids."""
    TV = 9000
    cfg0 = synth.config("8b_bs1", **dict(MID, V=4000), K=4, D=3, N=10)
    m = _model("d2t", cfg0, embed_rows=TV)
    rng = np.random.default_rng(3)
    d2t = np.sort(rng.choice(TV, size=cfg0.V, replace=False)).astype(np.int64)
    m.gpu["d2t"] = torch.from_numpy(d2t.astype(np.int32)).cuda()
    try:
        seqs, d, kv, tree = first_round(m, 3, cap_rounds=3, d2t=d2t,
                                         target_vocab=TV)
        run_chain(m, seqs, d, kv, tree, rounds=2, T=1.0, mode="keep",
                   d2t=d2t, TV=TV)
    finally:
        m.gpu.pop("d2t")


def test_draft_cache_capacity_rule():
    """A draft cache must hold at least one 32-key attention step in whole
    16-byte runs (cap a multiple of 8, at least 32): smaller or ragged
    capacities are rejected before anything is launched."""
    from eagle_draft_tree_amd import KVCache
    from eagle_draft_tree_amd._lib import EagleError
    m = _model("chain", synth.config("8b_bs1", **MID, K=1, D=3, N=3))
    cfg = m.cfg
    d = m.drafter(max_batch=1)
    S = d.shape.max_seed
    seed_src = torch.zeros(1, S, cfg.H, dtype=torch.float32, device="cuda")
    tok = torch.zeros(1, S, dtype=torch.int32, device="cuda")
    seed_len = torch.ones(1, dtype=torch.int32, device="cuda")
    for cap in (24, 36):
        k = torch.zeros(1, cfg.n_kv, cap, cfg.hd, dtype=tdtype(cfg), device="cuda")
        kv = KVCache.from_rows(k, k.clone(), torch.zeros(1, dtype=torch.int32, device="cuda"))
        with pytest.raises(EagleError) as e:
            d.draft_tree(seed_src, tok, seed_len, kv)
        assert e.value.code == 1  # invalid argument
    print("[cap] capacities 24 and 36 rejected", flush=True)
