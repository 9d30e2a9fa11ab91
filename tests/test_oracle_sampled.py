"""Pins of the oracle's sampled-children trees and their verification.

  * the Gumbel-top-k draws are sequential sampling without replacement:
    joint frequencies of the first two draws over many Philox key rows
    against q(x1) q(x2) / (1 - q(x1)) (chi-square), and the draws of
    different key rows are independent;
  * the sampled-row verification keeps the target law exactly: summing
    over every ordered draw of the children with its probability, the
    acceptance probabilities and the final residual of sampled_row_steps
    give an emitted-token law equal to softmax(target / T) (brute force on
    small vocabularies, K = 1..3);
  * a drafted tree with sampled children keeps every draw, in draw order,
    under its parent; its verification draws the bonus from the target
    alone at childless rows;
  * over seeded rounds, the first emitted token of a root with sampled
    children follows the target law (chi-square).
"""
import itertools

import numpy as np
from scipy import stats

import oracle as O
import synth


def _softmax(x, T):
    x = np.asarray(x, dtype=np.float64) / T
    e = np.exp(x - x.max())
    return e / e.sum()


def test_gumbel_top_k_is_sampling_without_replacement():
    V, K, T = 6, 2, 0.7
    rng = np.random.default_rng(11)
    lg = rng.normal(0, 1.5, V).astype(np.float32)
    q = _softmax(lg, T)
    n = 60000
    u = O.gumbel_uniforms(12345, 3, 1, np.arange(1, n + 1), V)
    counts = np.zeros((V, V))
    for i in range(n):
        toks, _ = O.sample_children(lg, T, K, u[i])
        counts[toks[0], toks[1]] += 1
    want = np.array([[q[a] * q[b] / (1 - q[a]) if a != b else 0.0 for b in range(V)]
                     for a in range(V)])
    assert counts.trace() == 0, "a token drawn twice"
    mask = want > 0
    chi = stats.chisquare(counts[mask], want[mask] * n)
    assert chi.pvalue > 1e-4, chi


def test_gumbel_rows_are_independent():
    """Draws of consecutive key rows: first tokens pair up as q x q."""
    V, T = 5, 1.0
    lg = np.array([0.3, -0.2, 1.1, 0.0, -1.0], dtype=np.float32)
    q = _softmax(lg, T)
    n = 40000
    u = O.gumbel_uniforms(7, 0, 0, np.arange(2 * n), V)
    first = np.array([O.sample_children(lg, T, 1, u[i])[0][0] for i in range(2 * n)])
    pairs = np.zeros((V, V))
    np.add.at(pairs, (first[0::2], first[1::2]), 1)
    chi = stats.chisquare(pairs.ravel(), np.outer(q, q).ravel() * n)
    assert chi.pvalue > 1e-4, chi


def _law_of_row(tl, dl, K, T):
    """Emitted-token law at one row: every ordered draw of K children from q
    without replacement, Algorithm 1's acceptances, the final residual."""
    V = len(tl)
    q = _softmax(dl, T)
    law = np.zeros(V)
    for seq in itertools.permutations(range(V), K):
        pr, rest = 1.0, 1.0
        for x in seq:
            pr *= q[x] / rest
            rest -= q[x]
        ratios, resid = O.sampled_row_steps(tl, dl, list(seq), T)
        stay = 1.0
        for x, r in zip(seq, ratios):
            a = min(1.0, r)
            law[x] += pr * stay * a
            stay *= 1.0 - a
        law += pr * stay * resid
    return law


def test_sampled_verification_keeps_target_law_exactly():
    rng = np.random.default_rng(5)
    for V, K in ((3, 1), (4, 2), (5, 3), (5, 2)):
        for T in (1.0, 0.6):
            tl = rng.normal(0, 1.2, V)
            dl = rng.normal(0, 1.2, V)
            law = _law_of_row(tl, dl, K, T)
            np.testing.assert_allclose(law, _softmax(tl, T), rtol=0, atol=1e-12)


def test_identical_draft_and_target_accept_first_child():
    V, K, T = 50, 4, 0.8
    lg = np.random.default_rng(2).normal(0, 1, V)
    ratios, _ = O.sampled_row_steps(lg, lg, [3, 7, 1, 9], T)
    assert ratios[0] >= 1.0 - 1e-12


CFG = synth.config("tiny", H=64, n_q=4, n_kv=2, hd=16, F=96, V=300, ctx=(20, 20),
                   D=3, K=3, N=21)


def _sampled_tree(seed, rnd, b=0):
    cfg = CFG
    W = O.Weights(cfg, synth.weights(cfg, 4))
    s = synth.seq_inputs(cfg, b)
    P = cfg.ctx[0]
    kk, vv = synth.prefix_kv(cfg, b, P)
    cap = P + 2 + (cfg.D - 1) * cfg.K + 8
    k = np.zeros((cfg.n_kv, cap, cfg.hd))
    v = np.zeros_like(k)
    k[:, :P] = O.store(kk, cfg.dtype)
    v[:, :P] = O.store(vv, cfg.dtype)
    kv = O.DraftKV(k, v)
    g = O.fuse(W, O.store(s["low"], "fp32"), O.store(s["mid"], "fp32"),
               O.store(s["high"], "fp32"))
    tree, info = O.draft_tree(W, kv, g, [s["token"]], P,
                              sample={"T": 1.0, "seed": seed, "rnd": rnd, "b": b})
    return cfg, tree, info


def test_sampled_tree_keeps_every_draw_in_order():
    cfg, tree, info = _sampled_tree(99, 0)
    assert tree["n_nodes"] == cfg.n_cand
    rows = O.draft_rows(cfg, tree, info)
    for v in range(tree["n_nodes"] + 1):
        nc = tree["n_child"][v]
        if nc == 0:
            continue
        e = 0 if v == 0 else 1 + tree["kv_slot"][v]
        node_id = -1 if v == 0 else None
        if v > 0:
            # the node whose slot is kv_slot[v]
            node_id = next(n["id"] for n in info["nodes"] if n.get("slot") == tree["kv_slot"][v])
        u = O.gumbel_uniforms(99, 0, 0, 0 if v == 0 else 1 + node_id, cfg.V)
        want, _ = O.sample_children(rows[e], 1.0, cfg.K, u)
        fc = tree["first_child"][v]
        assert list(tree["token"][fc:fc + nc]) == want, v


def test_sampled_root_first_token_law():
    """Root with sampled children, target at temperature 1: over rounds the
    first emitted token follows softmax(target)."""
    V, K, T = 8, 3, 1.0
    rng = np.random.default_rng(8)
    dl = rng.normal(0, 1, V).astype(np.float32)
    tl = rng.normal(0, 1, V).astype(np.float32)
    p = _softmax(tl, T)
    n = 20000
    ug = O.gumbel_uniforms(21, 0, 0, np.arange(n), V)
    uv = O.uniform01(22, O.STREAM_VERIFY, np.arange(n)[:, None], 0, 0,
                     np.append(np.arange(K), O.BONUS_DRAW)[None, :])
    counts = np.zeros(V)
    for i in range(n):
        kids, _ = O.sample_children(dl, T, K, ug[i])
        ci, tok, _ = O.verify_row_sampled(tl, dl, kids, T, lambda j: uv[i, j],
                                          lambda: uv[i, K])
        counts[kids[ci] if ci is not None else tok] += 1
    chi = stats.chisquare(counts, p * n)
    assert chi.pvalue > 1e-4, chi
