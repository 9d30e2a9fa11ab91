"""Pins of the oracle's tree verification and commit (no GPU).

The sampling pins use the property the pages fix for Algorithm 1: the emitted
tokens follow the target distribution exactly.  The per-row law is computed
by exhaustive enumeration over a grid of uniforms whose cell edges contain
every acceptance threshold (target probabilities are chosen rational), so the
enumeration is exact; the whole-tree law is checked by a chi-square test."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _logits_for(p, T=1.0):
    """Logits whose softmax at temperature T is p (p > 0)."""
    return (T * np.log(np.asarray(p, dtype=np.float64))).astype(np.float32)


def _exact_row_law(logits, kids, T, G, row_fn=O.verify_row):
    """Law of one verified row's outcome: enumerate u over cell midpoints
    (i + 1/2)/G of each draw that the row actually consumes."""
    law = {}

    def run(prefix, depth_weight):
        draws = list(prefix)
        consumed = []

        def u_child(i):
            consumed.append(("c", i))
            return draws[len(consumed) - 1] if len(consumed) <= len(draws) else None

        def u_bonus():
            consumed.append(("b", None))
            return draws[len(consumed) - 1] if len(consumed) <= len(draws) else None

        # run with a sentinel that aborts when a draw beyond the prefix is read
        class Need(Exception):
            pass

        def uc(i):
            v = u_child(i)
            if v is None:
                raise Need()
            return v

        def ub():
            v = u_bonus()
            if v is None:
                raise Need()
            return v

        try:
            ci, tok, _ = row_fn(logits, kids, T, uc, ub)
        except Need:
            for g in range(G):
                run(prefix + [(g + 0.5) / G], depth_weight / G)  # exact Fraction weights
            return
        key = ("child", kids[ci]) if ci is not None else ("tok", tok)
        law[key] = law.get(key, Fraction(0)) + depth_weight

    run([], Fraction(1))
    return law


@pytest.mark.parametrize("p,kids,G", [
    ([0.5, 0.25, 0.25], [0], 4),
    ([0.4, 0.3, 0.2, 0.1], [1, 2], 70),
    ([0.1, 0.2, 0.3, 0.4], [3, 0], 30),
    ([0.25, 0.25, 0.25, 0.25], [0, 1, 2], 12),
])
def test_sampling_row_law_is_target_exact(p, kids, G):
    law = _exact_row_law(_logits_for(p), kids, 1.0, G)
    for t, pt in enumerate(p):
        key = ("child", t) if t in kids else ("tok", t)
        assert abs(float(law.get(key, 0)) - pt) < 1e-9, (t, law)
    assert sum(law.values()) == 1


def test_point_mass_reading_is_needed_negative():
    """Using q = softmax(draft) as the proposal of a deterministic child is
    not lossless: V = {A, B}, child {A}, q = (0.9, 0.1), p = (0.5, 0.5) emits
    A with probability 5/9.  The exact-law check must catch that variant."""
    q = np.array([0.9, 0.1])

    def wrong_row(logits, kids, T, u_child, u_bonus):
        p = np.exp(np.asarray(logits, np.float64) / T)
        p /= p.sum()
        for i, c in enumerate(kids):
            if u_child(i) < min(1.0, p[c] / q[c]):
                return i, None, 1.0
            p = np.maximum(0.0, p - q)
            p /= p.sum()
        cdf = np.cumsum(p)
        return None, int(np.searchsorted(cdf, u_bonus(), side="right")), 1.0

    law = _exact_row_law(_logits_for([0.5, 0.5]), [0], 1.0, 90,
                         row_fn=wrong_row)
    assert abs(float(law[("child", 0)]) - 5 / 9) < 1e-9
    good = _exact_row_law(_logits_for([0.5, 0.5]), [0], 1.0, 90)
    assert good[("child", 0)] == Fraction(1, 2)


def test_sampling_temperature_scales_logits():
    p = np.array([0.4, 0.3, 0.2, 0.1])
    T = 0.6
    law = _exact_row_law(_logits_for(p, T), [1], T, 70)
    for t in range(4):
        key = ("child", t) if t == 1 else ("tok", t)
        assert abs(float(law[key]) - p[t]) < 1e-9


def _hand_tree(N, K, D, parents, tokens, slots=None):
    """Flattened tree from parent rows (row 0 = root) in canonical order."""
    cfg = synth.config("tiny", N=N, K=K, D=D)
    root = {"id": -1, "token": tokens[0], "parent": None, "depth": 0,
            "score": np.float32(0), "slot": -1}
    nodes = [root]
    sel = []
    for r in range(1, len(parents)):
        p = nodes[parents[r]]
        n = {"id": r - 1, "token": tokens[r], "parent": p,
             "depth": p["depth"] + 1, "score": np.float32(-r),
             "slot": -1 if slots is None else slots[r]}
        nodes.append(n)
        sel.append(n)
    return cfg, O.flatten(cfg, root, sel, 100)


def test_greedy_walk_hand_tree():
    #        root(7)
    #       /      \
    #     1(3)     2(5)
    #    /   \       \
    #  3(0)  4(9)    5(3)
    cfg, tree = _hand_tree(6, 2, 3, [-1, 0, 0, 1, 1, 2], [7, 3, 5, 0, 9, 3])
    V = 16
    lg = np.zeros((cfg.N + 1, V), dtype=np.float32)
    lg[0, 3] = 5.0          # root -> token 3 (row 1)
    lg[1, 9] = 4.0          # row 1 -> token 9 (row 4)
    lg[4, 11] = 2.0         # row 4 is a leaf: bonus 11
    r = O.verify(cfg, tree, lg, 0.0)
    assert r["accept_len"] == 2
    assert list(r["accepted_rows"][:2]) == [1, 4]
    assert list(r["tokens"][:3]) == [3, 9, 11]
    # first mismatch stops the walk; ties pick the lowest id
    lg2 = np.zeros((cfg.N + 1, V), dtype=np.float32)
    lg2[0, 5] = 1.0
    lg2[2, 8] = lg2[2, 4] = 3.0
    r2 = O.verify(cfg, tree, lg2, 0.0)
    assert r2["accept_len"] == 1 and list(r2["tokens"][:2]) == [5, 4]
    # no match at the root: zero accepted, bonus only
    lg3 = np.zeros((cfg.N + 1, V), dtype=np.float32)
    lg3[0, 12] = 1.0
    r3 = O.verify(cfg, tree, lg3, 0.0)
    assert r3["accept_len"] == 0 and r3["tokens"][0] == 12
    assert r3["tokens"][1] == -1


def _tiny_setup(seed=0, **kw):
    cfg = synth.config("tiny", **kw)
    W = O.Weights(cfg, synth.weights(cfg, seed))
    s = synth.seq_inputs(cfg, 0)
    P = cfg.ctx[0]
    cap = P + 4 + (cfg.D + 1) * cfg.K + cfg.N
    kk, vv = synth.prefix_kv(cfg, 0, P)
    k = np.zeros((cfg.n_kv, cap, cfg.hd))
    v = np.zeros_like(k)
    k[:, :P], v[:, :P] = kk, vv
    g = O.fuse(W, s["low"], s["mid"], s["high"])
    return cfg, W, O.DraftKV(k, v), g, s["token"], P


def test_draft_equals_target_accepts_greedy_chain():
    """With target logits equal to the draft logits, the accepted tokens are
    the drafter's own greedy continuation (computed here by plain causal
    decoding with no tree), as far as it lies in the tree."""
    cfg, W, kv, g, tok, P = _tiny_setup(D=4, K=3, N=12)
    kv_chain = kv.copy()
    tree, info = O.draft_tree(W, kv, g, [tok], P)
    target = O.score_rows(W, kv, tree, info)
    res = O.verify(cfg, tree, target, 0.0)
    # greedy chain by causal decoding
    out = O.layer(W, kv_chain, g, [tok], pos=[P], dest=[P],
                  visible=[np.arange(P + 1)])
    chain, src = [], out
    for d in range(cfg.D + 1):
        nxt = int(np.argmax(src["logits"][-1]))
        chain.append(nxt)
        if d == cfg.D:
            break
        src = O.layer(W, kv_chain, src["a"][-1:], [nxt], pos=[P + 1 + d],
                      dest=[P + 1 + d], visible=[np.arange(P + 2 + d)])
    a = res["accept_len"]
    assert a >= 1
    assert list(res["tokens"][: a + 1]) == chain[: a + 1]
    # the chain leaves the tree right after the accepted prefix
    v = int(res["accepted_rows"][a - 1])
    kids = range(tree["first_child"][v],
                 tree["first_child"][v] + tree["n_child"][v])
    assert a == cfg.D or chain[a] not in [tree["token"][c] for c in kids]


def _tree_law(tree, p_rows, n_kids_max):
    """Exact law of the emitted token sequence under the target, given the
    target distribution of each row: first token ~ p_root; if it is a child
    token, continue from that child's row."""
    law = {}

    def walk(v, prefix, prob):
        kids = {int(tree["token"][c]): c for c in
                range(tree["first_child"][v],
                      tree["first_child"][v] + tree["n_child"][v])}
        for t, pt in enumerate(p_rows[v]):
            if t in kids:
                walk(kids[t], prefix + (t,), prob * pt)
            else:
                key = prefix + (t,)
                law[key] = law.get(key, 0.0) + prob * pt

    walk(0, (), 1.0)
    return law


def test_sampling_whole_tree_chi_square():
    rng = np.random.default_rng(11)
    cfg, tree = _hand_tree(5, 2, 2, [-1, 0, 0, 1, 1], [4, 1, 3, 0, 2])
    V, T = 5, 0.8
    lg = (rng.standard_normal((cfg.N + 1, V)) * 1.5).astype(np.float32)
    p_rows = []
    for r in range(cfg.N + 1):
        w = np.exp((lg[r].astype(np.float64) - lg[r].max()) / T)
        p_rows.append(w / w.sum())
    law = _tree_law(tree, p_rows, 2)
    n = 60000
    counts = {}
    U = rng.random((n, cfg.N + 1, cfg.K + 1))
    for i in range(n):
        r = O.verify(cfg, tree, lg, T, U[i])
        key = tuple(int(x) for x in r["tokens"][: r["accept_len"] + 1])
        counts[key] = counts.get(key, 0) + 1
    assert set(counts) <= set(law)
    from scipy.stats import chisquare
    keys = sorted(law)
    obs = np.array([counts.get(k, 0) for k in keys], dtype=np.float64)
    exp = np.array([law[k] * n for k in keys])
    assert abs(exp.sum() - n) < 1e-6 * n
    stat, pval = chisquare(obs, exp)
    assert pval > 1e-4, (stat, pval)


def test_publication_fixture_row_map():
    """Accepted rows map to KV rows through flatten metadata, never through
    token equality: two nodes carry the same token on different branches."""
    fix = json.load(open(os.path.join(GOLDEN, "m75_publication_fixture.json")))
    assert fix["accepted_flatten_rows"] == fix["committed_kv_rows"]
    # root(9) -> rows 1 (tok 5, slot 0), 2 (tok 6, slot 1);
    # row 1 -> row 3 (tok 7); row 2 -> row 4 (tok 7, same token as row 3)
    cfg, tree = _hand_tree(4, 2, 3, [-1, 0, 0, 1, 2], [9, 5, 6, 7, 7],
                           slots=[-1, 0, 1, -1, 2])
    P_root = int(tree["position"][0])
    len_out = P_root + 1
    cap = len_out + 8
    k = np.zeros((1, cap, 2))
    for s in range(4):
        k[0, len_out + s] = [100 + s, 0]
    kv = O.DraftKV(k, k.copy())
    res = {"accept_len": 2, "accepted_rows": np.array([2, 4, -1]),
           "bonus": 3}
    new_len, seed_rows, seed_toks = O.commit(cfg, tree, res, kv)
    # row 2 (slot 1) -> position P_root+1; row 4 (slot 2, depth 2) kept
    assert new_len == len_out + 2
    assert kv.k[0, len_out + 0, 0] == 101
    assert kv.k[0, len_out + 1, 0] == 102
    assert seed_rows == [4] and seed_toks == [3]


@pytest.mark.parametrize("case", ["none", "expanded_last", "leaf_last"])
def test_commit_equals_explicit_concatenation(case):
    cfg, W, kv, g, tok, P = _tiny_setup(D=3, K=2, N=6)
    kv_before = None
    tree, info = O.draft_tree(W, kv, g, [tok], P)
    kv_before = kv.copy()
    len_out = P + 1
    n = tree["n_nodes"]
    # pick an accepted path by hand
    path = []
    if case != "none":
        v = 0
        while tree["n_child"][v] > 0:
            kids = list(range(tree["first_child"][v],
                              tree["first_child"][v] + tree["n_child"][v]))
            want_leaf = case == "leaf_last"
            nxt = kids[0]
            for c in kids:
                if (tree["kv_slot"][c] < 0) == want_leaf or tree["n_child"][c]:
                    nxt = c
                    break
            path.append(nxt)
            v = nxt
            if (case == "expanded_last" and tree["kv_slot"][v] >= 0
                    and len(path) >= 1):
                break
    a = len(path)
    res = {"accept_len": a,
           "accepted_rows": np.array(path + [-1] * (cfg.D - a)),
           "bonus": 17}
    new_len, seed_rows, seed_toks = O.commit(cfg, tree, res, kv)
    kept = [r for r in path if tree["kv_slot"][r] >= 0]
    if a and tree["kv_slot"][path[-1]] < 0:
        kept = path[:-1]
    want = np.concatenate(
        [kv_before.k[:, :len_out]] +
        [kv_before.k[:, len_out + tree["kv_slot"][r]][:, None] for r in kept],
        axis=1)
    assert new_len == len_out + len(kept)
    assert np.array_equal(kv.k[:, :new_len], want)
    if a == 0:
        assert seed_rows == [0] and seed_toks == [17]
    elif tree["kv_slot"][path[-1]] >= 0:
        assert seed_rows == [path[-1]] and seed_toks == [17]
    else:
        prev = path[-2] if a >= 2 else 0
        assert seed_rows == [prev, path[-1]]
        assert seed_toks == [int(tree["token"][path[-1]]), 17]
    assert n == cfg.N


def test_sampling_law_under_seeded_philox_draws():
    """The same whole-tree law, with every draw taken from the counter-based
    generator: round i of seed 2024 drives the i-th verification."""
    rng = np.random.default_rng(12)
    cfg, tree = _hand_tree(5, 2, 2, [-1, 0, 0, 1, 1], [4, 1, 3, 0, 2])
    V, T = 5, 0.7
    lg = (rng.standard_normal((cfg.N + 1, V)) * 1.5).astype(np.float32)
    p_rows = []
    for r in range(cfg.N + 1):
        w = np.exp((lg[r].astype(np.float64) - lg[r].max()) / T)
        p_rows.append(w / w.sum())
    law = _tree_law(tree, p_rows, 2)
    n = 40000
    draws = np.append(np.arange(cfg.K), O.BONUS_DRAW)
    U = O.uniform01(2024, O.STREAM_VERIFY, np.arange(n)[:, None, None], 3,
                    np.arange(cfg.N + 1)[None, :, None], draws[None, None, :])
    counts = {}
    for i in range(n):
        r = O.verify(cfg, tree, lg, T, U[i])
        key = tuple(int(x) for x in r["tokens"][: r["accept_len"] + 1])
        counts[key] = counts.get(key, 0) + 1
    # the seeded entry point draws exactly these numbers
    for i in (0, 17, n - 1):
        a = O.verify(cfg, tree, lg, T, seed=2024, rnd=i, b=3)
        b = O.verify(cfg, tree, lg, T, U[i])
        assert list(a["tokens"]) == list(b["tokens"])
    from scipy.stats import chisquare
    keys = sorted(law)
    obs = np.array([counts.get(k, 0) for k in keys], dtype=np.float64)
    exp = np.array([law[k] * n for k in keys])
    stat, pval = chisquare(obs, exp)
    assert pval > 1e-4, (stat, pval)


@pytest.mark.parametrize("case", ["none", "leaf_last"])
def test_reseed_commit_keeps_nothing_and_seeds_every_verified_row(case):
    """Full reseed: no draft row survives; the next seed pairs every verified
    row's target feature with the token that follows it, and the next draft
    call appends them at the root's position + 1."""
    cfg, W, kv, g, tok, P = _tiny_setup(D=3, K=2, N=6)
    tree, info = O.draft_tree(W, kv, g, [tok], P)
    kv_before = kv.copy()
    path = []
    if case != "none":
        v = 0
        while tree["n_child"][v] > 0:
            v = int(tree["first_child"][v] + tree["n_child"][v] - 1)
            path.append(v)
    a = len(path)
    res = {"accept_len": a,
           "accepted_rows": np.array(path + [-1] * (cfg.D - a)),
           "bonus": 21}
    new_len, rows, toks = O.commit(cfg, tree, res, kv, mode="reseed")
    assert new_len == P + 1
    assert rows == [0] + path
    assert toks == [int(tree["token"][r]) for r in path] + [21]
    assert np.array_equal(kv.k, kv_before.k)
    # the next round's seed rows land at P+1.. and see the prefix causally
    feats = np.stack([g[0] * (1 + 0.1 * i) for i in range(len(rows))])
    kv2 = kv.copy()
    tree2, info2 = O.draft_tree(W, kv2, feats, toks, new_len)
    assert info2["len_out"] == new_len + len(rows)
    assert tree2["position"][0] == new_len + len(rows) - 1
    kv3 = kv.copy()
    ref = O.layer(W, kv3, feats, toks, pos=np.arange(new_len, new_len + len(rows)),
                  dest=np.arange(new_len, new_len + len(rows)),
                  visible=[np.arange(new_len + i + 1) for i in range(len(rows))])
    lo, hi = new_len, new_len + len(rows)
    assert np.array_equal(kv2.k[:, lo:hi], kv3.k[:, lo:hi])
    assert np.array_equal(info2["root"]["a"], ref["a"][-1])


def test_reduced_vocabulary_map():
    """With an increasing draft->target id map d2t and a target embedding
    whose row d2t[i] equals the draft table's row i, the tree is the unmapped
    tree with every token sent through d2t."""
    cfg, W, kv, g, tok, P = _tiny_setup(D=3, K=3, N=8)
    kv0 = kv.copy()
    tree0, _ = O.draft_tree(W, kv0, g, [tok], P)
    V = cfg.V
    d2t = np.arange(V) * 3 + 1
    Vt = int(d2t[-1]) + 5
    rng = np.random.default_rng(3)
    Et = rng.standard_normal((Vt, cfg.H)) * 0.02
    Et[d2t] = W.embed
    W2 = O.Weights(cfg, {n: getattr(W, n) for n in O.Weights.NAMES})
    W2.embed = Et
    kv1 = kv.copy()
    root_tok = int(d2t[tok])
    tree1, _ = O.draft_tree(W2, kv1, g, [root_tok], P, d2t=d2t)
    n = tree0["n_nodes"]
    assert tree1["n_nodes"] == n
    for k in ("parent", "depth", "position", "kv_slot", "first_child",
              "n_child"):
        assert np.array_equal(tree1[k], tree0[k]), k
    assert np.array_equal(tree1["score"], tree0["score"])
    assert list(tree1["token"][1:n + 1]) == list(d2t[tree0["token"][1:n + 1]])
    assert tree1["token"][0] == root_tok
    assert np.array_equal(kv1.k, kv0.k)
