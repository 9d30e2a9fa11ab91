"""Pins of the oracle's EAGLE-2 tree growth, rerank and flatten, and of its
draft pass under tree masks (no GPU)."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _mock_expand(table):
    """expand() over a fixed {parent name: [(child name, confidence)]} table;
    tokens are the children's names."""
    def expand(parents, depth):
        out = []
        for p in parents:
            name = p.get("name", "root")
            kids = table.get(name, [])
            out.append([(c, np.float32(math.log(conf))) for c, conf in kids])
        return out
    return expand


def _named_root():
    return {"id": -1, "token": "root", "name": "root", "parent": None,
            "depth": 0, "score": np.float32(0.0)}


def test_worked_example_selects_connected_budget():
    fix = json.load(open(os.path.join(GOLDEN, "m75_tree_example.json")))
    # expansion of A/B needs names on the nodes before they are expanded
    table = fix["children"]

    def expand(parents, depth):
        return [[(c, np.float32(math.log(conf)))
                 for c, conf in table.get(p["token"], [])] for p in parents]

    sel, nodes = O.eagle2_tree(_named_root(), expand, fix["expansion_width"],
                               fix["max_depth"], fix["budget"])
    assert [n["token"] for n in sel] == fix["selected"]
    order = [n["token"] for n in sorted(nodes, key=O.select_key)]
    assert order == fix["global_order"]
    for n in nodes:
        assert abs(math.exp(float(n["score"])) - fix["path_values"][n["token"]]) < 1e-6
    # breadth-first order would have spent the last slot elsewhere
    bfs = [n["token"] for n in sorted(nodes, key=lambda n: (n["depth"], n["id"]))]
    assert bfs[:4] == fix["breadth_first_would_select"]
    assert set(bfs[:4]) != set(fix["selected"])


@pytest.mark.parametrize("bad", [
    dict(width=0), dict(width=1.5), dict(budget=-1), dict(depth=-2),
])
def test_argument_validation(bad):
    args = dict(width=2, depth=2, budget=3)
    args.update(bad)
    with pytest.raises(ValueError):
        O.eagle2_tree(_named_root(), lambda p, d: [[] for _ in p],
                      args["width"], args["depth"], args["budget"])


@pytest.mark.parametrize("kids", [
    [("x", 0.5), ("x", 0.2)],          # duplicate token under one parent
    [("x", 0.7), ("y", 0.6)],          # sibling mass above one
])
def test_record_validation(kids):
    with pytest.raises(ValueError):
        O.eagle2_tree(_named_root(),
                      lambda p, d: [[(t, np.float32(math.log(c)))
                                     for t, c in kids] for _ in p], 2, 1, 3)


def test_budget_zero_gives_empty_tree():
    sel, nodes = O.eagle2_tree(_named_root(), lambda p, d: 1 / 0, 2, 3, 0)
    assert sel == [] and nodes == []


def _random_expand(seed, K, V=50):
    rng = np.random.default_rng(seed)

    def expand(parents, depth):
        out = []
        for _ in parents:
            p = rng.dirichlet(np.full(V, 0.3))
            ids = np.argsort(-p)[:K]
            out.append([(int(t), np.float32(math.log(p[t])))
                        for t in sorted(ids)])
        return out
    return expand


@pytest.mark.parametrize("seed", range(6))
def test_selection_is_best_closed_subset_brute_force(seed):
    K, D, N = 2, 3, 4
    sel, nodes = O.eagle2_tree(_named_root(), _random_expand(seed, K), K, D, N)
    assert len(nodes) == K + (D - 1) * K * K
    ids = {n["id"] for n in sel}
    # ancestor closed
    for n in sel:
        assert n["parent"]["id"] == -1 or n["parent"]["id"] in ids
    # maximum total value over every size-N subset, unique under the order
    best = max(itertools.combinations(nodes, N),
               key=lambda c: (sum(float(n["score"]) for n in c),
                              [-k for k in sorted(n["depth"] for n in c)]))
    assert {n["id"] for n in best} == ids
    # values never increase along a path
    for n in nodes:
        if n["parent"]["id"] != -1:
            assert n["score"] <= n["parent"]["score"]


def test_expansion_keeps_only_newest_layer_best():
    K, D = 3, 4
    expanded = []

    def expand(parents, depth):
        expanded.append([p["id"] for p in parents])
        return _random_expand(7, K)(parents, depth)

    sel, nodes = O.eagle2_tree(_named_root(), expand, K, D, 100)
    assert expanded[0] == [-1]
    for d in range(1, D):
        layer_nodes = [n for n in nodes if n["depth"] == d]
        best = sorted(layer_nodes, key=O.select_key)[:K]
        assert expanded[d] == sorted(n["id"] for n in best)
    assert len(sel) == len(nodes) == K + (D - 1) * K * K


def _tiny(**kw):
    cfg = synth.config("tiny", **kw)
    W = O.Weights(cfg, synth.weights(cfg, 0))
    s = synth.seq_inputs(cfg, 0)
    P = cfg.ctx[0]
    cap = P + 4 + (cfg.D + 1) * cfg.K + cfg.N
    kk, vv = synth.prefix_kv(cfg, 0, P)
    k = np.zeros((cfg.n_kv, cap, cfg.hd))
    v = np.zeros_like(k)
    k[:, :P], v[:, :P] = kk, vv
    kv = O.DraftKV(k, v)
    g = O.fuse(W, s["low"], s["mid"], s["high"])
    return cfg, W, kv, g, s["token"], P


def test_flatten_invariants_tiny():
    cfg, W, kv, g, tok, P = _tiny()
    tree, info = O.draft_tree(W, kv, g, [tok], P)
    n = tree["n_nodes"]
    assert n == cfg.N
    assert len(info["nodes"]) == cfg.n_cand
    assert tree["position"][0] == P and tree["depth"][0] == 0
    for r in range(1, n + 1):
        p = tree["parent"][r]
        assert 0 <= p < r
        assert tree["depth"][r] == tree["depth"][p] + 1
        assert tree["position"][r] == P + tree["depth"][r]
        assert tree["score"][r] <= tree["score"][p]
        # ancestry mask = ancestors + self
        anc, a = set(), r
        while a != -1:
            anc.add(a)
            a = tree["parent"][a]
        bits = {j for j in range(n + 1)
                if (int(tree["mask"][r, j // 64]) >> (j % 64)) & 1}
        assert bits == anc
    # canonical order: (depth, parent row, token)
    keys = [(tree["depth"][r], tree["parent"][r], tree["token"][r])
            for r in range(1, n + 1)]
    assert keys == sorted(keys)
    # children contiguous and counted
    for r in range(n + 1):
        kids = [c for c in range(1, n + 1) if tree["parent"][c] == r]
        assert tree["n_child"][r] == len(kids)
        if kids:
            assert kids == list(range(tree["first_child"][r],
                                      tree["first_child"][r] + len(kids)))
    # a node with a child in the tree was expanded and owns a scratch slot
    for r in range(1, n + 1):
        if tree["n_child"][r] > 0:
            assert tree["kv_slot"][r] >= 0


def test_chain_tree_equals_causal_attention():
    """K=1: every node attends to the prefix plus its ancestors, which is
    plain causal attention over the chain appended to the prefix."""
    cfg, W, kv, g, tok, P = _tiny(K=1, D=4, N=4)
    kv0 = kv.copy()
    tree, info = O.draft_tree(W, kv, g, [tok], P, record=True)
    chain = [info["root"]] + [n for n in sorted(info["nodes"],
                                                key=lambda n: n["id"])]
    expanded = [n for n in chain[1:] if "a" in n]
    src = np.stack([g[0]] + [n["parent"]["a"] for n in expanded])
    toks = [tok] + [n["token"] for n in expanded]
    R = len(toks)
    out = O.layer(W, kv0, src, toks, pos=np.arange(P, P + R),
                  dest=np.arange(P, P + R),
                  visible=[np.arange(P + i + 1) for i in range(R)])
    got = np.stack([info["root"]["a"]] + [n["a"] for n in expanded])
    assert np.allclose(out["a"], got, rtol=1e-6, atol=1e-6)
    # the cache rows of the chain match the scratch rows
    for i, n in enumerate(expanded):
        assert np.allclose(kv.k[:, P + 1 + n["slot"]], kv0.k[:, P + 1 + i],
                           rtol=1e-6, atol=1e-6)


def test_branch_independence():
    """A node's output does not depend on K/V rows of non-ancestors."""
    cfg, W, kv, g, tok, P = _tiny()
    tree, info = O.draft_tree(W, kv, g, [tok], P, record=True)
    last = info["passes"][-1]
    node = last["rows"][0]
    len_out = P + 1
    vis = np.concatenate([np.arange(len_out), len_out + np.asarray(
        node["mask_slots"])])
    kv2 = kv.copy()
    others = [s for s in range(cfg.scratch_rows) if s not in node["mask_slots"]]
    kv2.k[:, [len_out + s for s in others]] += 5.0
    kv2.v[:, [len_out + s for s in others]] -= 3.0
    o = O.layer(W, kv2, node["parent"]["a"][None], [node["token"]],
                pos=[P + node["depth"]], dest=[len_out + node["slot"]],
                visible=[vis])
    assert np.array_equal(o["a"][0], node["a"])
    # and it does depend on an ancestor's rows
    kv3 = kv.copy()
    kv3.v[:, len_out + node["mask_slots"][0]] += 50.0
    o3 = O.layer(W, kv3, node["parent"]["a"][None], [node["token"]],
                 pos=[P + node["depth"]], dest=[len_out + node["slot"]],
                 visible=[vis])
    assert not np.array_equal(o3["a"][0], node["a"])


def test_root_only_trees():
    for kw in (dict(N=0), dict(D=0)):
        cfg, W, kv, g, tok, P = _tiny(**kw)
        tree, info = O.draft_tree(W, kv, g, [tok], P)
        assert tree["n_nodes"] == 0
        assert tree["token"][0] == tok and tree["n_child"][0] == 0
        # seed row still committed
        assert info["len_out"] == P + 1
        assert np.any(kv.k[:, P] != 0)
