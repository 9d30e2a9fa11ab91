"""Pins of the oracle's target tree layer (the target's verification forward
over the flattened draft tree under tree attention).

  * every root-to-leaf path of the tree gives, row for row, the outputs of
    a separate causal pass over that path alone (siblings and cousins are
    invisible; each row sees the prefix and its own ancestors);
  * with zero attention-output and down projections the block is the
    identity on its input, so the logits reduce to the closed form
    LM(rmsnorm(E[token]) * g_final).
"""
import numpy as np

import oracle as O
import synth

CFG = synth.config("tiny", H=64, n_q=4, n_kv=2, hd=16, F=96, V=200, ctx=(9, 9),
                   D=3, K=2, N=5)


def _weights(cfg, zero=()):
    w = synth.weights(cfg, 7)
    for n in zero:
        w[n] = np.zeros_like(w[n])
    return O.Weights(cfg, w)


def _tree(p_root):
    """root -> rows 1, 2; row 1 -> rows 3, 4; row 2 -> row 5 (canonical
    order: by depth, parent row, token id)."""
    parent = np.array([-1, 0, 0, 1, 1, 2])
    depth = np.array([0, 1, 1, 2, 2, 2])
    token = np.array([11, 3, 150, 7, 42, 99])
    return {"token": token, "parent": parent, "depth": depth,
            "position": p_root + depth, "n_nodes": 5}


def _prefix(cfg, P, cap):
    kk, vv = synth.prefix_kv(cfg, 0, P)
    k = np.zeros((cfg.n_kv, cap, cfg.hd))
    v = np.zeros_like(k)
    k[:, :P] = O.store(kk, cfg.dtype)
    v[:, :P] = O.store(vv, cfg.dtype)
    return O.DraftKV(k, v)


def test_paths_equal_separate_causal_passes():
    cfg = CFG
    W = _weights(cfg)
    P = 9
    tree = _tree(P)
    kv = _prefix(cfg, P, 40)
    full = O.target_tree_layer(W, kv.copy(), tree, P)
    leaves = [3, 4, 5]
    for leaf in leaves:
        path = O.tree_ancestors(tree, leaf)
        kv2 = _prefix(cfg, P, 40)
        x = O.store(W.embed[tree["token"][path]], "fp32")
        vis = [np.arange(P + i + 1) for i in range(len(path))]
        alone = O.block(W, kv2, x, pos=tree["position"][path],
                        dest=np.arange(P, P + len(path)), visible=vis)
        for i, r in enumerate(path):
            np.testing.assert_allclose(full["a"][r], alone["a"][i], rtol=1e-6, atol=1e-6)
            np.testing.assert_allclose(full["logits"][r], alone["logits"][i],
                                       rtol=1e-5, atol=1e-5)


def test_sibling_branch_is_invisible():
    """Changing the token of row 2 (a sibling branch of rows 1, 3, 4) leaves
    those rows' outputs unchanged and changes row 2's and row 5's."""
    cfg = CFG
    W = _weights(cfg)
    P = 9
    t1 = _tree(P)
    t2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in t1.items()}
    t2["token"][2] = 151
    a = O.target_tree_layer(W, _prefix(cfg, P, 40), t1, P)
    b = O.target_tree_layer(W, _prefix(cfg, P, 40), t2, P)
    for r in (0, 1, 3, 4):
        np.testing.assert_array_equal(a["logits"][r], b["logits"][r])
    for r in (2, 5):
        assert np.abs(a["logits"][r] - b["logits"][r]).max() > 1e-3


def test_identity_block_gives_closed_form_logits():
    cfg = CFG
    W = _weights(cfg, zero=("wo", "w_down"))
    P = 9
    tree = _tree(P)
    out = O.target_tree_layer(W, _prefix(cfg, P, 40), tree, P)
    e = W.embed[tree["token"]].astype(np.float64)
    nf = e / np.sqrt(np.mean(e * e, axis=1, keepdims=True) + cfg.eps) * W.g_final
    want = nf @ W.w_lm.T
    np.testing.assert_allclose(out["a"], e, rtol=0, atol=0)
    np.testing.assert_allclose(out["logits"], want, rtol=1e-5, atol=1e-5)


def test_cache_rows_follow_flattened_rows():
    """Row r's K/V lands in cache row len_in + r; the prefix is untouched."""
    cfg = CFG
    W = _weights(cfg)
    P = 9
    tree = _tree(P)
    kv = _prefix(cfg, P, 40)
    before = kv.k[:, :P].copy()
    out = O.target_tree_layer(W, kv, tree, P)
    np.testing.assert_array_equal(kv.k[:, :P], before)
    for r in range(tree["n_nodes"] + 1):
        np.testing.assert_array_equal(kv.k[:, P + r], out["k"][r])
        np.testing.assert_array_equal(kv.v[:, P + r], out["v"][r])
