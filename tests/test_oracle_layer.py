"""Pins of the oracle's draft layer, its selection margins and its random
numbers against closed forms, hand-worked cases and library routines (no GPU).

The draft layer is a LLaMA-style pre-norm block ("EAGLE-3 ... Training-Time
Test" summary page, 3.4 "The Draft Model Architecture in Detail"; section 6,
Limitation 6: pre-normalisation, SwiGLU, rotary embeddings, GQA).  Each pin
below picks weights for which that block has a short closed form, so that a
mistake in one place (the join order, where the residual is added, which
norm the MLP reads, gate/up roles, the GQA head map, the visibility set)
changes the result."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth

PIN = synth.Config("pin", H=16, n_q=4, n_kv=2, hd=4, F=16, V=12,
                   dtype="fp32", theta=10000.0, B=1, ctx=(5, 5), D=2, K=2,
                   N=3, T=0.0)


def _weights(cfg, rng, **fixed):
    H, F, V = cfg.H, cfg.F, cfg.V
    qd, kd = cfg.n_q * cfg.hd, cfg.n_kv * cfg.hd
    shapes = {"w_fuse": (H, 3 * H), "w_in": (H, 2 * H), "embed": (V, H),
              "wq": (qd, H), "wk": (kd, H), "wv": (kd, H), "wo": (H, qd),
              "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F),
              "w_lm": (V, H)}
    arr = {n: (rng.standard_normal(s) * 0.3).astype(np.float32)
           for n, s in shapes.items()}
    for g in ("g_attn", "g_mlp", "g_final"):
        arr[g] = (1.0 + 0.2 * rng.standard_normal(H)).astype(np.float32)
    arr.update({k: np.asarray(v, dtype=np.float32) for k, v in fixed.items()})
    return O.Weights(cfg, arr)


def _kv(cfg, rng, cap=12):
    k = rng.standard_normal((cfg.n_kv, cap, cfg.hd)).astype(np.float32)
    v = rng.standard_normal((cfg.n_kv, cap, cfg.hd)).astype(np.float32)
    return O.DraftKV(k, v)


def _one_row(W, kv, src, tok, P=5):
    """A seed-like row at position P seeing cache rows [0, P]."""
    return O.layer(W, kv, src[None], [tok], pos=[P], dest=[P],
                   visible=[np.arange(P + 1)])


def _rms(x, eps):
    return np.sqrt(np.mean(np.asarray(x, np.float64) ** 2) + eps)


def test_join_order_and_residual_placement():
    """W_I = [I, 0] gives x = src; with Wo = Wd = 0 both residual branches
    add nothing, so the draft state equals the source row.  W_I = [0, I]
    gives the token's embedding instead."""
    rng = np.random.default_rng(10)
    H = PIN.H
    eye, zero = np.eye(H), np.zeros((H, H))
    src = rng.standard_normal(H) * 3.0
    W = _weights(PIN, rng, w_in=np.hstack([eye, zero]), wo=np.zeros((H, 16)),
                 w_down=np.zeros((H, PIN.F)))
    out = _one_row(W, _kv(PIN, rng), O.store(src, "fp32"), 7)
    assert np.array_equal(out["x"][0], O.store(src, "fp32"))
    assert np.array_equal(out["a"][0], O.store(src, "fp32"))
    W2 = _weights(PIN, rng, w_in=np.hstack([zero, eye]), wo=np.zeros((H, 16)),
                  w_down=np.zeros((H, PIN.F)))
    out2 = _one_row(W2, _kv(PIN, rng), src, 7)
    assert np.array_equal(out2["a"][0], W2.embed[7])


def test_mlp_reads_its_own_norm_and_gate_up_roles():
    """x = src; Wq = Wk = Wv = 0 with every prefix V row equal to e_0 makes
    each head's attention output (P/(P+1)) e_0, and Wo = I adds it to x, so
    h = x + o differs from x.  With Wg = c*I, Wu = I, Wd = I:
    a = h + silu(c * n2) * n2, n2 = h / rms(h) * g_mlp.  The attention norm
    gets a very different gain, so an MLP that read n1 (or x) would fail, and
    c != 1 tells gate from up."""
    rng = np.random.default_rng(11)
    H, c, P = PIN.H, 2.5, 5
    eye = np.eye(H)
    src = O.store(rng.standard_normal(H) * 1.7, "fp32")
    g_mlp = O.store(1.0 + 0.3 * rng.standard_normal(H), "fp32")
    kv = _kv(PIN, rng)
    kv.v[:] = 0.0
    kv.v[:, :P, 0] = 1.0
    W = _weights(PIN, rng, w_in=np.hstack([eye, np.zeros((H, H))]),
                 wq=np.zeros((16, H)), wk=np.zeros((8, H)), wv=np.zeros((8, H)),
                 wo=eye, w_gate=c * eye, w_up=eye, w_down=eye,
                 g_mlp=g_mlp, g_attn=np.full(H, 3.0))
    out = _one_row(W, kv, src, 3, P=P)
    o = np.zeros((PIN.n_q, PIN.hd))
    o[:, 0] = P / (P + 1)
    h = src + o.reshape(-1)
    np.testing.assert_allclose(out["h"][0], h, rtol=1e-6, atol=1e-7)
    n2 = h / _rms(h, PIN.eps) * g_mlp
    want = h + (c * n2) / (1.0 + np.exp(-c * n2)) * n2
    np.testing.assert_allclose(out["a"][0], want, rtol=2e-6, atol=1e-6)
    swapped = h + n2 / (1.0 + np.exp(-n2)) * (c * n2)
    assert np.abs(out["a"][0] - swapped).max() > 1e-2


def test_attention_uniform_weights_gqa_map_and_visibility():
    """Wq = Wk = 0 makes every score 0, so each head's output is the plain
    mean of the V rows it sees.  Wv = 0 makes the row's own V zero.  kv head
    0 holds e_0 in every prefix row, kv head 1 holds 2*e_1: with 4 query heads
    over 2 kv heads, heads 0 and 1 must read kv head 0 and heads 2 and 3 kv
    head 1.  A huge V in a row outside the visible set must not leak in."""
    rng = np.random.default_rng(12)
    H, P = PIN.H, 5
    kv = _kv(PIN, rng)
    kv.v[:] = 0.0
    kv.v[0, :P, 0] = 1.0
    kv.v[1, :P, 1] = 2.0
    kv.v[:, P + 3] = 1e6                      # not visible
    qd = PIN.n_q * PIN.hd
    W = _weights(PIN, rng, wq=np.zeros((qd, H)), wk=np.zeros((8, H)),
                 wv=np.zeros((8, H)), wo=np.eye(H), w_down=np.zeros((H, PIN.F)),
                 w_in=np.hstack([np.eye(H), np.zeros((H, H))]))
    src = O.store(rng.standard_normal(H), "fp32")
    out = _one_row(W, kv, src, 2, P=P)
    f = P / (P + 1)                            # P ones out of P+1 rows
    want = np.zeros((PIN.n_q, PIN.hd))
    want[0, 0] = want[1, 0] = f
    want[2, 1] = want[3, 1] = 2 * f
    np.testing.assert_allclose(out["o"][0], want, rtol=1e-7, atol=1e-12)
    # Wo = I: the attention output lands on the residual unchanged
    np.testing.assert_allclose(out["a"][0], src + want.reshape(-1),
                               rtol=1e-6, atol=1e-7)


def test_attention_matches_torch_sdpa_with_gqa():
    """Random weights, three rows with tree-shaped visibility: the oracle's
    per-head attention equals torch's scaled_dot_product_attention with an
    explicit boolean mask and enable_gqa (float64, CPU)."""
    rng = np.random.default_rng(13)
    P, cap = 5, 12
    W = _weights(PIN, rng)
    kv = _kv(PIN, rng, cap)
    src = rng.standard_normal((3, PIN.H))
    dest = np.array([P, P + 1, P + 2])
    vis = [np.arange(P + 1), np.r_[np.arange(P), P + 1],
           np.r_[np.arange(P), P, P + 2]]
    out = O.layer(W, kv, src, [1, 4, 9], pos=[P, P + 1, P + 1], dest=dest,
                  visible=vis)
    mask = np.zeros((3, cap), dtype=bool)
    for r, v in enumerate(vis):
        mask[r, v] = True
    q = torch.from_numpy(out["q"]).permute(1, 0, 2)[None]           # [1,nq,R,hd]
    k = torch.from_numpy(kv.k)[None]                                 # [1,nkv,cap,hd]
    v = torch.from_numpy(kv.v)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=torch.from_numpy(mask)[None, None], enable_gqa=True)
    np.testing.assert_allclose(out["o"], ref[0].permute(1, 0, 2).numpy(),
                               rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------------------
# decision_margin on hand-built trees
# ---------------------------------------------------------------------------
def _node(nid, depth, score, parent, logits=None):
    n = {"id": nid, "depth": depth, "score": np.float32(score),
         "parent": parent}
    if logits is not None:
        n["logits"] = np.asarray(logits, dtype=np.float32)
    return n


def _hand_tree(final_third=-1.2, n1_gap=0.5):
    """K=2, D=2, N=3.  Root's logits have a 0.05 gap at the top-2 cut; n0's
    a 0.03 gap; n1's gap is `n1_gap`.  Values: n0 -0.3, n1 `final_third`
    (the 4th best overall), n0's children -0.7 / -1.0, n1's -1.5 / -2.0."""
    root = {"id": -1, "depth": 0, "score": np.float32(0),
            "logits": np.float32([2.0, 1.0, 0.95, -5.0])}
    n0 = _node(0, 1, -0.3, root, [3.0, 2.0, 1.97, -4.0])
    n1 = _node(1, 1, final_third, root, [1.0, 0.9, 0.9 - n1_gap, -4.0])
    kids = [_node(2, 2, -0.7, n0), _node(3, 2, -1.0, n0),
            _node(4, 2, -1.5, n1), _node(5, 2, -2.0, n1)]
    return {"nodes": [n0, n1] + kids}


def test_decision_margin_hand_worked():
    cfg = PIN.replace(K=2, D=2, N=3)
    # cuts that decide this tree: final top-3 (-1.0 vs -1.2 -> 0.2), the
    # root's top-2 (0.05, its 2nd child is near the final cut), n0's top-2
    # (0.03, its 2nd child is the last one selected)
    assert O.decision_margin(cfg, _hand_tree()) == pytest.approx(0.03, abs=1e-6)
    # n1's children lie far below every cut: its own top-2 gap does not count
    assert O.decision_margin(cfg, _hand_tree(n1_gap=1e-6)) == pytest.approx(
        0.03, abs=1e-6)
    # a near-tie at the final cut is caught
    assert O.decision_margin(cfg, _hand_tree(final_third=-1.0005)) == \
        pytest.approx(0.0005, abs=1e-6)


def test_decision_margin_expansion_cut():
    """D=3: the depth-2 layer (4 nodes) is cut to K=2 for expansion; the gap
    between its 2nd and 3rd values is a deciding margin."""
    cfg = PIN.replace(K=2, D=3, N=10)
    t = _hand_tree()
    t["nodes"][3]["score"] = np.float32(-1.0)
    t["nodes"][4]["score"] = np.float32(-1.0004)     # 3rd of depth 2
    assert O.decision_margin(cfg, t) == pytest.approx(0.0004, abs=1e-6)


def test_root_only_tree_has_no_margin():
    assert O.decision_margin(PIN, {"nodes": []}) == float("inf")


# ---------------------------------------------------------------------------
# Philox4x64-10
# ---------------------------------------------------------------------------
def _numpy_block(counter, key):
    """numpy's Philox bit generator adds one to its 256-bit counter before
    encrypting, so start it one below the counter wanted."""
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    c = (c - 1) % (1 << 256)
    words = np.array([(c >> (64 * i)) & ((1 << 64) - 1) for i in range(4)],
                     dtype=np.uint64)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=words)
    return [int(x) for x in bg.random_raw(4)]


def test_philox_matches_numpy_bit_generator():
    rng = np.random.default_rng(14)
    m = (1 << 64) - 1
    cases = [([0, 0, 0, 0], [0, 0]), ([1, 0, 0, 0], [5, 0]),
             ([m, 7, 0, 3], [m, m]), ([0, 1, 2, 3], [12345, 1])]
    for _ in range(40):
        cases.append(([int(x) for x in rng.integers(0, 2 ** 63, 4)],
                      [int(x) for x in rng.integers(0, 2 ** 63, 2)]))
    for ctr, key in cases:
        assert O.philox4x64(ctr, key) == _numpy_block(ctr, key), (ctr, key)


def test_philox_vectorised_equals_scalar():
    rng = np.random.default_rng(15)
    c = rng.integers(0, 2 ** 63, size=(4, 300), dtype=np.uint64)
    c[0, :5] = np.uint64((1 << 64) - 1)
    got = O.philox4x64_np(c[0], c[1], c[2], c[3], 99, 2)
    for i in range(c.shape[1]):
        want = O.philox4x64([int(c[w, i]) for w in range(4)], [99, 2])
        assert [int(got[w][i]) for w in range(4)] == want


def test_uniforms_layout_and_law():
    u = O.uniform01(7, O.STREAM_VERIFY, 3, np.arange(4)[:, None, None],
                    np.arange(50)[None, :, None], np.arange(64)[None, None, :])
    assert u.dtype == np.float32 and u.shape == (4, 50, 64)
    assert u.min() >= 0.0 and u.max() < 1.0
    # each value is a multiple of 2^-24 taken from the top bits of word 0
    x0 = O.philox4x64([5, 2, 1, 3], [7, O.STREAM_VERIFY])[0]
    assert u[1, 2, 5] == np.float32((x0 >> 40) * 2.0 ** -24)
    # uniform law: mean, variance and a coarse histogram
    flat = u.astype(np.float64).ravel()
    assert abs(flat.mean() - 0.5) < 0.01
    assert abs(flat.var() - 1 / 12) < 0.005
    h = np.histogram(flat, bins=10, range=(0, 1))[0] / flat.size
    assert np.all(np.abs(h - 0.1) < 0.01)
    # another stream or round gives other numbers
    u2 = O.uniform01(7, O.STREAM_DRAFT, 3, 1, 2, 5)
    u3 = O.uniform01(7, O.STREAM_VERIFY, 4, 1, 2, 5)
    assert u2 != u[1, 2, 5] and u3 != u[1, 2, 5]


def test_verify_uniforms_columns():
    cfg = PIN.replace(K=3, N=4)
    U = O.verify_uniforms(cfg, 11, 2, 5)
    assert U.shape == (cfg.N + 1, cfg.K + 1)
    assert U[3, 1] == O.uniform01(11, O.STREAM_VERIFY, 2, 5, 3, 1)
    assert U[3, cfg.K] == O.uniform01(11, O.STREAM_VERIFY, 2, 5, 3,
                                       O.BONUS_DRAW)
