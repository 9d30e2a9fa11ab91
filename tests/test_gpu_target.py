"""GPU parity of the target tree layer: the target's one-pass forward over
the flattened draft trees (tree attention under the trees' ancestor masks),
through the C ABI against the oracle's target_tree_layer on the same seeded
inputs, and its logits fed to the verification.  The trees come from the
library's own drafting (checked against the oracle first); the target is a
separate one-layer model of the drafter's shape with its own weights."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from harness import SEED, Model, as_np, first_round, stored, tol, tree_to_np

pytestmark = pytest.mark.gpu

MID = dict(H=1024, n_q=8, n_kv=2, hd=128, F=2816, V=8000, ctx=(200, 700),
           D=4, K=6, N=20)
CASES = {"mid": dict(MID, B=3), "mid_b23": dict(MID, B=23)}
_models = {}


def _models_for(name):
    if name not in _models:
        cfg = synth.config("8b_bs1", **CASES[name])
        print(f"[setup] draft and target models {name}", flush=True)
        _models[name] = (Model(cfg, seed=0), Model(cfg, seed=1))
    return _models[name]


def _close(cfg, got, want, what):
    atol, rtol = tol(cfg)
    np.testing.assert_allclose(got, want, atol=atol, rtol=rtol, err_msg=what)


@pytest.mark.parametrize("name", ["mid", "mid_b23"])
def test_target_layer_matches_oracle_and_feeds_verify(name):
    from eagle_draft_tree_amd import KVCache
    md, mt = _models_for(name)
    cfg = md.cfg
    B = cfg.B
    seqs, d, _, tree = first_round(md, B)
    print(f"[target] {name}: {B} trees drafted and equal", flush=True)
    # the target's committed prefix ends right before the root's position
    len_in = np.array([int(tree["position"][b, 0]) for b in range(B)], np.int32)
    cap = int(len_in.max() + cfg.N + 1 + 7) // 8 * 8
    k = torch.zeros(B, cfg.n_kv, cap, cfg.hd, dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    for b in range(B):
        kk, vv = synth.prefix_kv(cfg, 100 + b, int(len_in[b]))
        k[b, :, :len_in[b]] = stored(cfg, kk)
        v[b, :, :len_in[b]] = stored(cfg, vv)
    kv_cpu = (k.clone(), v.clone())
    kv = KVCache.from_rows(k.cuda(), v.cuda(), torch.from_numpy(len_in).cuda())
    dt = mt.drafter(max_batch=B)
    hidden = torch.empty(B, cfg.N + 1, cfg.H, dtype=torch.float32, device="cuda")
    logits, _ = dt.target_tree_layer(tree, kv, hidden=hidden)
    torch.cuda.synchronize()
    assert dt.device_status() == 0
    got_l = logits.cpu().numpy()
    got_h = hidden.cpu().numpy()
    for b in range(B):
        t = tree_to_np(tree, b)
        n = int(t["n_nodes"])
        okv = O.DraftKV(as_np(kv_cpu[0][b]), as_np(kv_cpu[1][b]))
        want = O.target_tree_layer(mt.oracle, okv, t, int(len_in[b]))
        _close(cfg, got_h[b, :n + 1], want["a"], f"hidden seq {b}")
        # fp32 activations on both sides; q, k and v are rounded to bf16 at
        # their storage points, where a last-bit difference before rounding
        # can flip one bf16 step: that leaves ~1e-4 in the outputs, while a
        # wrong mask, position or weight shows up at 1e-2 and above
        rel = np.abs(got_h[b, :n + 1] - want["a"]).max() / np.abs(want["a"]).max()
        assert rel < 1e-3, f"hidden off by {rel:.2e} relative"
        _close(cfg, got_l[b, :n + 1], want["logits"], f"logits seq {b}")
        assert not got_l[b, n + 1:].any(), "padding rows carry zero logits"
        # the tree rows' K/V landed at len_in + r; the prefix is untouched
        lo, hi = int(len_in[b]), int(len_in[b]) + n + 1
        _close(cfg, as_np(kv.k[b, :, lo:hi].cpu()), okv.k[:, lo:hi], "k rows")
        _close(cfg, as_np(kv.v_rows()[b, :, lo:hi].cpu()), okv.v[:, lo:hi], "v rows")
        assert torch.equal(kv.k[b, :, :lo].cpu(), kv_cpu[0][b, :, :lo])
    # the layer's logits drive the verification; both sides read the same
    # (library) logits, so accepted paths and tokens must agree exactly
    for T in (0.0, 1.0):
        res = d.verify(tree, logits, T, seed=SEED, round=3)
        torch.cuda.synchronize()
        for b, s in enumerate(seqs):
            w = O.verify(cfg, s.tree, got_l[b], T, seed=SEED, rnd=3, b=b)
            if T > 0 and w["margin"] < 1e-6:
                continue
            assert int(res["accept_len"][b]) == w["accept_len"], (T, b)
            assert np.array_equal(res["tokens"][b].cpu().numpy(), w["tokens"]), (T, b)
    print(f"[target] {name}: layer, cache rows and verification equal", flush=True)
