"""eagle_verify_tree_noalloc (no context, no workspace; static scratch)
against eagle_verify_tree on the same trees and target logits, through the
C ABI: two calls in a row, the second on a smaller batch."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from harness import (SEED, Model, cap_for, gpu_tree_round, make_seq,
                     target_logits, upload_batch)

pytestmark = pytest.mark.gpu

MID = dict(H=1024, n_q=8, n_kv=2, hd=128, F=2816, V=8000, ctx=(200, 700),
           D=4, K=6, N=20, B=3)


def _noalloc(d, B, tree, logits, T, rnd, kv_k, kv_v, cap):
    from eagle_draft_tree_amd import _lib
    i32 = dict(dtype=torch.int32, device="cuda")
    D, S = d.shape.depth, d.shape.max_seed
    out = {"accept_len": torch.full((B,), -7, **i32),
           "accepted_rows": torch.full((B, D), -7, **i32),
           "tokens": torch.full((B, D + 1), -7, **i32),
           "seed_rows": torch.full((B, S), -7, **i32),
           "seed_tokens": torch.full((B, S), -7, **i32),
           "seed_len": torch.full((B,), -7, **i32),
           "kv_len": torch.full((B,), -7, **i32)}
    cfg = d.shape.c_config()
    ct = d._c_tree({k: v[:B] for k, v in tree.items()})
    ckv = _lib.KV(kv_k.data_ptr(), kv_v.data_ptr(), cap, None,
                  out["kv_len"].data_ptr())
    st = _lib.lib().eagle_verify_tree_noalloc(
        ctypes.byref(cfg), B, ctypes.byref(ct), logits.data_ptr(), float(T),
        SEED, rnd, 0, ctypes.byref(ckv),
        *[out[k].data_ptr() for k in ("accept_len", "accepted_rows", "tokens",
                                      "seed_rows", "seed_tokens", "seed_len")],
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    return out


def test_noalloc_verify_matches_context_entry_point():
    from eagle_draft_tree_amd import KVCache
    cfg = synth.config("8b_bs1", **MID)
    m = Model(cfg)
    ctxs = synth.contexts(cfg)
    cap = cap_for(cfg, int(ctxs.max()))
    seqs = [make_seq(m, b, int(ctxs[b]), cap) for b in range(cfg.B)]
    d = m.drafter()
    kv, feats, tok, seed_len = upload_batch(m, seqs, cap)
    _, tree, _ = gpu_tree_round(d, m, seqs, kv, feats, tok, seed_len)
    tl = np.stack([target_logits(m, s) for s in seqs])
    for b, s in enumerate(seqs):          # lean towards the best child
        t = s.tree
        for v in range(t["n_nodes"] + 1):
            if t["n_child"][v]:
                kids = range(t["first_child"][v], t["first_child"][v] + t["n_child"][v])
                tl[b, v, t["token"][max(kids, key=lambda c: t["score"][c])]] += 8.0
    tl = torch.from_numpy(tl).cuda()
    for call, (B, T, rnd) in enumerate([(3, 1.0, 5), (2, 0.0, 6)]):
        print(f"[noalloc] call {call}: batch {B}, T={T}", flush=True)
        k1, v1 = kv.k[:B].clone(), kv.v[:B].clone()
        k2, v2 = kv.k[:B].clone(), kv.v[:B].clone()
        kv1 = KVCache(k1, v1, kv.length[:B].clone())
        kv_len1 = torch.empty(B, dtype=torch.int32, device="cuda")
        want = d.verify({k: v[:B] for k, v in tree.items()}, tl[:B].contiguous(),
                        T, seed=SEED, round=rnd, kv=kv1, kv_len_out=kv_len1)
        got = _noalloc(d, B, tree, tl[:B].contiguous(), T, rnd, k2, v2, cap)
        torch.cuda.synchronize()
        for k in ("accept_len", "accepted_rows", "tokens", "seed_rows",
                  "seed_tokens", "seed_len", "kv_len"):
            assert torch.equal(got[k], want[k]), (call, k, got[k], want[k])
        assert torch.equal(k2, k1) and torch.equal(v2, v1)
        print(f"[noalloc] call {call}: accepted {want['accept_len'].tolist()}",
              flush=True)
