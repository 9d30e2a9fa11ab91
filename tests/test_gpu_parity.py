"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on
the same seeded inputs.  Integer outputs (top-k ids, tree topology, masks,
slots, accepted lengths, tokens) must match exactly; floats within 2e-2
abs/rel in bf16 and 1e-4 in fp32."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from harness import (MARGIN, SEED, Model, as_np, assert_tree_equal, cap_for,
                     gpu_tree_round, make_seq, stored, target_logits, tdtype,
                     tol, tree_to_np, upload_batch)

pytestmark = pytest.mark.gpu

# a mid-size bf16 drafter: several tiles per GEMM, ragged vocab tile (8000 is
# not a multiple of 64), GQA 4, ragged contexts, batch 3
MID = dict(H=1024, n_q=8, n_kv=2, hd=128, F=2816, V=8000, ctx=(200, 700),
           D=4, K=6, N=20, B=3)

CASES = {
    "tiny": lambda: synth.config("tiny"),
    "mid": lambda: synth.config("8b_bs1", **MID),
    "mid_fp32": lambda: synth.config("tiny", H=512, n_q=8, n_kv=2, F=1376,
                                     V=2000, ctx=(90, 300), D=4, K=5, N=16,
                                     B=2),
    # batch 23 x 6 rows per sequence = 138 rows: the dense (MFMA-bound) GEMM
    # path, three 64-row blocks with a ragged last one, split K
    "mid_b23": lambda: synth.config("8b_bs1", **dict(MID, B=23, s_max=6)),
}

_models = {}


def model_for(name):
    if name not in _models:
        print(f"[setup] building model {name}", flush=True)
        _models[name] = Model(CASES[name]())
    return _models[name]


def _close(cfg, got, want, what=""):
    atol, rtol = tol(cfg)
    np.testing.assert_allclose(got, want, atol=atol, rtol=rtol, err_msg=what)


@pytest.mark.parametrize("name", ["tiny", "mid", "mid_fp32", "mid_b23"])
@pytest.mark.parametrize("rows", [1, 7, 64, 131])
def test_fuse_parity(name, rows):
    m = model_for(name)
    cfg = m.cfg
    d = m.drafter(max_batch=cfg.B)
    feats = synth.normal(synth.GenKey(1, "fuse-test", rows), (3, rows, cfg.H))
    low, mid, high = (stored(cfg, f) for f in feats)
    g = d.fuse(low.cuda(), mid.cuda(), high.cuda())
    torch.cuda.synchronize()
    want = O.fuse(m.oracle, as_np(low), as_np(mid), as_np(high))
    _close(cfg, as_np(g), want, "g")


@pytest.mark.parametrize("name", ["tiny", "mid", "mid_fp32", "mid_b23"])
def test_draft_step_parity(name):
    """One draft step over causal seed rows of several sequences."""
    m = model_for(name)
    cfg = m.cfg
    B, rps = cfg.B, cfg.s_max
    d = m.drafter()
    ctxs = synth.contexts(cfg)
    cap = cap_for(cfg, int(ctxs.max()))
    rng = np.random.default_rng(5)
    src = torch.from_numpy((rng.standard_normal((B * rps, cfg.H)) * 2.0).astype(np.float32))
    toks = rng.integers(0, cfg.V, size=B * rps).astype(np.int32)
    if B > 1:
        toks[rps * (B - 1) + 1] = -1        # a padding row
    K_all = torch.zeros(B, cfg.n_kv, cap, cfg.hd, dtype=tdtype(cfg))
    V_all = torch.zeros_like(K_all)
    for b in range(B):
        kk, vv = synth.prefix_kv(cfg, b, int(ctxs[b]))
        K_all[b, :, :ctxs[b]] = stored(cfg, kk)
        V_all[b, :, :ctxs[b]] = stored(cfg, vv)
    pos = np.array([ctxs[r // rps] + r % rps for r in range(B * rps)], np.int32)
    plen = pos + 1
    from eagle_draft_tree_amd import KVCache
    kv = KVCache.from_rows(K_all.cuda(), V_all.cuda(),
                           torch.tensor(ctxs, dtype=torch.int32).cuda())
    zero_mask = torch.zeros(B * rps, dtype=torch.int64, device="cuda")
    a, tid, tval, lse = d.draft_step(
        B, rps, src.cuda(), torch.from_numpy(toks).cuda(),
        torch.from_numpy(pos).cuda(), torch.from_numpy(pos).cuda(),
        torch.from_numpy(plen).cuda(),
        torch.tensor(ctxs + rps, dtype=torch.int32).cuda(), zero_mask, kv)
    torch.cuda.synchronize()
    for b in range(B):
        okv = O.DraftKV(as_np(K_all[b]), as_np(V_all[b]))
        rows = [r for r in range(b * rps, (b + 1) * rps) if toks[r] >= 0]
        out = O.layer(m.oracle, okv, as_np(src[rows]), toks[rows], pos=pos[rows],
                      dest=pos[rows], visible=[np.arange(plen[r]) for r in rows])
        _close(cfg, as_np(a[rows]), out["a"], f"a seq {b}")
        # activations are fp32 on both sides: the draft state tracks the
        # oracle to float precision (a systematic error shows up far above)
        rel = np.abs(as_np(a[rows]) - out["a"]).max() / np.abs(out["a"]).max()
        assert rel < 1e-4, f"draft state off by {rel:.2e} relative"
        for i, r in enumerate(rows):
            lg = out["logits"][i]
            srt = np.sort(lg.astype(np.float64))[::-1]
            if srt[cfg.K - 1] - srt[cfg.K] >= MARGIN:
                assert list(tid[r].cpu().numpy()) == list(O.topk_desc(lg, cfg.K))
            np.testing.assert_allclose(
                tval[r].cpu().numpy(), lg[tid[r].cpu().numpy()].astype(np.float64),
                atol=1e-4, rtol=1e-4, err_msg="topk logits")
            assert abs(float(lse[r]) - float(O.lse32(lg))) < 1e-4
        got_k = as_np(kv.k[b].cpu())
        for r in rows:
            _close(cfg, got_k[:, pos[r]], okv.k[:, pos[r]], "k row")
            _close(cfg, as_np(kv.v_rows()[b].cpu())[:, pos[r]], okv.v[:, pos[r]], "v row")
        # prefix untouched
        assert torch.equal(kv.k[b, :, :ctxs[b]].cpu(), K_all[b, :, :ctxs[b]])


def _run_tree_case(name, check_kv=True):
    m = model_for(name)
    cfg = m.cfg
    ctxs = synth.contexts(cfg)
    cap = cap_for(cfg, int(ctxs.max()))
    seqs = [make_seq(m, b, int(ctxs[b]), cap) for b in range(cfg.B)]
    d = m.drafter()
    kv, feats, tok, seed_len = upload_batch(m, seqs, cap)
    g, tree, len_out = gpu_tree_round(d, m, seqs, kv, feats, tok, seed_len)
    for b, s in enumerate(seqs):
        print(f"[tree] {name} seq {b} ctx {s.ctx} attempt {s.attempt} "
              f"margin {s.margin:.2e}", flush=True)
        _close(cfg, as_np(g[b]), s.g[0], "g")
        assert int(len_out[b]) == s.ctx + 1
        assert_tree_equal(cfg, tree_to_np(tree, b), s.tree)
        if check_kv:
            lo = s.ctx + 1
            hi = lo + (cfg.D - 1) * cfg.K
            _close(cfg, as_np(kv.k[b, :, s.ctx:hi].cpu()), s.kv.k[:, s.ctx:hi], "k")
            _close(cfg, as_np(kv.v_rows()[b, :, s.ctx:hi].cpu()), s.kv.v[:, s.ctx:hi], "v")
    return m, seqs, d, kv, tree


@pytest.mark.parametrize("name", ["tiny", "mid", "mid_fp32", "mid_b23"])
def test_draft_tree_parity(name):
    _run_tree_case(name)


@pytest.mark.parametrize("name", ["tiny", "mid", "mid_b23"])
def test_verify_greedy_parity_with_commit(name):
    m, seqs, d, kv, tree = _run_tree_case(name, check_kv=False)
    cfg = m.cfg
    B = len(seqs)
    tl = np.stack([target_logits(m, s) for s in seqs])
    # make some rows agree with the drafter so paths get accepted
    for b, s in enumerate(seqs):
        for r in range(0, s.tree["n_nodes"] + 1, 2):
            kids = range(s.tree["first_child"][r],
                         s.tree["first_child"][r] + s.tree["n_child"][r])
            if s.tree["n_child"][r] > 0:
                tl[b, r, s.tree["token"][list(kids)[-1]]] += 100.0
    res = d.verify(tree, torch.from_numpy(tl).cuda(), 0.0, kv=kv)
    torch.cuda.synchronize()
    for b, s in enumerate(seqs):
        want = O.verify(cfg, s.tree, tl[b], 0.0)
        assert int(res["accept_len"][b]) == want["accept_len"]
        assert np.array_equal(res["accepted_rows"][b].cpu().numpy(),
                              want["accepted_rows"])
        assert np.array_equal(res["tokens"][b].cpu().numpy(), want["tokens"])
        okv = s.kv.copy()
        new_len, srows, stoks = O.commit(cfg, s.tree, want, okv)
        assert int(res["kv_len"][b]) == new_len
        n = int(res["seed_len"][b])
        assert n == len(srows)
        assert list(res["seed_rows"][b, :n].cpu().numpy()) == srows
        assert list(res["seed_tokens"][b, :n].cpu().numpy()) == stoks
        _close(cfg, as_np(kv.k[b, :, :new_len].cpu()), okv.k[:, :new_len], "k commit")
        _close(cfg, as_np(kv.v_rows()[b, :, :new_len].cpu()), okv.v[:, :new_len], "v commit")


@pytest.mark.parametrize("name,T", [("tiny", 1.0), ("tiny", 0.6), ("mid", 1.0)])
def test_verify_sampling_parity(name, T):
    """Seeded rejection sampling: the library's Philox draws of (seed, round,
    sequence) against the oracle's own Philox, over several rounds."""
    m, seqs, d, kv, tree = _run_tree_case(name, check_kv=False)
    cfg = m.cfg
    hits = 0
    for rnd in range(6):
        tl = []
        for s in seqs:
            for att in range(20):
                t = target_logits(m, s, rnd, att)
                # sharpen towards the drafter so children get accepted
                t = (t * np.float32(3.0)).astype(np.float32)
                w = O.verify(cfg, s.tree, t, T, seed=SEED, rnd=rnd, b=s.b)
                if w["margin"] >= 1e-6:
                    break
            tl.append(t)
        tl = np.stack(tl)
        res = d.verify(tree, torch.from_numpy(tl).cuda(), T, seed=SEED, round=rnd)
        torch.cuda.synchronize()
        for b, s in enumerate(seqs):
            want = O.verify(cfg, s.tree, tl[b], T, seed=SEED, rnd=rnd, b=b)
            hits += want["accept_len"]
            assert int(res["accept_len"][b]) == want["accept_len"]
            assert np.array_equal(res["tokens"][b].cpu().numpy(), want["tokens"])
            assert np.array_equal(res["accepted_rows"][b].cpu().numpy(),
                                  want["accepted_rows"])
    print(f"[verify] {name} T={T} accepted tokens over rounds: {hits}")


def test_verify_explicit_uniforms_hook():
    """The replay entry point with caller-drawn uniforms follows the same
    Algorithm 1 walk as the oracle fed the same numbers."""
    m, seqs, d, kv, tree = _run_tree_case("tiny", check_kv=False)
    cfg = m.cfg
    for rnd in range(4):
        for att in range(20):
            t = (target_logits(m, seqs[0], rnd, att) * np.float32(3.0)).astype(np.float32)
            u = synth.uniforms(cfg, 0, rnd, cfg.N + 1, att)
            w = O.verify(cfg, seqs[0].tree, t, 1.0, u)
            if w["margin"] >= 1e-6:
                break
        res = d.verify(tree, torch.from_numpy(t[None]).cuda(), 1.0,
                       uniforms=torch.from_numpy(u[None]).cuda())
        torch.cuda.synchronize()
        assert int(res["accept_len"][0]) == w["accept_len"]
        assert np.array_equal(res["tokens"][0].cpu().numpy(), w["tokens"])


def test_device_status_capacity():
    """A cache too small for the scratch rows is reported, nothing written
    out of bounds, and the sequence yields an invalid tree."""
    m = model_for("tiny")
    cfg = m.cfg
    d = m.drafter()
    from eagle_draft_tree_amd import KVCache
    cap = cfg.ctx[0] + 8      # needs ctx + 1 + (D-1)K rows
    assert cap < cfg.ctx[0] + 1 + (cfg.D - 1) * cfg.K
    k = torch.zeros(1, cfg.n_kv, cap, cfg.hd, dtype=tdtype(cfg), device="cuda")
    kv = KVCache.from_rows(k, torch.zeros_like(k),
                 torch.tensor([cfg.ctx[0]], dtype=torch.int32, device="cuda"))
    src = torch.zeros(1, cfg.s_max, cfg.H, dtype=tdtype(cfg), device="cuda")
    tok = torch.tensor([[5, -1]], dtype=torch.int32, device="cuda")
    tree, len_out = d.draft_tree(src, tok, torch.ones(1, dtype=torch.int32,
                                                       device="cuda"), kv)
    st = d.device_status()
    assert st & (1 << 4)
    assert int(tree["n_nodes"][0]) == -1
    assert d.device_status() == 0
