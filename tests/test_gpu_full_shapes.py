"""GPU parity at the workloads' full shapes, through the C ABI against the
CPU oracle on the same seeded inputs:

  * 8B drafter, batch 1, context 2048, depth 6 / top-k 10 / 60 nodes, greedy
    verification, two chained rounds;
  * 8B drafter, batch 64, contexts drawn from U{512..4096}, the same tree,
    seeded rejection sampling at T = 1, every sequence checked;
  * 70B drafter (H 8192, 64 q / 8 kv heads, FFN 28672), context 4096,
    batch 1 greedy, and batch 16 with three sequences checked at T = 1;
  * 8B drafter, batch 8, context 16384, depth 8 / top-k 8 / 80 nodes (two
    mask words per row), T = 0.6, four chained verify -> commit -> fuse ->
    draft rounds.

Every tree array is bit-exact, every accepted length and token equal, and
draft states, scores and committed K/V rows within the bf16 tolerance.  The
oracle runs in float64 on the host and dominates the run time."""
import copy
import gc

import numpy as np
import pytest
import torch

import harness
import synth
from harness import SEED, Model, first_round, run_chain, say, tree_to_np, assert_tree_equal

pytestmark = pytest.mark.gpu

_held = {}


@pytest.fixture(autouse=True, scope="module")
def _progress_to_terminal(pytestconfig):
    """These tests run for minutes, mostly in the oracle: their progress
    lines bypass pytest's output capture."""
    harness._capman = pytestconfig.pluginmanager.getplugin("capturemanager")
    yield
    harness._capman = None


def _dims(cfg):
    return (cfg.H, cfg.n_q, cfg.n_kv, cfg.hd, cfg.F, cfg.V, cfg.dtype)


def _model(name):
    """One set of weights at a time (the 70B drafter's float64 oracle copy
    is 14 GB); workloads with the same drafter dimensions share it, each
    seeing its own batch, context and tree settings."""
    cfg = synth.config(name)
    base = _held.get("base")
    if base is None or _dims(base.cfg) != _dims(cfg):
        _held.clear()
        gc.collect()
        torch.cuda.empty_cache()
        say(f"[setup] weights for {name}")
        base = _held["base"] = Model(cfg)
    m = copy.copy(base)
    m.cfg = cfg
    m.oracle = copy.copy(base.oracle)
    m.oracle.cfg = cfg
    return m


def test_8b_bs1_two_rounds_greedy():
    m = _model("8b_bs1")
    seqs, d, kv, tree = first_round(m, 1, cap_rounds=3)
    say("[8b bs1] first tree equal")
    run_chain(m, seqs, d, kv, tree, rounds=2, T=0.0, mode="keep")


def test_8b_bs64_sampling_every_sequence():
    m = _model("8b_bs64")
    seqs, d, kv, tree = first_round(m, 64)
    say("[8b bs64] 64 trees equal")
    run_chain(m, seqs, d, kv, tree, rounds=1, T=1.0, mode="keep")


def test_long_context_bs8_four_chained_rounds():
    m = _model("long_bs8")
    seqs, d, kv, tree = first_round(m, 8, cap_rounds=5)
    for b in range(8):
        assert_tree_equal(m.cfg, tree_to_np(tree, b), seqs[b].tree)
    say("[long bs8] 8 trees equal (two mask words per row)")
    run_chain(m, seqs, d, kv, tree, rounds=4, T=0.6, mode="keep")


def test_70b_bs1_greedy():
    m = _model("70b_bs1")
    seqs, d, kv, tree = first_round(m, 1, cap_rounds=2)
    say("[70b bs1] tree equal")
    run_chain(m, seqs, d, kv, tree, rounds=1, T=0.0, mode="keep")


def test_70b_bs16_subset_sampling():
    """All 16 trees are drafted in one batch; sequences 0, 7 and 15 are
    compared with the oracle (tree, sampled verification, commit)."""
    m = _model("70b_bs1")
    check = (0, 7, 15)
    seqs, d, kv, tree = first_round(m, 16, check=check)
    say("[70b bs16] checked trees equal")
    from harness import ChainSeq, as_np, close
    from eagle_draft_tree_amd import COMMIT_KEEP
    cfg = m.cfg
    tl = np.zeros((16, cfg.N + 1, cfg.V), dtype=np.float32)
    chains = {}
    for b in check:
        c = ChainSeq(m, seqs[b], 1.0, "keep", boost=0.0 if b % 2 else 8.0)
        tl[b], want = c.verify(0)
        chains[b] = (c, want)
    kv_len = torch.empty(16, dtype=torch.int32, device="cuda")
    res = d.verify(tree, torch.from_numpy(tl).cuda(), 1.0, seed=SEED, round=0,
                   kv=kv, kv_len_out=kv_len, commit_mode=COMMIT_KEEP)
    torch.cuda.synchronize()
    for b, (c, want) in chains.items():
        assert int(res["accept_len"][b]) == want["accept_len"], b
        assert np.array_equal(res["tokens"][b].cpu().numpy(), want["tokens"])
        assert int(kv_len[b]) == c.new_len
        n = int(res["seed_len"][b])
        assert list(res["seed_rows"][b, :n].cpu().numpy()) == c.seed_rows
        close(cfg, as_np(kv.k[b, :, :c.new_len].cpu()), c.kv.k[:, :c.new_len], "k")
        close(cfg, as_np(kv.v_rows()[b, :, :c.new_len].cpu()), c.kv.v[:, :c.new_len], "v")
    # the unchecked sequences verified without error
    assert (res["accept_len"] >= 0).all()
