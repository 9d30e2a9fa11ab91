"""Pins of the oracle's numeric building blocks against library routines,
closed forms and invariants (no GPU)."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10.0,
        np.float32([0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9,
                    1.0 + 2 ** -9, -(1.0 + 2 ** -9), 3.0e38, 1e-40, -1e-42,
                    np.inf, -np.inf]),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = O.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(O.bf16_round(np.float32([np.nan]))[0])


def test_bf16_ties_to_even_closed_form():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa
    assert O.bf16_round(np.float32([1.0 + 2 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: goes to 1+2^-6 (even)
    assert O.bf16_round(np.float32([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
    assert O.store([1.0 + 2 ** -20], "fp32")[0] == np.float32(1.0 + 2 ** -20)


def test_rmsnorm_closed_form_and_invariance():
    x = np.array([[3.0, 4.0]])
    y = O.rmsnorm(x, np.ones(2), 0.0, "fp32")
    r = math.sqrt((9 + 16) / 2)
    assert np.allclose(y, [[3 / r, 4 / r]], rtol=1e-7)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64))
    g = 1 + 0.02 * rng.standard_normal(64)
    a = O.rmsnorm(x, g, 1e-5, "fp32")
    b = O.rmsnorm(7.5 * x, g, 1e-5 * 7.5 ** 2, "fp32")
    assert np.allclose(a, b, rtol=1e-6)
    u = O.rmsnorm(x, np.ones(64), 0.0, "fp32")
    assert np.allclose(np.sqrt(np.mean(u * u, axis=1)), 1.0, rtol=1e-6)


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(3)
    hd = 128
    q = rng.standard_normal(hd)
    k = rng.standard_normal(hd)
    assert np.array_equal(O.rope(q, 0, 500000.0), q)
    half = hd // 2
    for p in (1, 17, 4095, 16383):
        r = O.rope(q, p, 500000.0)
        n0 = q[:half] ** 2 + q[half:] ** 2
        n1 = r[:half] ** 2 + r[half:] ** 2
        assert np.allclose(n0, n1, rtol=1e-6)
    # q.k after rotation depends only on the position difference
    d1 = O.rope(q, 1000, 10000.0) @ O.rope(k, 990, 10000.0)
    d2 = O.rope(q, 30, 10000.0) @ O.rope(k, 20, 10000.0)
    assert abs(d1 - d2) < 1e-5 * (np.abs(q).sum() + np.abs(k).sum())


def test_rope_matches_complex_rotation():
    # pair (i, i + hd/2) as the complex number x_i + j x_{i+hd/2}, rotated by
    # exp(j * pos * theta^(-2i/hd))
    rng = np.random.default_rng(4)
    hd, pos, th = 64, 321, 10000.0
    x = rng.standard_normal(hd)
    z = (x[: hd // 2] + 1j * x[hd // 2:]) * np.exp(
        1j * pos * th ** (-np.arange(hd // 2) * 2.0 / hd))
    want = np.concatenate([z.real, z.imag])
    assert np.allclose(O.rope(x, pos, th), want, atol=1e-6)


def _tiny_weights(cfg, seed=0):
    return O.Weights(cfg, synth.weights(cfg, seed))


def test_fuse_block_identity():
    cfg = synth.config("tiny")
    W = _tiny_weights(cfg)
    H = cfg.H
    rng = np.random.default_rng(5)
    l, m, h = (rng.standard_normal((2, H)) for _ in range(3))
    eye, zero = np.eye(H), np.zeros((H, H))
    for blk, want in ((0, l), (1, m), (2, h)):
        mats = [zero, zero, zero]
        mats[blk] = eye
        W.w_fuse = np.concatenate(mats, axis=1)
        assert np.allclose(O.fuse(W, l, m, h), O.store(want, "fp32"))
    # g is a float32 activation whatever the storage type of the weights
    W.cfg = cfg.replace(dtype="bf16")
    W.w_fuse = np.concatenate([eye, zero, zero], axis=1)
    assert np.array_equal(O.fuse(W, l, m, h),
                          l.astype(np.float32).astype(np.float64))


def test_fuse_is_plain_matmul():
    cfg = synth.config("tiny")
    W = _tiny_weights(cfg)
    rng = np.random.default_rng(6)
    l, m, h = (rng.standard_normal((3, cfg.H)) for _ in range(3))
    t = torch.from_numpy(np.concatenate([l, m, h], 1)) @ torch.from_numpy(
        W.w_fuse).T
    assert np.allclose(O.fuse(W, l, m, h), t.float().numpy(), rtol=1e-6,
                       atol=1e-6)


def test_causal_attention_matches_torch_sdpa():
    rng = np.random.default_rng(7)
    n, hd = 37, 64
    q, k, v = (rng.standard_normal((n, hd)) for _ in range(3))
    ours = O.causal_attention(q, k, v)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], is_causal=True)[0, 0].numpy()
    assert np.allclose(ours, ref, atol=1e-12)


def test_tree_attention_matches_dense_masked_sdpa():
    # explicit boolean mask over [prefix | scratch] reproduces attend() on
    # each query's visible set
    rng = np.random.default_rng(8)
    P, S, hd = 50, 12, 32
    keys = rng.standard_normal((P + S, hd))
    vals = rng.standard_normal((P + S, hd))
    q = rng.standard_normal((6, hd))
    masks = [rng.random(S) < 0.4 for _ in range(6)]
    ours = []
    dense = np.zeros((6, P + S), dtype=bool)
    for i, m in enumerate(masks):
        vis = np.concatenate([np.arange(P), P + np.nonzero(m)[0]])
        ours.append(O.attend(q[i], keys[vis], vals[vis]))
        dense[i, vis] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(keys)[None],
        torch.from_numpy(vals)[None], attn_mask=torch.from_numpy(dense)[None])
    assert np.allclose(np.stack(ours), ref[0].numpy(), atol=1e-12)


def test_topk_and_lse_brute_force():
    rng = np.random.default_rng(9)
    lg = rng.standard_normal(4096).astype(np.float32)
    lg[100] = lg[200] = lg.max() + 1.0      # exact tie: lower id first
    ids = O.topk_desc(lg, 7)
    brute = sorted(range(len(lg)), key=lambda i: (-float(lg[i]), i))[:7]
    assert list(ids) == brute
    assert ids[0] == 100 and ids[1] == 200
    from scipy.special import logsumexp
    assert abs(float(O.lse32(lg)) - logsumexp(lg.astype(np.float64))) < 1e-5
    assert O.child_logprob(-1e30, 0.0) == np.float32(math.log(1e-12))


def test_silu_closed_form():
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
