"""Seeded generators: shapes, distributions and keyed random streams.

Every stream is a NumPy PCG64 generator built from
``SeedSequence(seed, spawn_key=(tag, *indices))`` so that any tensor (a weight
matrix, one sequence's prefix KV, one round's noise) can be regenerated on its
own, in any order, on any machine.  Large tensors are drawn in fixed 8M-element
chunks, each from its own child stream, so the values do not depend on how many
threads draw them.

Distributions (the workloads of the draft-and-verify path on LLaMA-shaped
drafters; no trained weights exist here, so all weights are random):
  * every weight matrix ~ N(0, 0.02^2); norm gains ~ 1 + N(0, 0.02^2)
  * low/mid/high target features ~ N(0, 1)
  * committed prefix K/V rows ~ N(0, 1)
  * root tokens ~ U{0..V-1}
  * target-logit noise ~ N(0, 2^2)
  * verification uniforms ~ U[0, 1)
"""
from __future__ import annotations

import dataclasses
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_CHUNK = 1 << 23


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    H: int            # draft / target hidden width
    n_q: int          # query heads
    n_kv: int         # key/value heads
    hd: int           # head dim
    F: int            # SwiGLU width
    V: int            # vocabulary
    dtype: str        # "bf16" or "fp32" storage
    theta: float      # RoPE base
    B: int            # batch (independent sequences)
    ctx: tuple        # (lo, hi) committed prefix length range, inclusive
    D: int            # tree depth (draft passes per round)
    K: int            # top-k per node and expansion width
    N: int            # verification budget (tree nodes, root excluded)
    T: float          # verify temperature; 0 = greedy
    rounds: int = 1   # chained draft/verify rounds
    s_max: int = 2    # seed rows per sequence per round (upper bound)
    eps: float = 1e-5

    @property
    def n_cand(self) -> int:
        return self.K + (self.D - 1) * self.K * self.K if self.D > 0 else 0

    @property
    def scratch_rows(self) -> int:
        return max(self.D - 1, 0) * self.K

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


_8B = dict(H=4096, n_q=32, n_kv=8, hd=128, F=14336, V=32000, dtype="bf16",
           theta=500000.0)
_70B = dict(H=8192, n_q=64, n_kv=8, hd=128, F=28672, V=32000, dtype="bf16",
            theta=500000.0)

CONFIGS = {
    # tiny fp32 drafter, one sequence, depth 3 / top-4 / 10 nodes
    "tiny": Config("tiny", H=256, n_q=4, n_kv=4, hd=64, F=688, V=4096,
                   dtype="fp32", theta=10000.0, B=1, ctx=(128, 128), D=3, K=4,
                   N=10, T=0.0),
    # LLaMA-3.1-8B-shaped drafter, batch 1, greedy verify
    "8b_bs1": Config("8b_bs1", B=1, ctx=(2048, 2048), D=6, K=10, N=60, T=0.0,
                     **_8B),
    # same shape, 64 independent trees, rejection-sampling verify at T=1
    "8b_bs64": Config("8b_bs64", B=64, ctx=(512, 4096), D=6, K=10, N=60,
                      T=1.0, **_8B),
    # LLaMA-3.3-70B-shaped drafter
    "70b_bs1": Config("70b_bs1", B=1, ctx=(4096, 4096), D=6, K=10, N=60,
                      T=0.0, **_70B),
    "70b_bs16": Config("70b_bs16", B=16, ctx=(4096, 4096), D=6, K=10, N=60,
                       T=1.0, **_70B),
    # chain drafting (top-1 per step, depth 3) at batch 16
    "8b_chain_bs16": Config("8b_chain_bs16", B=16, ctx=(512, 4096), D=3, K=1,
                            N=3, T=0.0, **_8B),
    # long-context reasoning shape: 16k prefix, 64 chained rounds
    "long_bs8": Config("long_bs8", B=8, ctx=(16384, 16384), D=8, K=8, N=80,
                       T=0.6, rounds=64, **_8B),
}


def config(name: str, **overrides) -> Config:
    return CONFIGS[name].replace(**overrides)


def _tag(s: str) -> int:
    return zlib.crc32(s.encode())


class GenKey:
    """A keyed stream: (seed, tag, indices...)."""

    def __init__(self, seed: int, tag: str, *idx: int):
        self.seed = int(seed)
        self.key = (_tag(tag),) + tuple(int(i) for i in idx)

    def rng(self, *sub: int) -> np.random.Generator:
        ss = np.random.SeedSequence(self.seed, spawn_key=self.key + tuple(sub))
        return np.random.Generator(np.random.PCG64(ss))


def normal(key: GenKey, shape, std=1.0, mean=0.0, threads=8) -> np.ndarray:
    """N(mean, std^2) float32 array; chunked so results are thread-count free."""
    shape = tuple(int(s) for s in np.atleast_1d(shape))
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)
    n_chunks = (n + _CHUNK - 1) // _CHUNK

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        key.rng(c).standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if n_chunks <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(n_chunks)))
    if std != 1.0:
        out *= np.float32(std)
    if mean != 0.0:
        out += np.float32(mean)
    return out.reshape(shape)


def uniform_ints(key: GenKey, shape, lo: int, hi: int) -> np.ndarray:
    """Integers uniform on [lo, hi] inclusive, int64."""
    return key.rng().integers(lo, hi + 1, size=shape, dtype=np.int64)


def weights(cfg: Config, seed: int = 0, threads: int = 8) -> dict:
    """Random-init drafter weights, all float32 numpy, layout [out, in]."""
    H, F, V = cfg.H, cfg.F, cfg.V
    qd, kd = cfg.n_q * cfg.hd, cfg.n_kv * cfg.hd
    shapes = {
        "w_fuse": (H, 3 * H),   # W_R: [l; m; h] -> g
        "w_in": (H, 2 * H),     # W_I: [g | a ; e] -> x
        "embed": (V, H),        # token embedding table
        "wq": (qd, H), "wk": (kd, H), "wv": (kd, H), "wo": (H, qd),
        "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F),
        "w_lm": (V, H),
    }
    out = {}
    for name, shp in shapes.items():
        out[name] = normal(GenKey(seed, "w", _tag(cfg.name), _tag(name)), shp,
                           std=0.02, threads=threads)
    for name in ("g_attn", "g_mlp", "g_final"):
        out[name] = normal(GenKey(seed, "w", _tag(cfg.name), _tag(name)), (H,),
                           std=0.02, mean=1.0)
    return out


def contexts(cfg: Config, seed: int = 0) -> np.ndarray:
    """Committed prefix length per sequence."""
    lo, hi = cfg.ctx
    if lo == hi:
        return np.full(cfg.B, lo, dtype=np.int64)
    return uniform_ints(GenKey(seed, "ctx", _tag(cfg.name)), (cfg.B,), lo, hi)


def seq_inputs(cfg: Config, b: int, attempt: int = 0, seed: int = 0) -> dict:
    """First-round seed of sequence b: low/mid/high features and root token."""
    k = GenKey(seed, "seq", _tag(cfg.name), b, attempt)
    feats = normal(GenKey(seed, "feat", _tag(cfg.name), b, attempt),
                   (3, cfg.H))
    tok = int(uniform_ints(k, (), 0, cfg.V - 1))
    return {"low": feats[0], "mid": feats[1], "high": feats[2], "token": tok}


def prefix_kv(cfg: Config, b: int, length: int, attempt: int = 0,
              seed: int = 0, threads: int = 8):
    """Committed draft-KV rows [n_kv, length, hd] for K and V, N(0, 1)."""
    kk = normal(GenKey(seed, "pk", _tag(cfg.name), b, attempt),
                (cfg.n_kv, length, cfg.hd), threads=threads)
    vv = normal(GenKey(seed, "pv", _tag(cfg.name), b, attempt),
                (cfg.n_kv, length, cfg.hd), threads=threads)
    return kk, vv


def seed_features(cfg: Config, b: int, rnd: int, row: int, attempt: int = 0,
                  seed: int = 0) -> np.ndarray:
    """Target low/mid/high features [3, H] at flattened tree row `row` of
    round `rnd` (the verify pass's feature taps, synthetic)."""
    return normal(GenKey(seed, "sf", _tag(cfg.name), b, rnd, row, attempt),
                  (3, cfg.H))


def target_noise(cfg: Config, b: int, rnd: int, rows: int, attempt: int = 0,
                 seed: int = 0) -> np.ndarray:
    """N(0, 2^2) noise [rows, V] added to draft logits to make target logits."""
    return normal(GenKey(seed, "tn", _tag(cfg.name), b, rnd, attempt),
                  (rows, cfg.V), std=2.0)


def uniforms(cfg: Config, b: int, rnd: int, rows: int, attempt: int = 0,
             seed: int = 0) -> np.ndarray:
    """U[0,1) draws [rows, K+1] for the verification of one tree."""
    r = GenKey(seed, "u", _tag(cfg.name), b, rnd, attempt).rng()
    return r.random((rows, cfg.K + 1), dtype=np.float32)
