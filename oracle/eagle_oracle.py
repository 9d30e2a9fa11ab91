"""Plain CPU oracle of the EAGLE-3 draft-and-verify hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg; nothing on the product path imports it.  It
shares no code with the HIP library.

Everything is NumPy float64.  A value that the method stores is rounded at the
storage point.  Weights and the draft KV cache (and the rotated queries that
meet it) use the drafter's storage type (bf16 or fp32); every activation
(fused feature g, layer input x, attention output o, residual h, SwiGLU
product t, draft state a, and the normalised GEMM inputs) is stored as
float32.  Logits, log-sum-exp, log-probabilities and tree scores are float32.

Sources (web pages; cited by title and section):
  [E3]  "EAGLE-3: Scaling up Inference Acceleration of Large Language Models
        via Training-Time Test" (paper summary page), sections 3.2 Big-Picture
        Architecture, 3.4 "Feature Extraction: What Changes from EAGLE to
        EAGLE-3", "The Draft Model Architecture in Detail", "The Inference
        Pipeline: Drafting and Verification", 6 Limitation 6 (LLaMA family:
        pre-normalisation, SwiGLU, rotary embeddings, GQA).
  [E1]  "EAGLE: Speculative Sampling Requires Rethinking Feature Uncertainty"
        (paper summary page), 3.4 "Tree-Structured Draft Generation",
        "Verification Phase: Multi-Round Speculative Sampling on Trees"
        (Algorithm 1), "The Full Inference Loop".
  [M75] "M7.5 - EAGLE Feature Drafting: Uncertainty, Dynamic Trees, HASS, and
        EAGLE-3", sections 0x05A-0x05D, 0x06A-0x06C, 0x08B, 0x08C, 0x09.

Readings where the pages are silent (each also listed in the design notes):
  * fusion and input FCs carry no bias; LM head has no bias;
  * precision: weights and draft KV in the storage type, activations float32;
  * the draft layer is a LLaMA pre-norm block: RMSNorm (eps 1e-5) -> attention
    with rotate-half RoPE -> residual -> RMSNorm -> SwiGLU -> residual; a final
    RMSNorm with its own gain precedes the LM head; the un-normed output `a`
    is the state fed to children;
  * draft confidences are softmax of raw logits (temperature 1);
  * node ids follow creation order with children of one parent created in
    ascending token id, parents taken in ascending node id (only exact score
    ties see this order);
  * verification of deterministic top-k children uses Algorithm 1 with point
    mass proposals; children are tested in ascending token id; the residual
    draw is an inverse CDF over ascending token id.

Parity pins for every function live in tests/test_oracle_*.py.
"""
from __future__ import annotations

import heapq
import math

import numpy as np

__all__ = [
    "LOG_EPS", "bf16_round", "store", "Weights", "rmsnorm", "rope", "silu",
    "fuse", "layer", "topk_desc", "lse32", "child_logprob", "DraftKV",
    "draft_tree", "select_key", "eagle2_tree", "flatten", "verify", "verify_row",
    "block", "tree_ancestors", "target_tree_layer", "gumbel_uniforms",
    "sample_children", "draft_rows", "sampled_row_steps", "verify_row_sampled",
    "verify_sampled",
    "commit", "decision_margin", "score_rows", "causal_attention", "attend",
    "philox4x64", "philox4x64_np", "uniform01", "verify_uniforms",
    "STREAM_VERIFY", "STREAM_DRAFT", "BONUS_DRAW",
]

# log of the confidence floor 1e-12 used for ranking ([M75] 0x06A), float32
LOG_EPS = float(np.float32(math.log(1e-12)))


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16, ties to even.

    bfloat16 keeps the top 16 bits of an IEEE float32.  Rounding adds half of
    the dropped range (0x7FFF) plus the lowest kept bit, then truncates.
    NaN stays NaN (quiet bit forced)."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    nan = np.isnan(x32)
    if nan.any():
        r = np.where(nan, (x32.view(np.uint32) | 0x00400000) & 0xFFFF0000, r)
    return r.view(np.float32).reshape(x32.shape)


def store(x, dtype: str) -> np.ndarray:
    """Value of `x` after it is stored in the drafter's storage type."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        x32 = bf16_round(x32)
    elif dtype != "fp32":
        raise ValueError(dtype)
    return x32.astype(np.float64)


class Weights:
    """Drafter weights as float64 copies of the stored values."""

    NAMES = ("w_fuse", "w_in", "embed", "wq", "wk", "wv", "wo", "w_gate",
             "w_up", "w_down", "w_lm", "g_attn", "g_mlp", "g_final")

    def __init__(self, cfg, arrays: dict):
        self.cfg = cfg
        for n in self.NAMES:
            setattr(self, n, store(arrays[n], cfg.dtype))


# ---------------------------------------------------------------------------
# elementwise pieces of the draft layer
# ---------------------------------------------------------------------------
def rmsnorm(x, gain, eps: float, dtype: str) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * gain, stored ([E3] Limitation 6: the
    LLaMA family uses pre-normalisation; RMSNorm is its norm)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return store(x / np.sqrt(ms + eps) * gain, dtype)


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding of the last axis (pairs i, i + hd/2).

    Angle of pair i at position p is p * theta^(-2i/hd), in float64; cos and
    sin are then rounded to float32.  `x` is [..., hd], `pos` broadcasts over
    the leading axes.  Result is unrounded float64."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    inv = theta ** (-(2.0 * i) / hd)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c = np.cos(ang).astype(np.float32).astype(np.float64)
    s = np.sin(ang).astype(np.float32).astype(np.float64)
    while c.ndim < x.ndim:
        c = c[..., None, :]
        s = s[..., None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


# ---------------------------------------------------------------------------
# (1) multi-layer feature fusion
# ---------------------------------------------------------------------------
def fuse(W: Weights, low, mid, high) -> np.ndarray:
    """g = W_R [l; m; h] for each row ([E3] "Change 2: The fusion FC layer";
    [M75] 0x08B): concat of the three k-dim taps, projected 3k -> k.  The
    taps arrive in the storage type; g is a float32 activation."""
    cat = np.concatenate([np.atleast_2d(low), np.atleast_2d(mid),
                          np.atleast_2d(high)], axis=-1).astype(np.float64)
    return store(cat @ W.w_fuse.T, "fp32")


# ---------------------------------------------------------------------------
# attention over a visible key set
# ---------------------------------------------------------------------------
def attend(q, keys, vals) -> np.ndarray:
    """softmax(q k^T / sqrt(hd)) v for one query vector, float64."""
    s = keys @ q / math.sqrt(q.shape[-1])
    s = s - s.max()
    p = np.exp(s)
    p /= p.sum()
    return p @ vals


def causal_attention(q, k, v) -> np.ndarray:
    """Plain causal attention over a chain: row i sees rows 0..i."""
    out = np.zeros_like(q, dtype=np.float64)
    for i in range(q.shape[0]):
        out[i] = attend(q[i], k[: i + 1], v[: i + 1])
    return out


# ---------------------------------------------------------------------------
# (2) one draft step: join + single decoder layer + LM head
# ---------------------------------------------------------------------------
class DraftKV:
    """One sequence's draft KV cache, [n_kv, cap, hd] float64 (stored values)."""

    def __init__(self, k, v):
        self.k = np.array(k, dtype=np.float64)
        self.v = np.array(v, dtype=np.float64)

    def copy(self):
        return DraftKV(self.k, self.v)


def layer(W: Weights, kv: DraftKV, src, tok, pos, dest, visible):
    """One draft pass over R query rows of one sequence.

    src [R,H]: fused target feature g (seed rows) or the parent's draft state a
    (tree rows) -- [E3] "The Draft Model Architecture in Detail" (input_i =
    [g_i; e_i], projected by a second FC) and "The Inference Pipeline" (a
    stands in for g at drafted positions); [M75] 0x08B u_t = W_I[r_t; e(x)].
    tok [R]: token whose embedding joins the row.  pos [R]: RoPE position.
    dest [R]: cache index receiving the row's K/V.  visible[r]: cache indices
    row r attends to ([M75] 0x08C: target prefix, draft ancestors, itself).

    Returns dict with x, q, k, v, o, h, t, a (stored values) and fp32 logits.
    """
    src = np.atleast_2d(np.asarray(src, dtype=np.float64))
    tok = np.asarray(tok, dtype=np.int64)
    x = store(np.concatenate([src, W.embed[tok]], axis=1) @ W.w_in.T, "fp32")
    return block(W, kv, x, pos, dest, visible)


def block(W: Weights, kv: DraftKV, x, pos, dest, visible):
    """The decoder block after the input: pre-norm attention with RoPE and
    GQA over the visible cache rows, residual, pre-norm SwiGLU, residual,
    then the final norm and the LM head ([E3] 6 "Limitation 6": the LLaMA
    block).  x [R,H] is the block input; every row's K/V is written to the
    cache before any row attends.  Returns dict with x, q, k, v, o, h, t, a
    (stored values) and fp32 logits."""
    cfg = W.cfg
    dt, eps = cfg.dtype, cfg.eps
    f32 = "fp32"
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    R = x.shape[0]
    nq, nkv, hd = cfg.n_q, cfg.n_kv, cfg.hd
    group = nq // nkv
    n1 = rmsnorm(x, W.g_attn, eps, f32)
    q = rope((n1 @ W.wq.T).reshape(R, nq, hd), pos, cfg.theta)
    k = rope((n1 @ W.wk.T).reshape(R, nkv, hd), pos, cfg.theta)
    v = (n1 @ W.wv.T).reshape(R, nkv, hd)
    q, k, v = store(q, dt), store(k, dt), store(v, dt)
    for r in range(R):
        kv.k[:, dest[r]] = k[r]
        kv.v[:, dest[r]] = v[r]
    o = np.zeros((R, nq, hd))
    for r in range(R):
        idx = np.asarray(visible[r], dtype=np.int64)
        for hh in range(nq):
            g = hh // group
            o[r, hh] = attend(q[r, hh], kv.k[g, idx], kv.v[g, idx])
    o = store(o, f32)
    h = store(x + o.reshape(R, nq * hd) @ W.wo.T, f32)
    n2 = rmsnorm(h, W.g_mlp, eps, f32)
    t = store(silu(n2 @ W.w_gate.T) * (n2 @ W.w_up.T), f32)
    a = store(h + t @ W.w_down.T, f32)
    nf = rmsnorm(a, W.g_final, eps, f32)
    logits = (nf @ W.w_lm.T).astype(np.float32)
    return {"x": x, "q": q, "k": k, "v": v, "o": o, "h": h, "t": t, "a": a,
            "logits": logits}


def topk_desc(logits, K: int) -> np.ndarray:
    """Ids of the K largest logits ordered by (-logit, id)."""
    lg = np.asarray(logits)
    order = np.lexsort((np.arange(lg.shape[-1]), -lg.astype(np.float64)))
    return order[:K]


def lse32(logits) -> np.float32:
    """log-sum-exp of one float32 logit row, computed in float64, as float32."""
    lg = np.asarray(logits, dtype=np.float64)
    m = lg.max()
    return np.float32(m + math.log(np.exp(lg - m).sum()))


def child_logprob(logit, lse) -> np.float32:
    """log(max(confidence, 1e-12)) of a child in float32 ([M75] 0x06A)."""
    lp = np.float32(np.float32(logit) - np.float32(lse))
    return np.float32(max(lp, np.float32(LOG_EPS)))


# ---------------------------------------------------------------------------
# (3) EAGLE-2 dynamic tree
# ---------------------------------------------------------------------------
def select_key(node):
    """Global order of [M75] 0x06B: higher value first, shallower, older."""
    return (-float(node["score"]), node["depth"], node["id"])


def _require_int(what: str, value, least: int):
    if isinstance(value, bool) or not isinstance(value, int) or value < least:
        raise ValueError(f"{what} has to be an int >= {least}, not {value!r}")


def _make_children(parent, proposals, created: list) -> list:
    """Append one parent's proposals to `created` as tree nodes.

    A proposal is (token, float32 log confidence).  The record rules of
    [M75] 0x06B are checked: a confidence is a probability (log <= 0, NaN
    refused, log 0 of an impossible token allowed), a token occurs once per
    parent, and the siblings' probabilities add up to at most one (1e-5 slack,
    since they arrive as float32 logs).  Value of a child = parent value +
    log(max(confidence, 1e-12)), accumulated in float32 ([M75] 0x06A)."""
    toks = [t for t, _ in proposals]
    logs = [np.float32(lc) for _, lc in proposals]
    where = f"under node {parent['id']}"
    if len(set(toks)) < len(toks):
        raise ValueError(f"a token is proposed twice {where}")
    if any(np.isnan(lc) or lc > np.float32(1e-6) for lc in logs):
        raise ValueError(f"a log confidence {where} is not the log of a "
                         f"probability: {[float(x) for x in logs]}")
    mass = math.fsum(math.exp(float(lc)) for lc in logs)
    if mass > 1.0 + 1e-5:
        raise ValueError(f"children {where} carry probability {mass:.6f} > 1")
    kids = []
    for tok, lc in zip(toks, logs):
        kids.append({"id": len(created), "token": tok, "parent": parent,
                     "depth": parent["depth"] + 1, "slot": -1,
                     "score": np.float32(parent["score"]
                                         + max(lc, np.float32(LOG_EPS)))})
        created.append(kids[-1])
    return kids


def eagle2_tree(root, expand, width: int, max_depth: int, budget: int):
    """EAGLE-2 dynamic tree ([M75] 0x06A-0x06B; [E3] 3.4 uses it with 10
    nodes kept per step).

    Growth goes one layer at a time.  Of the layer built last (at first: the
    root alone), the `width` nodes that come first in the global order
    (select_key) are handed to `expand(parents, depth)`, in ascending node id;
    it returns, per parent, (token, float32 log confidence) proposals, which
    become the next layer.  This repeats `max_depth` times.  Every node
    created along the way stays a candidate, and the `budget` candidates that
    come first in the global order are the tree.  Because a child's value
    never exceeds its parent's and ties go to the shallower node, that set is
    closed under ancestors.  A zero budget verifies nothing, so nothing is
    drafted.  Node ids count creation order.

    Argument and record errors raise ValueError (see _make_children).
    Returns (selected nodes in global order, every created node)."""
    _require_int("expansion width", width, 1)
    _require_int("verification budget", budget, 0)
    _require_int("maximum depth", max_depth, 0)
    created = []
    newest, depth = [root], 0
    while newest and depth < max_depth and budget > 0:
        parents = heapq.nsmallest(width, newest, key=select_key)
        parents.sort(key=lambda n: n["id"])
        proposals = expand(parents, depth)
        newest = [kid for par, props in zip(parents, proposals)
                  for kid in _make_children(par, props, created)]
        depth += 1
    return heapq.nsmallest(budget, created, key=select_key), created


def draft_tree(W: Weights, kv: DraftKV, seed_src, seed_tok, len_in: int,
               record: bool = False, d2t=None, sample=None):
    """Draft one tree for one sequence.

    Seed rows ([M75] 0x05A: [f_t, embed(x_{t+1})]) are appended to the draft
    KV at cache indices len_in.. and processed causally; the last seed row is
    the root.  Then EAGLE-2 growth (eagle2_tree) with width K, depth D and
    budget N, where expanding a node runs one draft pass over it and takes its
    top-K tokens as children (log confidence = logit - lse, float32).  Nodes
    expanded at depth d >= 1 get scratch slot (d-1)*K + rank (rank in
    ascending node id) at cache index len_out + slot, position P_root + d, and
    see the committed prefix, their ancestors' slots and their own slot.

    d2t: optional strictly increasing map from the drafter's reduced
    vocabulary (the LM head's rows) to target token ids ([M75] 0x08C: the
    draft head predicts over a configured sub-vocabulary with id maps).  Tree
    tokens, the embedding lookups and verification then use target ids; the
    map is increasing, so orders by draft id and by target id agree.

    sample: dict(T, seed, rnd, b) for sampled children ([E1] 3.4: at T > 0
    the children of a node are sampled from the draft distribution): each
    expanded node's K children are sample_children draws from softmax(logits
    / T) (Philox draws gumbel_uniforms of (seed, rnd, b, key row)), created in
    draw order, with log confidence log q(x) = logits[x] / T - lse(logits /
    T) in float32.  The budget must keep every created node (N >= K + (D-1)
    K^2), so that the children a node shows are all of its draws, in order --
    what the verification's sampling law needs.

    Mutates kv (seed rows + scratch rows).  Returns (tree, info)."""
    cfg = W.cfg
    K, D, N = cfg.K, cfg.D, cfg.N
    if sample is not None:
        if d2t is not None or N < cfg.n_cand:
            raise ValueError("sampled children keep every drafted node: need "
                             "N >= K + (D-1) K^2 and no reduced vocabulary")
    seed_src = np.atleast_2d(np.asarray(seed_src, dtype=np.float64))
    seed_tok = np.asarray(seed_tok, dtype=np.int64)
    s = len(seed_tok)
    len_out = len_in + s
    p_root = len_out - 1
    info = {"passes": [], "len_out": len_out, "nodes": []}

    out = layer(W, kv, seed_src, seed_tok,
                pos=np.arange(len_in, len_out), dest=np.arange(len_in, len_out),
                visible=[np.arange(0, len_in + i + 1) for i in range(s)])
    root = {"id": -1, "token": int(seed_tok[-1]), "parent": None, "depth": 0,
            "score": np.float32(0.0), "slot": -1, "a": out["a"][-1],
            "logits": out["logits"][-1], "mask_slots": []}
    info["root"] = root
    if record:
        info["passes"].append({"rows": [root], "out": out})

    def children(parents):
        res = []
        for p in parents:
            lg = p["logits"]
            if sample is not None:
                T = sample["T"]
                scaled = (np.asarray(lg, np.float32) / np.float32(T)).astype(np.float32)
                lse = lse32(scaled)
                key_row = 0 if p["id"] < 0 else 1 + p["id"]
                u = gumbel_uniforms(sample["seed"], sample["rnd"], sample["b"], key_row,
                                    len(lg))
                ids, m = sample_children(lg, T, K, u)
                info["sample_margin"] = min(info.get("sample_margin", float("inf")), m)
                res.append([(t, child_logprob(scaled[t], lse)) for t in ids])
                continue
            lse = lse32(lg)
            ids = sorted(int(i) for i in topk_desc(lg, K))
            res.append([(int(t) if d2t is None else int(d2t[t]),
                         child_logprob(lg[t], lse)) for t in ids])
        return res

    def expand(chosen, depth):
        if depth == 0:
            return children(chosen)
        for r, n in enumerate(chosen):
            n["slot"] = (depth - 1) * K + r
            n["mask_slots"] = n["parent"]["mask_slots"] + [n["slot"]]
        vis = [np.concatenate([np.arange(len_out),
                               len_out + np.asarray(n["mask_slots"])])
               for n in chosen]
        o = layer(W, kv, np.stack([n["parent"]["a"] for n in chosen]),
                  [n["token"] for n in chosen],
                  pos=np.full(len(chosen), p_root + depth),
                  dest=np.array([len_out + n["slot"] for n in chosen]),
                  visible=vis)
        for r, n in enumerate(chosen):
            n["a"] = o["a"][r]
            n["logits"] = o["logits"][r]
        if record:
            info["passes"].append({"rows": chosen, "out": o})
        return children(chosen)

    selected, nodes = eagle2_tree(root, expand, K, D, N)
    for n in selected:
        n["selected"] = True
    info["nodes"] = nodes
    info["sampled"] = sample is not None
    return flatten(cfg, root, selected, p_root), info


def draft_rows(cfg, tree, info) -> np.ndarray:
    """Draft logits of the expanded nodes, float32 [1 + (D-1) K, V]: row 0
    the root's, row 1 + s the node with scratch slot s (every node with
    children in the tree was expanded and has a slot)."""
    out = np.zeros((1 + max(cfg.D - 1, 0) * cfg.K, cfg.V), dtype=np.float32)
    out[0] = info["root"]["logits"]
    for n in info["nodes"]:
        if n.get("slot", -1) >= 0 and "logits" in n:
            out[1 + n["slot"]] = n["logits"]
    return out


def flatten(cfg, root, selected, p_root):
    """Flattened tree ([M75] 0x05C, 0x09: rows, positions, ancestry mask,
    retrieve map).  Row 0 is the root; rows 1..n are the selected nodes in
    ascending node id, i.e. by (depth, parent row, token id).  Arrays have
    N+1 rows; unused rows hold -1 (0 for score, n_child, mask)."""
    N = cfg.N
    W = (N + 1 + 63) // 64
    sel = sorted(selected, key=lambda n: n["id"])
    row_of = {id(root): 0}
    for r, n in enumerate(sel):
        row_of[id(n)] = r + 1
    n_rows = N + 1
    t = {k: np.full(n_rows, -1, dtype=np.int32) for k in
         ("token", "parent", "depth", "position", "kv_slot", "first_child")}
    t["n_child"] = np.zeros(n_rows, dtype=np.int32)
    t["score"] = np.zeros(n_rows, dtype=np.float32)
    t["mask"] = np.zeros((n_rows, W), dtype=np.uint64)
    t["n_nodes"] = len(sel)
    rows = [root] + sel
    for r, n in enumerate(rows):
        t["token"][r] = n["token"]
        t["parent"][r] = -1 if n["parent"] is None else row_of[id(n["parent"])]
        t["depth"][r] = n["depth"]
        t["position"][r] = p_root + n["depth"]
        t["kv_slot"][r] = n["slot"]
        t["score"][r] = n["score"]
        a = r
        while a != -1:
            t["mask"][r, a // 64] |= np.uint64(1) << np.uint64(a % 64)
            a = t["parent"][a]
    for r in range(1, len(rows)):
        p = t["parent"][r]
        if t["n_child"][p] == 0:
            t["first_child"][p] = r
        t["n_child"][p] += 1
    return t


def score_rows(W: Weights, kv: DraftKV, tree, info):
    """Draft logits at every flattened row (float32 [N+1, V]).

    Rows that were expanded already hold their logits.  The others (never
    expanded) are scored by one extra draft pass over them: source = parent's
    state, position = P_root + depth, K/V written to temporary cache rows past
    the scratch area (on a copy of `kv`), visibility = committed prefix, the
    ancestors' scratch rows and the row itself."""
    cfg = W.cfg
    N, K, D = cfg.N, cfg.K, cfg.D
    p_root = int(tree["position"][0])
    len_out = p_root + 1
    root = info["root"]
    out = np.zeros((N + 1, cfg.V), dtype=np.float32)
    out[0] = root["logits"]
    sel = sorted((n for n in info["nodes"] if n.get("selected")),
                 key=lambda n: n["id"])
    todo = []
    for r, n in enumerate(sel, start=1):
        if "logits" in n:
            out[r] = n["logits"]
        else:
            todo.append((r, n))
    if todo:
        kv2 = kv.copy()
        base = len_out + max(D - 1, 0) * K
        src = np.stack([n["parent"]["a"] for _, n in todo])
        vis = [np.concatenate([np.arange(len_out),
                               len_out + np.asarray(n["parent"]["mask_slots"],
                                                    dtype=np.int64),
                               [base + i]]) for i, (_, n) in enumerate(todo)]
        o = layer(W, kv2, src, [n["token"] for _, n in todo],
                  pos=np.array([p_root + n["depth"] for _, n in todo]),
                  dest=np.array([base + i for i in range(len(todo))]),
                  visible=vis)
        for i, (r, _) in enumerate(todo):
            out[r] = o["logits"][i]
    return out


# ---------------------------------------------------------------------------
# the target's verification forward over the flattened tree
# ---------------------------------------------------------------------------
def tree_ancestors(tree, r: int) -> list:
    """Flattened rows on the path from the root to row r, r included."""
    out = []
    while r >= 0:
        out.append(int(r))
        r = int(tree["parent"][r])
    return out[::-1]


def target_tree_layer(W: Weights, kv: DraftKV, tree, len_in: int):
    """One target decoder layer over the N+1 flattened tree rows in a single
    pass under tree attention ([E1] "The Full Inference Loop", Phase 2: the
    target processes the prompt plus the draft tree in one forward pass;
    [E3] 3.4 "The Inference Pipeline", Stage 2; [M75] 0x05C).  Row r takes
    the embedding of its token as input, rotates at its tree position,
    writes its K/V to cache row len_in + r, and sees the committed prefix
    [0, len_in) plus the rows of its own root-to-r path.  Returns the block
    outputs of rows 0..n_nodes: a [n+1, H] and float32 logits [n+1, V]
    (the target's next-token logits after each row)."""
    n = int(tree["n_nodes"])
    rows = list(range(n + 1))
    tok = np.asarray([tree["token"][r] for r in rows], dtype=np.int64)
    x = store(W.embed[tok], "fp32")
    vis = [np.concatenate([np.arange(len_in, dtype=np.int64),
                           len_in + np.asarray(tree_ancestors(tree, r), dtype=np.int64)])
           for r in rows]
    return block(W, kv, x, pos=np.asarray([tree["position"][r] for r in rows]),
                 dest=np.asarray([len_in + r for r in rows]), visible=vis)


def decision_margin(cfg, tree_info) -> float:
    """Smallest score gap at a selection boundary that decides the tree.

    Boundaries: each per-layer expansion cut (K-th vs K+1-th value among the
    layer's nodes), the final top-N cut, and the per-row top-K cut of a row
    whose K-th child lies within 2e-3 of the lowest value selected by either
    cut that sees it.  Inputs whose margin is below 1e-3 are redrawn."""
    nodes = tree_info.get("nodes", [])
    K, N, D = cfg.K, cfg.N, cfg.D
    inf = float("inf")
    margin = inf
    if not nodes:
        return margin
    by_depth = {}
    for n in nodes:
        by_depth.setdefault(n["depth"], []).append(n)
    cut_low = {}
    for d, layer_nodes in by_depth.items():
        sc = sorted((float(n["score"]) for n in layer_nodes), reverse=True)
        if d < D and len(sc) > K:
            margin = min(margin, sc[K - 1] - sc[K])
        cut_low[d] = sc[min(K, len(sc)) - 1] if d < D else inf
    allsc = sorted((float(n["score"]) for n in nodes), reverse=True)
    fin_low = allsc[min(N, len(allsc)) - 1] if N > 0 else inf
    if len(allsc) > N > 0:
        margin = min(margin, allsc[N - 1] - allsc[N])
    if tree_info.get("sampled"):
        # children are sampled: their draws decide, not per-row logit cuts
        return min(margin, tree_info.get("sample_margin", inf))
    # per-row top-K cuts
    parents = {}
    for n in nodes:
        parents.setdefault(id(n["parent"]), (n["parent"], []))[1].append(n)
    for p, kids in parents.values():
        lg = np.asarray(p["logits"], dtype=np.float64)
        srt = np.sort(lg)[::-1]
        if len(srt) <= K:
            continue
        gap = srt[K - 1] - srt[K]
        kth = min(float(c["score"]) for c in kids)
        d = kids[0]["depth"]
        low = min(cut_low.get(d, inf), fin_low)
        if kth + 2e-3 >= low:
            margin = min(margin, gap)
    return margin


# ---------------------------------------------------------------------------
# counter-based random numbers: Philox4x64-10
# ---------------------------------------------------------------------------
# Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3"
# (SC 2011): a 4 x 64-bit counter is encrypted under a 2 x 64-bit key by ten
# rounds of two 64x64->128 multiplications; the key is bumped by two Weyl
# constants between rounds.  Constants are the paper's for Philox4x64.
PHILOX_MUL = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
PHILOX_WEYL = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)
_M64 = (1 << 64) - 1

# random streams of the key's second word
STREAM_VERIFY = 0
STREAM_DRAFT = 1
# draw index of the residual (bonus) draw of a verified row
BONUS_DRAW = 63


def philox4x64(counter, key, rounds: int = 10):
    """One Philox4x64 block, plain Python integers.  counter: 4 words,
    key: 2 words.  Returns the 4 output words."""
    x = [int(c) & _M64 for c in counter]
    k0, k1 = int(key[0]) & _M64, int(key[1]) & _M64
    for _ in range(rounds):
        p0 = PHILOX_MUL[0] * x[0]
        p1 = PHILOX_MUL[1] * x[2]
        x = [(p1 >> 64) ^ x[1] ^ k0, p1 & _M64,
             (p0 >> 64) ^ x[3] ^ k1, p0 & _M64]
        k0 = (k0 + PHILOX_WEYL[0]) & _M64
        k1 = (k1 + PHILOX_WEYL[1]) & _M64
    return x


def _mulhilo64(a, m: int):
    """(high, low) 64-bit halves of a * m for a uint64 array, built from
    32-bit limbs so that no intermediate exceeds 64 bits."""
    a = a.astype(np.uint64)
    mask = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    a_lo, a_hi = a & mask, a >> s32
    m_lo, m_hi = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    ll = a_lo * m_lo
    lh = a_lo * m_hi
    hl = a_hi * m_lo
    hh = a_hi * m_hi
    mid = (ll >> s32) + (lh & mask) + (hl & mask)
    hi = hh + (lh >> s32) + (hl >> s32) + (mid >> s32)
    return hi, a * np.uint64(m)


def philox4x64_np(c0, c1, c2, c3, k0: int, k1: int):
    """philox4x64 over uint64 arrays of counters (same rounds, vectorised)."""
    x = [np.asarray(c, dtype=np.uint64).copy() for c in (c0, c1, c2, c3)]
    with np.errstate(over="ignore"):
        kk0, kk1 = np.uint64(k0 & _M64), np.uint64(k1 & _M64)
        for _ in range(10):
            h0, l0 = _mulhilo64(x[0], PHILOX_MUL[0])
            h1, l1 = _mulhilo64(x[2], PHILOX_MUL[1])
            x = [h1 ^ x[1] ^ kk0, l1, h0 ^ x[3] ^ kk1, l0]
            kk0 = kk0 + np.uint64(PHILOX_WEYL[0])
            kk1 = kk1 + np.uint64(PHILOX_WEYL[1])
    return x


def uniform01(seed: int, stream: int, rnd, b, row, draw) -> np.ndarray:
    """U[0,1) float32 draws: counter (draw, row, b, round), key (seed,
    stream); the top 24 bits of the block's first word, times 2^-24."""
    shape = np.broadcast(np.asarray(rnd), np.asarray(b), np.asarray(row),
                         np.asarray(draw)).shape
    c = [np.broadcast_to(np.asarray(v, dtype=np.uint64), shape)
         for v in (draw, row, b, rnd)]
    x0 = philox4x64_np(*c, seed, stream)[0]
    return ((x0 >> np.uint64(40)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def verify_uniforms(cfg, seed: int, rnd: int, b: int) -> np.ndarray:
    """The [N+1, K+1] draws a verification of sequence b in round `rnd`
    uses: column i < K for the i-th child of a row, column K the residual
    draw (draw index BONUS_DRAW)."""
    rows = np.arange(cfg.N + 1)[:, None]
    draws = np.append(np.arange(cfg.K), BONUS_DRAW)[None, :]
    return uniform01(seed, STREAM_VERIFY, rnd, b, rows, draws)


# ---------------------------------------------------------------------------
# sampled children ([E1] 3.4 "Tree-Structured Draft Generation": at T > 0 the
# k children of a node are sampled from the draft distribution)
# ---------------------------------------------------------------------------
def gumbel_uniforms(seed: int, rnd: int, b: int, key_row, V: int) -> np.ndarray:
    """U(0,1) draws for tokens 0..V-1 of one expanded node (float64): Philox
    key (seed, STREAM_DRAFT), counter (x // 4, key_row, b, round), token x
    takes output word x % 4; u = (top 24 bits + 1/2) * 2^-24, never 0 or 1.
    key_row is 0 for the root and 1 + node id for a drafted node; an array
    of key rows gives one row of draws per key [len, V]."""
    rows = np.atleast_1d(np.asarray(key_row, dtype=np.uint64))
    nq = (V + 3) // 4
    q = np.broadcast_to(np.arange(nq, dtype=np.uint64)[None, :], (len(rows), nq))
    kr = np.broadcast_to(rows[:, None], q.shape)
    words = philox4x64_np(q, kr, np.full(q.shape, b, np.uint64),
                          np.full(q.shape, rnd, np.uint64), seed, STREAM_DRAFT)
    w = np.stack(words, axis=-1).reshape(len(rows), -1)[:, :V]
    u = ((w >> np.uint64(40)).astype(np.float64) + 0.5) * 2.0 ** -24
    return u[0] if np.ndim(key_row) == 0 else u


def sample_children(logits, T: float, K: int, u) -> tuple:
    """K children drawn from q = softmax(logits / T) without replacement,
    in draw order: the Gumbel-top-k construction (Gumbel-max applied K
    times, each time over the tokens not yet drawn) -- x_i maximises
    logits[x] / T + G(x), G(x) = -log(-log u[x]), over the remaining tokens,
    ties to the lower id.  Returns (tokens, margin), margin = the smallest
    gap between consecutive perturbed values among the first K + 1."""
    lg = np.asarray(logits, dtype=np.float64)
    key = lg / T - np.log(-np.log(np.asarray(u, dtype=np.float64)))
    order = np.lexsort((np.arange(len(key)), -key))[: K + 1]
    vals = key[order]
    margin = float(np.min(vals[:-1] - vals[1:])) if len(vals) > 1 else float("inf")
    return [int(x) for x in order[:K]], margin


# ---------------------------------------------------------------------------
# (4) verification
# ---------------------------------------------------------------------------
def verify_row(logits, child_tokens, T: float, u_child, u_bonus):
    """One visited row of the verification walk.

    Greedy (T == 0): x* = argmax (lowest id on ties); the child carrying x* is
    accepted, else x* is the emitted token ([E1] 3.4, greedy tree drafting).

    Sampling (T > 0): Algorithm 1 of [E1] ("Multi-round sampling for tree
    structures") with target p = softmax(logits / T) and each child a point
    mass proposal (the children are the deterministic top-k, so p_hat_i puts
    all mass on t_i): child i is accepted when r_i < p(t_i) / 1; on rejection
    p <- norm(max(0, p - onehot(t_i))), i.e. t_i's mass is removed and p is
    renormalised; if every child is rejected one token is drawn from the
    final p by inverse CDF over ascending ids using u_bonus.

    `u_child(i)` / `u_bonus()` return the uniform for child i / the bonus.
    Returns (accepted child index or None, emitted token or None, margin)."""
    lg = np.asarray(logits, dtype=np.float64)
    if T == 0:
        x = int(np.argmax(lg))
        for i, c in enumerate(child_tokens):
            if c == x:
                return i, None, float("inf")
        return None, x, float("inf")
    w = np.exp((lg - lg.max()) / T)
    margin = float("inf")
    for i, c in enumerate(child_tokens):
        S = w.sum()
        u = float(u_child(i))
        thr = w[c] / S
        margin = min(margin, abs(u - thr))
        if u < thr:
            return i, None, margin
        w[c] = 0.0
    S = w.sum()
    ub = float(u_bonus())
    if not S > 0.0:
        # the children held all remaining mass: take the best other token
        lg2 = lg.copy()
        lg2[list(child_tokens)] = -np.inf
        return None, int(np.argmax(lg2)), 0.0
    cdf = np.cumsum(w) / S
    tok = int(np.searchsorted(cdf, ub, side="right"))
    tok = min(tok, len(w) - 1)
    while w[tok] == 0.0 and tok > 0:   # never land on a zero-mass token
        tok -= 1
    lo = cdf[tok - 1] if tok > 0 else 0.0
    margin = min(margin, abs(ub - cdf[tok]), abs(ub - lo) if tok > 0 else 1.0)
    return None, tok, margin


def verify(cfg, tree, target_logits, T: float, uniforms=None, seed=None,
           rnd: int = 0, b: int = 0):
    """Walk the flattened tree from the root ([E1] Algorithm 1, applied at
    each visited row; [E1] "The Full Inference Loop": a >= 0 accepted draft
    tokens plus one emitted token).

    target_logits [N+1, V] float32: row r holds the target's next-token
    logits after node r.  The draws: `uniforms` [N+1, K+1] (column i < K for
    the i-th child of that row in ascending token id, column K the residual
    draw), or, when it is None, the Philox draws of (seed, round rnd,
    sequence b) from verify_uniforms.
    Returns dict(accept_len, accepted_rows, tokens, bonus, margin)."""
    D, K = cfg.D, cfg.K
    if uniforms is None and T > 0 and seed is not None:
        uniforms = verify_uniforms(cfg, seed, rnd, b)
    v = 0
    acc = []
    margin = float("inf")
    while True:
        fc, nc = int(tree["first_child"][v]), int(tree["n_child"][v])
        kids = list(range(fc, fc + nc)) if nc > 0 else []
        ktok = [int(tree["token"][c]) for c in kids]
        u = uniforms[v] if uniforms is not None else None
        ci, tok, m = verify_row(target_logits[v], ktok, T,
                                (lambda i: u[i]) if u is not None else None,
                                (lambda: u[K]) if u is not None else None)
        margin = min(margin, m)
        if ci is not None:
            v = kids[ci]
            acc.append(v)
            continue
        bonus = tok
        break
    rows = np.full(D, -1, dtype=np.int32)
    rows[: len(acc)] = acc
    toks = np.full(D + 1, -1, dtype=np.int32)
    for i, r in enumerate(acc):
        toks[i] = tree["token"][r]
    toks[len(acc)] = bonus
    return {"accept_len": len(acc), "accepted_rows": rows, "tokens": toks,
            "bonus": bonus, "margin": margin}


def sampled_row_steps(target_logits, draft_logits, child_tokens, T: float):
    """The quantities of Algorithm 1 of [E1] ("Verification Phase:
    Multi-Round Speculative Sampling on Trees") at one row whose children
    were drawn from q = softmax(draft / T) without replacement: p =
    softmax(target / T); the i-th child's draft distribution p_hat_i is q
    with the earlier children's tokens removed, renormalised; child i is
    accepted with probability min(1, p(t_i) / p_hat_i(t_i)), and on
    rejection p <- norm(max(0, p - p_hat_i)).  A residual of zero mass (p
    equal to p_hat_i) restarts from the target distribution.
    Returns (ratios [k], the residual p after all k rejections)."""
    tl = np.asarray(target_logits, dtype=np.float64)
    dl = np.asarray(draft_logits, dtype=np.float64)
    p0 = np.exp((tl - tl.max()) / T)
    p0 /= p0.sum()
    q = np.exp((dl - dl.max()) / T)
    q /= q.sum()
    p = p0.copy()
    drawn, ratios = [], []
    for x in child_tokens:
        prop = q.copy()
        prop[drawn] = 0.0
        prop /= prop.sum()
        ratios.append(p[x] / prop[x])
        res = np.maximum(0.0, p - prop)
        z = res.sum()
        p = res / z if z > 0.0 else p0.copy()
        drawn.append(x)
    return ratios, p


def verify_row_sampled(target_logits, draft_logits, child_tokens, T: float,
                       u_child, u_bonus):
    """One visited row of the verification walk for sampled children
    (sampled_row_steps): child i is accepted when u_i < ratio_i; if every
    child is rejected, the emitted token is drawn from the final residual by
    inverse CDF over ascending ids with u_bonus.
    Returns (accepted child index or None, emitted token or None, margin)."""
    ratios, p = sampled_row_steps(target_logits, draft_logits, child_tokens, T)
    margin = float("inf")
    for i, r in enumerate(ratios):
        u = float(u_child(i))
        margin = min(margin, abs(u - r))
        if u < r:
            return i, None, margin
    ub = float(u_bonus())
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    tok = int(np.searchsorted(cdf, ub, side="right"))
    tok = min(tok, len(p) - 1)
    while p[tok] == 0.0 and tok > 0:
        tok -= 1
    lo = cdf[tok - 1] if tok > 0 else 0.0
    margin = min(margin, abs(ub - cdf[tok]), abs(ub - lo) if tok > 0 else 1.0)
    return None, tok, margin


def verify_sampled(cfg, tree, target_logits, draft_logit_rows, T: float,
                   uniforms=None, seed=None, rnd: int = 0, b: int = 0):
    """verify() for trees with sampled children: at each visited row v with
    children, verify_row_sampled against that row's draft logits
    (draft_logit_rows[0] for the root, [1 + kv_slot] for a drafted node);
    children are taken in flattened order, which is their draw order.  A row
    without children emits a token drawn from the target alone.  Draws as in
    verify()."""
    D, K = cfg.D, cfg.K
    if uniforms is None and seed is not None:
        uniforms = verify_uniforms(cfg, seed, rnd, b)
    v = 0
    acc = []
    margin = float("inf")
    while True:
        fc, nc = int(tree["first_child"][v]), int(tree["n_child"][v])
        kids = list(range(fc, fc + nc)) if nc > 0 else []
        ktok = [int(tree["token"][c]) for c in kids]
        u = uniforms[v]
        if nc > 0:
            e = 0 if v == 0 else 1 + int(tree["kv_slot"][v])
            ci, tok, m = verify_row_sampled(target_logits[v], draft_logit_rows[e], ktok, T,
                                            lambda i: u[i], lambda: u[K])
        else:
            ci, tok, m = verify_row(target_logits[v], [], T, None, lambda: u[K])
        margin = min(margin, m)
        if ci is not None:
            v = kids[ci]
            acc.append(v)
            continue
        bonus = tok
        break
    rows = np.full(D, -1, dtype=np.int32)
    rows[: len(acc)] = acc
    toks = np.full(D + 1, -1, dtype=np.int32)
    for i, r in enumerate(acc):
        toks[i] = tree["token"][r]
    toks[len(acc)] = bonus
    return {"accept_len": len(acc), "accepted_rows": rows, "tokens": toks,
            "bonus": bonus, "margin": margin}


# ---------------------------------------------------------------------------
# commit of the accepted path ([M75] 0x05D)
# ---------------------------------------------------------------------------
def commit(cfg, tree, result, kv: DraftKV, mode: str = "keep"):
    """Publish the accepted path into the draft KV and build the next seed.

    [M75] 0x05D commits accepted state, discards unaccepted tree rows and
    reseeds from the last verified target feature with the advanced token;
    row maps come from the flatten metadata, never from token equality.

    Draft row of node u (depth i) sits at position P_root + i and was computed
    from (parent state, token of u).  (row r, tok) below means "fused target
    feature at flattened row r, joined with token tok"; the next draft call
    appends such seed rows at the returned length.

    mode "keep": accepted nodes u_1..u_{a-1} each have a child in the tree, so
    each was expanded and owns a scratch row; u_a owns one only if it was
    expanded.  Kept rows move to cache index = position, and the seed supplies
    only the rows still missing:
      a == 0:                     [(row 0, bonus)]
      u_a expanded:               [(row u_a, bonus)]
      u_a not expanded:           [(row u_{a-1}, token u_a), (row u_a, bonus)]
    mode "reseed" ([E3] 3.4 Stage 2: the target's l, m, h at every verified
    position are fused for the next round): no draft row is kept; the seed is
    all a + 1 verified rows, [(row 0, tok u_1), (row u_1, tok u_2), ...,
    (row u_a, bonus)].
    Returns (new_len, seed_rows, seed_tokens)."""
    a = result["accept_len"]
    rows = list(result["accepted_rows"][:a])
    p_root = int(tree["position"][0])
    len_out = p_root + 1
    bonus = int(result["bonus"])
    if mode == "reseed":
        path = [0] + rows
        nxt = [int(tree["token"][r]) for r in rows] + [bonus]
        return len_out, path, nxt
    if mode != "keep":
        raise ValueError(mode)
    if a == 0:
        keep, seed = [], [(0, bonus)]
    elif tree["kv_slot"][rows[-1]] >= 0:
        keep, seed = rows, [(rows[-1], bonus)]
    else:
        prev = rows[-2] if a >= 2 else 0
        keep = rows[:-1]
        seed = [(prev, int(tree["token"][rows[-1]])), (rows[-1], bonus)]
    src = [len_out + int(tree["kv_slot"][r]) for r in keep]
    dst = [p_root + int(tree["depth"][r]) for r in keep]
    ksrc = kv.k[:, src].copy()
    vsrc = kv.v[:, src].copy()
    for i, dd in enumerate(dst):
        kv.k[:, dd] = ksrc[:, i]
        kv.v[:, dd] = vsrc[:, i]
    new_len = len_out + len(keep)
    return new_len, [s[0] for s in seed], [s[1] for s in seed]
