"""EAGLE-3 draft-and-verify hot path on MI355X (gfx950).

Thin PyTorch-facing binding over libeagle.so (include/eagle.h): every step of
the path runs in the library's HIP kernels; this module only allocates tensors
with torch and passes pointers.  Importing works without a GPU; calling needs
the built library and a gfx950 device.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import EagleError, check, lib

__all__ = ["DrafterShape", "Drafter", "KVCache", "EagleError", "lib",
           "WEIGHT_NAMES", "draw_uniforms", "COMMIT_KEEP", "COMMIT_RESEED"]

COMMIT_KEEP, COMMIT_RESEED = _lib.COMMIT_KEEP, _lib.COMMIT_RESEED

WEIGHT_NAMES = ("w_fuse", "w_in", "embed", "wq", "wk", "wv", "wo", "w_gate",
                "w_up", "w_down", "w_lm", "g_attn", "g_mlp", "g_final")


@dataclass(frozen=True)
class DrafterShape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    dtype: str          # "bf16" | "fp32"
    rope_theta: float
    depth: int
    topk: int
    budget: int
    max_batch: int
    max_seed: int = 2
    rms_eps: float = 1e-5
    target_vocab: int = 0   # 0: same as vocab; larger needs a d2t map

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def c_config(self) -> _lib.Config:
        return _lib.Config(self.hidden, self.n_q_heads, self.n_kv_heads,
                           self.head_dim, self.ffn, self.vocab,
                           0 if self.dtype == "bf16" else 1,
                           float(self.rope_theta), float(self.rms_eps),
                           self.depth, self.topk, self.budget, self.max_batch,
                           self.max_seed, self.target_vocab)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class KVCache:
    """Draft KV cache: k [B, n_kv, cap, hd] (key rows), v [B, n_kv, hd, cap]
    (values stored transposed), committed lengths [B] (int32); cap is a
    multiple of 8 and at least 32."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, length: torch.Tensor):
        assert k.dim() == 4 and v.dim() == 4 and k.is_contiguous() and v.is_contiguous()
        assert k.shape[:2] == v.shape[:2] and k.shape[2] == v.shape[3] and \
            k.shape[3] == v.shape[2], "v is [B, n_kv, hd, cap]"
        self.k, self.v = k, v
        self.length = length.to(torch.int32).contiguous()

    @classmethod
    def from_rows(cls, k: torch.Tensor, v_rows: torch.Tensor, length: torch.Tensor):
        """From key and value rows, both [B, n_kv, cap, hd]."""
        return cls(k.contiguous(), v_rows.transpose(-1, -2).contiguous(), length)

    def v_rows(self) -> torch.Tensor:
        """The values as rows, [B, n_kv, cap, hd] (a view)."""
        return self.v.transpose(-1, -2)

    @property
    def cap(self) -> int:
        return self.k.shape[2]

    def c_kv(self, len_in, len_out) -> _lib.KV:
        return _lib.KV(self.k.data_ptr(), self.v.data_ptr(), self.cap,
                       None if len_in is None else len_in.data_ptr(),
                       None if len_out is None else len_out.data_ptr())


class Drafter:
    """One drafter context: config, weights, workspace."""

    def __init__(self, shape: DrafterShape, weights: dict, device="cuda"):
        self.shape = shape
        L = lib()
        self._cfg = shape.c_config()
        nbytes = L.eagle_workspace_bytes(ctypes.byref(self._cfg))
        if nbytes == 0:
            raise EagleError(2, "eagle_workspace_bytes (config rejected)")
        self.weights = {}
        for n in WEIGHT_NAMES:
            t = weights[n]
            if t.dtype != shape.torch_dtype or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"weight {n}: need contiguous {shape.torch_dtype} on GPU")
            self.weights[n] = t
        d2t = weights.get("d2t")
        if d2t is not None:
            if d2t.dtype != torch.int32 or not d2t.is_contiguous() or not d2t.is_cuda:
                raise ValueError("d2t: need a contiguous int32 tensor on GPU")
            self.weights["d2t"] = d2t
        self._w = _lib.Weights(*[self.weights[n].data_ptr() for n in WEIGHT_NAMES],
                               None if d2t is None else d2t.data_ptr())
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        ctx = ctypes.c_void_p()
        check(L.eagle_create(ctypes.byref(self._cfg), ctypes.byref(self._w),
                             _ptr(self.workspace), nbytes, _stream(),
                             ctypes.byref(ctx)), "eagle_create")
        self._ctx = ctx

    def close(self):
        if getattr(self, "_ctx", None):
            lib().eagle_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------
    def profile(self, on: bool, resume: bool = False):
        mode = (2 if resume else 1) if on else 0
        check(lib().eagle_profile(self._ctx, mode), "eagle_profile")

    def profile_read(self) -> dict:
        import numpy as np
        n = len(_lib.PROFILE_CLASSES)
        ms = np.zeros(n, np.float32)
        cnt = np.zeros(n, np.int32)
        by = np.zeros(n, np.float64)
        fl = np.zeros(n, np.float64)
        check(lib().eagle_profile_read(
            self._ctx, n, ms.ctypes.data_as(ctypes.c_void_p),
            cnt.ctypes.data_as(ctypes.c_void_p),
            by.ctypes.data_as(ctypes.c_void_p),
            fl.ctypes.data_as(ctypes.c_void_p)), "eagle_profile_read")
        return {name: {"ms": float(ms[i]), "launches": int(cnt[i]),
                       "bytes": float(by[i]), "flops": float(fl[i])}
                for i, name in enumerate(_lib.PROFILE_CLASSES)}

    def device_status(self) -> int:
        st = ctypes.c_int32(0)
        check(lib().eagle_get_device_status(self._ctx, ctypes.byref(st),
                                            _stream()), "eagle_get_device_status")
        return int(st.value)

    def fuse(self, low, mid, high, out=None):
        rows = low.shape[0]
        if out is None:
            out = torch.empty(rows, self.shape.hidden, dtype=torch.float32,
                              device=low.device)
        check(lib().eagle_fuse_features(self._ctx, rows, _ptr(low), _ptr(mid),
                                        _ptr(high), _ptr(out), _stream()),
              "eagle_fuse_features")
        return out

    def draft_step(self, batch, rows_per_seq, src, token, position, dest,
                   prefix_len, scratch_base, scratch_mask, kv: KVCache,
                   a_out=None, topk_id=None, topk_logit=None, lse=None):
        R = batch * rows_per_seq
        dev = src.device
        K = self.shape.topk
        a_out = a_out if a_out is not None else torch.empty(
            R, self.shape.hidden, dtype=torch.float32, device=dev)
        topk_id = topk_id if topk_id is not None else torch.full(
            (R, K), -1, dtype=torch.int32, device=dev)
        topk_logit = topk_logit if topk_logit is not None else torch.full(
            (R, K), float("nan"), dtype=torch.float32, device=dev)
        lse = lse if lse is not None else torch.full(
            (R,), float("nan"), dtype=torch.float32, device=dev)
        ckv = kv.c_kv(None, None)
        check(lib().eagle_draft_step(
            self._ctx, batch, rows_per_seq, _ptr(src), _ptr(token),
            _ptr(position), _ptr(dest), _ptr(prefix_len), _ptr(scratch_base),
            _ptr(scratch_mask), ctypes.byref(ckv), _ptr(a_out), _ptr(topk_id),
            _ptr(topk_logit), _ptr(lse), _stream()), "eagle_draft_step")
        return a_out, topk_id, topk_logit, lse

    def alloc_tree(self, batch, device="cuda"):
        N1 = self.shape.budget + 1
        W = (N1 + 63) // 64
        i32 = dict(dtype=torch.int32, device=device)
        t = {n: torch.empty(batch, N1, **i32) for n in (
            "token", "parent", "depth", "position", "kv_slot", "first_child",
            "n_child")}
        t["score"] = torch.empty(batch, N1, dtype=torch.float32, device=device)
        t["mask"] = torch.empty(batch, N1, W, dtype=torch.int64, device=device)
        t["n_nodes"] = torch.empty(batch, **i32)
        return t

    @staticmethod
    def _c_tree(t) -> _lib.Tree:
        return _lib.Tree(*[t[n].data_ptr() for n in (
            "token", "parent", "depth", "position", "kv_slot", "first_child",
            "n_child", "score", "mask", "n_nodes")])

    def draft_tree(self, seed_src, seed_token, seed_len, kv: KVCache,
                   len_out=None, tree=None):
        """seed_src [B, max_seed, H] float32; seed_token [B, max_seed];
        seed_len [B].  Returns (tree dict, len_out [B])."""
        B = seed_src.shape[0]
        tree = tree if tree is not None else self.alloc_tree(B, seed_src.device)
        len_out = len_out if len_out is not None else torch.empty(
            B, dtype=torch.int32, device=seed_src.device)
        ckv = kv.c_kv(kv.length, len_out)
        ct = self._c_tree(tree)
        check(lib().eagle_draft_tree(self._ctx, B, _ptr(seed_src),
                                     _ptr(seed_token), _ptr(seed_len),
                                     ctypes.byref(ckv), ctypes.byref(ct),
                                     _stream()), "eagle_draft_tree")
        return tree, len_out

    def draft_tree_sampled(self, seed_src, seed_token, seed_len, kv: KVCache,
                           temperature, seed, round=0, len_out=None, tree=None,
                           draft_logits=None):
        """draft_tree with K children sampled (without replacement) at every
        expanded node.  Returns (tree, len_out, draft_logits [B, 1 + (D-1)K,
        V] fp32)."""
        B = seed_src.shape[0]
        sh = self.shape
        tree = tree if tree is not None else self.alloc_tree(B, seed_src.device)
        len_out = len_out if len_out is not None else torch.empty(
            B, dtype=torch.int32, device=seed_src.device)
        ne = 1 + max(sh.depth - 1, 0) * sh.topk
        if draft_logits is None:
            draft_logits = torch.zeros(B, ne, sh.vocab, dtype=torch.float32,
                                       device=seed_src.device)
        ckv = kv.c_kv(kv.length, len_out)
        ct = self._c_tree(tree)
        check(lib().eagle_draft_tree_sampled(
            self._ctx, B, _ptr(seed_src), _ptr(seed_token), _ptr(seed_len),
            ctypes.byref(ckv), ctypes.byref(ct), float(temperature), int(seed),
            int(round), _ptr(draft_logits), _stream()), "eagle_draft_tree_sampled")
        return tree, len_out, draft_logits

    def verify_sampled(self, tree, target_logits, draft_logits, temperature, seed=0,
                       round=0, kv: KVCache | None = None, kv_len_out=None,
                       commit_mode=_lib.COMMIT_KEEP):
        """verify() for trees from draft_tree_sampled."""
        B = tree["token"].shape[0]
        D, S = self.shape.depth, self.shape.max_seed
        i32 = dict(dtype=torch.int32, device=target_logits.device)
        out = {"accept_len": torch.empty(B, **i32),
               "accepted_rows": torch.empty(B, D, **i32),
               "tokens": torch.empty(B, D + 1, **i32),
               "seed_rows": torch.empty(B, S, **i32),
               "seed_tokens": torch.empty(B, S, **i32),
               "seed_len": torch.empty(B, **i32)}
        ckv = None
        if kv is not None:
            if kv_len_out is None:
                kv_len_out = torch.empty(B, **i32)
            out["kv_len"] = kv_len_out
            ckv = kv.c_kv(None, kv_len_out)
        ct = self._c_tree(tree)
        check(lib().eagle_verify_tree_sampled(
            self._ctx, B, ctypes.byref(ct), _ptr(target_logits), _ptr(draft_logits),
            float(temperature), int(seed), int(round), int(commit_mode),
            ctypes.byref(ckv) if ckv is not None else None,
            _ptr(out["accept_len"]), _ptr(out["accepted_rows"]), _ptr(out["tokens"]),
            _ptr(out["seed_rows"]), _ptr(out["seed_tokens"]), _ptr(out["seed_len"]),
            _stream()), "eagle_verify_tree_sampled")
        return out

    def verify(self, tree, target_logits, temperature=0.0, seed=0, round=0,
               kv: KVCache | None = None, kv_len_out=None, out=None,
               commit_mode=_lib.COMMIT_KEEP, uniforms=None):
        """Verify the trees; draws come from Philox(seed, round) unless
        explicit `uniforms` [B, N+1, K+1] are given."""
        B = tree["token"].shape[0]
        D = self.shape.depth
        S = self.shape.max_seed
        dev = target_logits.device
        i32 = dict(dtype=torch.int32, device=dev)
        if out is None:
            out = {"accept_len": torch.empty(B, **i32),
                   "accepted_rows": torch.empty(B, D, **i32),
                   "tokens": torch.empty(B, D + 1, **i32),
                   "seed_rows": torch.empty(B, S, **i32),
                   "seed_tokens": torch.empty(B, S, **i32),
                   "seed_len": torch.empty(B, **i32)}
        ckv = None
        if kv is not None:
            if kv_len_out is None:
                kv_len_out = torch.empty(B, **i32)
            out["kv_len"] = kv_len_out
            ckv = kv.c_kv(None, kv_len_out)
        ct = self._c_tree(tree)
        common = (_ptr(out["accept_len"]), _ptr(out["accepted_rows"]),
                  _ptr(out["tokens"]), _ptr(out["seed_rows"]),
                  _ptr(out["seed_tokens"]), _ptr(out["seed_len"]), _stream())
        kvp = ctypes.byref(ckv) if ckv is not None else None
        if uniforms is None:
            check(lib().eagle_verify_tree(
                self._ctx, B, ctypes.byref(ct), _ptr(target_logits),
                float(temperature), int(seed), int(round), int(commit_mode),
                kvp, *common), "eagle_verify_tree")
        else:
            check(lib().eagle_verify_tree_uniforms(
                self._ctx, B, ctypes.byref(ct), _ptr(target_logits),
                float(temperature), _ptr(uniforms), int(commit_mode), kvp,
                *common), "eagle_verify_tree_uniforms")
        return out


    def target_workspace_bytes(self, batch) -> int:
        n = lib().eagle_target_layer_workspace_bytes(ctypes.byref(self._cfg), int(batch))
        if n == 0:
            raise EagleError(2, "eagle_target_layer_workspace_bytes (shape rejected)")
        return int(n)

    def target_tree_layer(self, tree, kv: KVCache, logits=None, hidden=None,
                          workspace=None):
        """The target's one-pass forward over the flattened trees (this
        context's weights are the target layer's).  Returns (logits
        [B, N+1, V] fp32, hidden [B, N+1, H] fp32 or None)."""
        B = tree["token"].shape[0]
        N1 = self.shape.budget + 1
        dev = tree["token"].device
        if logits is None:
            logits = torch.empty(B, N1, self.shape.vocab, dtype=torch.float32, device=dev)
        if workspace is None:
            workspace = torch.empty(self.target_workspace_bytes(B), dtype=torch.uint8,
                                    device=dev)
        ckv = kv.c_kv(kv.length, None)
        ct = self._c_tree(tree)
        check(lib().eagle_target_tree_layer(
            self._ctx, B, ctypes.byref(ct), ctypes.byref(ckv), _ptr(workspace),
            workspace.numel(), None if hidden is None else _ptr(hidden), _ptr(logits),
            _stream()), "eagle_target_tree_layer")
        return logits, hidden


def draw_uniforms(seed, stream_id, round, batch, rows, draws, device="cuda"):
    """U[0,1) draws [batch, rows, draws] of the library's Philox generator."""
    out = torch.empty(batch, rows, draws, dtype=torch.float32, device=device)
    check(lib().eagle_draw_uniforms(int(seed), int(stream_id), int(round), batch,
                                    rows, draws, _ptr(out), _stream()),
          "eagle_draw_uniforms")
    return out
