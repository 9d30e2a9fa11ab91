"""ctypes view of libeagle.so (include/eagle.h).  Marshalling only."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libeagle.so")

EAGLE_OK = 0
STATUS_NAMES = {0: "ok", 1: "invalid argument", 2: "unsupported shape",
                3: "HIP launch or copy failed", 4: "KV capacity exceeded",
                5: "non-finite target logits", 6: "workspace too small"}
EXPORTS = ("eagle_workspace_bytes", "eagle_create", "eagle_destroy",
           "eagle_status_str", "eagle_get_device_status", "eagle_fuse_features",
           "eagle_draft_step", "eagle_draft_tree", "eagle_verify_tree",
           "eagle_verify_tree_uniforms", "eagle_verify_tree_noalloc",
           "eagle_draw_uniforms", "eagle_target_layer_workspace_bytes",
           "eagle_draft_tree_sampled", "eagle_verify_tree_sampled",
           "eagle_target_tree_layer",
           "eagle_profile", "eagle_profile_read")
COMMIT_KEEP, COMMIT_RESEED = 0, 1
STREAM_VERIFY, STREAM_DRAFT = 0, 1
PROFILE_CLASSES = ("gemm", "fuse", "attention", "merge", "tree", "verify")

c_int32_p = ctypes.c_void_p
vp = ctypes.c_void_p


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("depth", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("budget", ctypes.c_int32),
                ("max_batch", ctypes.c_int32), ("max_seed", ctypes.c_int32),
                ("target_vocab", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, vp) for n in (
        "w_fuse", "w_in", "embed", "wq", "wk", "wv", "wo", "w_gate", "w_up",
        "w_down", "w_lm", "g_attn", "g_mlp", "g_final", "d2t")]


class KV(ctypes.Structure):
    _fields_ = [("k", vp), ("v", vp), ("cap", ctypes.c_int32),
                ("len_in", vp), ("len_out", vp)]


class Tree(ctypes.Structure):
    _fields_ = [(n, vp) for n in (
        "token", "parent", "depth", "position", "kv_slot", "first_child",
        "n_child", "score", "mask", "n_nodes")]


class EagleError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(code, code)} ({code})")
        self.code = code


_lib = None


def lib():
    """Load libeagle.so; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m eagle_draft_tree_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.eagle_workspace_bytes.restype = ctypes.c_size_t
    L.eagle_workspace_bytes.argtypes = [ctypes.POINTER(Config)]
    L.eagle_create.restype = ctypes.c_int
    L.eagle_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights),
                               vp, ctypes.c_size_t, vp,
                               ctypes.POINTER(ctypes.c_void_p)]
    L.eagle_destroy.restype = None
    L.eagle_destroy.argtypes = [vp]
    L.eagle_status_str.restype = ctypes.c_char_p
    L.eagle_status_str.argtypes = [ctypes.c_int]
    L.eagle_get_device_status.restype = ctypes.c_int
    L.eagle_get_device_status.argtypes = [vp, ctypes.POINTER(ctypes.c_int32), vp]
    L.eagle_fuse_features.restype = ctypes.c_int
    L.eagle_fuse_features.argtypes = [vp, ctypes.c_int32, vp, vp, vp, vp, vp]
    L.eagle_draft_step.restype = ctypes.c_int
    L.eagle_draft_step.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp, vp,
                                   vp, vp, vp, vp, vp, ctypes.POINTER(KV), vp,
                                   vp, vp, vp, vp]
    L.eagle_draft_tree.restype = ctypes.c_int
    L.eagle_draft_tree.argtypes = [vp, ctypes.c_int32, vp, vp, vp,
                                   ctypes.POINTER(KV), ctypes.POINTER(Tree), vp]
    L.eagle_verify_tree.restype = ctypes.c_int
    L.eagle_verify_tree.argtypes = [vp, ctypes.c_int32, ctypes.POINTER(Tree),
                                    vp, ctypes.c_float, ctypes.c_uint64,
                                    ctypes.c_uint64, ctypes.c_int32,
                                    ctypes.POINTER(KV), vp, vp, vp, vp, vp, vp,
                                    vp]
    L.eagle_verify_tree_uniforms.restype = ctypes.c_int
    L.eagle_verify_tree_uniforms.argtypes = [
        vp, ctypes.c_int32, ctypes.POINTER(Tree), vp, ctypes.c_float, vp,
        ctypes.c_int32, ctypes.POINTER(KV), vp, vp, vp, vp, vp, vp, vp]
    L.eagle_verify_tree_noalloc.restype = ctypes.c_int
    L.eagle_verify_tree_noalloc.argtypes = [
        ctypes.POINTER(Config), ctypes.c_int32, ctypes.POINTER(Tree), vp,
        ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int32,
        ctypes.POINTER(KV), vp, vp, vp, vp, vp, vp, vp]
    L.eagle_draw_uniforms.restype = ctypes.c_int
    L.eagle_draw_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_uint64,
                                      ctypes.c_uint64, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, vp, vp]
    L.eagle_draft_tree_sampled.restype = ctypes.c_int
    L.eagle_draft_tree_sampled.argtypes = [vp, ctypes.c_int32, vp, vp, vp, ctypes.POINTER(KV),
                                           ctypes.POINTER(Tree), ctypes.c_float,
                                           ctypes.c_uint64, ctypes.c_uint64, vp, vp]
    L.eagle_verify_tree_sampled.restype = ctypes.c_int
    L.eagle_verify_tree_sampled.argtypes = [vp, ctypes.c_int32, ctypes.POINTER(Tree), vp, vp,
                                            ctypes.c_float, ctypes.c_uint64, ctypes.c_uint64,
                                            ctypes.c_int32, ctypes.POINTER(KV), vp, vp, vp,
                                            vp, vp, vp, vp]
    L.eagle_target_layer_workspace_bytes.restype = ctypes.c_size_t
    L.eagle_target_layer_workspace_bytes.argtypes = [ctypes.POINTER(Config), ctypes.c_int32]
    L.eagle_target_tree_layer.restype = ctypes.c_int
    L.eagle_target_tree_layer.argtypes = [vp, ctypes.c_int32, ctypes.POINTER(Tree),
                                          ctypes.POINTER(KV), vp, ctypes.c_size_t, vp, vp, vp]
    L.eagle_profile.restype = ctypes.c_int
    L.eagle_profile.argtypes = [vp, ctypes.c_int32]
    L.eagle_profile_read.restype = ctypes.c_int
    L.eagle_profile_read.argtypes = [vp, ctypes.c_int32, vp, vp, vp, vp]
    _lib = L
    return L


def check(code: int, where: str):
    if code != EAGLE_OK:
        raise EagleError(code, where)
