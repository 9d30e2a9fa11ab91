"""The C ABI library loads, exports every symbol include/eagle.h declares,
and rejects bad host arguments before touching a GPU (no GPU needed)."""
import ctypes
import os
import re

import pytest

from eagle_draft_tree_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eagle.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(eagle_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared()
    for want in ("eagle_fuse_features", "eagle_draft_tree", "eagle_verify_tree",
                 "eagle_draft_step", "eagle_create", "eagle_destroy",
                 "eagle_workspace_bytes", "eagle_status_str",
                 "eagle_get_device_status", "eagle_verify_tree_uniforms",
                 "eagle_draw_uniforms"):
        assert want in names
    assert set(names) == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for n in declared():
        assert hasattr(L, n), n


def _cfg(**kw):
    base = dict(hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn=688,
                vocab=4096, dtype=1, rope_theta=10000.0, rms_eps=1e-5, depth=3,
                topk=4, budget=10, max_batch=1, max_seed=2, target_vocab=0)
    base.update(kw)
    return _lib.Config(**base)


def test_workspace_bytes_and_config_validation():
    L = _lib.lib()
    ok = L.eagle_workspace_bytes(ctypes.byref(_cfg()))
    assert ok > 0 and ok % 256 == 0
    for bad in (dict(head_dim=96), dict(topk=0), dict(topk=17),
                dict(depth=10, topk=10), dict(budget=200), dict(dtype=7),
                dict(n_kv_heads=3), dict(max_batch=0), dict(hidden=100),
                dict(dtype=1, max_batch=64, topk=10, head_dim=64),
                dict(max_seed=17), dict(target_vocab=100), dict(target_vocab=-1),
                dict(max_seed=16, n_q_heads=16, n_kv_heads=1)):
        assert L.eagle_workspace_bytes(ctypes.byref(_cfg(**bad))) == 0, bad
    # larger batch needs more workspace
    small = L.eagle_workspace_bytes(ctypes.byref(_cfg(dtype=0, max_batch=1)))
    big = L.eagle_workspace_bytes(ctypes.byref(_cfg(dtype=0, max_batch=8)))
    assert big > small > 0


def test_null_arguments_rejected_on_host():
    L = _lib.lib()
    ctx = ctypes.c_void_p()
    w = _lib.Weights()
    assert L.eagle_create(ctypes.byref(_cfg()), ctypes.byref(w), None, 0, None,
                          ctypes.byref(ctx)) == 1
    assert L.eagle_fuse_features(None, 1, None, None, None, None, None) == 1
    assert L.eagle_draft_tree(None, 1, None, None, None, None, None, None) == 1
    assert L.eagle_verify_tree(None, 1, None, None, 0.0, 0, 0, 0, None, None,
                               None, None, None, None, None, None) == 1
    assert L.eagle_verify_tree_uniforms(None, 1, None, None, 1.0, None, 0, None,
                                        None, None, None, None, None, None,
                                        None) == 1
    # draw sizes are checked before anything is enqueued
    assert L.eagle_draw_uniforms(1, 0, 0, -1, 4, 4, None, None) == 1
    assert L.eagle_draw_uniforms(1, 0, 0, 70000, 4, 4, None, None) == 1
    assert L.eagle_draw_uniforms(1, 0, 0, 0, 4, 4, None, None) == 0
    assert L.eagle_draw_uniforms(1, 0, 0, 2, 4, 4, None, None) == 1
    st = ctypes.c_int32()
    assert L.eagle_get_device_status(None, ctypes.byref(st), None) == 1
    assert L.eagle_status_str(4) == b"draft KV cache capacity exceeded"
