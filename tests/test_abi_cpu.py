"""CPU-side checks of the C ABI: the library loads and exports every symbol
that include/*.h declares; host-side argument validation (no GPU work)."""
import ctypes
import glob
import os
import re

import pytest

from long_context_lm_token_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(ttt_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


def test_headers_declare_the_boundary():
    names = declared_functions()
    for n in ["ttt_model_create", "ttt_prefill", "ttt_decode", "ttt_get_weights", "ttt_reset",
              "ttt_model_destroy", "ttt_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(bd.LIB_PATH):
        pytest.skip("library not built")
    lib = ctypes.CDLL(bd.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_config_validation_errors_without_gpu():
    """Invalid configurations are rejected before any device call."""
    if not os.path.exists(bd.LIB_PATH):
        pytest.skip("library not built")
    from long_context_lm_token_amd import synth
    lib = bd.load()
    cfg = synth.get_config("tiny")
    c = bd.make_config(cfg)
    c.window = c.mini_batch - 1          # k < b is not allowed
    h = ctypes.c_void_p()
    w = bd.TTTWeights()
    rc = lib.ttt_model_create(ctypes.byref(c), ctypes.byref(w), None, ctypes.byref(h))
    assert rc == -1 and b"window" in lib.ttt_last_error()
    c = bd.make_config(cfg)
    c.head_dim = 24
    assert lib.ttt_model_create(ctypes.byref(c), ctypes.byref(w), None, ctypes.byref(h)) == -1
    c = bd.make_config(cfg)
    rc = lib.ttt_model_create(ctypes.byref(c), ctypes.byref(w), None, ctypes.byref(h))
    assert rc == -1 and b"NULL" in lib.ttt_last_error()
    assert not h.value
    assert lib.ttt_prefill(None, None, 1, None, None) == -1
    assert lib.ttt_decode(None, 1, None, None, None) == -1


def test_mini_batch_alignment_rejected_at_create():
    """A chunk size the weight-gradient products cannot contract over (K = b:
    a multiple of 8 for bf16, of 4 for fp32) is rejected before any device
    work, not at the first complete chunk."""
    if not os.path.exists(bd.LIB_PATH):
        pytest.skip("library not built")
    from long_context_lm_token_amd import synth
    lib = bd.load()
    w = bd.TTTWeights()
    h = ctypes.c_void_p()
    for dtype, b in [("bf16", 12), ("bf16", 1), ("fp32", 6), ("fp32", 1)]:
        cfg = synth.get_config("tiny", dtype=dtype, mini_batch=b, window=64)
        c = bd.make_config(cfg)
        rc = lib.ttt_model_create(ctypes.byref(c), ctypes.byref(w), None, ctypes.byref(h))
        assert rc == -1 and b"mini_batch" in lib.ttt_last_error(), (dtype, b, lib.ttt_last_error())
        assert not h.value
    # aligned sizes pass this check and fail later, on the NULL weights
    for dtype, b in [("bf16", 40), ("fp32", 4)]:
        c = bd.make_config(synth.get_config("tiny", dtype=dtype, mini_batch=b, window=64))
        assert lib.ttt_model_create(ctypes.byref(c), ctypes.byref(w), None, ctypes.byref(h)) == -1
        assert b"NULL" in lib.ttt_last_error()


def test_noalloc_attention_rejects_oversize_before_any_device_call():
    """The allocation-free attention forward checks its split partials
    against the static scratch (16 Mi floats) on the host."""
    if not os.path.exists(bd.LIB_PATH):
        pytest.skip("library not built")
    lib = bd.load()
    rc = lib.ttt_k_attn_fwd_noalloc(1, None, None, None, 9216, None, None, 2, 1024, 24, 128, 8192, 8192, 0.1, 4,
                                    None)
    assert rc == -1 and b"static scratch" in lib.ttt_k_last_error()
    assert b"25559040" in lib.ttt_k_last_error()          # 4 splits * 2 * 1024 rows * (3072 + 48)
    rc = lib.ttt_k_attn_fwd_noalloc(1, None, None, None, 9216, None, None, 1, 1024, 24, 128, 8192, 8192, 0.1, 17,
                                    None)
    assert rc == -1 and b"nsplit" in lib.ttt_k_last_error()


def test_prof_sample_rejects_bad_arguments_without_gpu():
    """Launch-timing selection is validated on the host."""
    if not os.path.exists(bd.LIB_PATH):
        pytest.skip("library not built")
    lib = bd.load()
    assert lib.ttt_prof_sample(None, 4) == -1 and b"NULL" in lib.ttt_last_error()
    assert lib.ttt_prof_begin(None, 6) == -1
