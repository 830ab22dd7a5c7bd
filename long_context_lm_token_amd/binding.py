"""Thin ctypes binding of libttt.so (argument marshalling only).

The names follow the C ABI in include/ttt.h: ttt_model_create, ttt_prefill,
ttt_decode, ttt_get_weights, ttt_reset, ttt_model_destroy. torch is used only
to own device buffers and to name the stream. Loading raises if the built
library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libttt.so")

TTT_FP32, TTT_BF16 = 0, 1
TTT_GELU, TTT_SWIGLU = 0, 1
TTT_UP, TTT_GATE, TTT_DOWN = 0, 1, 2
PROF = {"gemm": 0, "attn_fwd": 1, "attn_bwd": 2, "ce": 3, "mlp_up": 4, "gemm_span": 5, "gemm_chunk": 6,
        "gemm_sgd": 7, "attn_dq": 8, "attn_dkdv": 9, "norm": 10, "other": 11, "all": 12}
PROF_NCLASS = 12

c_i32, c_i64, c_f32, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class TTTConfig(ctypes.Structure):
    _fields_ = [("vocab", c_i32), ("d_model", c_i32), ("n_blocks", c_i32), ("n_heads", c_i32),
                ("head_dim", c_i32), ("mlp_kind", c_i32), ("mlp_hidden", c_i32),
                ("n_ttt_blocks", c_i32), ("ttt_hidden", c_i32), ("static_hidden", c_i32),
                ("rope", c_i32), ("rope_theta", c_f32), ("norm_eps", c_f32), ("window", c_i32),
                ("mini_batch", c_i32), ("lr", c_f32), ("dtype", c_i32), ("batch", c_i32),
                ("max_positions", c_i64), ("prefill_span", c_i32), ("max_device_bytes", c_i64),
                ("forward_only", c_i32), ("mh_heads", c_i32)]


_PP = ctypes.POINTER(c_vp)


class TTTWeights(ctypes.Structure):
    _fields_ = [("embed", c_vp), ("final_norm", c_vp), ("lm_head", c_vp), ("attn_norm", _PP),
                ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP), ("mlp_norm", _PP),
                ("w_up", _PP), ("w_gate", _PP), ("w_down", _PP), ("s_up", _PP), ("s_gate", _PP),
                ("s_down", _PP)]


class TTTError(RuntimeError):
    pass


_lib = None


def load():
    """Load libttt.so (raises TTTError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise TTTError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    lib.ttt_model_create.argtypes = [ctypes.POINTER(TTTConfig), ctypes.POINTER(TTTWeights), c_vp,
                                     ctypes.POINTER(c_vp)]
    lib.ttt_prefill.argtypes = [c_vp, c_vp, c_i64, c_vp, c_vp]
    lib.ttt_decode.argtypes = [c_vp, c_i64, c_vp, c_vp, c_vp]
    lib.ttt_get_weights.argtypes = [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]
    lib.ttt_reset.argtypes = [c_vp, c_vp]
    lib.ttt_model_destroy.argtypes = [c_vp]
    lib.ttt_model_destroy.restype = None
    lib.ttt_last_error.restype = ctypes.c_char_p
    lib.ttt_k_last_error.restype = ctypes.c_char_p
    lib.ttt_stream_length.argtypes = [c_vp]
    lib.ttt_stream_length.restype = c_i64
    lib.ttt_device_bytes.argtypes = [c_vp]
    lib.ttt_device_bytes.restype = c_i64
    lib.ttt_device_bytes_by_part.argtypes = [c_vp, c_vp]
    lib.ttt_model_create_session.argtypes = [c_vp, c_i32, c_i64, c_i32, c_i64, c_vp, ctypes.POINTER(c_vp)]
    lib.ttt_prof_begin.argtypes = [c_vp, c_i32]
    lib.ttt_prof_sample.argtypes = [c_vp, c_i32]
    lib.ttt_prof_end.argtypes = [c_vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i64),
                                 ctypes.POINTER(ctypes.c_double)]
    lib.ttt_prof_end_classes.argtypes = [c_vp, c_i32, c_vp, c_vp, c_vp, c_vp]
    lib.ttt_k_gemm.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_i64, c_i64, c_vp, c_i64, c_i64,
                               c_vp, c_i64, c_i64, c_vp, c_i64, c_i64, c_vp, c_i64, c_i64, c_vp, c_i64, c_i64,
                               c_f32, ctypes.c_uint32, c_i32, c_vp, c_i64, c_vp]
    lib.ttt_k_qkv_rope.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp,
                                   c_vp, c_i32, c_vp]
    lib.ttt_k_gemm_tile.argtypes = [c_i32]
    lib.ttt_k_gemm_tile.restype = None
    lib.ttt_k_gemm_operands.argtypes = [c_i32]
    lib.ttt_k_gemm_operands.restype = None
    lib.ttt_k_attn_fwd.argtypes = [c_i32, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                   c_i64, c_i32, c_f32, c_i32, c_vp, c_vp]
    lib.ttt_k_attn_fwd_noalloc.argtypes = [c_i32, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32,
                                           c_i32, c_i64, c_i32, c_f32, c_i32, c_vp]
    lib.ttt_k_attn_bwd.argtypes = [c_i32, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32,
                                   c_i32, c_i32, c_i32, c_i64, c_i32, c_f32, c_i32, c_vp]
    lib.ttt_k_attn_fwd_kernel.argtypes = [c_i32]
    lib.ttt_k_attn_fwd_kernel.restype = None
    lib.ttt_k_attn_splits.argtypes = [c_i32, c_i32, c_i32, c_i64]
    lib.ttt_k_attn_delta.argtypes = [c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]
    lib.ttt_k_ce.argtypes = [c_i32, c_vp, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_f32, c_vp, c_vp, c_vp, c_vp]
    lib.ttt_k_rmsnorm_fwd.argtypes = [c_i32, c_vp, c_i32, c_i32, c_vp, c_f32, c_vp, c_vp, c_vp]
    lib.ttt_k_rmsnorm_bwd.argtypes = [c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp, c_i32, c_vp]
    _lib = lib
    return lib


def check(rc, kernel=False):
    if rc != 0:
        lib = load()
        msg = (lib.ttt_k_last_error() if kernel else lib.ttt_last_error()).decode()
        raise TTTError(f"TTT error {rc}: {msg}")


def stream_ptr(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return c_vp(s.cuda_stream)


def ptr(t):
    return c_vp(t.data_ptr()) if t is not None else c_vp(0)


def make_config(cfg: dict, batch=1, max_positions=None, prefill_span=0, max_device_bytes=0,
                forward_only=False) -> TTTConfig:
    mp = max_positions if max_positions is not None else cfg["seq_len"] + 1
    return TTTConfig(vocab=cfg["vocab"], d_model=cfg["d_model"], n_blocks=cfg["n_blocks"],
                     n_heads=cfg["n_heads"], head_dim=cfg["head_dim"],
                     mlp_kind=TTT_SWIGLU if cfg["mlp"] == "swiglu" else TTT_GELU,
                     mlp_hidden=cfg["mlp_hidden"], n_ttt_blocks=cfg["n_ttt_blocks"],
                     ttt_hidden=cfg["ttt_hidden"], static_hidden=cfg["static_hidden"],
                     rope=1 if cfg["rope"] else 0, rope_theta=cfg["rope_theta"],
                     norm_eps=cfg["norm_eps"], window=cfg["window"], mini_batch=cfg["mini_batch"],
                     lr=cfg["lr"], dtype=TTT_BF16 if cfg["dtype"] == "bf16" else TTT_FP32,
                     batch=batch, max_positions=mp, prefill_span=prefill_span,
                     max_device_bytes=max_device_bytes, forward_only=1 if forward_only else 0,
                     mh_heads=cfg.get("mh_heads", 0))


# ---------------------------------------------------------------------------
# C-ABI names
# ---------------------------------------------------------------------------

def ttt_model_create(cfg: TTTConfig, weights: dict, L: int, stream=None):
    """weights: name -> device tensor ([in][out]); returns (handle, keepalive)."""
    lib = load()
    arrays = {}

    def per_block(key):
        vals = [weights.get(f"{l}.{key}") for l in range(L)]
        if all(v is None for v in vals):
            return None
        arr = (c_vp * L)(*[v.data_ptr() if v is not None else 0 for v in vals])
        arrays[key] = arr
        return ctypes.cast(arr, _PP)

    w = TTTWeights(embed=weights["embed"].data_ptr(), final_norm=weights["final_norm"].data_ptr(),
                   lm_head=weights["lm_head"].data_ptr(), attn_norm=per_block("attn_norm"),
                   wq=per_block("wq"), wk=per_block("wk"), wv=per_block("wv"), wo=per_block("wo"),
                   mlp_norm=per_block("mlp_norm"), w_up=per_block("w_up"), w_gate=per_block("w_gate"),
                   w_down=per_block("w_down"), s_up=per_block("s_up"), s_gate=per_block("s_gate"),
                   s_down=per_block("s_down"))
    h = c_vp()
    check(lib.ttt_model_create(ctypes.byref(cfg), ctypes.byref(w), stream_ptr(stream), ctypes.byref(h)))
    return h, arrays


def ttt_model_create_session(base, batch, max_positions, prefill_span=0, max_device_bytes=0, stream=None):
    h = c_vp()
    check(load().ttt_model_create_session(base, batch, max_positions, prefill_span, max_device_bytes,
                                          stream_ptr(stream), ctypes.byref(h)))
    return h


def ttt_prefill(h, tokens, n, losses, stream=None):
    check(load().ttt_prefill(h, ptr(tokens), n, ptr(losses), stream_ptr(stream)))


def ttt_decode(h, n_new, tokens_out, losses, stream=None):
    check(load().ttt_decode(h, n_new, ptr(tokens_out), ptr(losses), stream_ptr(stream)))


def ttt_get_weights(h, seq, block, mat, dst, stream=None):
    check(load().ttt_get_weights(h, seq, block, mat, ptr(dst), stream_ptr(stream)))


def ttt_reset(h, stream=None):
    check(load().ttt_reset(h, stream_ptr(stream)))


def ttt_model_destroy(h):
    load().ttt_model_destroy(h)


# ---------------------------------------------------------------------------
# convenience wrapper
# ---------------------------------------------------------------------------

class TTTModel:
    """Owns one library model; tokens and losses are torch device tensors."""

    def __init__(self, cfg: dict, weights: dict, batch=1, max_positions=None, prefill_span=0,
                 max_device_bytes=0, stream=None, forward_only=False):
        self.cfg = cfg
        self.batch = batch
        self.c = make_config(cfg, batch, max_positions, prefill_span, max_device_bytes, forward_only)
        self.h, self._keep = ttt_model_create(self.c, weights, cfg["n_blocks"], stream)
        self.stream = stream

    def session(self, batch=1, max_positions=None, prefill_span=0, max_device_bytes=0, stream=None):
        """A new model sharing this one's frozen and initial fast weights
        (ttt_model_create_session), with its own sequences and state."""
        obj = TTTModel.__new__(TTTModel)
        obj.cfg = self.cfg
        obj.batch = batch
        obj.c = None
        obj._keep = None
        mp = max_positions if max_positions is not None else self.cfg["seq_len"] + 1
        obj.h = ttt_model_create_session(self.h, batch, mp, prefill_span, max_device_bytes, stream)
        obj.stream = stream
        return obj

    def bytes_by_part(self):
        """{shared, fast, cache, work}: device bytes by the terms of Eq. 13."""
        out = (c_i64 * 4)()
        check(load().ttt_device_bytes_by_part(self.h, out))
        return dict(zip(["shared", "fast", "cache", "work"], list(out)))

    def prefill(self, tokens: torch.Tensor, want_losses=True):
        tokens = tokens.to(torch.int32).contiguous()
        if tokens.dim() == 1:
            tokens = tokens[None]
        B, n = tokens.shape
        assert B == self.batch and tokens.is_cuda
        losses = torch.empty((B, n), dtype=torch.float32, device=tokens.device) if want_losses else None
        ttt_prefill(self.h, tokens, n, losses, self.stream)
        return losses

    def decode(self, n_new: int, want_losses=True):
        dev = torch.device("cuda")
        out = torch.empty((self.batch, n_new), dtype=torch.int32, device=dev)
        losses = torch.empty((self.batch, n_new), dtype=torch.float32, device=dev) if want_losses else None
        ttt_decode(self.h, n_new, out, losses, self.stream)
        return out, losses

    def get_weights(self, seq: int, block: int, mat: str):
        d, ht = self.cfg["d_model"], self.cfg["ttt_hidden"]
        code = {"w_up": TTT_UP, "w_gate": TTT_GATE, "w_down": TTT_DOWN}[mat]
        shape = (ht, d) if code == TTT_DOWN else (d, ht)
        nh = self.cfg.get("mh_heads", 0)
        if nh > 1:
            shape = (nh, ht // nh, d // nh) if code == TTT_DOWN else (nh, d // nh, ht // nh)
        dst = torch.empty(shape, dtype=torch.float32, device="cuda")
        ttt_get_weights(self.h, seq, block, code, dst, self.stream)
        return dst

    def reset(self):
        ttt_reset(self.h, self.stream)

    def stream_length(self):
        return load().ttt_stream_length(self.h)

    def device_bytes(self):
        return load().ttt_device_bytes(self.h)

    def prof_begin(self, cls: str, every: int = 1):
        """Time the launches of class `cls` (every `every`-th one)."""
        check(load().ttt_prof_begin(self.h, PROF[cls]))
        if every != 1:
            check(load().ttt_prof_sample(self.h, every))

    def prof_end(self):
        ms, n, work = ctypes.c_double(), c_i64(), ctypes.c_double()
        check(load().ttt_prof_end(self.h, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(work)))
        return ms.value, n.value, work.value

    def prof_end_classes(self):
        """Per-class (ms, launches, flops, bytes) dicts keyed by class name."""
        n = PROF_NCLASS
        ms, fl, by = (ctypes.c_double * n)(), (ctypes.c_double * n)(), (ctypes.c_double * n)()
        k = (c_i64 * n)()
        check(load().ttt_prof_end_classes(self.h, n, ms, k, fl, by))
        names = {v: kname for kname, v in PROF.items()}
        return {names[c]: dict(ms=ms[c], launches=k[c], flops=fl[c], bytes=by[c]) for c in range(n)}

    def close(self):
        if self.h:
            ttt_model_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
