"""Seeded synthetic inputs: model configurations, random-init weights, Zipf tokens.

This module holds no arithmetic of the method itself. It only produces inputs
(shapes, hyper-parameters, N(0, 0.02) weights and token streams) that are
handed, identically, to the CPU oracle and to the HIP library.

Model shapes and hyper-parameters are the workloads named for the TTT-E2E
method ("End-to-End Test-Time Training for Long Context"); see the technical
review "TTT-E2E: Learning a Long Context into Weights", section 5 (8K window,
1K chunks) and section 6 (MLPs of the last quarter of the blocks are the fast
weights; each of those blocks also has a static MLP branch).

Token recipe: ids are drawn i.i.d. from a Zipf(1.1) law over the vocabulary
(rank r in 1..V with P(r) proportional to r^-1.1, id = r - 1). One random span
of S ids is then written at every position j*P .. j*P+S-1, so that the stream
repeats itself at a distance P. P = 2*window (for the tiny config: 128), which
places the repeats just beyond the attention window: only the fast weights can
carry them across.
"""
from __future__ import annotations

import copy
import numpy as np
import torch

# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------

_BASE = dict(rope_theta=10000.0, norm_eps=1e-6)

CONFIGS = {
    # tiny fp32: vocab 256, d=64, 4 blocks, 4 heads x 16, GELU hidden 128;
    # last block: trainable MLP(h=64) + static MLP(h=64); no RoPE.
    "tiny": dict(_BASE, vocab=256, d_model=64, n_blocks=4, n_heads=4, head_dim=16,
                 mlp="gelu", mlp_hidden=128, n_ttt_blocks=1, ttt_hidden=64,
                 static_hidden=64, rope=False, window=64, mini_batch=32, lr=0.1,
                 dtype="fp32", seq_len=512, span=64, period=128),
    # 125M-shape bf16
    "125m": dict(_BASE, vocab=32000, d_model=768, n_blocks=12, n_heads=12, head_dim=64,
                 mlp="gelu", mlp_hidden=3072, n_ttt_blocks=3, ttt_hidden=1536,
                 static_hidden=1536, rope=True, window=1024, mini_batch=512, lr=0.01,
                 dtype="bf16", seq_len=8192, span=256, period=2048),
    # 1B-shape bf16
    "1b": dict(_BASE, vocab=32000, d_model=2048, n_blocks=24, n_heads=16, head_dim=128,
               mlp="swiglu", mlp_hidden=5632, n_ttt_blocks=6, ttt_hidden=2816,
               static_hidden=2816, rope=True, window=2048, mini_batch=1024, lr=0.01,
               dtype="bf16", seq_len=32768, span=512, period=4096),
    # "TTT-E2E all layers MH" at the 125M shape: every block has its regular
    # (static) GELU MLP of hidden 3072 beside a fast multi-head MLP of 12
    # heads, each mapping its 64 columns through a hidden of 64 (768 in all)
    "125m_mh": dict(_BASE, vocab=32000, d_model=768, n_blocks=12, n_heads=12, head_dim=64,
                    mlp="gelu", mlp_hidden=3072, n_ttt_blocks=12, ttt_hidden=768,
                    static_hidden=3072, mh_heads=12, rope=True, window=1024, mini_batch=512,
                    lr=0.01, dtype="bf16", seq_len=8192, span=256, period=2048),
    # 3B-shape bf16 prefill, 1 x 128K
    "3b": dict(_BASE, vocab=32000, d_model=3072, n_blocks=28, n_heads=24, head_dim=128,
               mlp="swiglu", mlp_hidden=8192, n_ttt_blocks=7, ttt_hidden=4096,
               static_hidden=4096, rope=True, window=8192, mini_batch=1024, lr=0.005,
               dtype="bf16", seq_len=131072, span=1024, period=16384),
}


def get_config(name: str, **overrides) -> dict:
    """Return a copy of a named configuration with optional overrides."""
    cfg = copy.deepcopy(CONFIGS[name])
    cfg.update(overrides)
    cfg["name"] = name
    return cfg


def tail_start(cfg: dict) -> int:
    """Index of the first block whose MLP is a fast weight."""
    return cfg["n_blocks"] - cfg["n_ttt_blocks"]


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

def weight_shapes(cfg: dict) -> dict:
    """Name -> shape, every matrix in [in][out] layout (y = x @ W)."""
    V, d, L = cfg["vocab"], cfg["d_model"], cfg["n_blocks"]
    hq = cfg["n_heads"] * cfg["head_dim"]
    t0 = tail_start(cfg)
    shapes = {"embed": (V, d), "final_norm": (d,), "lm_head": (d, V)}
    glu = cfg["mlp"] == "swiglu"
    for l in range(L):
        p = f"{l}."
        shapes[p + "attn_norm"] = (d,)
        shapes[p + "wq"] = (d, hq)
        shapes[p + "wk"] = (d, hq)
        shapes[p + "wv"] = (d, hq)
        shapes[p + "wo"] = (hq, d)
        shapes[p + "mlp_norm"] = (d,)
        h = cfg["ttt_hidden"] if l >= t0 else cfg["mlp_hidden"]
        nh = cfg.get("mh_heads", 0)
        if l >= t0 and nh > 1:
            # multi-head fast MLP: [head][in][out] per head
            dh, hh = d // nh, h // nh
            shapes[p + "w_up"] = (nh, dh, hh)
            if glu:
                shapes[p + "w_gate"] = (nh, dh, hh)
            shapes[p + "w_down"] = (nh, hh, dh)
        else:
            shapes[p + "w_up"] = (d, h)
            if glu:
                shapes[p + "w_gate"] = (d, h)
            shapes[p + "w_down"] = (h, d)
        if l >= t0:
            hs = cfg["static_hidden"]
            shapes[p + "s_up"] = (d, hs)
            if glu:
                shapes[p + "s_gate"] = (d, hs)
            shapes[p + "s_down"] = (hs, d)
    return shapes


def torch_dtype(cfg: dict):
    return torch.float32 if cfg["dtype"] == "fp32" else torch.bfloat16


def make_weights(cfg: dict, seed: int = 0, device="cpu", std: float = 0.02) -> dict:
    """i.i.d. N(0, std) matrices, unit norm gains, in the config's dtype.

    Each tensor has its own generator seeded from (seed, tensor index), so the
    values do not depend on which other tensors are generated. bf16 configs
    round the fp32 draws to bf16 (round to nearest even); both the oracle and
    the HIP library receive exactly these values.
    """
    dt = torch_dtype(cfg)
    out = {}
    for i, (name, shape) in enumerate(weight_shapes(cfg).items()):
        if len(shape) == 1:
            out[name] = torch.ones(shape, dtype=dt, device=device)
            continue
        g = torch.Generator(device=device)
        g.manual_seed(seed * 1000003 + i * 7919 + 12345)
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
        out[name] = t.to(dt)
    return out


def weights_to_numpy(w: dict) -> dict:
    """fp32 numpy copies (exact for bf16 values) for the oracle."""
    return {k: v.detach().float().cpu().numpy() for k, v in w.items()}


# --------------------------------------------------------------------------
# tokens
# --------------------------------------------------------------------------

def zipf_tokens(vocab: int, n: int, rng: np.random.Generator, s: float = 1.1) -> np.ndarray:
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    p = ranks ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def make_tokens(cfg: dict, n_ids: int, seq: int = 0, seed: int = 1,
                span: int | None = None, period: int | None = None) -> np.ndarray:
    """One stream of n_ids Zipf(1.1) ids with a repeated span (int32)."""
    rng = np.random.default_rng(seed * 100003 + seq)
    ids = zipf_tokens(cfg["vocab"], n_ids, rng)
    S = cfg["span"] if span is None else span
    P = cfg["period"] if period is None else period
    if S > 0 and P > 0:
        rep = zipf_tokens(cfg["vocab"], S, rng)
        for j0 in range(0, n_ids, P):
            m = min(S, n_ids - j0)
            ids[j0:j0 + m] = rep[:m]
    return ids


def make_batch(cfg: dict, batch: int, n_ids: int, seed: int = 1) -> np.ndarray:
    """[batch][n_ids] int32, sequence s seeded with (seed, s)."""
    return np.stack([make_tokens(cfg, n_ids, seq=s, seed=seed) for s in range(batch)])
