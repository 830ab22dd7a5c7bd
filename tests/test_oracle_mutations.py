"""Planted mistakes in the oracle (on the CPU) must be caught by the pins.

Each case patches one plausible error into the oracle - a dropped term, a
wrong sign, a shifted window edge, a transposed operand - and checks that the
finite-difference or autograd pins then fail.
"""
import numpy as np
import pytest

from oracle import ttt_oracle as O
from tests import test_oracle_pins as pins


def _fd_gap(cfg):
    b = cfg["mini_batch"]
    w, ids = pins.setup(cfg, 2 * b + 1)
    orc = O.Oracle(cfg, w)
    orc.prefill(ids[: b + 1])
    orc.ids = [int(t) for t in ids]
    _, G, _ = orc.chunk_objective(1)
    rng = np.random.default_rng(1)
    D = {k: rng.standard_normal(v.shape) for k, v in orc.W.items()}

    def A(t):
        loss, _, _ = orc.chunk_objective(1, W={k: orc.W[k] + t * D[k] for k in orc.W})
        return loss.mean()
    fd = (A(1e-5) - A(-1e-5)) / 2e-5
    an = sum(np.sum(G[k] * D[k]) for k in G)
    return abs(fd - an) / abs(an)


def test_unpatched_gap_is_small():
    assert _fd_gap(pins.small_cfg()) < 1e-6


@pytest.mark.parametrize("mutation", ["norm_term", "rope_sign", "attn_transpose", "swiglu_term"])
def test_planted_backward_mistakes_fail_fd(monkeypatch, mutation):
    if mutation == "norm_term":
        monkeypatch.setattr(O, "rmsnorm_bwd", lambda x, g, r, dy: r * g * dy)
    elif mutation == "rope_sign":
        monkeypatch.setattr(O, "rope_inv", O.rope)
    elif mutation == "attn_transpose":
        orig = O.window_attention_bwd

        def bad(q, K, V, P, do):
            dq, dK, dV = orig(q, K, V, P, do)
            return dq, dV, dK
        monkeypatch.setattr(O, "window_attention_bwd", bad)
    elif mutation == "swiglu_term":
        orig_sig = O.sigmoid
        monkeypatch.setattr(O, "sigmoid", lambda x: orig_sig(x) * (1 + 1e-3))
    assert _fd_gap(pins.small_cfg()) > 1e-4


def test_planted_window_edge_fails_count(monkeypatch):
    def bad(qpos, kpos, window):
        qp = np.asarray(qpos)[:, None]
        kp = np.asarray(kpos)[None, :]
        return (kp <= qp) & (kp >= qp - window)
    monkeypatch.setattr(O, "window_mask", bad)
    with pytest.raises(AssertionError):
        pins.test_p9_visible_pairs_eq1()
