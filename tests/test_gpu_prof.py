"""The library's launch timing (include/ttt_prof.h): events attached to the
kernels' own dispatches, every launch or every n-th one of a class, and no
effect on results."""
import math

import numpy as np
import pytest
import torch

from long_context_lm_token_amd import binding as bd, synth
from tests.gpu_util import dev_weights

pytestmark = pytest.mark.gpu


def _model(cfg, n):
    wd, _ = dev_weights(cfg, seed=0, std=0.05)
    return bd.TTTModel(cfg, wd, batch=1, max_positions=n + 8)


def _prefill(model, toks):
    model.reset()
    out = model.prefill(toks).cpu().numpy()
    torch.cuda.synchronize()
    return out


def test_timing_all_classes_sampled_and_results_unchanged():
    # bf16 with head dim 128: the direct-to-LDS products and attention kernels
    cfg = synth.get_config("tiny", vocab=512, d_model=256, n_blocks=4, n_heads=2, head_dim=128, mlp="swiglu",
                           mlp_hidden=512, n_ttt_blocks=2, ttt_hidden=256, static_hidden=256, rope=True,
                           window=128, mini_batch=64, lr=0.05, dtype="bf16", span=32, period=256)
    n = 4 * cfg["mini_batch"] + 5
    toks = torch.as_tensor(synth.make_batch(cfg, 1, n, seed=3)).cuda()
    model = _model(cfg, n)
    plain = _prefill(model, toks)

    model.prof_begin("all")
    timed = _prefill(model, toks)
    classes = model.prof_end_classes()
    np.testing.assert_array_equal(timed, plain)
    seen = {c: v for c, v in classes.items() if v["launches"] > 0}
    assert {"gemm_chunk", "gemm_sgd", "attn_fwd", "ce", "norm"} <= set(seen), sorted(seen)
    for c, v in seen.items():
        assert v["ms"] > 0, c
    n_chunk = seen["gemm_chunk"]["launches"]

    for every in (1, 3, 8):
        model.prof_begin("gemm_chunk", every=every)
        got = _prefill(model, toks)
        sub = model.prof_end_classes()
        np.testing.assert_array_equal(got, plain)
        assert sub["gemm_chunk"]["launches"] == math.ceil(n_chunk / every)
        assert sub["gemm_chunk"]["ms"] > 0
        assert sum(v["launches"] for c, v in sub.items() if c != "gemm_chunk") == 0
    model.close()
