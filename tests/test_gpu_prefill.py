"""End-to-end parity of ttt_prefill / ttt_decode / ttt_get_weights (through
the C ABI) with the CPU fp64 oracle on the same seeded inputs.

Tolerances: fp32 models - per-token loss within 1e-4 absolute, fast weights
within 1e-4 relative (Frobenius) and their change W - W_0 within 1e-3
relative; bf16 models - loss within 2e-2 absolute, final weights within 2e-2
relative Frobenius and the change within 5e-2 relative.
"""
import numpy as np
import pytest
import torch

from long_context_lm_token_amd import binding as bd, synth
from oracle import ttt_oracle as O
from tests.gpu_util import compare_weights, dev_weights

pytestmark = pytest.mark.gpu

FP32_TOL = dict(loss=1e-4, w=1e-4, dw=1e-3)
BF16_TOL = dict(loss=2e-2, w=2e-2, dw=5e-2)


def small_cfg(**kw):
    base = dict(vocab=64, d_model=64, n_blocks=4, n_heads=4, head_dim=16, mlp="swiglu", mlp_hidden=96,
                n_ttt_blocks=2, ttt_hidden=48, static_hidden=48, rope=True, window=48, mini_batch=16,
                lr=0.5, dtype="fp32", span=16, period=96)
    base.update(kw)
    return synth.get_config("tiny", **base)


def run_prefill(cfg, n_ids, batch=1, std=0.02, cuts=None, seed=0, span=0):
    wd, wn = dev_weights(cfg, seed=seed, std=std)
    toks = synth.make_batch(cfg, batch, n_ids, seed=seed + 1)
    model = bd.TTTModel(cfg, wd, batch=batch, max_positions=n_ids + 64, prefill_span=span)
    cuts = cuts or [0, n_ids]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        parts.append(model.prefill(torch.as_tensor(toks[:, a:b]).cuda()).cpu().numpy())
    torch.cuda.synchronize()
    g_loss = np.concatenate(parts, axis=1)
    o_loss, ors = O.prefill(cfg, wn, toks)
    return model, wn, g_loss, o_loss, ors, toks


def check_losses(g, o, tol):
    assert np.isnan(g[:, 0]).all()
    err = np.abs(g[:, 1:] - o[:, 1:]).max()
    assert err <= tol, err
    return err


def test_tiny_fp32_config():
    """The tiny fp32 workload as specified: 512 labelled positions, b=32, k=64."""
    cfg = synth.get_config("tiny")
    model, wn, g, o, ors, _ = run_prefill(cfg, cfg["seq_len"] + 1)
    check_losses(g, o, FP32_TOL["loss"])
    compare_weights(cfg, model, ors, wn, FP32_TOL["w"], FP32_TOL["dw"])
    model.close()


@pytest.mark.parametrize("mlp,rope", [("swiglu", True), ("gelu", False)])
def test_two_tail_blocks_fp32(mlp, rope):
    """Gradients cross a tail block's attention (dQ over the window, dK/dV in chunk)."""
    cfg = small_cfg(mlp=mlp, rope=rope)
    model, wn, g, o, ors, _ = run_prefill(cfg, 6 * 16 + 5, std=0.2)
    check_losses(g, o, FP32_TOL["loss"])
    compare_weights(cfg, model, ors, wn, FP32_TOL["w"], FP32_TOL["dw"])
    model.close()


def test_streaming_batch_and_reset_fp32():
    cfg = small_cfg()
    n = 7 * 16 + 3
    cuts = [0, 5, 33, 34, 80, n]
    model, wn, g, o, ors, toks = run_prefill(cfg, n, batch=3, std=0.2, cuts=cuts, span=24)
    check_losses(g, o, FP32_TOL["loss"])
    compare_weights(cfg, model, ors, wn, FP32_TOL["w"], FP32_TOL["dw"])
    assert model.stream_length() == n
    # reset, then the same calls reproduce the run bit for bit (deterministic kernels)
    model.reset()
    again = np.concatenate([model.prefill(torch.as_tensor(toks[:, a:b]).cuda()).cpu().numpy()
                            for a, b in zip(cuts[:-1], cuts[1:])], axis=1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(again[:, 1:], g[:, 1:])
    # and a one-shot prefill agrees with the streamed one (summation order may differ)
    model.reset()
    once = model.prefill(torch.as_tensor(toks).cuda()).cpu().numpy()
    torch.cuda.synchronize()
    np.testing.assert_allclose(once[:, 1:], g[:, 1:], rtol=0, atol=1e-5)
    model.close()


def test_decode_fp32_teacher_forced():
    """Decode = prefill of the stream it generates (updates after full chunks)."""
    cfg = small_cfg()
    wd, wn = dev_weights(cfg, std=0.2)
    prompt = synth.make_batch(cfg, 2, 41, seed=3)
    model = bd.TTTModel(cfg, wd, batch=2, max_positions=200)
    model.prefill(torch.as_tensor(prompt).cuda())
    n_new = 45
    gen, gl = model.decode(n_new)
    torch.cuda.synchronize()
    gen = gen.cpu().numpy()
    gl = gl.cpu().numpy()
    for s in range(2):
        orc = O.Oracle(cfg, wn)
        orc.prefill(prompt[s])
        lo = []
        for t in gen[s]:
            # the oracle's logits of the last position must rank the GPU's id first
            z = orc.last_logits
            assert z[t] >= z.max() - 1e-4
            lo.append(orc.prefill([int(t)])[0])
        np.testing.assert_allclose(gl[s], lo, atol=FP32_TOL["loss"], rtol=0)
        ors = [orc]
        compare_weights(cfg, model, [None] * s + ors, wn, FP32_TOL["w"], FP32_TOL["dw"], seqs=[s])
    model.close()


def test_bf16_small_model():
    """bf16 path (head dim 64, SwiGLU, RoPE) on a small model, several chunks."""
    cfg = small_cfg(dtype="bf16", vocab=512, d_model=256, n_heads=4, head_dim=64, mlp_hidden=512,
                    ttt_hidden=256, static_hidden=256, n_blocks=4, n_ttt_blocks=2, window=128,
                    mini_batch=64, lr=0.05, span=32, period=256)
    model, wn, g, o, ors, _ = run_prefill(cfg, 5 * 64 + 9, std=0.05)
    check_losses(g, o, BF16_TOL["loss"])
    compare_weights(cfg, model, ors, wn, BF16_TOL["w"], BF16_TOL["dw"])
    model.close()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_products_split_over_k(dtype):
    """Every product that may split over K split in two (the GEMM test hook):
    the chunk loop's norms then take the partial sums of the products that
    feed them (head dX, MLP and QKV input gradients into the norm backward;
    the down projection and its residual into the next norm forward) in place
    of the reduce kernel. Two tail blocks, several chunks, against the oracle
    at the unsplit runs' bounds."""
    lib = bd.load()
    if dtype == "fp32":
        cfg, n, std, tol = small_cfg(), 6 * 16 + 5, 0.2, FP32_TOL
    else:
        cfg = small_cfg(dtype="bf16", vocab=512, d_model=256, n_heads=4, head_dim=64, mlp_hidden=512,
                        ttt_hidden=256, static_hidden=256, n_blocks=4, n_ttt_blocks=2, window=128,
                        mini_batch=64, lr=0.05, span=32, period=256)
        n, std, tol = 5 * 64 + 9, 0.05, BF16_TOL
    lib.ttt_k_gemm_tile(2 << 8)  # automatic tiles, two K splits
    try:
        model, wn, g, o, ors, _ = run_prefill(cfg, n, std=std)
    finally:
        lib.ttt_k_gemm_tile(0)
    check_losses(g, o, tol["loss"])
    compare_weights(cfg, model, ors, wn, tol["w"], tol["dw"])
    model.close()


def test_bf16_two_sequences_head_dim_128():
    """bf16 with head dim 128 (the direct-to-LDS attention kernels) and two
    sequences (per-sequence strides of every product, incl. the weight
    gradients read MN-major), several chunks, against the oracle."""
    cfg = small_cfg(dtype="bf16", vocab=512, d_model=256, n_heads=2, head_dim=128, mlp_hidden=512,
                    ttt_hidden=256, static_hidden=256, n_blocks=4, n_ttt_blocks=2, window=128,
                    mini_batch=64, lr=0.05, span=32, period=256)
    model, wn, g, o, ors, _ = run_prefill(cfg, 4 * 64 + 5, batch=2, std=0.05)
    check_losses(g, o, BF16_TOL["loss"])
    compare_weights(cfg, model, ors, wn, BF16_TOL["w"], BF16_TOL["dw"])
    model.close()


def test_decode_bf16_head_dim_128():
    """bf16 decode with head dim 128 (one-row Q/K/V products with the rotary
    epilogue, one-query attention), across a chunk boundary, against the
    oracle fed the generated ids."""
    cfg = small_cfg(dtype="bf16", vocab=512, d_model=256, n_heads=2, head_dim=128, mlp_hidden=512,
                    ttt_hidden=256, static_hidden=256, n_blocks=4, n_ttt_blocks=2, window=128,
                    mini_batch=64, lr=0.05, span=32, period=256)
    wd, wn = dev_weights(cfg, std=0.05)
    prompt = synth.make_batch(cfg, 2, 41, seed=3)
    model = bd.TTTModel(cfg, wd, batch=2, max_positions=200)
    model.prefill(torch.as_tensor(prompt).cuda())
    gen, gl = model.decode(45)
    torch.cuda.synchronize()
    gen = gen.cpu().numpy()
    gl = gl.cpu().numpy()
    for s in range(2):
        orc = O.Oracle(cfg, wn)
        orc.prefill(prompt[s])
        lo = []
        for t in gen[s]:
            z = orc.last_logits
            assert z[t] >= z.max() - 5e-2     # the GPU's id is (within bf16 noise) the oracle's argmax
            lo.append(orc.prefill([int(t)])[0])
        np.testing.assert_allclose(gl[s], lo, atol=BF16_TOL["loss"], rtol=0)
    model.close()


def test_forward_only_is_the_static_model():
    """forward_only: every position scored at W_init in one causal pass (the
    oracle's static losses; with a window as long as the stream, full causal
    attention), and the fast weights never move."""
    cfg = small_cfg(window=128, mini_batch=32, span=16, period=64)
    n = 3 * 32 + 7
    wd, wn = dev_weights(cfg, std=0.2)
    toks = synth.make_batch(cfg, 2, n, seed=4)
    model = bd.TTTModel(cfg, wd, batch=2, max_positions=n + 8, forward_only=True)
    g = model.prefill(torch.as_tensor(toks).cuda()).cpu().numpy()
    torch.cuda.synchronize()
    for s in range(2):
        ref = O.Oracle(cfg, wn).static_losses(toks[s])
        np.testing.assert_allclose(g[s, 1:], ref, rtol=0, atol=FP32_TOL["loss"])
        t0 = cfg["n_blocks"] - cfg["n_ttt_blocks"]
        for l in range(t0, cfg["n_blocks"]):
            for name in ("w_up", "w_gate", "w_down"):
                got = model.get_weights(s, l, name).cpu().numpy()
                np.testing.assert_array_equal(got, wn[f"{l}.{name}"])
    model.close()


@pytest.mark.parametrize("cuts", [None, [0, 37, 38, 150, 301]])
def test_frozen_ring_wraps_over_many_spans_fp32(cuts):
    """Frozen-prefix passes of 16 positions (about 19 of them, the prefix
    stream running at most two ahead of the chunk loop) over a frozen-block
    K/V ring of 64 slots (window 48 + span 16), which wraps four times; the
    tail ring (48 + 16 -> 64 slots) wraps too. Whole stream and uneven pieces."""
    cfg = small_cfg()
    n = 301
    model, wn, g, o, ors, _ = run_prefill(cfg, n, std=0.2, span=16, cuts=cuts)
    check_losses(g, o, FP32_TOL["loss"])
    compare_weights(cfg, model, ors, wn, FP32_TOL["w"], FP32_TOL["dw"])
    model.close()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_window_equal_to_chunk(dtype):
    """k = b, the smallest window the method allows: the first query of a
    chunk sees one key, the last sees b."""
    kw = dict(window=16, mini_batch=16)
    if dtype == "bf16":
        kw.update(dtype="bf16", vocab=512, d_model=256, n_heads=2, head_dim=128, mlp_hidden=512,
                  ttt_hidden=256, static_hidden=256, window=64, mini_batch=64, lr=0.05, span=32, period=256)
    cfg = small_cfg(**kw)
    b = cfg["mini_batch"]
    model, wn, g, o, ors, _ = run_prefill(cfg, 5 * b + 3, std=0.2 if dtype == "fp32" else 0.05, span=b)
    tol = FP32_TOL if dtype == "fp32" else BF16_TOL
    check_losses(g, o, tol["loss"])
    compare_weights(cfg, model, ors, wn, tol["w"], tol["dw"])
    model.close()


@pytest.mark.parametrize("hd", [64, 128])
def test_bf16_chunk_not_a_multiple_of_64(hd):
    """bf16 with b = 40: the weight-gradient products cannot read the
    activations MN-major (b not a multiple of 64), so they take
    token-contiguous transposed copies; ragged chunk-sized tiles everywhere."""
    cfg = small_cfg(dtype="bf16", vocab=512, d_model=256, n_heads=256 // hd, head_dim=hd, mlp_hidden=512,
                    ttt_hidden=256, static_hidden=256, n_blocks=4, n_ttt_blocks=2, window=80,
                    mini_batch=40, lr=0.05, span=32, period=160)
    model, wn, g, o, ors, _ = run_prefill(cfg, 6 * 40 + 7, batch=2, std=0.05, span=64)
    check_losses(g, o, BF16_TOL["loss"])
    compare_weights(cfg, model, ors, wn, BF16_TOL["w"], BF16_TOL["dw"])
    model.close()
