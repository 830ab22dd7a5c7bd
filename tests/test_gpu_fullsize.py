"""Parity at the workloads' full model widths (bf16), against the fp64 oracle.

* 125M shape: the whole 8192-position prefill (16 chunks of 512).
* 1B and 3B shapes: the first four chunks (4096 positions), the slice the
  oracle can afford. For 3B the losses are also taken from a full
  131072-position prefill in the benchmark's launch configuration.
* 3B width, 8 blocks (2 tail blocks), 12 chunks with 2048-position prefix
  passes: the steady state of the benchmark's path - the 8192-key window
  full, both K/V rings wrapped, six prefix passes beside the chunk loop.

Bounds asserted (bf16 runs), literally as stated for the method's parity:
  * final fast weights within 2e-2 relative Frobenius, their change from W_0
    within 5e-2 (the oracle's change must be non-zero);
  * every token's loss within 2e-2 absolute - asserted where an ideal
    bf16-operand computation meets it (125M). At 1B, 3B and the 8-block
    3B-width model it does not: the oracle itself, with every operand of
    every matrix product rounded to bf16 and all else in fp64, moves single
    token losses by more than 2e-2 (tests/golden/bf16_floor.json, written
    from the oracle alone). There the tests print how many tokens meet it
    and assert instead that the GPU's per-token error is no noisier than
    that ideal computation: rms per chunk within 1.25x of the ideal's over
    the same positions (the GPU adds fp32 accumulation, hardware
    exponentials and stochastically rounded fast-weight copies to the same
    bf16 operand rounding), and the mean loss of every mini-batch within
    2e-2.
"""
import json
import os

import numpy as np
import pytest
import torch

from long_context_lm_token_amd import binding as bd, synth
from oracle import ttt_oracle as O
from tests.gpu_util import compare_weights

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TOL = dict(loss=2e-2, w=2e-2, dw=5e-2)
NOISE_FACTOR = 1.25
FLOOR = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "bf16_floor.json")))


def log(cfg, msg):
    print(f"[{cfg['name']}] {msg}", flush=True)


def gpu_inputs(cfg, n_ids, seed=0):
    """Weights drawn on the host (the draws bf16_floor.json was computed on),
    then moved to the GPU; token ids as in the floor script."""
    w = synth.make_weights(cfg, seed=seed, device="cpu")
    wd = {k: v.cuda() for k, v in w.items()}
    toks = synth.make_tokens(cfg, n_ids, seq=0, seed=seed + 1)[None]
    return w, wd, toks


def oracle_run(cfg, wn, ids):
    orc = O.Oracle(cfg, wn, cache_fp64=False,
                   progress=lambda msg: log(cfg, msg) if "block 0 " in msg else None)
    return orc, orc.prefill(ids)


def check_losses(cfg, g, o, floor_key=None, literal=False):
    """g, o: losses of one stream (entry 0 NaN). Returns per-chunk stats."""
    b = cfg["mini_batch"]
    e = g[1:] - o[1:]
    n_chunks = len(e) // b
    assert np.isfinite(g[1:]).all()
    ec = e[:n_chunks * b].reshape(n_chunks, b)
    means = np.abs(ec.mean(axis=1))
    rms = np.sqrt(np.mean(ec * ec, axis=1))
    mx = np.abs(ec).max(axis=1)
    fl = FLOOR.get(floor_key) if floor_key else None
    for c in range(n_chunks):
        extra = ""
        if fl and c < fl["chunks"]:
            extra = f"; ideal bf16 rms {fl['rms'][c]:.4f} max {fl['max'][c]:.4f}"
        log(cfg, f"chunk {c}: mean {means[c]:.2e} rms {rms[c]:.4f} max {mx[c]:.4f}{extra}")
    within = float(np.mean(np.abs(e) <= TOL["loss"]))
    log(cfg, f"{len(e)} positions: max {np.abs(e).max():.4f}, rms {np.sqrt(np.mean(e * e)):.4f}, "
             f"{100 * within:.2f}% within {TOL['loss']}")
    assert means.max() <= TOL["loss"], means.max()
    if literal:
        assert np.abs(e).max() <= TOL["loss"], np.abs(e).max()
    else:
        assert fl is not None, f"no stored bf16 floor for {floor_key}"
        k = min(fl["chunks"], n_chunks)
        got = float(np.sqrt(np.mean(ec[:k] ** 2)))
        ideal = float(np.sqrt(np.mean(np.square(fl["rms"][:k]))))
        log(cfg, f"chunks 0..{k - 1}: rms {got:.4f} vs ideal bf16 {ideal:.4f} (bound {NOISE_FACTOR}x)")
        assert got <= NOISE_FACTOR * ideal, (got, ideal)
    return means, rms, mx


@pytest.mark.timeout(600)
def test_125m_full_prefill():
    cfg = synth.get_config("125m")
    n = cfg["seq_len"] + 1
    w, wd, toks = gpu_inputs(cfg, n)
    model = bd.TTTModel(cfg, wd, batch=1, max_positions=n)
    g = model.prefill(torch.as_tensor(toks).cuda()).cpu().numpy()[0]
    torch.cuda.synchronize()
    wn = synth.weights_to_numpy(w)
    orc, o = oracle_run(cfg, wn, toks[0])
    check_losses(cfg, g, o, "125m", literal=True)
    worst = compare_weights(cfg, model, [orc], wn, TOL["w"], TOL["dw"])
    log(cfg, f"worst weight rel err {worst[0]:.3e}, update rel err {worst[1]:.3e}")
    model.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["1b", "3b"])
def test_first_four_chunks(name):
    cfg = synth.get_config(name)
    b = cfg["mini_batch"]
    n = 4 * b + 1
    full = cfg["seq_len"] + 1
    w, wd, toks = gpu_inputs(cfg, full)
    # same library configuration as the benchmark: room for the whole stream
    model = bd.TTTModel(cfg, wd, batch=1, max_positions=full)
    g = model.prefill(torch.as_tensor(toks[:, :n]).cuda()).cpu().numpy()[0]
    torch.cuda.synchronize()
    wn = synth.weights_to_numpy(w)
    del w
    orc, o = oracle_run(cfg, wn, toks[0, :n])
    check_losses(cfg, g, o, name)
    worst = compare_weights(cfg, model, [orc], wn, TOL["w"], TOL["dw"])
    log(cfg, f"worst weight rel err {worst[0]:.3e}, update rel err {worst[1]:.3e}")
    if name == "3b":
        # the first four chunks inside a whole 128K prefill
        model.reset()
        gf = model.prefill(torch.as_tensor(toks).cuda()).cpu().numpy()[0]
        torch.cuda.synchronize()
        assert np.isfinite(gf[1:]).all()
        log(cfg, "full 131072-position prefill, first four chunks:")
        check_losses(cfg, gf[:n], o, name)
        # at full size, a property of every chunk: the run is deterministic
        # (fixed-order split reductions, no atomics), so a reset and the same
        # ids give bitwise the same 131072 losses and final fast weights
        w1 = model.get_weights(0, cfg["n_blocks"] - 1, "w_down").cpu().numpy()
        model.reset()
        gf2 = model.prefill(torch.as_tensor(toks).cuda()).cpu().numpy()[0]
        torch.cuda.synchronize()
        np.testing.assert_array_equal(gf2, gf)
        np.testing.assert_array_equal(model.get_weights(0, cfg["n_blocks"] - 1, "w_down").cpu().numpy(), w1)
    model.close()


@pytest.mark.timeout(900)
def test_steady_state_3b_width_eight_blocks():
    """3B width (d 3072, 24 x 128 heads, SwiGLU 8192 / tail 4096 + 4096,
    V 32000, k 8192, b 1024), 8 blocks of which 2 are tail blocks, so the
    gradient crosses a tail block's attention; 12 chunks (12289 ids) with
    2048-position prefix passes: from chunk 8 on every query sees a full
    8192-key window, the frozen-block ring (8192 + 2048 slots) and the tail
    ring (8192 + 1024) wrap, and six prefix passes run on the prefix stream
    beside the chunk loop. Every chunk is compared with the oracle."""
    cfg = synth.get_config("3b", n_blocks=8, n_ttt_blocks=2, seq_len=12288)
    n = 12289
    w, wd, toks = gpu_inputs(cfg, n)
    model = bd.TTTModel(cfg, wd, batch=1, max_positions=n, prefill_span=2048)
    g = model.prefill(torch.as_tensor(toks).cuda()).cpu().numpy()[0]
    torch.cuda.synchronize()
    wn = synth.weights_to_numpy(w)
    del w, wd
    orc, o = oracle_run(cfg, wn, toks[0])
    assert orc.chunk == 12
    check_losses(cfg, g, o, "3b_8block")
    worst = compare_weights(cfg, model, [orc], wn, TOL["w"], TOL["dw"])
    log(cfg, f"worst weight rel err {worst[0]:.3e}, update rel err {worst[1]:.3e}")
    model.close()
