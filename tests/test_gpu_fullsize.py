"""Parity at the workloads' full model sizes (bf16), against the CPU oracle.

* 125M shape: the whole 8192-position prefill (16 chunks of 512).
* 1B and 3B shapes: the first four chunks (4096 positions), the slice the
  oracle can afford. For 3B the losses are also taken from a full
  131072-position prefill in the benchmark's launch configuration.

Tolerances (bf16), against the fp64 oracle:
  * the per-token loss averaged over each mini-batch within 2e-2 absolute;
  * final fast weights within 2e-2 relative Frobenius, their change from W_0
    within 5e-2;
  * each token's loss: within 2e-2 at the 125M shape. At the 1B and 3B shapes
    bf16 operands alone move single-token losses further than that, so there
    the rms and the largest per-token error must stay within 1.5x of what the
    oracle's bf16 operand mode (every activation operand of a matrix product
    rounded to bf16, all else fp64) deviates from fp64 on the first chunk -
    a bound computed from the oracle alone.
"""
import numpy as np
import pytest
import torch

from long_context_lm_token_amd import binding as bd, synth
from oracle import ttt_oracle as O
from tests.gpu_util import compare_weights

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TOL = dict(loss=2e-2, w=2e-2, dw=5e-2)
FLOOR_FACTOR = 1.5


def log(cfg, msg):
    print(f"[{cfg['name']}] {msg}", flush=True)


def gpu_inputs(cfg, n_ids, seed=0):
    w = synth.make_weights(cfg, seed=seed, device="cuda")
    toks = synth.make_batch(cfg, 1, n_ids, seed=seed + 1)
    return w, toks


def oracle_run(cfg, wn, ids):
    orc = O.Oracle(cfg, wn, cache_fp64=False,
                   progress=lambda msg: log(cfg, msg) if "block 0 " in msg else None)
    return orc, orc.prefill(ids)


def bf16_floor(cfg, wn, ids, o_first):
    """(rms, max) of |bf16-operand-mode loss - fp64 loss| over the first chunk."""
    b = cfg["mini_batch"]
    ob = O.Oracle(cfg, wn, cache_fp64=False).static_losses(ids[:b + 1], operands="bf16")
    e = ob - o_first[1:b + 1]
    return float(np.sqrt(np.mean(e * e))), float(np.abs(e).max())


def check_losses(cfg, g, o, floor=None):
    b = cfg["mini_batch"]
    e = g[1:] - o[1:]
    n_chunks = len(e) // b
    worst_mean = max(abs(float(e[c * b:(c + 1) * b].mean())) for c in range(n_chunks))
    rms, mx = float(np.sqrt(np.mean(e * e))), float(np.abs(e).max())
    log(cfg, f"loss vs fp64 oracle over {len(e)} positions: worst mini-batch mean {worst_mean:.2e}, "
             f"rms {rms:.4f}, max {mx:.4f}" + (f"; bf16 floor rms {floor[0]:.4f} max {floor[1]:.4f}" if floor else ""))
    assert np.isfinite(g[1:]).all()
    assert worst_mean <= TOL["loss"], worst_mean
    if floor is None:
        assert mx <= TOL["loss"], mx
    else:
        assert rms <= FLOOR_FACTOR * floor[0], (rms, floor)
        assert mx <= FLOOR_FACTOR * floor[1], (mx, floor)


@pytest.mark.timeout(600)
def test_125m_full_prefill():
    cfg = synth.get_config("125m")
    n = cfg["seq_len"] + 1
    w, toks = gpu_inputs(cfg, n)
    model = bd.TTTModel(cfg, w, batch=1, max_positions=n)
    g = model.prefill(torch.as_tensor(toks).cuda()).cpu().numpy()[0]
    torch.cuda.synchronize()
    wn = synth.weights_to_numpy(w)
    orc, o = oracle_run(cfg, wn, toks[0])
    check_losses(cfg, g, o)
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
    w, toks = gpu_inputs(cfg, full)
    # same library configuration as the benchmark: room for the whole stream
    model = bd.TTTModel(cfg, w, batch=1, max_positions=full)
    g = model.prefill(torch.as_tensor(toks[:, :n]).cuda()).cpu().numpy()[0]
    torch.cuda.synchronize()
    wn = synth.weights_to_numpy(w)
    orc, o = oracle_run(cfg, wn, toks[0, :n])
    floor = bf16_floor(cfg, wn, toks[0], o)
    check_losses(cfg, g, o, floor)
    worst = compare_weights(cfg, model, [orc], wn, TOL["w"], TOL["dw"])
    log(cfg, f"worst weight rel err {worst[0]:.3e}, update rel err {worst[1]:.3e}")
    if name == "3b":
        # the first four chunks inside a whole 128K prefill
        model.reset()
        gf = model.prefill(torch.as_tensor(toks).cuda()).cpu().numpy()[0]
        torch.cuda.synchronize()
        assert np.isfinite(gf[1:]).all()
        log(cfg, "full 131072-position prefill, first four chunks:")
        check_losses(cfg, gf[:n], o, floor)
    model.close()
