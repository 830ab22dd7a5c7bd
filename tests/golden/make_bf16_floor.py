"""Write tests/golden/bf16_floor.json: how far an ideal bf16-operand forward
deviates from the fp64 one, per chunk, on the full-size parity workloads.

Calls only the oracle (and the seeded input generators). For each workload the
static model (the initial weights, no update) is run chunk by chunk twice over
the same ids, once in fp64 and once with every operand of every matrix product
rounded to bf16 (the oracle's bf16 operand mode), and the per-token loss
differences are summarised per chunk (rms, max). The GPU parity tests print
these beside their own errors; they are a diagnostic of the arithmetic, not a
parity bound.

Usage: python tests/golden/make_bf16_floor.py [workload ...]
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from long_context_lm_token_amd import synth  # noqa: E402
from oracle import ttt_oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bf16_floor.json")

# name -> (config name, overrides, ids generated, chunks summarised)
WORKLOADS = {
    "125m": ("125m", {}, 8193, 1),
    "1b": ("1b", {}, 32769, 1),
    "3b": ("3b", {}, 131073, 1),
    # 3B-width, 8 blocks (2 tail blocks), 12 chunks: the steady-state slice
    "3b_8block": ("3b", dict(n_blocks=8, n_ttt_blocks=2, seq_len=12288), 12289, 12),
}


def workload_inputs(name):
    cname, over, n_ids, n_chunks = WORKLOADS[name]
    cfg = synth.get_config(cname, **over)
    w = synth.weights_to_numpy(synth.make_weights(cfg, seed=0, device="cpu"))
    ids = synth.make_tokens(cfg, n_ids, seq=0, seed=1)
    return cfg, w, ids, n_chunks


def static_chunk_losses(orc, ids, n_chunks, rnd):
    """Losses of positions [0, n_chunks*b) of the static model, one chunk at a
    time with the K/V of earlier chunks from the cache (as in prefill)."""
    b = orc.cfg["mini_batch"]
    orc.reset()
    out = []
    for c in range(n_chunks):
        z, tape = orc.forward(list(ids[c * b:(c + 1) * b]), c * b, rnd=rnd)
        loss, _ = O.cross_entropy(z, np.asarray(ids[c * b + 1:(c + 1) * b + 1]))
        out.append(loss)
        orc._commit_kv(tape)
        print(f"  chunk {c} done", flush=True)
    return np.concatenate(out)


def floor(name):
    cfg, w, ids, n_chunks = workload_inputs(name)
    orc = O.Oracle(cfg, w, cache_fp64=False)
    t = time.time()
    ref = static_chunk_losses(orc, ids, n_chunks, None)
    low = static_chunk_losses(orc, ids, n_chunks, O.bf16_round)
    b = cfg["mini_batch"]
    e = (low - ref).reshape(n_chunks, b)
    rec = dict(chunks=n_chunks, mini_batch=b,
               rms=[float(np.sqrt(np.mean(r * r))) for r in e],
               max=[float(np.abs(r).max()) for r in e],
               rms_all=float(np.sqrt(np.mean(e * e))), max_all=float(np.abs(e).max()),
               frac_within_2e_2=float(np.mean(np.abs(e) <= 2e-2)))
    print(name, json.dumps(rec), f"{time.time() - t:.0f}s", flush=True)
    return rec


def main(names):
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    data["_about"] = ("per-token |bf16-operand oracle loss - fp64 oracle loss| of the static model "
                      "(initial weights), per chunk; written by tests/golden/make_bf16_floor.py")
    for n in names:
        data[n] = floor(n)
        json.dump(data, open(OUT, "w"), indent=1)


if __name__ == "__main__":
    main(sys.argv[1:] or list(WORKLOADS))
