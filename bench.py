"""Benchmark: TTT-E2E prefill on the 3B-shaped model, 1 x 131072 tokens, 1 GPU.

A step is one whole prefill of the batch (ttt_reset + ttt_prefill of 131073
ids = 131072 labelled positions: the frozen prefix over the whole sequence,
then 128 chunks of b = 1024 with forward, CE, tail backward and the fused SGD
step). Inputs (weights, tokens) are resident in HBM before the timed region.

Prints one JSON line (rank 0): tokens/s, ms per step, seconds per 1K tokens,
the roofline of the dominant kernel measured with HIP events on the library's
stream, and the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM bytes per launch of the roofline kernel, measured with rocprofv3 counters
# (FETCH_SIZE, WRITE_SIZE) and scaled by the same counters on a plain copy; the
# record names the hash of the GEMM source it was taken on and is ignored once
# that source changes
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "mlp_up_traffic_3b_span.md")
GEMM_SOURCE = os.path.join(ROOT, "long_context_lm_token_amd", "csrc", "gemm.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_bytes(kernel_class):
    """Stored HBM bytes per launch for the kernel class, or None."""
    if kernel_class != "mlp_up" or not os.path.exists(TRAFFIC_RECORD):
        return None
    text = open(TRAFFIC_RECORD).read()
    h = re.search(r"gemm_source_sha256:\s*([0-9a-f]{64})", text)
    v = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not h or not v:
        return None
    if hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest() != h.group(1):
        return None
    return int(v.group(1))


def probe():
    """Counter probe: the span MLP up-projection GEMM of the 3B shape (the
    roofline kernel, fused SwiGLU epilogue, same launch path as a prefill) and
    a plain device copy of known size, a few launches each."""
    import torch
    from long_context_lm_token_amd import binding as bd, synth
    cfg = synth.get_config("3b")
    M, N, K = 16384, 2 * cfg["mlp_hidden"], cfg["d_model"]
    lib = bd.load()
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    A = (torch.randn((M, K), device="cuda", generator=g) * 0.02).bfloat16()
    Bw = (torch.randn((N, K), device="cuda", generator=g) * 0.02).bfloat16()
    C = torch.empty((M, N // 2), device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        bd.check(lib.ttt_k_gemm(1, 3, 0, M, N, K, bd.ptr(A), K, 0, bd.ptr(Bw), K, 0, bd.ptr(C), N // 2, 0,
                                None, 0, 0, None, 0, 0, None, 0, 0, 0.0, 0, 1, None, 0, bd.stream_ptr()),
                 kernel=True)
    n_copy = 64 << 20  # fp32 elements: 256 MiB read + 256 MiB written per copy
    src = torch.ones(n_copy, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "mlp_up", "M": M, "N": N, "K": K, "copy_bytes_each_way": n_copy * 4}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="3b")
    ap.add_argument("--seq-len", type=int, default=None)
    ap.add_argument("--span", type=int, default=0,
                    help="rows per frozen-prefix pass (0: the library default)")
    ap.add_argument("--batch", type=int, default=1,
                    help="independent sequences per step (the length sweep: 16 x 8192, 4 x 32768)")
    ap.add_argument("--prof-class", default="mlp_up",
                    help="kernel class timed with HIP events during the timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-positions", type=int, default=None,
                    help="labelled positions of the CPU-oracle sample (default: one chunk)")
    ap.add_argument("--full-attention", action="store_true",
                    help="measure the static full-attention baseline instead: window = the stream, no "
                         "inner loop, the top blocks in 16K-row passes (same kernels)")
    ap.add_argument("--decode", action="store_true",
                    help="after the timed prefills, greedy-decode up to the next chunk boundary and "
                         "through the update it triggers, timed separately (reported under 'decode')")
    ap.add_argument("--probe", action="store_true",
                    help="run only the roofline kernel and a plain copy (for rocprofv3 counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if args.probe:
        probe()
        return

    import numpy as np
    import torch
    from long_context_lm_token_amd import binding as bd, synth

    cfg = synth.get_config(args.config)
    T = args.seq_len or cfg["seq_len"]
    if args.full_attention:
        cfg = dict(cfg, window=T + 1, mini_batch=min(16384, T))
    B = args.batch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] config {args.config}: generating weights on the GPU")
    w = synth.make_weights(cfg, seed=0, device="cuda")
    toks = torch.as_tensor(synth.make_batch(cfg, B, T + 1, seed=1)).to(dev)
    stream = torch.cuda.current_stream()
    # room for the decode measurement's tokens (up to one chunk) when asked
    max_pos = T + 1 + (cfg["mini_batch"] if args.decode else 0)
    model = bd.TTTModel(cfg, w, batch=B, max_positions=max_pos, stream=stream, prefill_span=args.span,
                        forward_only=args.full_attention)
    log(f"[bench] model created, library device bytes {model.device_bytes() / 2**30:.1f} GiB")
    if args.no_cpu_baseline:
        del w
        torch.cuda.empty_cache()

    def step():
        model.reset()
        model.prefill(toks, want_losses=True)

    for i in range(args.warmup):
        t0 = time.time()
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i} {time.time() - t0:.2f}s")
    model.prof_begin(args.prof_class)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
        torch.cuda.synchronize()
        log(f"[bench] step {i} done")
    t1 = time.perf_counter()
    k_ms, k_launch, k_work = model.prof_end()
    ms_step = (t1 - t0) * 1000 / args.steps
    tok = B * T
    value = tok / (ms_step / 1000)

    # algorithmic work of the whole step (flops), for the step-level roofline
    d, V, L, nt = cfg["d_model"], cfg["vocab"], cfg["n_blocks"], cfg["n_ttt_blocks"]
    hq = cfg["n_heads"] * cfg["head_dim"]
    m = 3 if cfg["mlp"] == "swiglu" else 2
    h, ht, b, k = cfg["mlp_hidden"], cfg["ttt_hidden"], cfg["mini_batch"], cfg["window"]
    pairs = sum(min(p + 1, k) for p in range(T))
    fwd = 2 * T * L * (2 * d * hq + 2 * d * hq + m * d * h) + 2 * T * V * d + 4 * hq * L * pairs
    bwd = (2 * T * V * d + (nt - 1) * (8 * T * d * hq + 4 * hq * pairs + 2 * hq * T * (b + 1)
                                       + 2 * T * m * d * h) + nt * 2 * T * m * d * ht + 2 * T * d * ht) * B
    step_flops = fwd * B + (0 if args.full_attention else bwd)
    peak_bf16 = 2.5e15

    if args.prof_class == "ce":
        achieved = k_work / (k_ms / 1000) / 1e9 if k_ms > 0 else 0.0
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": 8000.0, "unit": "GB/s",
                "frac": round(achieved / 8000.0, 4), "traffic": None}
    else:
        achieved = k_work / (k_ms / 1000) / 1e12 if k_ms > 0 else 0.0
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": 2500.0, "unit": "TFLOP/s",
                "frac": round(achieved / 2500.0, 4), "traffic": traffic_bytes(args.prof_class)}
    roof.update({"kernel": args.prof_class, "launches": k_launch,
                 "avg_launch_us": round(k_ms * 1000 / max(k_launch, 1), 2),
                 "step_frac": round(step_flops / peak_bf16 / (ms_step / 1000), 4),
                 # the span passes run concurrently with the chunk loop, so
                 # per-launch times include the shared GPU
                 "overlapped": True})

    dec = None
    if args.decode:
        dec = decode_timing(model, B, T + 1, cfg["mini_batch"])

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, w, toks, args.cpu_positions)

    out = {
        "metric": "TTT-E2E prefill tokens/s + s per 1K tokens, 3B-shape 128K ctx, 1 GPU",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 2),
        "s_per_1k_tokens": round(ms_step / 1000 / (tok / 1000), 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (Zipf(1.1) ids with a repeated 1024-id span; N(0,0.02) bf16 weights)",
        "config": {"workload": (f"{args.config}-shape static full-attention prefill (no inner loop), {B} x {T} tokens"
                                if args.full_attention else
                                f"{args.config}-shape TTT-E2E prefill, {B} x {T} tokens, b={b}, k={k}"),
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if dec is not None:
        out["decode"] = dec
    print(json.dumps(out), flush=True)
    model.close()


def decode_timing(model, B, n_ids, b):
    """Greedy decode after a full prefill of n_ids ids: the tokens before the
    next chunk boundary (forward of one position each), then the token whose
    arrival completes a chunk (the chunk's backward and SGD step run before
    its forward), each timed between synchronisations."""
    import torch
    n_lab = n_ids - 1
    plain = b - 1 - (n_lab % b)  # decoded ids that complete no chunk
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if plain:
        model.decode(plain)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    model.decode(1)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    log(f"[bench] decode: {plain} plain tokens {(t1 - t0) * 1000 / max(plain, 1):.2f} ms each, "
        f"update token {(t2 - t1) * 1000:.2f} ms")
    return {"batch": B, "plain_tokens": plain, "ms_per_token": round((t1 - t0) * 1000 / max(plain, 1), 3),
            "update_token_ms": round((t2 - t1) * 1000, 3),
            "ms_per_token_incl_update": round((t2 - t0) * 1000 / (plain + 1), 3)}


def cpu_baseline(cfg, w, toks, positions):
    """The oracle (numpy fp64) on this host: the first chunk of the same stream."""
    import numpy as np
    import torch
    from long_context_lm_token_amd import synth
    from oracle import ttt_oracle as O

    n = positions or cfg["mini_batch"]
    log(f"[bench] cpu baseline: copying weights to host, oracle over {n} positions")
    wn = synth.weights_to_numpy(w)
    ids = toks[0, : n + 1].cpu().numpy()
    cores = len(os.sched_getaffinity(0))
    orc = O.Oracle(cfg, wn, cache_fp64=False, progress=lambda msg: log(f"[bench] {msg}"))
    t0 = time.perf_counter()
    orc.prefill(ids)
    dt = time.perf_counter() - t0
    log(f"[bench] cpu baseline {dt:.1f}s")
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"oracle prefill of the first {n} labelled positions (one full chunk: forward of all "
                      f"blocks, CE, tail backward, SGD step) of the same {cfg['name']} stream",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
