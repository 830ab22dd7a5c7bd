"""Benchmark: TTT-E2E prefill on the 3B-shaped model, 1 x 131072 tokens, 1 GPU.

A step is one whole prefill of the batch (ttt_reset + ttt_prefill of 131073
ids = 131072 labelled positions: the frozen prefix over the whole sequence,
then 128 chunks of b = 1024 with forward, CE, tail backward and the fused SGD
step). Inputs (weights, tokens) are resident in HBM before the timed region.

Prints one JSON line (rank 0): tokens/s, ms per step, seconds per 1K tokens,
the roofline of the dominant kernel class (the one with the largest share of
kernel time in a profiled step), measured with HIP events attached to the
dispatches of every 8th launch of that class over the timed steps (each timed
dispatch costs its stream a few microseconds), every class's roofline fraction from the
profiled step, the config-4 greedy decode (2048 tokens, two update pauses) and
the CPU oracle timed on a bounded sample of the same workload beside the GPU
on the same sample.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
MFMA_PEAK = 2.5e15   # MI355X dense bf16 MFMA, flop/s
HBM_PEAK = 8.0e12    # MI355X HBM3E, bytes/s
# HBM bytes per launch, measured with rocprofv3 counters (FETCH_SIZE,
# WRITE_SIZE) and scaled by the same counters on a plain copy: per kernel
# class of the 3B prefill, and for the frozen prefix's MLP up-projection alone.
# Each record names the hash of the sources it was taken on and is ignored once
# they change.
CLASS_TRAFFIC = os.path.join(ROOT, "profiles", "prefill_3b_128k_class_counters.md")
CLASS_SOURCES = [os.path.join(ROOT, "long_context_lm_token_amd", "csrc", f)
                 for f in ("gemm.hip", "attention.hip", "elementwise.hip", "runtime.cpp")]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "mlp_up_traffic_3b_span.md")
GEMM_SOURCE = os.path.join(ROOT, "long_context_lm_token_amd", "csrc", "gemm.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_bytes(kernel_class, config):
    """Stored HBM bytes per launch for the kernel class (3B prefill), or None."""
    if config != "3b":
        return None
    if kernel_class == "mlp_up":
        if not os.path.exists(TRAFFIC_RECORD):
            return None
        text = open(TRAFFIC_RECORD).read()
        h = re.search(r"gemm_source_sha256:\s*([0-9a-f]{64})", text)
        v = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
        if not h or not v or hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest() != h.group(1):
            return None
        return int(v.group(1))
    if not os.path.exists(CLASS_TRAFFIC):
        return None
    text = open(CLASS_TRAFFIC).read()
    h = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    v = re.search(r"traffic_bytes_per_launch %s:\s*([0-9]+)" % re.escape(kernel_class), text)
    if not h or not v:
        return None
    cur = hashlib.sha256(b"".join(open(f, "rb").read() for f in CLASS_SOURCES)).hexdigest()
    return int(v.group(1)) if cur == h.group(1) else None


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
    ap.add_argument("--prof-class", default=None,
                    help="kernel class timed with HIP events during the timed steps (default: the class "
                         "with the largest share of kernel time in the profiled step)")
    ap.add_argument("--prof-every", type=int, default=8,
                    help="during the timed steps, time every N-th launch of the roofline class (1: all; each "
                         "timed dispatch costs its stream a few microseconds)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-positions", type=int, default=None,
                    help="labelled positions of the CPU-oracle sample (default: one chunk)")
    ap.add_argument("--full-attention", action="store_true",
                    help="measure the static full-attention baseline instead: window = the stream, no "
                         "inner loop, the top blocks in 16K-row passes (same kernels)")
    ap.add_argument("--decode", type=int, default=2048,
                    help="after the timed prefills, greedy-decode this many tokens (0: none), timed in "
                         "segments between the chunk updates it triggers (reported under 'decode')")
    ap.add_argument("--sessions", default=None,
                    help="comma-separated session counts S (e.g. 1,4,16): measure the serving budget M(S) "
                         "and the prefill throughput of S concurrent sessions sharing one model's weights, "
                         "each on its own stream, beside one lockstep batch of S sequences")
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
    if args.sessions:
        sessions_bench(args)
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
    max_pos = T + 1 + max(args.decode, 0)
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
    # one profiled step (outside the timed region): every launch under its class
    model.prof_begin("all")
    t0 = time.time()
    step()
    torch.cuda.synchronize()
    prof_all = model.prof_end_classes()
    log(f"[bench] profiled step {time.time() - t0:.2f}s")
    classes = class_table(prof_all)
    prof_class = args.prof_class or max(classes, key=lambda c: classes[c]["ms_per_step"])
    log(f"[bench] roofline class: {prof_class}")
    model.prof_begin(prof_class, every=args.prof_every)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
        torch.cuda.synchronize()
        log(f"[bench] step {i} done")
    t1 = time.perf_counter()
    timed = model.prof_end_classes()
    k_ms = sum(v["ms"] for v in timed.values())
    k_launch = sum(v["launches"] for v in timed.values())
    k_flops = sum(v["flops"] for v in timed.values())
    k_bytes = sum(v["bytes"] for v in timed.values())
    ms_step = (t1 - t0) * 1000 / args.steps
    tok = B * T
    value = tok / (ms_step / 1000)

    # algorithmic work of the whole step (flops), for the step-level roofline:
    # forward of every block and the head; backward through the head and the
    # tail blocks (attention only above the first tail block), the fast
    # weights' gradients; a multi-head fast MLP costs 1/heads of a dense one
    d, V, L, nt = cfg["d_model"], cfg["vocab"], cfg["n_blocks"], cfg["n_ttt_blocks"]
    hq = cfg["n_heads"] * cfg["head_dim"]
    m = 3 if cfg["mlp"] == "swiglu" else 2
    h, ht, hs, b, k = cfg["mlp_hidden"], cfg["ttt_hidden"], cfg["static_hidden"], cfg["mini_batch"], cfg["window"]
    nh = cfg.get("mh_heads", 0)
    ht_eff = ht / nh if nh > 1 else ht
    pairs = sum(min(p + 1, k) for p in range(T))
    fwd = (2 * T * L * 4 * d * hq + 2 * T * (L - nt) * m * d * h + 2 * T * nt * m * d * (hs + ht_eff)
           + 2 * T * V * d + 4 * hq * L * pairs)
    bwd = (2 * T * V * d + (nt - 1) * (8 * T * d * hq + 4 * hq * pairs + 2 * hq * T * (b + 1)
                                       + 2 * T * m * d * (hs + ht_eff)) + nt * 2 * T * m * d * ht_eff
           + 2 * T * d * ht_eff) * B
    step_flops = fwd * B + (0 if args.full_attention else bwd)
    peak_bf16 = 2.5e15

    if k_bytes / HBM_PEAK > k_flops / MFMA_PEAK:
        achieved = k_bytes / (k_ms / 1000) / 1e9 if k_ms > 0 else 0.0
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": round(achieved * 1e9 / HBM_PEAK, 4), "traffic": traffic_bytes(prof_class, args.config)}
    else:
        achieved = k_flops / (k_ms / 1000) / 1e12 if k_ms > 0 else 0.0
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK / 1e12, "unit": "TFLOP/s",
                "frac": round(achieved * 1e12 / MFMA_PEAK, 4), "traffic": traffic_bytes(prof_class, args.config)}
    roof.update({"kernel": prof_class, "launches": k_launch, "sampled_every": args.prof_every,
                 "avg_launch_us": round(k_ms * 1000 / max(k_launch, 1), 2),
                 "step_frac": round(step_flops / peak_bf16 / (ms_step / 1000), 4),
                 # the span passes run concurrently with the chunk loop, so
                 # per-launch times include the shared GPU
                 "overlapped": True,
                 "share_of_kernel_time": classes.get(prof_class, {}).get("share")})

    dec = None
    if args.decode > 0:
        dec = decode_timing(model, B, T + 1, cfg["mini_batch"], args.decode)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, w, toks, args.cpu_positions, model)

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
        "classes": classes,
        "cpu_baseline": cpu,
    }
    if dec is not None:
        out["decode"] = dec
    print(json.dumps(out), flush=True)
    model.close()


def sessions_bench(args):
    """Serving S sessions (technical review, section 11.2, Eq. 13): S models
    sharing one model's frozen and initial fast weights, each prefilling its
    own stream of seq_len ids on its own HIP stream, all enqueued before one
    synchronisation; memory by the terms of Eq. 13 from the library's own
    accounting; beside it one model with a lockstep batch of S sequences."""
    import torch
    from long_context_lm_token_amd import binding as bd, synth
    cfg = synth.get_config(args.config)
    T = args.seq_len or 8192
    counts = [int(x) for x in args.sessions.split(",")]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] sessions: config {args.config}, {T} ids per session, S in {counts}")
    w = synth.make_weights(cfg, seed=0, device="cuda")
    base = bd.TTTModel(cfg, w, batch=1, max_positions=T + 1, prefill_span=args.span)
    del w
    torch.cuda.empty_cache()
    toks = torch.as_tensor(synth.make_batch(cfg, max(counts), T + 1, seed=1)).to(dev)
    rows = []
    for S in counts:
        sess = [base] + [base.session(max_positions=T + 1, prefill_span=args.span) for _ in range(S - 1)]
        streams = [torch.cuda.Stream() for _ in range(S)]
        for x, st in zip(sess, streams):
            x.stream = st
        parts = {k: 0 for k in ("shared", "fast", "cache", "work")}
        for i, x in enumerate(sess):
            p = x.bytes_by_part()
            for k in ("fast", "cache", "work"):
                parts[k] += p[k]
            parts["shared"] = p["shared"]

        def run_all():
            for i, (x, st) in enumerate(zip(sess, streams)):
                with torch.cuda.stream(st):
                    x.reset()
                    x.prefill(toks[i:i + 1], want_losses=False)
            torch.cuda.synchronize()

        run_all()  # warm-up
        t0 = time.perf_counter()
        for _ in range(args.steps):
            run_all()
        dt = (time.perf_counter() - t0) / args.steps
        for x in sess[1:]:
            x.close()
        base.stream = None
        del sess
        # the same S sequences as one lockstep batch
        bat = base.session(batch=S, max_positions=T + 1, prefill_span=args.span)
        bat.reset()
        bat.prefill(toks[:S], want_losses=False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            bat.reset()
            bat.prefill(toks[:S], want_losses=False)
            torch.cuda.synchronize()
        dtb = (time.perf_counter() - t0) / args.steps
        pb = bat.bytes_by_part()
        bat.close()
        per = {k: parts[k] // S for k in ("fast", "cache", "work")}
        row = {"S": S, "tokens_per_s": round(S * T / dt, 1), "s_per_step": round(dt, 4),
               "M_S_GiB": round((parts["shared"] + parts["fast"] + parts["cache"] + parts["work"]) / 2**30, 3),
               "M_shared_GiB": round(parts["shared"] / 2**30, 3),
               "per_session_GiB": {k: round(v / 2**30, 3) for k, v in per.items()},
               "batched_tokens_per_s": round(S * T / dtb, 1),
               "batched_M_GiB": round(sum(pb.values()) / 2**30, 3)}
        log(f"[bench] S={S}: {json.dumps(row)}")
        rows.append(row)
    base.close()
    print(json.dumps({"metric": "TTT-E2E prefill tokens/s of S concurrent sessions and the serving budget M(S)",
                      "config": {"workload": f"{args.config}-shape, {T} ids per session, b={cfg['mini_batch']}, "
                                             f"k={cfg['window']}"},
                      "sessions": rows}), flush=True)


def decode_timing(model, B, n_ids, b, n_new):
    """Greedy decode of n_new ids after a full prefill of n_ids ids (the
    technical review's Algorithm 3): segments of ids that complete no chunk
    (forward of one position each) and the single ids whose arrival completes
    a chunk (that chunk's backward and SGD step run before their forward),
    each segment timed between synchronisations."""
    import torch
    segs = []
    done, n_lab = 0, n_ids - 1
    while done < n_new:
        plain = min(b - 1 - (n_lab % b), n_new - done)   # ids that complete no chunk
        if plain:
            segs.append(("plain", plain))
            done += plain
            n_lab += plain
        if done < n_new:
            segs.append(("update", 1))
            done += 1
            n_lab += 1
    times = []
    torch.cuda.synchronize()
    for kind, n in segs:
        t0 = time.perf_counter()
        model.decode(n, want_losses=False)
        torch.cuda.synchronize()
        times.append((kind, n, time.perf_counter() - t0))
    plain_n = sum(n for k, n, _ in times if k == "plain")
    plain_t = sum(t for k, _, t in times if k == "plain")
    upd = [round(t * 1000, 3) for k, _, t in times if k == "update"]
    total = sum(t for _, _, t in times)
    log(f"[bench] decode {n_new}: {plain_t * 1000 / max(plain_n, 1):.2f} ms per plain token, update tokens {upd} ms")
    return {"batch": B, "tokens": n_new, "ms_per_token": round(plain_t * 1000 / max(plain_n, 1), 3),
            "update_token_ms": upd, "seconds": round(total, 3),
            "tokens_per_s": round(B * n_new / total, 1),
            "ms_per_token_incl_updates": round(total * 1000 / n_new, 3)}


def class_table(prof):
    """Per disjoint kernel class of one profiled step: time, share of kernel
    time, achieved rates and the fraction of the class's roofline (the larger
    of its algorithmic flops at the bf16 MFMA peak and its algorithmic bytes
    at the HBM peak, over its measured time)."""
    names = ["gemm_span", "gemm_chunk", "gemm_sgd", "attn_fwd", "attn_dq", "attn_dkdv", "ce", "norm", "other"]
    tot = sum(prof[n]["ms"] for n in names) or 1.0
    out = {}
    for n in names:
        v = prof[n]
        t = v["ms"] / 1000
        t_f, t_b = v["flops"] / MFMA_PEAK, v["bytes"] / HBM_PEAK
        out[n] = {"ms_per_step": round(v["ms"], 2), "share": round(v["ms"] / tot, 4), "launches": v["launches"],
                  "tflops": round(v["flops"] / t / 1e12, 1) if t > 0 else 0.0,
                  "gbs": round(v["bytes"] / t / 1e9, 1) if t > 0 else 0.0,
                  "bound": "mfma" if t_f >= t_b else "hbm",
                  "frac": round(max(t_f, t_b) / t, 4) if t > 0 else 0.0}
    return out


def cpu_baseline(cfg, w, toks, positions, model):
    """The oracle (numpy fp64) on this host: the first chunk of the same
    stream; the GPU library timed on the same sample beside it."""
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
    # the GPU on the same sample: reset + prefill of the same n+1 ids (median of 5)
    part = toks[:, : n + 1].contiguous()
    gt = []
    for _ in range(6):
        model.reset()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        model.prefill(part)
        torch.cuda.synchronize()
        gt.append(time.perf_counter() - t0)
    g_dt = float(np.median(gt[1:]))
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "gpu_same_sample": round(n / g_dt, 1),
            "sample": f"oracle prefill of the first {n} labelled positions (one full chunk: forward of all "
                      f"blocks, CE, tail backward, SGD step) of the same {cfg['name']} stream",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
