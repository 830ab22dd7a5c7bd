"""Helpers shared by the GPU parity tests (marshalling and comparisons only)."""
import numpy as np
import torch

from long_context_lm_token_amd import binding, synth


def dev_weights(cfg, seed=0, std=0.02):
    """Seeded weights on the GPU (dtype of the config) and their oracle copy."""
    w = synth.make_weights(cfg, seed=seed, device="cpu", std=std)
    wd = {k: v.cuda() for k, v in w.items()}
    return wd, synth.weights_to_numpy(w)


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def fast_names(cfg):
    return ["w_up", "w_gate", "w_down"] if cfg["mlp"] == "swiglu" else ["w_up", "w_down"]


def compare_weights(cfg, model, oracles, w_np, tol_w, tol_dw, seqs=None):
    """Final fast weights (relative Frobenius) and their change from W_0."""
    t0 = cfg["n_blocks"] - cfg["n_ttt_blocks"]
    worst = (0.0, 0.0)
    for s, orc in enumerate(oracles):
        if seqs is not None and s not in seqs:
            continue
        for l in range(t0, cfg["n_blocks"]):
            for name in fast_names(cfg):
                g = model.get_weights(s, l, name).cpu().numpy().astype(np.float64)
                o = orc.fast_weight(l, name)
                w0 = w_np[f"{l}.{name}"].astype(np.float64)
                e_w = rel_fro(g, o)
                e_dw = rel_fro(g - w0, o - w0)
                assert np.linalg.norm(o - w0) > 0, "the oracle's update vanished"
                assert e_w <= tol_w, (s, l, name, e_w)
                assert e_dw <= tol_dw, (s, l, name, e_dw)
                worst = (max(worst[0], e_w), max(worst[1], e_dw))
    return worst


def to_dev(a, dtype):
    return torch.as_tensor(np.ascontiguousarray(a)).to(dtype).cuda()


def kdt(dtype):
    return binding.TTT_BF16 if dtype == torch.bfloat16 else binding.TTT_FP32
