"""CPU fp64 oracle of the TTT-E2E prefill / decode inner loop.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module. It shares no code with the HIP
library and is deliberately plain: numpy fp64, one chunk at a time, every
step written out, backward derived by hand.

What it computes follows the pages on "End-to-End Test-Time Training for Long
Context":
  * per-token loss: cross entropy of the next token, natural log
    (b-lab.team summary, "Test-Time Training (Inner Loop)", loss function;
    technical review "TTT-E2E: Learning a Long Context into Weights",
    section 2.2 and Eq. 3);
  * mini-batch update W_i = W_{i-1} - eta * (1/b) * sum of per-token gradients
    taken at W_{i-1}, every target in a chunk scored before the update
    (summary, "Mini-Batch Gradient Descent"; review section 5, Eq. 9);
  * the prefill loop of the review's section 7, Algorithm 1 (fresh copy of the
    initial fast weights, causal masking inside a chunk, loss recorded before
    the update, gradient, SGD step, keep only the windowed attention state);
  * sliding-window causal attention with window k >= b (summary,
    "Integration with Sliding-Window Attention"; review Eq. 1 and section 5);
  * fast weights = MLPs of the last quarter of the blocks; embeddings, norms
    and attention frozen; each such block also has a static MLP branch
    (summary, "Implementation Details for TTT"; review section 6);
  * decoding updates only after a full mini-batch of generated tokens
    (summary, "Decoding Multiple Tokens"; review section 7, Algorithm 3).
  * the "TTT-E2E all layers MH" variant (config key mh_heads > 1; summary,
    "Alternative Derivation", step 4; review section 8, Table 1 and the
    paragraph on splitting a width-D map into H heads): every block carries
    a fast MLP split into mh_heads independent heads, each a small MLP from
    its slice of the normalised state (width d / mh_heads, hidden
    ttt_hidden / mh_heads) back to the same slice, trained by the same
    next-token loss and inner update as the final design.

Readings of points the pages leave open (each is listed in the design doc):
  * position p has input x_p and label x_{p+1}; chunk c is positions
    [c*b, (c+1)*b) counted from the first id of the stream;
  * key j is visible to query p iff p-k < j <= p (min(p+1, k) keys, the
    bound N_window <= T*k of the review's Eq. 1);
  * K/V of earlier chunks are kept as computed (at their own W) and are
    constants of the gradient; they are not recomputed after an update;
  * frozen modules are differentiated through, never updated;
  * the static branch shares the block's pre-MLP RMSNorm and is summed into
    the residual with the trainable branch;
  * RMSNorm eps 1e-6, no biases, untied LM head, final RMSNorm before it;
  * MHA, scale 1/sqrt(hd), RoPE theta 10000 on pairs (i, i+hd/2) at absolute
    positions (configs with rope only); GELU is the exact erf form, SwiGLU is
    W_down(silu(x W_gate) * (x W_up));
  * plain SGD (no momentum, decay or clipping), one joint step over all fast
    matrices; a chunk that is not yet complete is scored at the current W and
    never applied.
  * all-layers MH variant: n_ttt_blocks = n_blocks; each block's fast
    multi-head MLP sits beside its regular (static) MLP, sharing the pre-MLP
    RMSNorm, both summed into the residual; per-head weights are stored
    [head][in][out].

bf16 operand mode (static_losses(..., operands="bf16")): the bf16 runs compute
every matrix product from bf16 operands with wider accumulation. In this mode
the forward rounds each operand of a matrix product that is not a stored
weight to bf16 - an fp32 value rounded to nearest even - and keeps everything
else in fp64. Those operands are the normalised activations, q and k after
RoPE, v, the attention weights P = softmax(q k^T / sqrt(hd)) (the operand of
the P v product), the attention output, the MLP activation and the final
normalised state. It measures what bf16 operands alone do to the losses (a
diagnostic; no parity bound is derived from it) and is not used for
gradients.
"""
from __future__ import annotations

import math
import numpy as np
from scipy.special import erf

__all__ = ["Oracle", "rmsnorm_fwd", "rmsnorm_bwd", "gelu", "gelu_grad", "rope",
           "rope_inv", "window_attention", "window_attention_bwd", "cross_entropy",
           "sgd_step", "visible_pairs", "prefill", "bf16_round"]


# --------------------------------------------------------------------------
# elementary operations (each a textbook definition)
# --------------------------------------------------------------------------

def rmsnorm_fwd(x, g, eps):
    """y = x * (mean(x^2) + eps)^(-1/2) * g, row-wise; also returns r."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * g, r


def rmsnorm_bwd(x, g, r, dy):
    """dx of rmsnorm_fwd: r*g*dy - x * r^3 * mean(x*g*dy)."""
    return r * g * dy - x * (r ** 3) * np.mean(x * g * dy, axis=-1, keepdims=True)


def gelu(x):
    """x * Phi(x) with the exact normal CDF."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def gelu_grad(x):
    """Phi(x) + x * phi(x)."""
    return 0.5 * (1.0 + erf(x / math.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def rope_angles(pos, hd, theta):
    """[len(pos)][hd/2] angles p * theta^(-2i/hd) in fp64."""
    i = np.arange(hd // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / hd)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def rope(x, pos, theta):
    """Rotate pairs (i, i + hd/2) of x [m][H][hd] by the angles of pos."""
    hd = x.shape[-1]
    a = rope_angles(pos, hd, theta)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : hd // 2], x[..., hd // 2:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_inv(x, pos, theta):
    """Inverse rotation (the transpose of rope), used for its backward."""
    hd = x.shape[-1]
    a = rope_angles(pos, hd, theta)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : hd // 2], x[..., hd // 2:]
    return np.concatenate([x1 * c + x2 * s, -x1 * s + x2 * c], axis=-1)


def bf16_round(x):
    """Round to bf16: to fp32 (nearest even), then keep the top 16 bits of the
    fp32 pattern, rounding the dropped 16 to nearest with ties to even (the
    bf16 format: fp32's sign and exponent, 7 stored mantissa bits)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    bits = ((bits + 0x7FFF + lsb) >> 16) << 16
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def _same(x):
    return x


def window_mask(qpos, kpos, window):
    """Visible iff qpos - window < kpos <= qpos."""
    qp = np.asarray(qpos)[:, None]
    kp = np.asarray(kpos)[None, :]
    return (kp <= qp) & (kp > qp - window)


def visible_pairs(T, window):
    """Number of (query, key) pairs the window admits over T positions."""
    return int(sum(min(p + 1, window) for p in range(T)))


def window_attention(q, K, V, qpos, kpos, window, rnd=None):
    """Softmax attention per head restricted to the window.

    q [m][H][hd], K/V [n][H][hd]; returns o [m][H][hd] and P [H][m][n].
    With rnd (bf16 operand mode) the product with V takes rnd(P); P is then
    None.
    """
    hd = q.shape[-1]
    mask = window_mask(qpos, kpos, window)
    qh, Kh, Vh = q.transpose(1, 0, 2), K.transpose(1, 0, 2), V.transpose(1, 0, 2)
    s = (qh @ Kh.transpose(0, 2, 1)) / math.sqrt(hd)          # [H][m][n]
    s = np.where(mask[None], s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    P = e / e.sum(axis=-1, keepdims=True)
    if rnd is not None:
        return (rnd(P) @ Vh).transpose(1, 0, 2), None
    o = (P @ Vh).transpose(1, 0, 2)                           # [m][H][hd]
    return o, P


def window_attention_bwd(q, K, V, P, do):
    """Gradients of window_attention given P: returns dq, dK, dV."""
    hd = q.shape[-1]
    qh, Kh, Vh, doh = (a.transpose(1, 0, 2) for a in (q, K, V, do))
    dP = doh @ Vh.transpose(0, 2, 1)                               # [H][m][n]
    dS = P * (dP - np.sum(dP * P, axis=-1, keepdims=True))
    dq = (dS @ Kh).transpose(1, 0, 2) / math.sqrt(hd)
    dK = (dS.transpose(0, 2, 1) @ qh).transpose(1, 0, 2) / math.sqrt(hd)
    dV = (P.transpose(0, 2, 1) @ doh).transpose(1, 0, 2)
    return dq, dK, dV


def cross_entropy(z, labels):
    """Per-row natural-log CE and its gradient softmax - onehot."""
    zmax = z.max(axis=-1, keepdims=True)
    e = np.exp(z - zmax)
    ssum = e.sum(axis=-1, keepdims=True)
    lse = (np.log(ssum) + zmax)[:, 0]
    loss = lse - z[np.arange(len(labels)), labels]
    p = e / ssum
    p[np.arange(len(labels)), labels] -= 1.0
    return loss, p


def sgd_step(w, g, lr):
    """W <- W - lr * G (the inner update of Eq. 9 / Eq. 3)."""
    return w - lr * g


# --------------------------------------------------------------------------
# the model and the inner loop, one sequence
# --------------------------------------------------------------------------

class Oracle:
    """One sequence's TTT-E2E state: fast weights, attention cache, stream."""

    def __init__(self, cfg: dict, weights: dict, cache_fp64: bool | None = None, progress=None):
        self.cfg = cfg
        self.progress = progress        # optional callable(str), called once per block
        self.w32 = weights              # fp32 (bf16-exact) numpy arrays, [in][out]
        total = sum(v.size for v in weights.values())
        self._keep64 = (total < 300_000_000) if cache_fp64 is None else cache_fp64
        self._w64 = {}
        L = cfg["n_blocks"]
        self.t0 = L - cfg["n_ttt_blocks"]
        self.glu = cfg["mlp"] == "swiglu"
        self.mh = cfg.get("mh_heads", 0) > 1
        self.fast_names = ["w_up", "w_gate", "w_down"] if self.glu else ["w_up", "w_down"]
        self.reset()

    # ---- parameters ----
    def p(self, name):
        """fp64 view of a frozen parameter."""
        if name in self._w64:
            return self._w64[name]
        v = self.w32[name].astype(np.float64)
        if self._keep64:
            self._w64[name] = v
        return v

    def reset(self):
        """Fresh copy of the initial fast weights, empty cache and stream."""
        self.W = {(l, n): self.w32[f"{l}.{n}"].astype(np.float64)
                  for l in range(self.t0, self.cfg["n_blocks"]) for n in self.fast_names}
        L = self.cfg["n_blocks"]
        H, hd = self.cfg["n_heads"], self.cfg["head_dim"]
        self.K = [np.zeros((0, H, hd)) for _ in range(L)]
        self.V = [np.zeros((0, H, hd)) for _ in range(L)]
        self.ids = []
        self.chunk = 0                   # next chunk to apply
        self.last_logits = None

    # ---- forward over positions [p0, p0+m) with the cache for keys < p0 ----
    def forward(self, ids, p0, W=None, keep=False, rnd=None):
        """Return logits [m][V] and a tape of what the backward needs.

        Keys before p0 come from the cache as stored; keys in [p0, p0+m) come
        from this pass. If keep, the tape keeps tail-block intermediates.
        rnd: operand rounding of the bf16 operand mode (forward only).
        """
        cfg = self.cfg
        r = _same if rnd is None else rnd
        assert rnd is None or not keep
        W = self.W if W is None else W
        H, hd, eps = cfg["n_heads"], cfg["head_dim"], cfg["norm_eps"]
        win = cfg["window"]
        m = len(ids)
        pos = np.arange(p0, p0 + m)
        lo = max(0, p0 - win + 1)
        kpos = np.arange(lo, p0 + m)
        x = self.p("embed")[np.asarray(ids)]
        tape = {"pos": pos, "kpos": kpos, "blocks": {}, "kv": []}
        for l in range(cfg["n_blocks"]):
            pre = f"{l}."
            u, r1 = rmsnorm_fwd(x, self.p(pre + "attn_norm"), eps)
            ur = r(u)
            q = (ur @ self.p(pre + "wq")).reshape(m, H, hd)
            k = (ur @ self.p(pre + "wk")).reshape(m, H, hd)
            v = r((ur @ self.p(pre + "wv")).reshape(m, H, hd))
            if cfg["rope"]:
                q = rope(q, pos, cfg["rope_theta"])
                k = rope(k, pos, cfg["rope_theta"])
            q, k = r(q), r(k)
            Kw = np.concatenate([self.K[l][lo:p0], k], axis=0)
            Vw = np.concatenate([self.V[l][lo:p0], v], axis=0)
            o, P = window_attention(q, Kw, Vw, pos, kpos, win, rnd=rnd)
            a = o.reshape(m, H * hd)
            y = x + r(a) @ self.p(pre + "wo")
            n, r2 = rmsnorm_fwd(y, self.p(pre + "mlp_norm"), eps)
            nr = r(n)
            rec = None
            if l >= self.t0:
                fast = self._mh_mlp if self.mh else self._mlp
                mt, mt_rec = fast(nr, W[(l, "w_up")], W.get((l, "w_gate")), W[(l, "w_down")], r)
                ms, ms_rec = self._mlp(nr, self.p(pre + "s_up"),
                                       self.p(pre + "s_gate") if self.glu else None,
                                       self.p(pre + "s_down"), r)
                xn = y + mt + ms
                if keep:
                    rec = dict(x=x, u=u, r1=r1, q=q, Kw=Kw, Vw=Vw, P=None, a=a, y=y, n=n,
                               r2=r2, mt=mt_rec, ms=ms_rec, nk_cache=p0 - lo)
            else:
                mo, _ = self._mlp(nr, self.p(pre + "w_up"),
                                  self.p(pre + "w_gate") if self.glu else None,
                                  self.p(pre + "w_down"), r)
                xn = y + mo
            tape["kv"].append((k, v))
            if rec is not None:
                tape["blocks"][l] = rec
            x = xn
            if self.progress:
                self.progress(f"oracle forward block {l} positions {p0}..{p0 + m - 1}")
        f, rf = rmsnorm_fwd(x, self.p("final_norm"), eps)
        z = r(f) @ self.p("lm_head")
        tape.update(xL=x, rf=rf, f=f)
        return z, tape

    def _mlp(self, n, Wup, Wgate, Wdown, r=_same):
        hu = n @ Wup
        if self.glu:
            hg = n @ Wgate
            act = hg * sigmoid(hg) * hu
        else:
            hg = None
            act = gelu(hu)
        return r(act) @ Wdown, dict(hu=hu, hg=hg, act=act)

    def _mh_mlp(self, n, Wup, Wgate, Wdown, r=_same):
        """Multi-head MLP: head i maps columns [i*dh, (i+1)*dh) of n through
        its own MLP (Wup[i]: [dh][hh], Wdown[i]: [hh][dh]) back to the same
        columns."""
        nh, dh, _ = Wup.shape
        m = n.shape[0]
        nH = n.reshape(m, nh, dh).transpose(1, 0, 2)             # [nh][m][dh]
        hu = nH @ Wup                                            # [nh][m][hh]
        if self.glu:
            hg = nH @ Wgate
            act = hg * sigmoid(hg) * hu
        else:
            hg = None
            act = gelu(hu)
        out = (r(act) @ Wdown).transpose(1, 0, 2).reshape(m, nh * dh)
        return out, dict(hu=hu, hg=hg, act=act)

    def _mh_mlp_bwd(self, n, rec, Wup, Wgate, Wdown, dout, need_dn):
        """Gradients of one multi-head MLP, head by head (the chain rule of
        _mlp_bwd applied to each head's own slice)."""
        nh, dh, _ = Wup.shape
        m = n.shape[0]
        nH = n.reshape(m, nh, dh).transpose(1, 0, 2)
        doH = dout.reshape(m, nh, dh).transpose(1, 0, 2)         # [nh][m][dh]
        dact = doH @ Wdown.transpose(0, 2, 1)                    # [nh][m][hh]
        dWdown = rec["act"].transpose(0, 2, 1) @ doH             # [nh][hh][dh]
        if self.glu:
            hg, hu = rec["hg"], rec["hu"]
            sg = sigmoid(hg)
            dhu = dact * hg * sg
            dhg = dact * hu * sg * (1.0 + hg * (1.0 - sg))
            dWgate = nH.transpose(0, 2, 1) @ dhg                 # [nh][dh][hh]
            dnH = (dhu @ Wup.transpose(0, 2, 1) + dhg @ Wgate.transpose(0, 2, 1)) if need_dn else None
        else:
            dhu = dact * gelu_grad(rec["hu"])
            dWgate = None
            dnH = (dhu @ Wup.transpose(0, 2, 1)) if need_dn else None
        dWup = nH.transpose(0, 2, 1) @ dhu
        dn = dnH.transpose(1, 0, 2).reshape(m, nh * dh) if need_dn else None
        return dWup, dWgate, dWdown, dn

    def _mlp_bwd(self, n, rec, Wup, Wgate, Wdown, dout, need_dn):
        """Gradients of one MLP branch: (dWup, dWgate, dWdown, dn)."""
        dact = dout @ Wdown.T
        dWdown = rec["act"].T @ dout
        if self.glu:
            hg, hu = rec["hg"], rec["hu"]
            sg = sigmoid(hg)
            silu = hg * sg
            dhu = dact * silu
            dhg = dact * hu * sg * (1.0 + hg * (1.0 - sg))
            dWgate = n.T @ dhg
            dWup = n.T @ dhu
            dn = (dhu @ Wup.T + dhg @ Wgate.T) if need_dn else None
        else:
            dhu = dact * gelu_grad(rec["hu"])
            dWgate = None
            dWup = n.T @ dhu
            dn = (dhu @ Wup.T) if need_dn else None
        return dWup, dWgate, dWdown, dn

    # ---- backward: gradient of (1/b) * sum of chunk losses wrt the fast weights ----
    def backward(self, tape, dz, W=None):
        """dz = d(chunk objective)/d(logits) [m][V]; returns {(l, name): G}."""
        cfg = self.cfg
        W = self.W if W is None else W
        H, hd = cfg["n_heads"], cfg["head_dim"]
        m = dz.shape[0]
        G = {}
        df = dz @ self.p("lm_head").T
        dx = rmsnorm_bwd(tape["xL"], self.p("final_norm"), tape["rf"], df)
        for l in range(cfg["n_blocks"] - 1, self.t0 - 1, -1):
            rec = tape["blocks"][l]
            pre = f"{l}."
            # MLP sublayer: x_out = y + MLP_t(n) + MLP_s(n)
            need = l > self.t0
            fast_bwd = self._mh_mlp_bwd if self.mh else self._mlp_bwd
            dWu, dWg, dWd, dn_t = fast_bwd(rec["n"], rec["mt"], W[(l, "w_up")],
                                           W.get((l, "w_gate")), W[(l, "w_down")], dx, need)
            G[(l, "w_up")] = dWu
            G[(l, "w_down")] = dWd
            if self.glu:
                G[(l, "w_gate")] = dWg
            if not need:
                break
            _, _, _, dn_s = self._mlp_bwd(rec["n"], rec["ms"], self.p(pre + "s_up"),
                                          self.p(pre + "s_gate") if self.glu else None,
                                          self.p(pre + "s_down"), dx, True)
            dy = dx + rmsnorm_bwd(rec["y"], self.p(pre + "mlp_norm"), rec["r2"], dn_t + dn_s)
            # attention sublayer: y = x + attn(RMSNorm(x)) @ Wo
            da = dy @ self.p(pre + "wo").T
            do = da.reshape(m, H, hd)
            _, P = window_attention(rec["q"], rec["Kw"], rec["Vw"], tape["pos"], tape["kpos"],
                                    cfg["window"])
            dq, dK, dV = window_attention_bwd(rec["q"], rec["Kw"], rec["Vw"], P, do)
            nc = rec["nk_cache"]
            dk, dv = dK[nc:], dV[nc:]          # cached keys are constants
            if cfg["rope"]:
                dq = rope_inv(dq, tape["pos"], cfg["rope_theta"])
                dk = rope_inv(dk, tape["pos"], cfg["rope_theta"])
            du = (dq.reshape(m, -1) @ self.p(pre + "wq").T + dk.reshape(m, -1) @ self.p(pre + "wk").T
                  + dv.reshape(m, -1) @ self.p(pre + "wv").T)
            dx = dy + rmsnorm_bwd(rec["x"], self.p(pre + "attn_norm"), rec["r1"], du)
            if self.progress:
                self.progress(f"oracle backward block {l}")
        return G

    # ---- one chunk: score at W_c, gradient, update ----
    def chunk_objective(self, c, W=None):
        """Mean loss of chunk c at W (cache as stored) and its gradient."""
        b = self.cfg["mini_batch"]
        ids = self.ids[c * b:(c + 1) * b]
        labels = np.asarray(self.ids[c * b + 1:(c + 1) * b + 1])
        z, tape = self.forward(ids, c * b, W=W, keep=True)
        loss, dz = cross_entropy(z, labels)
        G = self.backward(tape, dz / b, W=W)
        return loss, G, tape

    def _commit_kv(self, tape):
        for l, (k, v) in enumerate(tape["kv"]):
            self.K[l] = np.concatenate([self.K[l], k], axis=0)
            self.V[l] = np.concatenate([self.V[l], v], axis=0)

    def prefill(self, new_ids):
        """Append ids; return the loss of every position labelled by them.

        Entry i is the loss of predicting new id i (position len(old ids)+i-1);
        it is NaN for the first id of a stream, which has no predecessor.
        """
        cfg = self.cfg
        b, lr = cfg["mini_batch"], cfg["lr"]
        n_old = len(self.ids)
        self.ids.extend(int(t) for t in new_ids)
        n_ids = len(self.ids)
        n_lab = n_ids - 1
        loss_at = {}
        while (self.chunk + 1) * b <= n_lab:
            c = self.chunk
            loss, G, tape = self.chunk_objective(c)
            for i, v in enumerate(loss):
                loss_at[c * b + i] = v
            for key in self.W:
                self.W[key] = sgd_step(self.W[key], G[key], lr)
            self._commit_kv(tape)
            self.chunk += 1
        p0 = self.chunk * b
        if p0 < n_ids:
            z, _ = self.forward(self.ids[p0:n_ids], p0)
            if n_lab > p0:
                loss, _ = cross_entropy(z[: n_lab - p0], np.asarray(self.ids[p0 + 1:n_ids]))
                for i, v in enumerate(loss):
                    loss_at[p0 + i] = v
            self.last_logits = z[-1]
        out = np.full(len(new_ids), np.nan)
        for i in range(len(new_ids)):
            pos = n_old + i - 1
            if pos >= 0:
                out[i] = loss_at[pos]
        return out

    def static_losses(self, ids, operands=None):
        """Losses of a whole stream in one pass at the current W (no updates).

        operands="bf16": the bf16 operand mode (module docstring)."""
        assert operands in (None, "bf16")
        saveK, saveV = self.K, self.V
        L = self.cfg["n_blocks"]
        H, hd = self.cfg["n_heads"], self.cfg["head_dim"]
        self.K = [np.zeros((0, H, hd)) for _ in range(L)]
        self.V = [np.zeros((0, H, hd)) for _ in range(L)]
        try:
            z, _ = self.forward(list(ids[:-1]), 0, rnd=bf16_round if operands else None)
        finally:
            self.K, self.V = saveK, saveV
        loss, _ = cross_entropy(z, np.asarray(ids[1:]))
        return loss

    def fast_weight(self, block, name):
        """Current fast matrix in [in][out] layout (fp64); [head][in][out]
        for the multi-head variant."""
        return self.W[(block, name)]


def prefill(cfg, weights, tokens):
    """Batch helper: independent sequences; returns (losses [B][n], oracles)."""
    tokens = np.atleast_2d(np.asarray(tokens))
    outs, ors = [], []
    for s in range(tokens.shape[0]):
        o = Oracle(cfg, weights)
        outs.append(o.prefill(tokens[s]))
        ors.append(o)
    return np.stack(outs), ors
