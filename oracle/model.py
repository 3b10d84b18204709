"""Decoder with LoRA over a frozen (dequantized) base: forward, hand-derived
backward, LM head, SFT and DPO losses, one SGD step.  Oracle.

Test infrastructure only; see ``oracle/__init__.py``.

Everything is plain numpy in the dtype of the inputs (float64 for parity and
finite differences, float32 for the timed CPU baseline).  No blocking, no
fusion: each function is the textbook definition written out.

What the pages fix (page title, section):
* only the LoRA adapter trains over a frozen base, and plain LoRA only
  ("Soup: Fine-Tune an 8B Model on a 4 GB GPU", "The Core Idea: Layer
  Streaming" and its "FAQ");
* the layer stack is read again during backward (same page, same section:
  streaming is slower because it re-reads each layer) -- so a layer's backward
  may recompute its forward; results do not depend on it;
* DPO's reference log-probabilities come from the same base with the adapter
  switched off ("Show HN: Fine-tune an 8B model on a 4 GB laptop GPU", first
  paragraph);
* streamed execution equals resident execution bit for bit (axbrief.com
  article, "Beyond Memory: The Layer Streaming Breakthrough").

Readings where the pages are silent (they print no formulas):
* the decoder is the Llama/Qwen form reachable through a causal-LM loader
  (axbrief.com article, "The Architecture of Low-VRAM Alignment"): pre-norm
  RMSNorm, q/k/v/o projections without bias, rotate-half RoPE with positions
  restarting at 0 for every sequence, causal softmax attention with grouped
  key/value heads (q head h reads kv head h // (n_heads / n_kv_heads)),
  SwiGLU MLP (silu(gate) * up, then down), residual connections;
* LoRA on a projection: y = x W + s (x A) B with A [in, r], B [r, out],
  s = alpha / r; "adapter disabled" skips the branch;
* weights are kept as W^T = [out, in] (the causal-LM storage order), so
  y = x @ Wt.T;
* SFT loss: mean over every position t < S-1 of every sequence of
  -log p(token[t+1] | tokens[:t+1]);
* DPO loss: -log sigmoid(beta * ((pc - rc) - (pr - rr))) with each term the
  sum of response-token log-probabilities of the chosen (c) or rejected (r)
  sequence under the policy (p) or reference (r) model;
* SGD: theta <- theta - lr * grad, no momentum, no decay.
"""
import numpy as np


# --------------------------------------------------------------------------
# elementary ops
# --------------------------------------------------------------------------

def rmsnorm(h, g, eps):
    """y = g * h / sqrt(mean(h^2) + eps) over the last axis; returns (y, rstd)."""
    rstd = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return g * h * rstd, rstd


def rmsnorm_backward(h, g, rstd, dy):
    """d/dh of rmsnorm for a frozen gain g:
    dx = rstd * (g dy) - rstd^3 / H * h * sum(g dy h)."""
    H = h.shape[-1]
    gdy = g * dy
    return rstd * gdy - (rstd ** 3) / H * h * np.sum(gdy * h, axis=-1, keepdims=True)


def rope_tables(seq_len, head_dim, theta, dtype):
    """cos/sin [S, d/2] for positions 0..S-1 and inverse frequencies
    theta^(-2j/d), j = 0..d/2-1 (computed in float64)."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / head_dim)
    ang = np.arange(seq_len, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x, cos, sin):
    """Rotate-half RoPE.  x [n_seq, S, heads, d]; cos/sin [S, d/2].
    The pair (x_j, x_{j+d/2}) is rotated by the angle of position p."""
    half = x.shape[-1] // 2
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_backward(dy, cos, sin):
    """Transpose of the rotation: rotate the gradient by minus the angle."""
    half = dy.shape[-1] // 2
    c = cos[None, :, None, :]
    s = sin[None, :, None, :]
    d1, d2 = dy[..., :half], dy[..., half:]
    return np.concatenate([d1 * c + d2 * s, d2 * c - d1 * s], axis=-1)


def attention(q, k, v):
    """Causal GQA attention.  q [n_seq, S, nq, d], k/v [n_seq, S, nkv, d].
    Returns o [n_seq, S, nq, d] and the probabilities P [n_seq, nq, S, S]."""
    n_seq, S, nq, d = q.shape
    nkv = k.shape[2]
    group = nq // nkv
    scale = 1.0 / np.sqrt(d)
    o = np.zeros_like(q)
    P = np.zeros((n_seq, nq, S, S), dtype=q.dtype)
    mask = np.triu(np.ones((S, S), dtype=bool), k=1)    # key j > query i
    for b in range(n_seq):
        for h in range(nq):
            kv = h // group
            s = (q[b, :, h, :] @ k[b, :, kv, :].T) * q.dtype.type(scale)
            s = np.where(mask, -np.inf, s)
            s = s - s.max(axis=-1, keepdims=True)
            e = np.exp(s)
            p = e / e.sum(axis=-1, keepdims=True)
            P[b, h] = p
            o[b, :, h, :] = p @ v[b, :, kv, :]
    return o, P


def attention_backward(q, k, v, P, do):
    """Gradients of causal GQA attention: dS = P * (dP - rowsum(dP * P));
    dq = scale dS k; dk = scale dS^T q and dv = P^T do, summed over the q heads
    that share a kv head."""
    n_seq, S, nq, d = q.shape
    nkv = k.shape[2]
    group = nq // nkv
    scale = q.dtype.type(1.0 / np.sqrt(d))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(n_seq):
        for h in range(nq):
            kv = h // group
            p = P[b, h]
            dp = do[b, :, h, :] @ v[b, :, kv, :].T
            ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
            dq[b, :, h, :] = (ds @ k[b, :, kv, :]) * scale
            dk[b, :, kv, :] += (ds.T @ q[b, :, h, :]) * scale
            dv[b, :, kv, :] += p.T @ do[b, :, h, :]
    return dq, dk, dv


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    return x * sigmoid(x)


def silu_grad(x):
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


def log_sigmoid(x):
    """log sigma(x) = -softplus(-x), evaluated without overflow."""
    return -np.logaddexp(0.0, -x)


# --------------------------------------------------------------------------
# LoRA linear
# --------------------------------------------------------------------------

def lora_linear(x, Wt, A=None, B=None, s=1.0, enabled=True):
    """y = x Wt^T + s (x A) B.  x [M, K], Wt [N, K] (frozen), A [K, r], B [r, N].
    With the adapter disabled (or absent) y = x Wt^T."""
    y = x @ Wt.T
    if enabled and A is not None:
        y = y + x.dtype.type(s) * ((x @ A) @ B)
    return y


def lora_linear_backward(x, Wt, A, B, s, dy, enabled=True):
    """Reverse of ``lora_linear`` with the base frozen.
    With u = dy B^T:  dx = dy Wt + s u A^T,  dA = s x^T u,  dB = s (x A)^T dy.
    Returns (dx, dA, dB); dA/dB are None for a projection without adapter."""
    dx = dy @ Wt
    if A is None or not enabled:
        return dx, None, None
    sc = x.dtype.type(s)
    u = dy @ B.T
    dx = dx + sc * (u @ A.T)
    dA = sc * (x.T @ u)
    dB = sc * ((x @ A).T @ dy)
    return dx, dA, dB


# --------------------------------------------------------------------------
# decoder layer
# --------------------------------------------------------------------------

PROJ = ("q", "k", "v", "o", "gate", "up", "down")


class Config:
    """Shapes and hyper-parameters of a Llama/Qwen-style decoder."""

    def __init__(self, n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn,
                 vocab, rms_eps, rope_theta, lora_rank, lora_alpha,
                 lora_targets=("q", "v"), tied=False):
        self.n_layers = n_layers
        self.hidden = hidden
        self.n_heads = n_heads
        self.n_kv_heads = n_kv_heads
        self.head_dim = head_dim
        self.ffn = ffn
        self.vocab = vocab
        self.rms_eps = rms_eps
        self.rope_theta = rope_theta
        self.lora_rank = lora_rank
        self.lora_alpha = lora_alpha
        self.lora_targets = tuple(lora_targets)
        self.tied = tied

    @property
    def lora_scale(self):
        return self.lora_alpha / self.lora_rank

    def proj_shape(self, name):
        """(out N, in K) of projection ``name`` as stored (W^T)."""
        H, F = self.hidden, self.ffn
        qd = self.n_heads * self.head_dim
        kvd = self.n_kv_heads * self.head_dim
        return {"q": (qd, H), "k": (kvd, H), "v": (kvd, H), "o": (H, qd),
                "gate": (F, H), "up": (F, H), "down": (H, F)}[name]


def layer_forward(cfg, lw, lora, h, n_seq, adapter_enabled=True):
    """One decoder layer.  h [T, H] with T = n_seq * S (sequences back to back).

    lw:   dict with the frozen, dequantized projections lw[name] = Wt [N, K]
          and the RMSNorm gains lw["attn_norm"], lw["mlp_norm"] [H].
    lora: dict name -> (A, B) for the adapted projections.
    Returns (out [T, H], cache for ``layer_backward``).
    """
    T, H = h.shape
    S = T // n_seq
    nq, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    s = cfg.lora_scale
    dt = h.dtype

    def proj(name, x):
        A, B = lora.get(name, (None, None))
        return lora_linear(x, lw[name], A, B, s, adapter_enabled)

    n1, r1 = rmsnorm(h, lw["attn_norm"], cfg.rms_eps)
    q = proj("q", n1).reshape(n_seq, S, nq, d)
    k = proj("k", n1).reshape(n_seq, S, nkv, d)
    v = proj("v", n1).reshape(n_seq, S, nkv, d)
    cos, sin = rope_tables(S, d, cfg.rope_theta, dt)
    qr = rope(q, cos, sin)
    kr = rope(k, cos, sin)
    o, P = attention(qr, kr, v)
    o = o.reshape(T, nq * d)
    h2 = h + proj("o", o)
    n2, r2 = rmsnorm(h2, lw["mlp_norm"], cfg.rms_eps)
    g = proj("gate", n2)
    u = proj("up", n2)
    a = silu(g) * u
    out = h2 + proj("down", a)
    cache = dict(h=h, n1=n1, r1=r1, qr=qr, kr=kr, v=v, P=P, o=o, h2=h2, n2=n2,
                 r2=r2, g=g, u=u, a=a, cos=cos, sin=sin, n_seq=n_seq,
                 adapter_enabled=adapter_enabled)
    return out, cache


def layer_backward(cfg, lw, lora, cache, dout):
    """Hand-derived reverse of ``layer_forward``.  Returns (dh [T, H],
    grads dict name -> (dA, dB) for the adapted projections)."""
    T, H = dout.shape
    n_seq = cache["n_seq"]
    S = T // n_seq
    nq, nkv, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    s = cfg.lora_scale
    en = cache["adapter_enabled"]
    grads = {}

    def proj_bwd(name, x, dy):
        A, B = lora.get(name, (None, None))
        dx, dA, dB = lora_linear_backward(x, lw[name], A, B, s, dy, en)
        if dA is not None:
            grads[name] = (dA, dB)
        return dx

    # MLP: out = h2 + down(silu(g) * u)
    dh2 = dout.copy()
    da = proj_bwd("down", cache["a"], dout)
    g, u = cache["g"], cache["u"]
    dg = da * u * silu_grad(g)
    du = da * silu(g)
    dn2 = proj_bwd("gate", cache["n2"], dg) + proj_bwd("up", cache["n2"], du)
    dh2 = dh2 + rmsnorm_backward(cache["h2"], lw["mlp_norm"], cache["r2"], dn2)
    # attention block: h2 = h + o_proj(attn(rope(q), rope(k), v))
    do = proj_bwd("o", cache["o"], dh2).reshape(n_seq, S, nq, d)
    dqr, dkr, dv = attention_backward(cache["qr"], cache["kr"], cache["v"],
                                      cache["P"], do)
    dq = rope_backward(dqr, cache["cos"], cache["sin"]).reshape(T, nq * d)
    dk = rope_backward(dkr, cache["cos"], cache["sin"]).reshape(T, nkv * d)
    dv = dv.reshape(T, nkv * d)
    n1 = cache["n1"]
    dn1 = proj_bwd("q", n1, dq) + proj_bwd("k", n1, dk) + proj_bwd("v", n1, dv)
    dh = dh2 + rmsnorm_backward(cache["h"], lw["attn_norm"], cache["r1"], dn1)
    return dh, grads


# --------------------------------------------------------------------------
# LM head
# --------------------------------------------------------------------------

def head_logprobs(cfg, head, h, targets):
    """Final RMSNorm, logits = n W_lm^T, logp_t = logits[t, y_t] - logsumexp_t.

    head: dict with "final_norm" [H], "lm_head" [V, H] (the embedding when the
    model ties them).  targets int [T]; a negative target gives logp 0 (no
    prediction at that position).  Returns (logp [T], cache)."""
    n, r = rmsnorm(h, head["final_norm"], cfg.rms_eps)
    logits = n @ head["lm_head"].T
    m = logits.max(axis=-1, keepdims=True)
    lse = (m + np.log(np.sum(np.exp(logits - m), axis=-1, keepdims=True)))[:, 0]
    valid = targets >= 0
    idx = np.where(valid, targets, 0)
    logp = np.where(valid, logits[np.arange(len(idx)), idx] - lse, 0.0).astype(h.dtype)
    return logp, dict(h=h, n=n, r=r, logits=logits, lse=lse, targets=targets)


def head_backward(cfg, head, cache, dlogp):
    """dh from d(loss)/d(logp): dlogits = dlogp (onehot(y) - softmax),
    dn = dlogits W_lm, then the final RMSNorm backward."""
    logits, lse, targets = cache["logits"], cache["lse"], cache["targets"]
    valid = targets >= 0
    p = np.exp(logits - lse[:, None])
    dlogits = -p * dlogp[:, None]
    rows = np.nonzero(valid)[0]
    dlogits[rows, targets[rows]] += dlogp[rows]
    dlogits[~valid] = 0.0
    dn = dlogits @ head["lm_head"]
    return rmsnorm_backward(cache["h"], head["final_norm"], cache["r"], dn)


# --------------------------------------------------------------------------
# losses
# --------------------------------------------------------------------------

def sft_targets(tokens):
    """Targets for next-token prediction: position t of each sequence predicts
    token t+1; the last position of every sequence has none (-1)."""
    tokens = np.asarray(tokens)
    t = np.full(tokens.shape, -1, dtype=np.int64)
    t[:, :-1] = tokens[:, 1:]
    return t.reshape(-1)


def sft_loss(logp, targets):
    """Mean negative log-likelihood over positions with a target.
    Returns (loss, dloss/dlogp)."""
    valid = targets >= 0
    n = int(valid.sum())
    loss = -np.sum(logp[valid]) / n
    dlogp = np.where(valid, -1.0 / n, 0.0).astype(logp.dtype)
    return loss, dlogp


def response_mask(seq_len, prompt_len, n_seq):
    """Positions whose target is a response token: t = prompt_len-1 .. S-2 in
    every sequence (they predict tokens prompt_len .. S-1)."""
    m = np.zeros((n_seq, seq_len), dtype=bool)
    m[:, prompt_len - 1:seq_len - 1] = True
    return m.reshape(-1)


def dpo_loss(logp_policy, logp_ref, seq_len, prompt_len, beta):
    """DPO on one preference pair laid out as two sequences (chosen, rejected).

    pc, pr = summed response log-probs under the policy, rc, rr under the
    reference; z = beta ((pc - rc) - (pr - rr)); loss = -log sigmoid(z).
    Returns (loss, dloss/dlogp_policy [T], z)."""
    mask = response_mask(seq_len, prompt_len, 2)
    S = seq_len
    pc = np.sum(logp_policy[:S][mask[:S]])
    pr = np.sum(logp_policy[S:][mask[S:]])
    rc = np.sum(logp_ref[:S][mask[:S]])
    rr = np.sum(logp_ref[S:][mask[S:]])
    z = beta * ((pc - rc) - (pr - rr))
    loss = -log_sigmoid(z)
    g = beta * sigmoid(-z)          # -dloss/dpc = dloss/dpr
    d = np.zeros_like(logp_policy)
    d[:S][mask[:S]] = -g
    d[S:][mask[S:]] = g
    return loss, d, z


# --------------------------------------------------------------------------
# whole steps
# --------------------------------------------------------------------------

def embed(head, tokens):
    """h0 = rows of the (frozen) embedding table."""
    return head["embed"][np.asarray(tokens).reshape(-1)]


def forward_stack(cfg, layers, lora, head, tokens, adapter_enabled=True,
                  dequantize_layer=None):
    """Forward over the stack.  ``layers`` is a list of per-layer weight dicts,
    or, when ``dequantize_layer`` is given, of opaque records that it turns
    into weight dicts one layer at a time (the streamed schedule)."""
    n_seq = np.asarray(tokens).shape[0]
    h = embed(head, tokens)
    inputs = []
    for i in range(cfg.n_layers):
        lw = layers[i] if dequantize_layer is None else dequantize_layer(layers[i])
        inputs.append(h)
        h, _ = layer_forward(cfg, lw, lora[i], h, n_seq, adapter_enabled)
    return h, inputs


def backward_stack(cfg, layers, lora, head, inputs, dh_top, n_seq,
                   dequantize_layer=None):
    """Backward from the top, recomputing each layer's forward from its saved
    input.  Returns (dh0, grads list per layer)."""
    grads = [None] * cfg.n_layers
    dh = dh_top
    for i in reversed(range(cfg.n_layers)):
        lw = layers[i] if dequantize_layer is None else dequantize_layer(layers[i])
        _, cache = layer_forward(cfg, lw, lora[i], inputs[i], n_seq, True)
        dh, grads[i] = layer_backward(cfg, lw, lora[i], cache, dh)
    return dh, grads


def sgd(lora, grads, lr):
    """theta <- theta - lr * grad for every adapter matrix (returns new dicts)."""
    out = []
    for lo, gr in zip(lora, grads):
        new = {}
        for name, (A, B) in lo.items():
            dA, dB = gr[name]
            new[name] = (A - A.dtype.type(lr) * dA, B - B.dtype.type(lr) * dB)
        out.append(new)
    return out


def sft_step(cfg, layers, lora, head, tokens, lr, dequantize_layer=None):
    """One LoRA-SFT step.  Returns dict(loss, logp, grads, lora_new, dh0)."""
    tokens = np.asarray(tokens)
    n_seq = tokens.shape[0]
    hL, inputs = forward_stack(cfg, layers, lora, head, tokens, True, dequantize_layer)
    targets = sft_targets(tokens)
    logp, hc = head_logprobs(cfg, head, hL, targets)
    loss, dlogp = sft_loss(logp, targets)
    dh = head_backward(cfg, head, hc, dlogp)
    dh0, grads = backward_stack(cfg, layers, lora, head, inputs, dh, n_seq,
                                dequantize_layer)
    return dict(loss=loss, logp=logp, grads=grads, lora_new=sgd(lora, grads, lr),
                dh0=dh0, targets=targets)


def dpo_step(cfg, layers, lora, head, chosen, rejected, prompt_len, beta, lr,
             dequantize_layer=None):
    """One LoRA-DPO step on one pair.  The reference log-probs come from the
    same frozen base run again with the adapter switched off; no second copy
    of the weights exists.  Returns dict(loss, z, logp_policy, logp_ref, grads,
    lora_new)."""
    tokens = np.stack([np.asarray(chosen), np.asarray(rejected)])
    S = tokens.shape[1]
    targets = sft_targets(tokens)
    h_ref, _ = forward_stack(cfg, layers, lora, head, tokens, False, dequantize_layer)
    logp_ref, _ = head_logprobs(cfg, head, h_ref, targets)
    hL, inputs = forward_stack(cfg, layers, lora, head, tokens, True, dequantize_layer)
    logp_pol, hc = head_logprobs(cfg, head, hL, targets)
    loss, dlogp, z = dpo_loss(logp_pol, logp_ref, S, prompt_len, beta)
    dh = head_backward(cfg, head, hc, dlogp)
    _, grads = backward_stack(cfg, layers, lora, head, inputs, dh, 2, dequantize_layer)
    return dict(loss=loss, z=z, logp_policy=logp_pol, logp_ref=logp_ref,
                grads=grads, lora_new=sgd(lora, grads, lr))


# --------------------------------------------------------------------------
# other preference losses over the same streamed base
# --------------------------------------------------------------------------
# The pages list ORPO, SimPO and KTO as running over layer streaming (axbrief
# article, "The Architecture of Low-VRAM Alignment"; the evermx page); they
# give no formulas.  The plainest readings, on one pair laid out as two
# sequences (chosen, rejected) with response targets at positions
# prompt_len-1 .. S-2:
#   SimPO  u = beta (mean_c - mean_r) - gamma,  loss = -log sigmoid(u)
#          (mean_* = average response log-prob; reference-free)
#   ORPO   loss = -mean_c - lam * log sigmoid(odds_c - odds_r),
#          odds(m) = m - log(1 - exp(m))  (log-odds of the average token
#          probability exp(m); reference-free)
#   KTO    r_* = sum_* (policy) - sum_* (reference); chosen desirable,
#          rejected undesirable, reference point 0:
#          loss = (1 - sigmoid(beta r_c)) + (1 - sigmoid(-beta r_r))
# Each returns (loss, dloss/dlogp_policy [2S], aux dict).

def _pair_stats(logp, seq_len, prompt_len):
    mask = response_mask(seq_len, prompt_len, 2)
    S = seq_len
    n_c = int(mask[:S].sum())
    n_r = int(mask[S:].sum())
    s_c = np.sum(logp[:S][mask[:S]])
    s_r = np.sum(logp[S:][mask[S:]])
    return mask, n_c, n_r, s_c, s_r


def simpo_loss(logp, seq_len, prompt_len, beta, gamma):
    mask, n_c, n_r, s_c, s_r = _pair_stats(logp, seq_len, prompt_len)
    S = seq_len
    u = beta * (s_c / n_c - s_r / n_r) - gamma
    loss = -log_sigmoid(u)
    g = sigmoid(-u)                       # -dloss/du
    d = np.zeros_like(logp)
    d[:S][mask[:S]] = -g * beta / n_c
    d[S:][mask[S:]] = g * beta / n_r
    return loss, d, dict(u=u)


def log_odds(m):
    """log(p / (1 - p)) for p = exp(m), m < 0."""
    return m - np.log(-np.expm1(m))


def orpo_loss(logp, seq_len, prompt_len, lam):
    mask, n_c, n_r, s_c, s_r = _pair_stats(logp, seq_len, prompt_len)
    S = seq_len
    m_c, m_r = s_c / n_c, s_r / n_r
    v = log_odds(m_c) - log_odds(m_r)
    loss = -m_c - lam * log_sigmoid(v)
    # d log_odds / dm = 1 / (1 - exp(m))
    dv_c = 1.0 / (-np.expm1(m_c))
    dv_r = 1.0 / (-np.expm1(m_r))
    g = lam * sigmoid(-v)                 # -dloss/dv from the odds term
    d = np.zeros_like(logp)
    d[:S][mask[:S]] = (-1.0 - g * dv_c) / n_c
    d[S:][mask[S:]] = (g * dv_r) / n_r
    return loss, d, dict(v=v)


def kto_loss(logp_policy, logp_ref, seq_len, prompt_len, beta):
    mask, n_c, n_r, pc, pr = _pair_stats(logp_policy, seq_len, prompt_len)
    _, _, _, rc, rr = _pair_stats(logp_ref, seq_len, prompt_len)
    S = seq_len
    r_c, r_r = pc - rc, pr - rr
    loss = (1.0 - sigmoid(beta * r_c)) + (1.0 - sigmoid(-beta * r_r))
    sc = sigmoid(beta * r_c)
    sr = sigmoid(-beta * r_r)
    d = np.zeros_like(logp_policy)
    d[:S][mask[:S]] = -beta * sc * (1.0 - sc)
    d[S:][mask[S:]] = beta * sr * (1.0 - sr)
    return loss, d, dict(r_c=r_c, r_r=r_r)


def pref_step(cfg, layers, lora, head, chosen, rejected, prompt_len, kind, beta, param, lr):
    """One LoRA step with a preference loss ``kind`` (dpo, simpo, orpo, kto);
    param is gamma (simpo) or lambda (orpo).  Reference log-probs, when the
    loss uses them, come from the same base with the adapter off."""
    tokens = np.stack([np.asarray(chosen), np.asarray(rejected)])
    S = tokens.shape[1]
    targets = sft_targets(tokens)
    ref = None
    if kind in ("dpo", "kto"):
        h_ref, _ = forward_stack(cfg, layers, lora, head, tokens, False)
        ref, _ = head_logprobs(cfg, head, h_ref, targets)
    hL, inputs = forward_stack(cfg, layers, lora, head, tokens, True)
    logp, hc = head_logprobs(cfg, head, hL, targets)
    if kind == "dpo":
        loss, dlogp, aux = dpo_loss(logp, ref, S, prompt_len, beta)
    elif kind == "simpo":
        loss, dlogp, a = simpo_loss(logp, S, prompt_len, beta, param)
        aux = a["u"]
    elif kind == "orpo":
        loss, dlogp, a = orpo_loss(logp, S, prompt_len, param)
        aux = a["v"]
    else:
        loss, dlogp, a = kto_loss(logp, ref, S, prompt_len, beta)
        aux = a["r_c"]
    dh = head_backward(cfg, head, hc, dlogp)
    _, grads = backward_stack(cfg, layers, lora, head, inputs, dh, 2)
    return dict(loss=loss, aux=aux, logp_policy=logp, logp_ref=ref, grads=grads,
                lora_new=sgd(lora, grads, lr))
