"""Pins for the oracle's decoder, head and losses (oracle.model): brute-force
loops, closed forms, invariants and float64 central finite differences."""
import math

import numpy as np
import pytest

from oracle import model as om
from oracle import nf4


def _tiny_cfg(n_heads=2, n_kv=1, tied=False, targets=("q", "v")):
    return om.Config(n_layers=2, hidden=32, n_heads=n_heads, n_kv_heads=n_kv,
                     head_dim=8, ffn=48, vocab=50, rms_eps=1e-5,
                     rope_theta=1e4, lora_rank=4, lora_alpha=8.0,
                     lora_targets=targets, tied=tied)


def _tiny_model(cfg, seed=0, dtype=np.float64, b_zero=False):
    rng = np.random.default_rng(seed)
    layers, lora = [], []
    for _ in range(cfg.n_layers):
        lw = {}
        for p in om.PROJ:
            N, K = cfg.proj_shape(p)
            lw[p] = (rng.standard_normal((N, K)) * 0.2).astype(dtype)
        lw["attn_norm"] = (1 + 0.1 * rng.standard_normal(cfg.hidden)).astype(dtype)
        lw["mlp_norm"] = (1 + 0.1 * rng.standard_normal(cfg.hidden)).astype(dtype)
        layers.append(lw)
        lo = {}
        for p in cfg.lora_targets:
            N, K = cfg.proj_shape(p)
            A = (rng.standard_normal((K, cfg.lora_rank)) * 0.2).astype(dtype)
            B = np.zeros((cfg.lora_rank, N), dtype) if b_zero else \
                (rng.standard_normal((cfg.lora_rank, N)) * 0.2).astype(dtype)
            lo[p] = (A, B)
        lora.append(lo)
    emb = (rng.standard_normal((cfg.vocab, cfg.hidden)) * 0.5).astype(dtype)
    lm = emb if cfg.tied else (rng.standard_normal((cfg.vocab, cfg.hidden)) * 0.3).astype(dtype)
    head = dict(embed=emb, lm_head=lm,
                final_norm=(1 + 0.1 * rng.standard_normal(cfg.hidden)).astype(dtype))
    return layers, lora, head


# ------------------------------------------------------------------ basics

def test_lora_linear_bruteforce_loops():
    rng = np.random.default_rng(1)
    M, K, N, r, s = 3, 5, 4, 2, 1.5
    x, Wt = rng.standard_normal((M, K)), rng.standard_normal((N, K))
    A, B = rng.standard_normal((K, r)), rng.standard_normal((r, N))
    y = om.lora_linear(x, Wt, A, B, s)
    for m in range(M):
        for n in range(N):
            base = sum(x[m, k] * Wt[n, k] for k in range(K))
            t = [sum(x[m, k] * A[k, j] for k in range(K)) for j in range(r)]
            low = sum(t[j] * B[j, n] for j in range(r))
            assert abs(y[m, n] - (base + s * low)) < 1e-12
    assert np.array_equal(om.lora_linear(x, Wt, A, B, s, enabled=False), x @ Wt.T)


def test_b_zero_gives_base_output_bitwise():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 16)).astype(np.float32)
    Wt = rng.standard_normal((9, 16)).astype(np.float32)
    A = rng.standard_normal((16, 4)).astype(np.float32)
    B = np.zeros((4, 9), np.float32)
    assert np.array_equal(om.lora_linear(x, Wt, A, B, 2.0), x @ Wt.T)
    dy = rng.standard_normal((7, 9)).astype(np.float32)
    dx, dA, dB = om.lora_linear_backward(x, Wt, A, B, 2.0, dy)
    assert np.array_equal(dA, np.zeros_like(A))
    assert np.array_equal(dx, dy @ Wt)
    # whole layer: adapter on with B = 0 equals adapter off, bit for bit
    cfg = _tiny_cfg()
    layers, lora, head = _tiny_model(cfg, dtype=np.float32, b_zero=True)
    h = head["embed"][np.arange(12) % cfg.vocab]
    on, _ = om.layer_forward(cfg, layers[0], lora[0], h, 2, True)
    off, _ = om.layer_forward(cfg, layers[0], lora[0], h, 2, False)
    assert np.array_equal(on, off)


def test_rmsnorm_bruteforce_and_scale_invariance():
    rng = np.random.default_rng(3)
    h = rng.standard_normal((4, 10))
    g = rng.standard_normal(10)
    y, r = om.rmsnorm(h, g, 0.0)
    for t in range(4):
        ms = sum(v * v for v in h[t]) / 10
        for i in range(10):
            assert abs(y[t, i] - g[i] * h[t, i] / math.sqrt(ms)) < 1e-12
    y2, _ = om.rmsnorm(h * 37.0, g, 0.0)
    assert np.allclose(y, y2, rtol=1e-13, atol=0)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(4)
    S, d, theta = 9, 8, 1e4
    x = rng.standard_normal((1, S, 3, d))
    cos, sin = om.rope_tables(S, d, theta, np.float64)
    y = om.rope(x, cos, sin)
    half = d // 2
    for p in range(S):
        for j in range(half):
            ang = p * theta ** (-2.0 * j / d)
            z = (x[0, p, :, j] + 1j * x[0, p, :, j + half]) * np.exp(1j * ang)
            assert np.allclose(y[0, p, :, j], z.real, atol=1e-12)
            assert np.allclose(y[0, p, :, j + half], z.imag, atol=1e-12)
    assert np.array_equal(y[0, 0], x[0, 0])                       # position 0
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))
    assert np.allclose(om.rope_backward(y, cos, sin), x, atol=1e-12)


def test_attention_bruteforce_and_special_cases():
    rng = np.random.default_rng(5)
    n_seq, S, nq, nkv, d = 2, 5, 4, 2, 3
    q = rng.standard_normal((n_seq, S, nq, d))
    k = rng.standard_normal((n_seq, S, nkv, d))
    v = rng.standard_normal((n_seq, S, nkv, d))
    o, P = om.attention(q, k, v)
    for b in range(n_seq):
        for h in range(nq):
            kv = h // 2
            for i in range(S):
                w = [math.exp(sum(q[b, i, h, e] * k[b, j, kv, e] for e in range(d)) / math.sqrt(d))
                     for j in range(i + 1)]
                z = sum(w)
                for e in range(d):
                    ref = sum(w[j] / z * v[b, j, kv, e] for j in range(i + 1))
                    assert abs(o[b, i, h, e] - ref) < 1e-12
    assert np.allclose(P.sum(-1), 1.0)
    assert np.all(np.triu(P[0, 0], 1) == 0)
    o1, _ = om.attention(q[:, :1], k[:, :1], v[:, :1])     # S = 1 returns v
    assert np.allclose(o1[:, 0, :, :], v[:, 0, [0, 0, 1, 1], :])


# ------------------------------------------------------------------ gradients

def _fd(f, x, idx, eps=1e-6):
    old = x[idx]
    x[idx] = old + eps
    fp = f()
    x[idx] = old - eps
    fm = f()
    x[idx] = old
    return (fp - fm) / (2 * eps)


@pytest.mark.parametrize("n_heads,n_kv", [(2, 1), (2, 2)])
def test_layer_backward_finite_differences(n_heads, n_kv):
    cfg = _tiny_cfg(n_heads, n_kv)
    layers, lora, head = _tiny_model(cfg, seed=9)
    lw, lo = layers[0], lora[0]
    rng = np.random.default_rng(10)
    n_seq, S = 2, 6
    h = rng.standard_normal((n_seq * S, cfg.hidden))
    R = rng.standard_normal((n_seq * S, cfg.hidden))

    def loss():
        out, _ = om.layer_forward(cfg, lw, lo, h, n_seq)
        return float(np.sum(out * R))

    _, cache = om.layer_forward(cfg, lw, lo, h, n_seq)
    dh, grads = om.layer_backward(cfg, lw, lo, cache, R)
    for idx in [(0, 0), (3, 7), (6, 31), (11, 15)]:
        assert abs(_fd(loss, h, idx) - dh[idx]) < 1e-6 * max(1, abs(dh[idx]))
    for p in cfg.lora_targets:
        A, B = lo[p]
        dA, dB = grads[p]
        for idx in [(0, 0), (5, 3), (31, 2)]:
            assert abs(_fd(loss, A, idx) - dA[idx]) < 1e-6 * max(1, abs(dA[idx]))
        for idx in [(0, 0), (3, 7), (1, B.shape[1] - 1)]:
            assert abs(_fd(loss, B, idx) - dB[idx]) < 1e-6 * max(1, abs(dB[idx]))


def test_all_projections_adapted_finite_differences():
    cfg = _tiny_cfg(targets=om.PROJ)
    layers, lora, head = _tiny_model(cfg, seed=12)
    lw, lo = layers[0], lora[0]
    rng = np.random.default_rng(13)
    h = rng.standard_normal((6, cfg.hidden))
    R = rng.standard_normal((6, cfg.hidden))

    def loss():
        return float(np.sum(om.layer_forward(cfg, lw, lo, h, 1)[0] * R))

    _, cache = om.layer_forward(cfg, lw, lo, h, 1)
    _, grads = om.layer_backward(cfg, lw, lo, cache, R)
    for p in om.PROJ:
        A, B = lo[p]
        dA, dB = grads[p]
        assert abs(_fd(loss, A, (1, 1)) - dA[1, 1]) < 1e-6 * max(1, abs(dA[1, 1]))
        assert abs(_fd(loss, B, (2, 3)) - dB[2, 3]) < 1e-6 * max(1, abs(dB[2, 3]))


def test_head_backward_finite_differences():
    cfg = _tiny_cfg()
    _, _, head = _tiny_model(cfg, seed=14)
    rng = np.random.default_rng(15)
    h = rng.standard_normal((8, cfg.hidden))
    targets = np.array([3, 7, -1, 0, 49, 12, -1, 5])
    wts = rng.standard_normal(8)

    def loss():
        return float(np.sum(om.head_logprobs(cfg, head, h, targets)[0] * wts))

    logp, hc = om.head_logprobs(cfg, head, h, targets)
    assert logp[2] == 0 and logp[6] == 0
    dh = om.head_backward(cfg, head, hc, wts)
    assert np.all(dh[2] == 0) and np.all(dh[6] == 0)
    for idx in [(0, 0), (4, 9), (7, 31)]:
        assert abs(_fd(loss, h, idx) - dh[idx]) < 1e-6 * max(1, abs(dh[idx]))


def test_sft_step_finite_differences_and_sgd():
    cfg = _tiny_cfg()
    layers, lora, head = _tiny_model(cfg, seed=16)
    tokens = np.random.default_rng(17).integers(0, cfg.vocab, (2, 7))
    res = om.sft_step(cfg, layers, lora, head, tokens, lr=0.1)

    def loss():
        hL, _ = om.forward_stack(cfg, layers, lora, head, tokens)
        t = om.sft_targets(tokens)
        return float(om.sft_loss(om.head_logprobs(cfg, head, hL, t)[0], t)[0])

    assert abs(loss() - res["loss"]) < 1e-12
    for layer in range(cfg.n_layers):
        for p in ("q", "v"):
            A, B = lora[layer][p]
            dA, dB = res["grads"][layer][p]
            assert abs(_fd(loss, A, (2, 1)) - dA[2, 1]) < 1e-7 + 1e-6 * abs(dA[2, 1])
            assert abs(_fd(loss, B, (1, 5)) - dB[1, 5]) < 1e-7 + 1e-6 * abs(dB[1, 5])
            A1, B1 = res["lora_new"][layer][p]
            assert np.allclose(A1, A - 0.1 * dA, rtol=0, atol=1e-15)
            assert np.allclose(B1, B - 0.1 * dB, rtol=0, atol=1e-15)


def test_dpo_step_finite_differences():
    cfg = _tiny_cfg()
    layers, lora, head = _tiny_model(cfg, seed=18)
    rng = np.random.default_rng(19)
    prompt = rng.integers(0, cfg.vocab, 3)
    ch = np.concatenate([prompt, rng.integers(0, cfg.vocab, 5)])
    rj = np.concatenate([prompt, rng.integers(0, cfg.vocab, 5)])
    beta = 0.5
    res = om.dpo_step(cfg, layers, lora, head, ch, rj, 3, beta, 0.1)
    tokens = np.stack([ch, rj])
    t = om.sft_targets(tokens)

    def loss():
        ref = om.head_logprobs(cfg, head, om.forward_stack(cfg, layers, lora, head, tokens, False)[0], t)[0]
        pol = om.head_logprobs(cfg, head, om.forward_stack(cfg, layers, lora, head, tokens, True)[0], t)[0]
        return float(om.dpo_loss(pol, ref, 8, 3, beta)[0])

    assert abs(loss() - res["loss"]) < 1e-12
    A, B = lora[1]["q"]
    dA, dB = res["grads"][1]["q"]
    assert abs(_fd(loss, A, (0, 2)) - dA[0, 2]) < 1e-7 + 1e-6 * abs(dA[0, 2])
    assert abs(_fd(loss, B, (3, 6)) - dB[3, 6]) < 1e-7 + 1e-6 * abs(dB[3, 6])


# ------------------------------------------------------------------ closed forms

def test_zero_lm_head_gives_ln_vocab():
    cfg = _tiny_cfg()
    layers, lora, head = _tiny_model(cfg, dtype=np.float32)
    head = dict(head, lm_head=np.zeros_like(head["lm_head"]))
    tokens = np.random.default_rng(20).integers(0, cfg.vocab, (1, 9))
    res = om.sft_step(cfg, layers, lora, head, tokens, lr=0.1)
    assert abs(res["loss"] - math.log(cfg.vocab)) < 1e-6
    assert np.all(res["grads"][0]["q"][0] == 0)      # no signal reaches the adapter


def test_dpo_policy_equals_reference_gives_ln2():
    cfg = _tiny_cfg()
    layers, lora, head = _tiny_model(cfg, dtype=np.float32, b_zero=True)
    rng = np.random.default_rng(21)
    prompt = rng.integers(0, cfg.vocab, 4)
    ch = np.concatenate([prompt, rng.integers(0, cfg.vocab, 6)])
    rj = np.concatenate([prompt, rng.integers(0, cfg.vocab, 6)])
    res = om.dpo_step(cfg, layers, lora, head, ch, rj, 4, 0.1, 0.1)
    assert res["z"] == 0.0
    assert res["loss"] == np.float32(math.log(2.0)) or abs(res["loss"] - math.log(2)) < 1e-7
    assert np.array_equal(res["logp_policy"], res["logp_ref"])


def test_dpo_loss_symmetry_and_gradient_closed_form():
    rng = np.random.default_rng(22)
    S, P, beta = 10, 4, 0.3
    lp = rng.standard_normal(2 * S)
    lr_ = rng.standard_normal(2 * S)
    loss, d, z = om.dpo_loss(lp, lr_, S, P, beta)
    swap = np.concatenate([lp[S:], lp[:S]])
    swap_r = np.concatenate([lr_[S:], lr_[:S]])
    loss2, _, z2 = om.dpo_loss(swap, swap_r, S, P, beta)
    assert abs(z + z2) < 1e-12
    assert abs((loss - loss2) - (-z)) < 1e-12
    sig = 1 / (1 + math.exp(z))
    mask = om.response_mask(S, P, 2)
    assert np.allclose(d[:S][mask[:S]], -beta * sig) and np.allclose(d[S:][mask[S:]], beta * sig)
    assert np.all(d[~mask] == 0)
    assert mask.reshape(2, S)[0].tolist() == [False] * 3 + [True] * 6 + [False]


def test_causality():
    cfg = _tiny_cfg()
    layers, lora, head = _tiny_model(cfg, seed=23)
    tokens = np.random.default_rng(24).integers(0, cfg.vocab, (1, 10))
    t = om.sft_targets(tokens)
    lp1 = om.head_logprobs(cfg, head, om.forward_stack(cfg, layers, lora, head, tokens)[0], t)[0]
    tok2 = tokens.copy()
    tok2[0, 6] = (tok2[0, 6] + 1) % cfg.vocab
    t2 = om.sft_targets(tok2)
    lp2 = om.head_logprobs(cfg, head, om.forward_stack(cfg, layers, lora, head, tok2)[0], t2)[0]
    assert np.array_equal(lp1[:5], lp2[:5])       # positions < 5 never see token 6
    assert not np.array_equal(lp1[5:], lp2[5:])


def test_streamed_equals_resident_bitwise():
    """Dequantizing layer by layer inside the loop gives the same bits as
    dequantizing the whole stack up front."""
    cfg = _tiny_cfg()
    layers, lora, head = _tiny_model(cfg, dtype=np.float32)
    records = []
    for lw in layers:
        rec = {p: nf4.quantize(lw[p]) + (lw[p].shape,) for p in om.PROJ}
        rec["attn_norm"], rec["mlp_norm"] = lw["attn_norm"], lw["mlp_norm"]
        records.append(rec)

    def deq(rec):
        out = {p: nf4.dequantize(rec[p][0], rec[p][1], int(np.prod(rec[p][2]))).reshape(rec[p][2])
               for p in om.PROJ}
        out["attn_norm"], out["mlp_norm"] = rec["attn_norm"], rec["mlp_norm"]
        return out

    resident = [deq(r) for r in records]
    tokens = np.random.default_rng(25).integers(0, cfg.vocab, (1, 8))
    a = om.sft_step(cfg, resident, lora, head, tokens, 0.1)
    b = om.sft_step(cfg, records, lora, head, tokens, 0.1, dequantize_layer=deq)
    assert a["loss"] == b["loss"]
    for la, lb in zip(a["grads"], b["grads"]):
        for p in la:
            assert np.array_equal(la[p][0], lb[p][0]) and np.array_equal(la[p][1], lb[p][1])


def test_float32_oracle_agrees_with_float64():
    cfg = _tiny_cfg()
    l64, lo64, h64 = _tiny_model(cfg, seed=26)
    cast = lambda d: {k: (v.astype(np.float32) if isinstance(v, np.ndarray) else v) for k, v in d.items()}
    l32 = [cast(l) for l in l64]
    lo32 = [{p: (A.astype(np.float32), B.astype(np.float32)) for p, (A, B) in lo.items()} for lo in lo64]
    h32 = cast(h64)
    tokens = np.random.default_rng(27).integers(0, cfg.vocab, (1, 12))
    r64 = om.sft_step(cfg, l64, lo64, h64, tokens, 0.1)
    r32 = om.sft_step(cfg, l32, lo32, h32, tokens, 0.1)
    assert abs(r32["loss"] - r64["loss"]) < 1e-5 * abs(r64["loss"])
    dA64 = r64["grads"][0]["q"][0]
    dA32 = r32["grads"][0]["q"][0]
    assert np.linalg.norm(dA32 - dA64) < 1e-4 * np.linalg.norm(dA64)
