"""Pins for the oracle's SimPO / ORPO / KTO losses: finite differences of the
loss in the log-probs, closed forms at symmetric points, limits."""
import math

import numpy as np

from oracle import model as om

S, P = 12, 4


def _logp(seed):
    return -np.abs(np.random.default_rng(seed).standard_normal(2 * S)) - 0.05


def _fd_check(f, lp, d):
    eps = 1e-6
    mask = om.response_mask(S, P, 2)
    for t in range(2 * S):
        x = lp.copy()
        x[t] += eps
        hi = f(x)
        x[t] -= 2 * eps
        lo = f(x)
        g = (hi - lo) / (2 * eps)
        assert abs(g - d[t]) < 1e-7, (t, g, d[t])
        if not mask[t]:
            assert d[t] == 0


def test_simpo_gradient_and_closed_form():
    lp = _logp(1)
    loss, d, aux = om.simpo_loss(lp, S, P, 2.0, 0.5)
    _fd_check(lambda x: om.simpo_loss(x, S, P, 2.0, 0.5)[0], lp, d)
    # equal averages: u = -gamma, loss = log(1 + e^gamma)
    same = np.concatenate([lp[:S], lp[:S]])
    l2, _, a2 = om.simpo_loss(same, S, P, 2.0, 0.5)
    assert abs(a2["u"] + 0.5) < 1e-15 and abs(l2 - math.log1p(math.exp(0.5))) < 1e-12


def test_orpo_gradient_and_closed_form():
    lp = _logp(2)
    loss, d, aux = om.orpo_loss(lp, S, P, 0.1)
    _fd_check(lambda x: om.orpo_loss(x, S, P, 0.1)[0], lp, d)
    # log-odds of p: m = log p
    for p in (0.1, 0.5, 0.9):
        assert abs(om.log_odds(math.log(p)) - math.log(p / (1 - p))) < 1e-12
    # identical pair: odds term = lam * ln 2, NLL = -mean
    same = np.concatenate([lp[:S], lp[:S]])
    l2, _, _ = om.orpo_loss(same, S, P, 0.1)
    m = np.mean(lp[:S][om.response_mask(S, P, 1)])
    assert abs(l2 - (-m + 0.1 * math.log(2))) < 1e-12


def test_kto_gradient_and_closed_form():
    lp, lr = _logp(3), _logp(4)
    loss, d, aux = om.kto_loss(lp, lr, S, P, 0.1)
    _fd_check(lambda x: om.kto_loss(x, lr, S, P, 0.1)[0], lp, d)
    # policy == reference: both rewards 0, loss = 1/2 + 1/2
    l2, d2, _ = om.kto_loss(lp, lp, S, P, 0.1)
    assert l2 == 1.0
    assert np.allclose(d2[:S][om.response_mask(S, P, 1)], -0.1 * 0.25)


def test_dpo_matches_kto_free_limit():
    # DPO and KTO agree in sign of the chosen-side gradient (push chosen up)
    lp, lr = _logp(5), _logp(6)
    _, dd, _ = om.dpo_loss(lp, lr, S, P, 0.1)
    _, dk, _ = om.kto_loss(lp, lr, S, P, 0.1)
    m = om.response_mask(S, P, 2)
    assert np.all(dd[:S][m[:S]] < 0) and np.all(dk[:S][m[:S]] < 0)
    assert np.all(dd[S:][m[S:]] > 0) and np.all(dk[S:][m[S:]] > 0)


def test_pref_step_dpo_equals_dpo_step():
    from tests.test_oracle_model import _tiny_cfg, _tiny_model
    cfg = _tiny_cfg()
    layers, lora, head = _tiny_model(cfg, seed=31)
    rng = np.random.default_rng(32)
    pr = rng.integers(0, cfg.vocab, 3)
    ch = np.concatenate([pr, rng.integers(0, cfg.vocab, 5)])
    rj = np.concatenate([pr, rng.integers(0, cfg.vocab, 5)])
    a = om.dpo_step(cfg, layers, lora, head, ch, rj, 3, 0.2, 0.1)
    b = om.pref_step(cfg, layers, lora, head, ch, rj, 3, "dpo", 0.2, 0.0, 0.1)
    assert a["loss"] == b["loss"]
    assert np.array_equal(a["grads"][1]["v"][1], b["grads"][1]["v"][1])


def test_pref_step_finite_differences():
    from tests.test_oracle_model import _fd, _tiny_cfg, _tiny_model
    cfg = _tiny_cfg()
    layers, lora, head = _tiny_model(cfg, seed=33)
    rng = np.random.default_rng(34)
    pr = rng.integers(0, cfg.vocab, 3)
    ch = np.concatenate([pr, rng.integers(0, cfg.vocab, 5)])
    rj = np.concatenate([pr, rng.integers(0, cfg.vocab, 5)])
    for kind, beta, param in (("simpo", 2.0, 0.5), ("orpo", 0.0, 0.1), ("kto", 0.1, 0.0)):
        res = om.pref_step(cfg, layers, lora, head, ch, rj, 3, kind, beta, param, 0.1)
        A, B = lora[0]["q"]
        dA, dB = res["grads"][0]["q"]

        def loss():
            return float(om.pref_step(cfg, layers, lora, head, ch, rj, 3, kind, beta, param,
                                      0.1)["loss"])
        assert abs(_fd(loss, A, (1, 2)) - dA[1, 2]) < 1e-7 + 1e-6 * abs(dA[1, 2]), kind
        assert abs(_fd(loss, B, (2, 5)) - dB[2, 5]) < 1e-7 + 1e-6 * abs(dB[2, 5]), kind
