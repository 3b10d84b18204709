"""GPU parity of whole training steps through the C ABI.

* SFT on the tiny decoder (2 layers, hidden 256, 4 heads, FFN 688, vocab
  1024, seq 64; LoRA r=8, alpha=16 on q, v; B = 0 then one SGD step, lr 0.1):
  step 1 compares loss, log-probs and dB (dA is exactly 0 on both sides) and
  the updated adapters; the oracle's updated adapters are then loaded into
  the GPU and step 2 compares again with dA != 0.
* DPO on the tiny decoder: policy == reference (B = 0) gives ln 2 and equal
  log-probs bit for bit; with B != 0 loss, z and gradients match the oracle.
* streamed (host RAM or file) and resident runs are bit-identical, and the
  scheduler copies exactly the expected number of layer records.
"""
import math
import os
import sys
import tempfile

import numpy as np
import pytest

import synth
from oracle import model as om
from tests.modelbuild import assert_close, gpu_model, oracle_model, rel

pytestmark = pytest.mark.gpu
TINY = synth.WORKLOADS["tiny"]
LR = 0.1
# Two sequences of 128 tokens (256 per step), GQA, every projection adapted:
# all forward projections (K = 256 or 704, multiples of 64) run the 256 x 256
# forward NF4 kernel, with C_F32 and residual (C_F32_RES) outputs.
SMALL256 = dict(wid=5, n_layers=2, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                ffn=704, vocab=1024, rms_eps=1e-5, rope_theta=1e4, lora_rank=8,
                lora_alpha=16.0, tied=False, n_seq=2, seq_len=128)
ALL7 = ("q", "k", "v", "o", "gate", "up", "down")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


def _dev_tokens(torch, tokens):
    from layer_streamed_nf4_double_amd.trainer import sft_targets
    tok = torch.from_numpy(np.ascontiguousarray(tokens.reshape(-1).astype(np.int32))).cuda()
    tgt = torch.from_numpy(sft_targets(tokens)).cuda()
    return tok, tgt


def _grads(m, w, targets=("q", "v")):
    out = []
    for layer in range(w["n_layers"]):
        d = {}
        for p in targets:
            A, B, dA, dB = m.get_lora(layer, p)
            d[p] = (A, B, dA, dB)
        out.append(d)
    return out


def _run_sft(torch, m, tokens, lr=LR):
    tok, tgt = _dev_tokens(torch, tokens)
    n_seq, S = tokens.shape
    loss = m.sft_step(tok, tgt, n_seq, S, lr)
    m.sync()
    return float(loss[0].item()), m.logp[: n_seq * S].cpu().numpy().copy()


def test_sft_tiny_two_steps_vs_oracle(torch):
    w = TINY
    tokens = synth.sft_tokens(w)
    say("[sft-tiny] oracle")
    cfg, layers, lora, head = oracle_model(w, b_zero=True)
    o1 = om.sft_step(cfg, layers, lora, head, tokens, LR)
    say("[sft-tiny] gpu stream_host step 1")
    m = gpu_model(w, "stream_host", b_zero=True)
    loss1, logp1 = _run_sft(torch, m, tokens)
    g1 = _grads(m, w)
    assert abs(loss1 - o1["loss"]) <= 2e-2 * abs(o1["loss"])
    assert_close(logp1, o1["logp"], 2e-2, "logp step 1")
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            A, B, dA, dB = g1[layer][p]
            odA, odB = o1["grads"][layer][p]
            assert np.all(dA == 0) and np.all(odA == 0), "dA must vanish at B = 0"
            assert_close(dB, odB, 5e-2, f"dB L{layer} {p} step 1")
            oA, oB = o1["lora_new"][layer][p]
            assert np.array_equal(A, oA.astype(np.float32)), "A unchanged by SGD at dA = 0"
            assert_close(B, oB, 5e-2, f"B' L{layer} {p}")
    # step 2 from identical parameters: the oracle's updated adapters
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            A, B = o1["lora_new"][layer][p]
            m.set_lora(layer, p, A.astype(np.float32), B.astype(np.float32))
    say("[sft-tiny] gpu step 2")
    o2 = om.sft_step(cfg, layers, o1["lora_new"], head, tokens, LR)
    loss2, logp2 = _run_sft(torch, m, tokens)
    g2 = _grads(m, w)
    assert abs(loss2 - o2["loss"]) <= 2e-2 * abs(o2["loss"])
    assert_close(logp2, o2["logp"], 2e-2, "logp step 2")
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            _, _, dA, dB = g2[layer][p]
            odA, odB = o2["grads"][layer][p]
            assert np.abs(odA).max() > 0
            assert_close(dA, odA, 5e-2, f"dA L{layer} {p} step 2")
            assert_close(dB, odB, 5e-2, f"dB L{layer} {p} step 2")
    m.close()


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def _dpo_bars(od, beta):
    """(loss bar, z bar).  z is a small difference of large log-prob sums:
    2e-2 relative with a floor of beta.  The loss -log sigmoid(z) is a
    function of z alone, so besides 2e-2 relative it may move by what z's bar
    allows through d loss / dz = -sigmoid(-z) (for large z the loss is
    exponentially small and its relative error equals z's absolute error)."""
    z = float(od["z"])
    zbar = 2e-2 * max(abs(z), beta)
    sig = 1.0 / (1.0 + math.exp(z))
    return max(2e-2 * abs(float(od["loss"])), sig * zbar), zbar


def _two_step_record(torch, m, w, tokens):
    rec = []
    for _ in range(2):
        loss, logp = _run_sft(torch, m, tokens)
        rec.append((np.float32(loss), logp, _grads(m, w)))
    return rec


def _assert_bit_identical(a, b):
    for (la, pa, ga), (lb, pb, gb) in zip(a, b):
        assert _bits(la) == _bits(lb)
        assert np.array_equal(_bits(pa), _bits(pb))
        for da, db in zip(ga, gb):
            for p in da:
                for x, y in zip(da[p], db[p]):
                    assert np.array_equal(_bits(x), _bits(y))


def _status(fn, *args):
    from layer_streamed_nf4_double_amd import _lib as L
    try:
        fn(*args)
    except L.LsnError as e:
        return e.status
    return L.LSN_OK


def test_calls_out_of_order_fail_and_change_nothing(torch):
    """Calls that break the pass contract return LSN_ERR_STATE (bad pass
    arguments LSN_ERR_INVALID) before enqueueing anything: the context is not
    poisoned, and the two SFT steps that follow give the same bits as on a
    fresh model."""
    from layer_streamed_nf4_double_amd import _lib as L
    w = dict(TINY, n_layers=3)
    tokens = synth.tokens((1, 64), w["vocab"], 5)
    say("[order] fresh model")
    ref = gpu_model(w, "stream_host", b_zero=False, max_tokens=64)
    a = _two_step_record(torch, ref, w, tokens)
    ref.close()
    say("[order] misuse, then the same steps")
    m = gpu_model(w, "stream_host", b_zero=False, max_tokens=64)
    h = torch.zeros(64, w["hidden"], device="cuda")
    ST, INV = L.LSN_ERR_STATE, L.LSN_ERR_INVALID
    assert _status(L.lsn_forward_layer, m.ctx, 0, h, h) == ST          # outside a pass
    L.lsn_begin_pass(m.ctx, L.LSN_PASS_FWD, 1, 64)
    assert _status(L.lsn_forward_layer, m.ctx, 1, h, h) == ST          # layer 0 comes first
    assert _status(L.lsn_backward_layer, m.ctx, 0, h, h, h) == ST      # not a backward pass
    assert _status(L.lsn_begin_pass, m.ctx, L.LSN_PASS_FWD, 1, 60) == INV   # seq_len % 8
    assert _status(L.lsn_begin_pass, m.ctx, L.LSN_PASS_FWD, 2, 64) == INV   # > max_tokens
    L.lsn_set_adapter_enabled(m.ctx, 0)
    assert _status(L.lsn_begin_pass, m.ctx, L.LSN_PASS_BWD, 1, 64) == ST
    L.lsn_set_adapter_enabled(m.ctx, 1)
    L.lsn_begin_pass(m.ctx, L.LSN_PASS_BWD, 1, 64)
    L.lsn_set_adapter_enabled(m.ctx, 0)
    assert _status(L.lsn_backward_layer, m.ctx, 2, h, h, h) == ST      # adapters switched off
    assert b"adapters" in L._lib.lsn_last_error(m.ctx)
    L.lsn_set_adapter_enabled(m.ctx, 1)
    b = _two_step_record(torch, m, w, tokens)
    m.close()
    _assert_bit_identical(a, b)


@pytest.mark.parametrize("n_layers", [2, 5])
def test_streamed_equals_resident_bitwise(torch, n_layers):
    w = dict(TINY, n_layers=n_layers)
    tokens = synth.tokens((2, 64), w["vocab"], 77)
    say(f"[stream==resident] L={n_layers}")
    res = gpu_model(w, "resident", b_zero=False, max_tokens=128)
    a = _two_step_record(torch, res, w, tokens)
    res.close()
    st = gpu_model(w, "stream_host", b_zero=False, max_tokens=128)
    b = _two_step_record(torch, st, w, tokens)
    loads, nbytes, _ = st.stats()
    from layer_streamed_nf4_double_amd import _lib as L
    assert not L.lsn_file_direct_io(st.ctx)  # no file source
    st.close()
    _assert_bit_identical(a, b)
    # forward copies all L records, backward reuses the last two; the next
    # step's forward reuses the two the backward ended on
    L_ = n_layers
    want = (L_ + max(L_ - 2, 0)) + (max(L_ - 2, 0) + max(L_ - 2, 0))
    assert loads == want, (loads, want)
    with tempfile.TemporaryDirectory() as d:
        fm = gpu_model(w, "stream_file", b_zero=False, max_tokens=128,
                       store_path=os.path.join(d, "store.bin"))
        c = _two_step_record(torch, fm, w, tokens)
        say(f"[stream==resident] file source reads with O_DIRECT: {L.lsn_file_direct_io(fm.ctx)}")
        fm.close()
    _assert_bit_identical(a, c)


@pytest.mark.parametrize("mode,tied", [("stream_host", False), ("stream_file", False),
                                       ("stream_host", True)])
def test_head_on_host_matches_device_head(torch, mode, tied, tmp_path):
    """Embedding and LM-head tables in pinned host memory, W_lm streamed
    through the layer slots in two chunks (768 + 256 rows here).  Two SFT
    steps equal, bitwise, the run with the tables on the device and the same
    768-row chunks, and match the oracle within the parity bar.  The head
    displaces the two records the backward would have reused, so each step
    loads two more."""
    w = dict(TINY, n_layers=3, tied=tied)
    tokens = synth.sft_tokens(w)
    say(f"[head-on-host] {mode} tied={tied} oracle")
    cfg, layers, lora, head = oracle_model(w, b_zero=False)
    o = om.sft_step(cfg, layers, lora, head, tokens, LR)
    dev = gpu_model(w, "stream_host", b_zero=False, head_chunk_rows=768)
    a = _two_step_record(torch, dev, w, tokens)
    la, _, _ = dev.stats()
    dev.close()
    store = str(tmp_path / "store.bin") if mode == "stream_file" else None
    host = gpu_model(w, mode, b_zero=False, head_on_host=True, store_path=store)
    b = _two_step_record(torch, host, w, tokens)
    lb, _, _ = host.stats()
    host.close()
    assert lb - la == 4, (la, lb)
    lb0, pb0, _ = b[0]
    assert abs(float(lb0) - o["loss"]) <= 2e-2 * abs(o["loss"])
    assert_close(pb0, o["logp"], 2e-2, "logp vs oracle")
    _assert_bit_identical(a, b)


def test_head_on_host_dpo(torch):
    """The fused DPO step with the head tables on the host: both head passes
    (reference and policy) stream W_lm; policy == reference at B = 0 gives
    ln 2, and B != 0 equals, bitwise, the device-table run with the same
    chunks."""
    w = dict(TINY, n_layers=2)
    S, P, beta = 64, 16, 0.1
    rng_tok = synth.tokens((P,), w["vocab"], 88, synth.TID_PROMPT)
    ch = np.concatenate([rng_tok, synth.tokens((S - P,), w["vocab"], 88, synth.TID_CHOSEN)])
    rj = np.concatenate([rng_tok, synth.tokens((S - P,), w["vocab"], 88, synth.TID_REJECTED)])
    tok, tgt = _dev_tokens(torch, np.stack([ch, rj]))
    m = gpu_model(w, "stream_host", b_zero=True, max_tokens=2 * S, head_on_host=True)
    out = m.dpo_step(tok, tgt, S, P, beta, None)
    m.sync()
    assert abs(float(out.cpu().numpy()[0]) - math.log(2.0)) <= 1e-7
    m.close()
    res = []
    for hoh in (False, True):
        m = gpu_model(w, "stream_host", b_zero=False, max_tokens=2 * S, head_on_host=hoh,
                      head_chunk_rows=768)
        out = m.dpo_step(tok, tgt, S, P, beta, LR)
        m.sync()
        res.append((out.cpu().numpy()[:6].copy(), _grads(m, w)))
        m.close()
    (o0, g0), (o1, g1) = res
    assert np.array_equal(_bits(o0), _bits(o1))
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            for x, y in zip(g0[layer][p], g1[layer][p]):
                assert np.array_equal(_bits(x), _bits(y))


def test_wide_heads_long_sequence_vs_oracle(torch):
    """head_dim 272 (> 256) and a 2304-token sequence (> 2048): the shapes
    for which RoPE and the causal softmax run their scalar kernels instead of
    the 16-byte ones.  One SFT step with B != 0 against the oracle."""
    w = dict(TINY, n_layers=1, n_heads=1, n_kv_heads=1, head_dim=272, seq_len=2304)
    tokens = synth.sft_tokens(w)
    say("[wide-heads] oracle")
    cfg, layers, lora, head = oracle_model(w, b_zero=False)
    o = om.sft_step(cfg, layers, lora, head, tokens, LR)
    say("[wide-heads] gpu stream_host")
    m = gpu_model(w, "stream_host", b_zero=False)
    loss, logp = _run_sft(torch, m, tokens)
    g = _grads(m, w)
    m.close()
    assert abs(loss - o["loss"]) <= 2e-2 * abs(o["loss"])
    assert_close(logp, o["logp"], 2e-2, "logp")
    for p in ("q", "v"):
        _, _, dA, dB = g[0][p]
        oA, oB = o["grads"][0][p]
        assert_close(dA, oA, 5e-2, f"dA {p}")
        assert_close(dB, oB, 5e-2, f"dB {p}")


def _load_layer_from(m, w, layer, src_layer):
    """Loads the record built from layer src_layer's seeded weights as layer."""
    from layer_streamed_nf4_double_amd import _lib as L
    ones = np.full(w["hidden"], 0x3F80, np.uint16)
    codes, absmax = [], []
    for p in synth.PROJ:
        c, a = L.lsn_nf4_quantize(synth.layer_weights_f32(w, src_layer, p))
        codes.append(c)
        absmax.append(a)
    m.load_layer(layer, codes, absmax, ones, ones)


@pytest.mark.parametrize("mode", ["resident", "stream_host", "stream_file"])
def test_reloaded_layer_record_takes_effect(torch, mode, tmp_path):
    """A layer record rewritten between steps is what the next step uses.
    After a streamed step, layer 0 still sits in a device slot (the next
    forward would reuse it), and with the file source its record also sits
    in the reader's staging buffers; neither old copy may be served.  The
    step after the rewrite equals, bitwise, the step of a model built with
    the new record from the start."""
    w = dict(TINY, n_layers=4)
    tokens = synth.tokens((2, 64), w["vocab"], 91)
    store = (lambda n: str(tmp_path / f"{n}.bin")) if mode == "stream_file" else (lambda n: None)
    say(f"[reload] {mode}")
    m = gpu_model(w, mode, b_zero=False, max_tokens=128, store_path=store("a"))
    _, logp0 = _run_sft(torch, m, tokens, lr=None)
    _load_layer_from(m, w, 0, 3)
    loss_a, logp_a = _run_sft(torch, m, tokens, lr=None)
    ga = _grads(m, w)
    m.close()
    f = gpu_model(w, mode, b_zero=False, max_tokens=128, store_path=store("b"))
    _load_layer_from(f, w, 0, 3)
    loss_b, logp_b = _run_sft(torch, f, tokens, lr=None)
    gb = _grads(f, w)
    f.close()
    assert not np.array_equal(_bits(logp0), _bits(logp_a)), "the new record changed nothing"
    _assert_bit_identical([(np.float32(loss_a), logp_a, ga)], [(np.float32(loss_b), logp_b, gb)])


def test_dpo_tiny(torch):
    w = dict(TINY)
    S, P, beta = 64, 16, 0.1
    rng_tok = synth.tokens((P,), w["vocab"], 88, synth.TID_PROMPT)
    ch = np.concatenate([rng_tok, synth.tokens((S - P,), w["vocab"], 88, synth.TID_CHOSEN)])
    rj = np.concatenate([rng_tok, synth.tokens((S - P,), w["vocab"], 88, synth.TID_REJECTED)])
    tokens = np.stack([ch, rj])
    tok, tgt = _dev_tokens(torch, tokens)
    # policy == reference: B = 0
    say("[dpo-tiny] B=0 -> ln 2")
    m = gpu_model(w, "stream_host", b_zero=True, max_tokens=2 * S)
    out = m.dpo_step(tok, tgt, S, P, beta, None)
    m.sync()
    o = out.cpu().numpy()
    assert o[1] == 0.0, "z must be exactly 0 when the adapter contributes nothing"
    assert abs(float(o[0]) - math.log(2.0)) <= 1e-7
    assert np.array_equal(_bits(m.logp[:2 * S].cpu().numpy()),
                          _bits(m.logp_ref[:2 * S].cpu().numpy()))
    m.close()
    # B != 0: parity with the oracle
    say("[dpo-tiny] B!=0 vs oracle")
    cfg, layers, lora, head = oracle_model(w, b_zero=False)
    od = om.dpo_step(cfg, layers, lora, head, ch, rj, P, beta, LR)
    m = gpu_model(w, "stream_host", b_zero=False, max_tokens=2 * S)
    out = m.dpo_step(tok, tgt, S, P, beta, LR)
    m.sync()
    o = out.cpu().numpy()
    # z = beta * (difference of ~2.6e3-nat log-prob sums) cancels; its bar is
    # 2e-2 relative with a floor of beta (one nat of log-prob difference)
    lbar, zbar = _dpo_bars(od, beta)
    assert abs(o[0] - od["loss"]) <= lbar
    assert abs(o[1] - od["z"]) <= zbar
    assert_close(m.logp[:2 * S].cpu().numpy(), od["logp_policy"], 2e-2, "policy logp")
    assert_close(m.logp_ref[:2 * S].cpu().numpy(), od["logp_ref"], 2e-2, "reference logp")
    g = _grads(m, w)
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            _, _, dA, dB = g[layer][p]
            odA, odB = od["grads"][layer][p]
            assert_close(dA, odA, 5e-2, f"DPO dA L{layer} {p}")
            assert_close(dB, odB, 5e-2, f"DPO dB L{layer} {p}")
    m.close()


def test_all_projections_adapted_gqa(torch):
    """Every projection adapted, grouped kv heads, two sequences."""
    w = dict(TINY, n_heads=4, n_kv_heads=2, n_layers=2)
    targets = synth.PROJ
    tokens = synth.tokens((2, 32), w["vocab"], 91)
    say("[all-targets gqa]")
    cfg, layers, lora, head = oracle_model(w, b_zero=False, lora_targets=targets)
    o = om.sft_step(cfg, layers, lora, head, tokens, LR)
    m = gpu_model(w, "stream_host", b_zero=False, lora_targets=targets, max_tokens=64,
                  max_seq_len=32)
    loss, logp = _run_sft(torch, m, tokens)
    assert abs(loss - o["loss"]) <= 2e-2 * abs(o["loss"])
    assert_close(logp, o["logp"], 2e-2, "logp")
    g = _grads(m, w, targets)
    for layer in range(w["n_layers"]):
        for p in targets:
            _, _, dA, dB = g[layer][p]
            odA, odB = o["grads"][layer][p]
            assert_close(dA, odA, 5e-2, f"dA L{layer} {p}")
            assert_close(dB, odB, 5e-2, f"dB L{layer} {p}")
    m.close()


def _dpo_record(torch, m, w, tok, tgt, S, P, beta, fused):
    rec = []
    for _ in range(2):
        out = m.dpo_step(tok, tgt, S, P, beta, LR, fused=fused)
        m.sync()
        rec.append((out[:6].cpu().numpy().copy(), m.logp[:2 * S].cpu().numpy().copy(),
                    m.logp_ref[:2 * S].cpu().numpy().copy(), _grads(m, w)))
    return rec


def test_dpo_fused_reference_pass_bitwise(torch):
    """The reference forward run on the same layer copy as the policy forward
    gives the same bits as a separate adapter-off pass, with 2L instead of 3L
    record copies per step (minus the 2 reused at each pass boundary)."""
    w = dict(TINY, n_layers=5)
    S, P, beta = 64, 16, 0.1
    pr = synth.tokens((P,), w["vocab"], 89, synth.TID_PROMPT)
    ch = np.concatenate([pr, synth.tokens((S - P,), w["vocab"], 89, synth.TID_CHOSEN)])
    rj = np.concatenate([pr, synth.tokens((S - P,), w["vocab"], 89, synth.TID_REJECTED)])
    tok, tgt = _dev_tokens(torch, np.stack([ch, rj]))
    say("[dpo fused vs separate]")
    sep = gpu_model(w, "stream_host", b_zero=False, max_tokens=2 * S)
    a = _dpo_record(torch, sep, w, tok, tgt, S, P, beta, fused=False)
    loads_sep = sep.stats()[0]
    sep.close()
    fus = gpu_model(w, "stream_host", b_zero=False, max_tokens=2 * S)
    b = _dpo_record(torch, fus, w, tok, tgt, S, P, beta, fused=True)
    loads_fus = fus.stats()[0]
    fus.close()
    for (oa, la, ra, ga), (ob, lb, rb, gb) in zip(a, b):
        assert np.array_equal(_bits(oa), _bits(ob))
        assert np.array_equal(_bits(la), _bits(lb)) and np.array_equal(_bits(ra), _bits(rb))
        for da, db in zip(ga, gb):
            for p in da:
                for x, y in zip(da[p], db[p]):
                    assert np.array_equal(_bits(x), _bits(y))
    L_ = w["n_layers"]
    assert loads_sep == (3 * L_ - 2) + (3 * L_ - 4), loads_sep
    assert loads_fus == (2 * L_ - 2) + (2 * L_ - 4), loads_fus


@pytest.mark.parametrize("kind,beta,param", [("simpo", 2.0, 0.5), ("orpo", 0.0, 0.1),
                                             ("kto", 0.1, 0.0), ("dpo", 0.1, 0.0)])
def test_preference_losses_tiny(torch, kind, beta, param):
    w = dict(TINY)
    S, P = 64, 16
    pr = synth.tokens((P,), w["vocab"], 90, synth.TID_PROMPT)
    ch = np.concatenate([pr, synth.tokens((S - P,), w["vocab"], 90, synth.TID_CHOSEN)])
    rj = np.concatenate([pr, synth.tokens((S - P,), w["vocab"], 90, synth.TID_REJECTED)])
    tok, tgt = _dev_tokens(torch, np.stack([ch, rj]))
    say(f"[pref {kind}]")
    cfg, layers, lora, head = oracle_model(w, b_zero=False)
    od = om.pref_step(cfg, layers, lora, head, ch, rj, P, kind, beta, param, LR)
    m = gpu_model(w, "stream_host", b_zero=False, max_tokens=2 * S)
    out = m.pref_step(kind, tok, tgt, S, P, beta, param, LR)
    m.sync()
    o = out.cpu().numpy()
    assert abs(o[0] - od["loss"]) <= 2e-2 * abs(od["loss"]), (o[0], od["loss"])
    assert_close(m.logp[:2 * S].cpu().numpy(), od["logp_policy"], 2e-2, "policy logp")
    g = _grads(m, w)
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            _, _, dA, dB = g[layer][p]
            odA, odB = od["grads"][layer][p]
            assert_close(dA, odA, 5e-2, f"{kind} dA L{layer} {p}")
            assert_close(dB, odB, 5e-2, f"{kind} dB L{layer} {p}")
    m.close()


def test_adapter_export_import_round_trip(torch, tmp_path):
    """Saved adapters load back bit for bit into a fresh context and change
    the model's output (they are not inert)."""
    from layer_streamed_nf4_double_amd import adapter as ad
    w = dict(TINY)
    tokens = synth.sft_tokens(w)
    say("[adapter export/import]")
    m = gpu_model(w, "stream_host", b_zero=False)
    _run_sft(torch, m, tokens)                       # one step: adapters move
    ad.save_adapter(m, str(tmp_path / "adapter"))
    want = _grads(m, w)
    loss_m, _ = _run_sft(torch, m, tokens, lr=None)  # forward with trained adapters
    m.close()
    fresh = gpu_model(w, "stream_host", b_zero=True)
    loss_base, _ = _run_sft(torch, fresh, tokens, lr=None)
    ad.load_adapter(fresh, str(tmp_path / "adapter"))
    got = _grads(fresh, w)
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            assert np.array_equal(_bits(got[layer][p][0]), _bits(want[layer][p][0]))
            assert np.array_equal(_bits(got[layer][p][1]), _bits(want[layer][p][1]))
    loss_loaded, _ = _run_sft(torch, fresh, tokens, lr=None)
    fresh.close()
    assert _bits(np.float32(loss_loaded)) == _bits(np.float32(loss_m))
    assert loss_loaded != loss_base


def test_auto_source_and_preflight(torch):
    from layer_streamed_nf4_double_amd import adapter as ad
    from layer_streamed_nf4_double_amd.trainer import LayerStreamedLoRA
    w = dict(TINY)
    m = LayerStreamedLoRA(w, "auto")
    assert m.mode == "stream_host"          # a 2-layer tiny stack fits in RAM
    m.close()
    f = LayerStreamedLoRA(w, "stream_file")  # no store_path: a temporary store file
    path = f.cfg.store_path.decode()
    assert os.path.exists(path)
    f.close()
    assert not os.path.exists(path)         # removed with the model that made it
    free, _ = torch.cuda.mem_get_info()
    with pytest.raises(ad.NoFit):           # a workspace larger than the card
        ad.plan_run(1, 1, free + (1 << 30), free, 1 << 40)


def test_sft_large_vocab_multichunk_head_vs_oracle(torch):
    """One SFT step with a 70000-entry vocabulary at 2 x 152 tokens: the LM
    head runs three vocabulary chunks (32768, 32768, 4464 rows: online
    log-sum-exp across chunks and the expected-row accumulator rescaled to
    the running max chunk by chunk, then dh from it) on the 256 x 256 bf16
    kernels with a ragged row tile and a ragged last column tile.  A head
    backward after a logprobs pass that kept no accumulator is refused."""
    w = dict(SMALL256, n_layers=1, vocab=70000, n_seq=2, seq_len=152)
    tokens = synth.sft_tokens(w)
    say("[sft-vocab70000] oracle")
    cfg, layers, lora, head = oracle_model(w, b_zero=False, lora_targets=ALL7)
    o = om.sft_step(cfg, layers, lora, head, tokens, LR)
    say("[sft-vocab70000] gpu stream_host")
    m = gpu_model(w, "stream_host", b_zero=False, lora_targets=ALL7)
    loss, logp = _run_sft(torch, m, tokens)
    g = _grads(m, w, ALL7)
    assert abs(loss - o["loss"]) <= 2e-2 * abs(o["loss"])
    assert_close(logp, o["logp"], 2e-2, "logp")
    for p in ALL7:
        _, _, dA, dB = g[0][p]
        oA, oB = o["grads"][0][p]
        assert_close(dA, oA, 5e-2, f"dA {p}")
        assert_close(dB, oB, 5e-2, f"dB {p}")
    from layer_streamed_nf4_double_amd import _lib as L
    T = w["n_seq"] * w["seq_len"]
    _, tgt = _dev_tokens(torch, tokens)
    hL = m.hs[w["n_layers"]][:T]
    L.lsn_lm_head_logprobs(m.ctx, hL, tgt, m.logp[:T], 0)
    with pytest.raises(L.LsnError):
        L.lsn_lm_head_backward(m.ctx, hL, tgt, m.dlogp[:T], m.dh[:T])


def test_sft_256_tokens_all_projections_vs_oracle(torch):
    """One SFT step at 256 tokens with B != 0 on all seven projections (the
    forward NF4 GEMMs run the 256 x 256 kernel), then streamed == resident
    bitwise."""
    w = SMALL256
    tokens = synth.sft_tokens(w)
    say("[sft-256] oracle")
    cfg, layers, lora, head = oracle_model(w, b_zero=False, lora_targets=ALL7)
    o = om.sft_step(cfg, layers, lora, head, tokens, LR)
    say("[sft-256] gpu stream_host")
    m = gpu_model(w, "stream_host", b_zero=False, lora_targets=ALL7)
    loss, logp = _run_sft(torch, m, tokens)
    g = _grads(m, w, ALL7)
    assert abs(loss - o["loss"]) <= 2e-2 * abs(o["loss"])
    assert_close(logp, o["logp"], 2e-2, "logp")
    for layer in range(w["n_layers"]):
        for p in ALL7:
            _, _, dA, dB = g[layer][p]
            oA, oB = o["grads"][layer][p]
            assert_close(dA, oA, 5e-2, f"dA L{layer} {p}")
            assert_close(dB, oB, 5e-2, f"dB L{layer} {p}")
    say("[sft-256] gpu resident")
    r = gpu_model(w, "resident", b_zero=False, lora_targets=ALL7)
    loss_r, logp_r = _run_sft(torch, r, tokens)
    assert np.array_equal(np.float32(loss_r).view(np.uint32), np.float32(loss).view(np.uint32))
    assert np.array_equal(logp_r.view(np.uint32), logp.view(np.uint32))
    gr = _grads(r, w, ALL7)
    for layer in range(w["n_layers"]):
        for p in ALL7:
            for u, v in zip(g[layer][p], gr[layer][p]):
                assert np.array_equal(np.asarray(u).view(np.uint32), np.asarray(v).view(np.uint32))


# 512 tokens with an FFN of 8208 features (64 x 128 + 16): the gate|up GEMM
# takes the SwiGLU epilogue (unsplit 256 x 256 tiles of 128 features), whose
# last feature tile is ragged; every projection adapted, so the epilogue also
# adds the gate and up low-rank columns and the backward rebuilds a for the
# down adapter.
RAGGED_FFN = dict(wid=6, n_layers=2, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                  ffn=8208, vocab=1024, rms_eps=1e-5, rope_theta=1e4, lora_rank=8,
                  lora_alpha=16.0, tied=False, n_seq=2, seq_len=256)


def test_sft_swiglu_epilogue_ragged_ffn_vs_oracle(torch):
    """SFT step with the fused SwiGLU epilogue on a ragged feature count
    against the oracle, then streamed == resident bitwise."""
    w = RAGGED_FFN
    tokens = synth.sft_tokens(w)
    say("[sft-ragged-ffn] oracle")
    cfg, layers, lora, head = oracle_model(w, b_zero=False, lora_targets=ALL7)
    o = om.sft_step(cfg, layers, lora, head, tokens, LR)
    say("[sft-ragged-ffn] gpu stream_host")
    m = gpu_model(w, "stream_host", b_zero=False, lora_targets=ALL7)
    loss, logp = _run_sft(torch, m, tokens)
    g = _grads(m, w, ALL7)
    m.close()
    assert abs(loss - o["loss"]) <= 2e-2 * abs(o["loss"])
    assert_close(logp, o["logp"], 2e-2, "logp")
    for layer in range(w["n_layers"]):
        for p in ALL7:
            _, _, dA, dB = g[layer][p]
            oA, oB = o["grads"][layer][p]
            assert_close(dA, oA, 5e-2, f"dA L{layer} {p}")
            assert_close(dB, oB, 5e-2, f"dB L{layer} {p}")
    say("[sft-ragged-ffn] gpu resident (bitwise)")
    r = gpu_model(w, "resident", b_zero=False, lora_targets=ALL7)
    loss_r, logp_r = _run_sft(torch, r, tokens)
    gr = _grads(r, w, ALL7)
    r.close()
    assert np.array_equal(_bits(np.float32(loss_r)), _bits(np.float32(loss)))
    assert np.array_equal(_bits(logp_r), _bits(logp))
    for layer in range(w["n_layers"]):
        for p in ALL7:
            for u, v in zip(g[layer][p], gr[layer][p]):
                assert np.array_equal(_bits(np.asarray(u)), _bits(np.asarray(v)))


# The 8B layer shape at the bench's 512 tokens (hidden 4096, 32 q / 8 kv heads
# of 128, FFN 14336, the same seeded layers as the 8B workload), two layers and
# a 1024-entry vocabulary so that the float64 oracle stays within seconds.
LLAMA8B_2L = dict(synth.WORKLOADS["llama3.1-8b-shaped"], n_layers=2, vocab=1024)


@pytest.fixture(scope="module")
def llama2l_oracle():
    return oracle_model(LLAMA8B_2L, b_zero=False)


def test_sft_llama8b_layer_shape_vs_oracle(torch, llama2l_oracle):
    """One streamed SFT step at the full 8B layer shape (the kernels and launch
    configuration the bench times) against the oracle; then streamed ==
    resident bitwise at this shape."""
    w = LLAMA8B_2L
    tokens = synth.sft_tokens(w)
    say("[sft-8b-shape] oracle")
    cfg, layers, lora, head = llama2l_oracle
    o = om.sft_step(cfg, layers, lora, head, tokens, LR)
    say("[sft-8b-shape] gpu stream_host")
    m = gpu_model(w, "stream_host", b_zero=False)
    loss, logp = _run_sft(torch, m, tokens)
    g = _grads(m, w)
    assert abs(loss - o["loss"]) <= 2e-2 * abs(o["loss"])
    assert_close(logp, o["logp"], 2e-2, "logp")
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            _, _, dA, dB = g[layer][p]
            oA, oB = o["grads"][layer][p]
            assert_close(dA, oA, 5e-2, f"dA L{layer} {p}")
            assert_close(dB, oB, 5e-2, f"dB L{layer} {p}")
    m.close()
    say("[sft-8b-shape] gpu resident (bitwise)")
    r = gpu_model(w, "resident", b_zero=False)
    loss_r, logp_r = _run_sft(torch, r, tokens)
    gr = _grads(r, w)
    r.close()
    assert np.array_equal(_bits(np.float32(loss_r)), _bits(np.float32(loss)))
    assert np.array_equal(_bits(logp_r), _bits(logp))
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            for u, v in zip(g[layer][p], gr[layer][p]):
                assert np.array_equal(_bits(np.asarray(u)), _bits(np.asarray(v)))


def test_dpo_llama8b_layer_shape_vs_oracle(torch, llama2l_oracle):
    """One streamed DPO step (fused reference pass) on one 2 x 512-token pair
    at the full 8B layer shape against the oracle."""
    w = LLAMA8B_2L
    S, beta = w["seq_len"], synth.DPO_PAIR["beta"]
    P = synth.dpo_prompt_len(w)
    ch, rj = synth.dpo_pair(w)
    tok, tgt = _dev_tokens(torch, np.stack([ch, rj]))
    say("[dpo-8b-shape] oracle")
    cfg, layers, lora, head = llama2l_oracle
    od = om.dpo_step(cfg, layers, lora, head, ch, rj, P, beta, LR)
    say("[dpo-8b-shape] gpu stream_host")
    m = gpu_model(w, "stream_host", b_zero=False, max_tokens=2 * S)
    out = m.dpo_step(tok, tgt, S, P, beta, LR)
    m.sync()
    o = out.cpu().numpy()
    lbar, zbar = _dpo_bars(od, beta)
    assert abs(o[0] - od["loss"]) <= lbar
    assert abs(o[1] - od["z"]) <= zbar
    assert_close(m.logp[:2 * S].cpu().numpy(), od["logp_policy"], 2e-2, "policy logp")
    assert_close(m.logp_ref[:2 * S].cpu().numpy(), od["logp_ref"], 2e-2, "reference logp")
    g = _grads(m, w)
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            _, _, dA, dB = g[layer][p]
            odA, odB = od["grads"][layer][p]
            assert_close(dA, odA, 5e-2, f"DPO dA L{layer} {p}")
            assert_close(dB, odB, 5e-2, f"DPO dB L{layer} {p}")
    m.close()


def test_sft_qwen3b_layer_shape_vs_oracle(torch):
    """One streamed SFT step at the 3B layer shape (hidden 2048, 16 q / 2 kv
    heads of 128, FFN 11008, tied embedding, RoPE theta 1e6, eps 1e-6), two
    layers, vocabulary 1024, 512 tokens, against the oracle; then the same
    step with the base resident gives the same bits."""
    w = dict(synth.WORKLOADS["qwen2.5-3b-shaped"], n_layers=2, vocab=1024)
    tokens = synth.sft_tokens(w)
    say("[sft-3b-shape] oracle")
    cfg, layers, lora, head = oracle_model(w, b_zero=False)
    o = om.sft_step(cfg, layers, lora, head, tokens, LR)
    say("[sft-3b-shape] gpu stream_host")
    m = gpu_model(w, "stream_host", b_zero=False)
    loss, logp = _run_sft(torch, m, tokens)
    g = _grads(m, w)
    m.close()
    assert abs(loss - o["loss"]) <= 2e-2 * abs(o["loss"])
    assert_close(logp, o["logp"], 2e-2, "logp")
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            _, _, dA, dB = g[layer][p]
            oA, oB = o["grads"][layer][p]
            assert_close(dA, oA, 5e-2, f"dA L{layer} {p}")
            assert_close(dB, oB, 5e-2, f"dB L{layer} {p}")
    say("[sft-3b-shape] gpu resident (bitwise)")
    r = gpu_model(w, "resident", b_zero=False)
    loss_r, logp_r = _run_sft(torch, r, tokens)
    gr = _grads(r, w)
    r.close()
    assert np.array_equal(_bits(np.float32(loss_r)), _bits(np.float32(loss)))
    assert np.array_equal(_bits(logp_r), _bits(logp))
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            for u, v in zip(g[layer][p], gr[layer][p]):
                assert np.array_equal(_bits(np.asarray(u)), _bits(np.asarray(v)))


def test_dpo_qwen3b_layer_shape_vs_oracle_and_resident(torch):
    """One streamed DPO step (fused reference pass) on a 2 x 512-token pair at
    the 3B layer shape (tied embedding, GQA 16/2, FFN 11008), two layers and
    a 1024-entry vocabulary, against the oracle; the same step with the base
    resident gives the same bits (loss, z, the four sums, both log-prob
    vectors, A, B, dA, dB)."""
    w = dict(synth.WORKLOADS["qwen2.5-3b-shaped"], n_layers=2, vocab=1024)
    S, beta = w["seq_len"], synth.DPO_PAIR["beta"]
    P = synth.dpo_prompt_len(w)
    ch, rj = synth.dpo_pair(w)
    tok, tgt = _dev_tokens(torch, np.stack([ch, rj]))
    say("[dpo-3b-shape] oracle")
    cfg, layers, lora, head = oracle_model(w, b_zero=False)
    od = om.dpo_step(cfg, layers, lora, head, ch, rj, P, beta, LR)
    runs = {}
    for mode in ("stream_host", "resident"):
        say(f"[dpo-3b-shape] gpu {mode}")
        m = gpu_model(w, mode, b_zero=False, max_tokens=2 * S)
        out = m.dpo_step(tok, tgt, S, P, beta, LR)
        m.sync()
        runs[mode] = (out[:6].cpu().numpy().copy(), m.logp[:2 * S].cpu().numpy().copy(),
                      m.logp_ref[:2 * S].cpu().numpy().copy(), _grads(m, w))
        m.close()
    o, logp, logp_ref, g = runs["stream_host"]
    lbar, zbar = _dpo_bars(od, beta)
    assert abs(o[0] - od["loss"]) <= lbar
    assert abs(o[1] - od["z"]) <= zbar
    assert_close(logp, od["logp_policy"], 2e-2, "policy logp")
    assert_close(logp_ref, od["logp_ref"], 2e-2, "reference logp")
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            _, _, dA, dB = g[layer][p]
            odA, odB = od["grads"][layer][p]
            assert_close(dA, odA, 5e-2, f"DPO dA L{layer} {p}")
            assert_close(dB, odB, 5e-2, f"DPO dB L{layer} {p}")
    r = runs["resident"]
    for a, b in zip((o, logp, logp_ref), r[:3]):
        assert np.array_equal(_bits(a), _bits(b))
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            for u, v in zip(g[layer][p], r[3][layer][p]):
                assert np.array_equal(_bits(np.asarray(u)), _bits(np.asarray(v)))


def test_sft_ragged_sequence_groups(torch):
    """Three sequences with layer_tokens = 2 x seq_len: each layer runs a
    group of two sequences, then a group of one, on its record.  Every
    projection adapted (GQA).  Resident == host-streamed bitwise (loss,
    log-probs, A, B, dA, dB), one step against the oracle (loss and log-probs
    within 2e-2, adapter gradients within 5e-2), and the record copies are
    those of the ungrouped step."""
    w = dict(SMALL256, n_seq=3, seq_len=64)
    S, n = w["seq_len"], w["n_seq"]
    tokens = synth.sft_tokens(w)
    runs, loads = {}, {}
    for mode in ("resident", "stream_host"):
        say(f"[sft groups] {mode}")
        m = gpu_model(w, mode, b_zero=False, lora_targets=ALL7, layer_tokens=2 * S)
        l0 = m.stats()[0]
        loss, logp = _run_sft(torch, m, tokens)
        loads[mode] = m.stats()[0] - l0
        runs[mode] = (loss, logp, _grads(m, w, ALL7))
        m.close()
    a, b = runs["resident"], runs["stream_host"]
    assert np.float32(a[0]).view(np.uint32) == np.float32(b[0]).view(np.uint32)
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    for la, lb in zip(a[2], b[2]):
        for p in ALL7:
            for x, y in zip(la[p], lb[p]):
                assert np.array_equal(np.asarray(x, np.float32).view(np.uint32),
                                      np.asarray(y, np.float32).view(np.uint32)), p
    assert loads["stream_host"] == 2 * w["n_layers"] - 2, loads
    say("[sft groups] oracle")
    cfg, layers, lora, head = oracle_model(w, b_zero=False, lora_targets=ALL7)
    o = om.sft_step(cfg, layers, lora, head, tokens, LR)
    loss, logp, g = b
    assert abs(loss - o["loss"]) <= 2e-2 * abs(o["loss"]), (loss, o["loss"])
    assert_close(logp, o["logp"], 2e-2, "logp")
    for layer in range(w["n_layers"]):
        for p in ALL7:
            _, _, dA, dB = g[layer][p]
            odA, odB = o["grads"][layer][p]
            assert_close(dA, odA, 5e-2, f"dA L{layer} {p}")
            assert_close(dB, odB, 5e-2, f"dB L{layer} {p}")
