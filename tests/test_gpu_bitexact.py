"""The pages' own correctness bar, through the C ABI: streamed training is
bit-exact against a run with the base resident ("Show HN: Fine-tune an 8B
model on a 4 GB laptop GPU", first paragraph, which states it for the DPO
reference pass; axbrief.com article, "Beyond Memory: The Layer Streaming
Breakthrough"), also with the process capped to the streamed run's memory
(the evermx page's notebook caps a T4 to 4 GB and asserts bit identity).

* DPO steps, fused and separate reference pass, resident == host-streamed ==
  file-streamed, bitwise; the fused form at the full 8B layer shape; the
  chosen and rejected sequences run one after the other on each record
  (layer_tokens), also against the oracle.
* SFT with 3 and 4 slots, and the exact record-copy counts.
* Fault injection: slots filled with NaN bytes before every copy, copies
  delayed on the copy stream, layers delayed on the compute stream: the
  bits do not change (a missing wait would read a poisoned or stale slot).
* A truncated store file: LSN_ERR_IO, then LSN_ERR_STATE on later calls.
* Memory: resident peak - streamed peak is (L - n_slots) records; the
  streamed peak is the workspace plus the trainer's activations (no second
  copy of the weights for the DPO reference model: "Show HN", second
  paragraph, gives a forced second copy as +730 MB, one copy of the weights).
* Resume: two steps == one step, adapters read out and written into a fresh
  context, one step.
* A decoder whose q|k|v width is below hidden, against the oracle.
"""
import math
import os
import sys

import numpy as np
import pytest

import synth
from oracle import model as om
from tests.modelbuild import assert_close, gpu_model, oracle_model

pytestmark = pytest.mark.gpu
TINY = synth.WORKLOADS["tiny"]
LR = 0.1
LLAMA8B_2L = dict(synth.WORKLOADS["llama3.1-8b-shaped"], n_layers=2, vocab=1024)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def _dev(torch, tokens, vocab):
    from layer_streamed_nf4_double_amd.trainer import device_batch, sft_targets
    tokens = np.asarray(tokens)
    return device_batch(tokens, sft_targets(tokens), vocab)


def _adapters(m, w, targets=("q", "v")):
    return [{p: m.get_lora(layer, p) for p in targets} for layer in range(w["n_layers"])]


def _same(a, b, what):
    """Nested tuples/lists/dicts of arrays and scalars, bit for bit."""
    if isinstance(a, dict):
        assert a.keys() == b.keys(), what
        for k in a:
            _same(a[k], b[k], f"{what}.{k}")
    elif isinstance(a, (list, tuple)):
        assert len(a) == len(b), what
        for i, (x, y) in enumerate(zip(a, b)):
            _same(x, y, f"{what}[{i}]")
    else:
        assert np.array_equal(_bits(a), _bits(b)), what


def _pair(w, wid=89):
    S = w["seq_len"]
    P = S // 4
    pr = synth.tokens((P,), w["vocab"], wid, synth.TID_PROMPT)
    ch = np.concatenate([pr, synth.tokens((S - P,), w["vocab"], wid, synth.TID_CHOSEN)])
    rj = np.concatenate([pr, synth.tokens((S - P,), w["vocab"], wid, synth.TID_REJECTED)])
    return ch, rj, P


def _dpo_steps(torch, m, w, tok, tgt, P, fused, steps=2, beta=0.1):
    S = w["seq_len"]
    rec = []
    for _ in range(steps):
        out = m.dpo_step(tok, tgt, S, P, beta, LR, fused=fused)
        m.sync()
        rec.append((out[:6].cpu().numpy().copy(), m.logp[:2 * S].cpu().numpy().copy(),
                    m.logp_ref[:2 * S].cpu().numpy().copy(), _adapters(m, w)))
    return rec


def _sft_steps(torch, m, w, tok, tgt, n_seq, S, steps=2, lr=LR):
    rec = []
    for _ in range(steps):
        loss = m.sft_step(tok, tgt, n_seq, S, lr)
        m.sync()
        rec.append((loss[:1].cpu().numpy().copy(), m.logp[:n_seq * S].cpu().numpy().copy(),
                    _adapters(m, w)))
    return rec


@pytest.mark.parametrize("fused", [True, False])
def test_dpo_streamed_equals_resident_bitwise(torch, fused, tmp_path):
    """Two DPO steps (loss, z, pc, pr, rc, rr, both log-prob vectors, A, B,
    dA, dB after each step) give the same bits with the base resident,
    streamed from pinned host memory and streamed from a store file."""
    w = dict(TINY, n_layers=5)
    ch, rj, P = _pair(w)
    tok, tgt = _dev(torch, np.stack([ch, rj]), w["vocab"])
    S = w["seq_len"]
    runs = {}
    for mode in ("resident", "stream_host", "stream_file"):
        say(f"[dpo bitwise] fused={fused} {mode}")
        store = str(tmp_path / f"{mode}.bin") if mode == "stream_file" else None
        m = gpu_model(w, mode, b_zero=False, max_tokens=2 * S, store_path=store)
        runs[mode] = _dpo_steps(torch, m, w, tok, tgt, P, fused)
        m.close()
    assert np.abs(runs["resident"][0][0][1]) > 0, "z must be non-zero (B != 0)"
    _same(runs["resident"], runs["stream_host"], "host")
    _same(runs["resident"], runs["stream_file"], "file")


def test_dpo_llama8b_layer_shape_streamed_equals_resident(torch):
    """One fused DPO step on a 2 x 512-token pair at the full 8B layer shape
    (the kernels and launch shapes the bench times): resident == streamed,
    bitwise."""
    w = LLAMA8B_2L
    S, beta = w["seq_len"], synth.DPO_PAIR["beta"]
    P = synth.dpo_prompt_len(w)
    ch, rj = synth.dpo_pair(w)
    tok, tgt = _dev(torch, np.stack([ch, rj]), w["vocab"])
    runs = {}
    for mode in ("resident", "stream_host"):
        say(f"[dpo-8b bitwise] {mode}")
        m = gpu_model(w, mode, b_zero=False, max_tokens=2 * S)
        runs[mode] = _dpo_steps(torch, m, w, tok, tgt, P, True, steps=1, beta=beta)
        m.close()
        torch.cuda.empty_cache()
    _same(runs["resident"], runs["stream_host"], "8B DPO")


@pytest.mark.parametrize("shape", ["tiny", "llama8b-layer"])
def test_dpo_sequence_groups(torch, shape):
    """layer_tokens = seq_len: each layer runs the chosen and then the
    rejected sequence on its record (fused reference pass).  Resident ==
    host-streamed bitwise over two steps, the record copies per step are
    those of the ungrouped step, and (tiny) one step against the oracle:
    losses and log-probs within 2e-2, adapter gradients within 5e-2."""
    w = dict(TINY, n_layers=5) if shape == "tiny" else LLAMA8B_2L
    S = w["seq_len"]
    if shape == "tiny":
        ch, rj, P = _pair(w)
        beta = 0.1
    else:
        P, beta = synth.dpo_prompt_len(w), synth.DPO_PAIR["beta"]
        ch, rj = synth.dpo_pair(w)
    tok, tgt = _dev(torch, np.stack([ch, rj]), w["vocab"])
    steps = 2 if shape == "tiny" else 1
    runs, loads = {}, {}
    for mode in ("resident", "stream_host"):
        say(f"[dpo groups {shape}] {mode}")
        m = gpu_model(w, mode, b_zero=False, max_tokens=2 * S, layer_tokens=S)
        l0 = m.stats()[0]
        runs[mode] = _dpo_steps(torch, m, w, tok, tgt, P, True, steps=steps, beta=beta)
        loads[mode] = m.stats()[0] - l0
        m.close()
        torch.cuda.empty_cache()
    _same(runs["resident"], runs["stream_host"], f"grouped DPO {shape}")
    L_ = w["n_layers"]
    assert loads["stream_host"] == (2 * L_ - 2) + (steps - 1) * (2 * L_ - 4), loads
    if shape != "tiny":
        return
    say("[dpo groups tiny] vs oracle")
    cfg, layers, lora, head = oracle_model(w, b_zero=False)
    od = om.dpo_step(cfg, layers, lora, head, ch, rj, P, beta, LR)
    m = gpu_model(w, "stream_host", b_zero=False, max_tokens=2 * S, layer_tokens=S)
    out = m.dpo_step(tok, tgt, S, P, beta, LR)
    m.sync()
    o = out[:6].cpu().numpy().astype(np.float64)
    assert abs(o[0] - od["loss"]) <= 2e-2 * abs(od["loss"]), (o[0], od["loss"])
    assert_close(m.logp[:2 * S].cpu().numpy(), od["logp_policy"], 2e-2, "policy logp")
    assert_close(m.logp_ref[:2 * S].cpu().numpy(), od["logp_ref"], 2e-2, "reference logp")
    for layer in range(L_):
        for p in ("q", "v"):
            _, _, dA, dB = m.get_lora(layer, p)
            odA, odB = od["grads"][layer][p]
            assert_close(dA, odA, 5e-2, f"grouped dA L{layer} {p}")
            assert_close(dB, odB, 5e-2, f"grouped dB L{layer} {p}")
    m.close()


@pytest.mark.parametrize("n_slots", [3, 4])
def test_more_slots_equal_resident_and_copy_less(torch, n_slots, tmp_path):
    """SFT with 3 and 4 device slots: bitwise equal to resident, from host
    memory and from a store file, and each pass reuses the n_slots records
    the previous pass left behind: L + (2 * steps - 1)(L - n_slots) copies."""
    w = dict(TINY, n_layers=8)
    tokens = synth.tokens((2, 64), w["vocab"], 77)
    tok, tgt = _dev(torch, tokens, w["vocab"])
    res = gpu_model(w, "resident", b_zero=False, max_tokens=128)
    a = _sft_steps(torch, res, w, tok, tgt, 2, 64, steps=3)
    res.close()
    for mode in ("stream_host", "stream_file"):
        say(f"[slots={n_slots}] {mode}")
        store = str(tmp_path / "store.bin") if mode == "stream_file" else None
        m = gpu_model(w, mode, b_zero=False, max_tokens=128, n_slots=n_slots, store_path=store)
        b = _sft_steps(torch, m, w, tok, tgt, 2, 64, steps=3)
        loads = m.stats()[0]
        m.close()
        _same(a, b, f"{mode} n_slots={n_slots}")
        L_ = w["n_layers"]
        assert loads == L_ + 5 * (L_ - n_slots), (loads, n_slots)


@pytest.mark.parametrize("case", ["host-copy-delay", "host-compute-delay", "file-copy-delay",
                                  "head-on-host-both", "slots3-both"])
def test_fault_injection_leaves_bits_unchanged(torch, case, tmp_path):
    """Every slot filled with 0xFF bytes (NaN) just before each copy into
    it, with copies delayed on the copy stream or layers delayed on the
    compute stream (3 ms each): two SFT steps give the same bits as without
    the faults.  A compute that ran before its copy finished, or a copy that
    overwrote a slot before its last reader finished, would read NaN or a
    stale record."""
    from layer_streamed_nf4_double_amd import _lib as L
    w = dict(TINY, n_layers=5)
    tokens = synth.tokens((2, 64), w["vocab"], 81)
    tok, tgt = _dev(torch, tokens, w["vocab"])
    kw = dict(b_zero=False, max_tokens=128)
    mode = "stream_file" if case.startswith("file") else "stream_host"
    if case.startswith("head"):
        kw["head_on_host"] = True
    if case.startswith("slots3"):
        kw["n_slots"] = 3
    copy_delay = 3000 if ("copy" in case or "both" in case) else 0
    compute_delay = 3000 if ("compute" in case or "both" in case) else 0
    recs = []
    for faults in (False, True):
        say(f"[faults] {case} faults={faults}")
        store = str(tmp_path / f"s{int(faults)}.bin") if mode == "stream_file" else None
        m = gpu_model(w, mode, store_path=store, **kw)
        if faults:
            L.lsn_set_fault_injection(m.ctx, copy_delay, compute_delay, True)
        recs.append(_sft_steps(torch, m, w, tok, tgt, 2, 64))
        m.close()
    assert np.all(np.isfinite(recs[1][0][1]))
    _same(recs[0], recs[1], case)


def test_fault_injection_rejects_bad_delays(torch):
    from layer_streamed_nf4_double_amd import _lib as L
    m = gpu_model(TINY, "stream_host", b_zero=True)
    with pytest.raises(L.LsnError) as e:
        L.lsn_set_fault_injection(m.ctx, -1, 0, False)
    assert e.value.status == L.LSN_ERR_INVALID
    with pytest.raises(L.LsnError):
        L.lsn_set_fault_injection(m.ctx, 0, 200000, False)
    m.close()


def test_truncated_store_file_io_error_then_state(torch, tmp_path):
    """A store file cut short after two records: the step fails with
    LSN_ERR_IO when the scheduler reaches the third record, and the
    poisoned context answers every later call with LSN_ERR_STATE; closing
    it still works."""
    from layer_streamed_nf4_double_amd import _lib as L
    w = dict(TINY, n_layers=4)
    tokens = synth.tokens((1, 64), w["vocab"], 83)
    tok, tgt = _dev(torch, tokens, w["vocab"])
    path = str(tmp_path / "store.bin")
    m = gpu_model(w, "stream_file", b_zero=False, store_path=path)
    rec = L.lsn_record_bytes(m.ctx)
    os.truncate(path, 2 * rec)
    with pytest.raises(L.LsnError) as e:
        m.sft_step(tok, tgt, 1, 64, LR)
    assert e.value.status == L.LSN_ERR_IO, e.value
    assert b"layer 2" in L._lib.lsn_last_error(m.ctx)
    for call in (lambda: L.lsn_sync(m.ctx), lambda: L.lsn_zero_grads(m.ctx),
                 lambda: L.lsn_begin_pass(m.ctx, L.LSN_PASS_FWD, 1, 64)):
        with pytest.raises(L.LsnError) as e2:
            call()
        assert e2.value.status == L.LSN_ERR_STATE
    m.close()


def _r512(n):
    return (n + 511) // 512 * 512


def _trainer_bytes(w, T, n_layers):
    """Device bytes the trainer allocates beside the workspace, as the torch
    allocator counts them (each allocation rounded up to 512 B): L + 1 saved
    layer inputs, two reference-pass buffers and dh ([T, hidden] fp32 each),
    logp, logp_ref, dlogp ([T]) and the 8-float loss vector."""
    H = w["hidden"]
    return (n_layers + 4) * _r512(T * H * 4) + 3 * _r512(T * 4) + _r512(32)


def _peak_of_step(torch, w, mode, T, step, **kw):
    """(device bytes the model holds after construction, peak during the
    step, workspace bytes, record bytes), all relative to what was allocated
    before the model."""
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    m = gpu_model(w, mode, b_zero=False, max_tokens=T, **kw)
    held = torch.cuda.memory_allocated() - base
    torch.cuda.reset_peak_memory_stats()
    step(m)
    m.sync()
    peak = torch.cuda.max_memory_allocated() - base
    ws = m.ws_bytes
    from layer_streamed_nf4_double_amd import _lib as L
    rb = L.lsn_record_bytes(m.ctx)
    m.close()
    del m
    gc.collect()
    torch.cuda.empty_cache()
    return held, peak, ws, rb


# torch's caching allocator gives a large allocation a segment rounded up to
# 2 MiB and leaves an unsplit tail of under 1 MiB inside the block, which its
# statistics count: the granularity of the memory accounting below
SEG_TAIL = 1 << 20


def test_peak_memory_accounting(torch):
    """At the 8B layer shape with 4 layers: the step allocates no device
    memory (its peak is what the model holds after construction), and what
    the model holds is the workspace plus the trainer's activation tensors
    (to the allocator's granularity).  The workspaces differ by exactly
    (L - 2) records between resident and streamed runs (L - 3 with three
    slots), and so do the peaks; a DPO step's peak is the same account at
    2 x 512 tokens (the reference model is the same streamed base: no second
    copy of the weights), also with one sequence per layer group, whose
    workspace lies between the SFT and the one-batch DPO workspaces."""
    w = dict(synth.WORKLOADS["llama3.1-8b-shaped"], n_layers=4, vocab=1024)
    S = w["seq_len"]
    L_ = w["n_layers"]
    tokens = synth.sft_tokens(w)
    tok, tgt = _dev(torch, tokens, w["vocab"])
    sft = lambda m: m.sft_step(tok, tgt, 1, S, LR)  # noqa: E731
    out = {}
    for name, mode, kw in (("resident", "resident", {}), ("stream2", "stream_host", {}),
                           ("stream3", "stream_host", {"n_slots": 3})):
        say(f"[memory] {name}")
        held, peak, ws, rb = _peak_of_step(torch, w, mode, S, sft, **kw)
        say(f"  held {held} peak {peak} workspace {ws} record {rb}")
        assert peak == held, (name, peak, held)
        extra = held - (_r512(ws) + _trainer_bytes(w, S, L_))
        assert 0 <= extra < SEG_TAIL, (name, held, ws, extra)
        out[name] = (peak, ws, rb)
    (pr, wr, rb), (ps, ws, _), (p3, w3, _) = out["resident"], out["stream2"], out["stream3"]
    assert wr - ws == (L_ - 2) * rb and wr - w3 == (L_ - 3) * rb
    assert abs((pr - ps) - (L_ - 2) * rb) < SEG_TAIL and abs((pr - p3) - (L_ - 3) * rb) < SEG_TAIL
    ch, rj = synth.dpo_pair(w)
    dtok, dtgt = _dev(torch, np.stack([ch, rj]), w["vocab"])
    P = synth.dpo_prompt_len(w)
    say("[memory] streamed DPO")
    held, peak, wd, _ = _peak_of_step(torch, w, "stream_host", 2 * S,
                                      lambda m: m.dpo_step(dtok, dtgt, S, P, 0.1, LR))
    assert peak == held, (peak, held)
    assert 0 <= held - (_r512(wd) + _trainer_bytes(w, 2 * S, L_)) < SEG_TAIL, (held, wd)
    # one sequence per layer group: the same account with the smaller
    # workspace, which the step does not exceed either
    say("[memory] streamed DPO, one sequence per layer group")
    held_g, peak_g, wg, _ = _peak_of_step(torch, w, "stream_host", 2 * S,
                                          lambda m: m.dpo_step(dtok, dtgt, S, P, 0.1, LR),
                                          layer_tokens=S)
    assert peak_g == held_g, (peak_g, held_g)
    assert 0 <= held_g - (_r512(wg) + _trainer_bytes(w, 2 * S, L_)) < SEG_TAIL, (held_g, wg)
    assert ws < wg < wd and held_g < held, (ws, wg, wd, held_g, held)


def test_capped_memory_run_equals_resident(torch):
    """The pages' capped-card check: the process's allocator is capped to
    what the streamed run needs (workspace + activations + 64 MiB), the
    context refuses a workspace beyond that budget, the resident model does
    not fit under the cap, and the capped streamed steps equal the uncapped
    resident steps bit for bit."""
    from layer_streamed_nf4_double_amd import _lib as L
    w = dict(synth.WORKLOADS["llama3.1-8b-shaped"], n_layers=4, vocab=1024)
    S = w["seq_len"]
    tokens = synth.sft_tokens(w)
    tok, tgt = _dev(torch, tokens, w["vocab"])
    say("[cap] resident, uncapped")
    r = gpu_model(w, "resident", b_zero=False)
    a = _sft_steps(torch, r, w, tok, tgt, 1, S)
    r.close()
    del r
    from layer_streamed_nf4_double_amd.trainer import make_config
    ws = L.lsn_workspace_bytes(make_config(w, "stream_host"))
    cap = ws + _trainer_bytes(w, S, w["n_layers"]) + (64 << 20)
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    total = torch.cuda.get_device_properties(0).total_memory
    used = torch.cuda.memory_allocated()
    torch.cuda.set_per_process_memory_fraction((cap + used) / total)
    try:
        with pytest.raises((torch.cuda.OutOfMemoryError, RuntimeError)):
            gpu_model(w, "resident", b_zero=False)
        torch.cuda.empty_cache()
        say(f"[cap] streamed under a {cap / 2**20:.0f} MiB cap")
        m = gpu_model(w, "stream_host", b_zero=False, vram_budget=ws)
        b = _sft_steps(torch, m, w, tok, tgt, 1, S)
        m.close()
        del m
        with pytest.raises(L.LsnError) as e:
            gpu_model(w, "stream_host", b_zero=False, vram_budget=ws - 4096)
        assert e.value.status == L.LSN_ERR_NOFIT
    finally:
        torch.cuda.empty_cache()
        torch.cuda.set_per_process_memory_fraction(1.0)
    _same(a, b, "capped streamed vs resident")


def test_resume_from_adapters_bitwise(torch):
    """Two SFT steps equal one step, the adapters read out (lsn_get_lora)
    and written into a fresh context (lsn_set_lora), then one more step:
    the adapter is the whole trained state ("Soup: Fine-Tune an 8B Model on
    a 4 GB GPU", "Why Layer Streaming Matters Beyond the Laptop")."""
    w = dict(TINY, n_layers=3)
    tokens = synth.tokens((1, 64), w["vocab"], 85)
    tok, tgt = _dev(torch, tokens, w["vocab"])
    say("[resume] two steps")
    m = gpu_model(w, "stream_host", b_zero=False)
    a = _sft_steps(torch, m, w, tok, tgt, 1, 64, steps=2)
    m.close()
    say("[resume] one step, save, fresh context, one step")
    m = gpu_model(w, "stream_host", b_zero=False)
    _sft_steps(torch, m, w, tok, tgt, 1, 64, steps=1)
    saved = {(l, p): m.get_lora(l, p)[:2] for l in range(w["n_layers"]) for p in ("q", "v")}
    m.close()
    f = gpu_model(w, "stream_host", b_zero=True)
    for (l, p), (A, B) in saved.items():
        f.set_lora(l, p, A, B)
    b = _sft_steps(torch, f, w, tok, tgt, 1, 64, steps=1)
    f.close()
    _same(a[1], b[0], "resumed step")


def test_narrow_attention_width_vs_oracle(torch):
    """q|k|v narrower than hidden (hidden 256, 2 q heads and 1 kv head of
    32: q|k|v width 128, attention output 64 -> o -> 256): one SFT step
    against the oracle with every projection adapted; the fp32 output
    gradients of down and o (T x 256) are cast to bf16 in a buffer sized for
    the larger of the two widths."""
    w = dict(TINY, n_layers=2, n_heads=2, n_kv_heads=1, head_dim=32)
    targets = synth.PROJ
    tokens = synth.tokens((2, 64), w["vocab"], 93)
    cfg, layers, lora, head = oracle_model(w, b_zero=False, lora_targets=targets)
    o = om.sft_step(cfg, layers, lora, head, tokens, LR)
    m = gpu_model(w, "stream_host", b_zero=False, lora_targets=targets, max_tokens=128)
    tok, tgt = _dev(torch, tokens, w["vocab"])
    loss = float(m.sft_step(tok, tgt, 2, 64, LR)[0].item())
    m.sync()
    assert abs(loss - o["loss"]) <= 2e-2 * abs(o["loss"])
    assert_close(m.logp[:128].cpu().numpy(), o["logp"], 2e-2, "logp")
    for layer in range(w["n_layers"]):
        for p in targets:
            _, _, dA, dB = m.get_lora(layer, p)
            oA, oB = o["grads"][layer][p]
            assert_close(dA, oA, 5e-2, f"dA L{layer} {p}")
            assert_close(dB, oB, 5e-2, f"dB L{layer} {p}")
    m.close()


def test_out_of_range_target_is_nan_not_a_read(torch):
    """A target id >= vocab reads no LM-head row: its log-prob is NaN (so
    the loss is NaN) and the step finishes with every other log-prob
    finite.  The host check refuses such a batch before it reaches the
    device."""
    from layer_streamed_nf4_double_amd.trainer import check_ids
    w = dict(TINY)
    tokens = synth.tokens((1, 64), w["vocab"], 87)
    tgt_np = np.append(tokens[0, 1:], -1).astype(np.int32)
    tgt_np[5] = w["vocab"] + 1000
    with pytest.raises(ValueError):
        check_ids(tokens, tgt_np, w["vocab"])
    m = gpu_model(w, "stream_host", b_zero=False)
    tok = torch.from_numpy(tokens.reshape(-1).astype(np.int32)).cuda()
    tgt = torch.from_numpy(tgt_np).cuda()
    loss = float(m.sft_step(tok, tgt, 1, 64, None)[0].item())
    m.sync()
    logp = m.logp[:64].cpu().numpy()
    m.close()
    assert math.isnan(loss) and math.isnan(logp[5])
    assert np.all(np.isfinite(np.delete(logp, 5)))


def test_serialized_run_equals_async_run(torch, tmp_path):
    """The same SFT and DPO steps in a child process whose HIP runtime waits
    before and after every kernel and every copy (AMD_SERIALIZE_KERNEL=3,
    AMD_SERIALIZE_COPY=3: nothing overlaps, so no copy can race a kernel)
    give the same bits as this process's asynchronous run, where record
    copies overlap the layers' kernels."""
    import subprocess
    from tests import serial_run
    ref = serial_run.run()
    out = tmp_path / "serial.npz"
    env = dict(os.environ, AMD_SERIALIZE_KERNEL="3", AMD_SERIALIZE_COPY="3")
    say("[serialized] child process with serialized kernels and copies")
    r = subprocess.run([sys.executable, "-u", os.path.join(os.path.dirname(__file__), "serial_run.py"),
                        str(out)], env=env, capture_output=True, text=True, timeout=240)
    say(r.stdout[-500:] + r.stderr[-1500:])
    assert r.returncode == 0
    got = np.load(out)
    assert len(got.files) == len(ref)
    for i, a in enumerate(ref):
        assert np.array_equal(_bits(got[f"arr_{i}"]), _bits(a)), f"array {i} differs"
