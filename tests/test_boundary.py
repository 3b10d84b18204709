"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every symbol the header declares, and its host NF4 codec agrees bit for bit
with the oracle's."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import nf4 as onf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from layer_streamed_nf4_double_amd import _lib as L
    return L


def _declared():
    src = open(os.path.join(ROOT, "include", "lsn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lsn_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = _lib()
    raw = ctypes.CDLL(L.LIB_PATH)
    names = _declared()
    assert len(names) >= 25
    for n in names:
        assert hasattr(raw, n), f"{n} declared in lsn.h but not exported"
    assert set(names) == set(L.EXPORTED), "binding and header disagree"


def test_codebook_bit_equal_to_oracle():
    L = _lib()
    cb = L.lsn_nf4_codebook()
    assert np.array_equal(cb.view(np.uint32), onf4.codebook().view(np.uint32))


def _adversarial():
    c = onf4.codebook()
    m = onf4.midpoints()
    rng = np.random.default_rng(5)
    blocks = []
    b = np.zeros(64, np.float32); b[0] = 1.0; b[1:16] = m; b[16:31] = c[:15]
    blocks.append(b)                                               # exact ties / levels
    blocks.append(np.zeros(64, np.float32))                         # all-zero block
    b = np.full(64, -0.0, np.float32); b[5] = -3.0; blocks.append(b)
    b = (rng.standard_normal(64) * 1e-30).astype(np.float32); blocks.append(b)  # tiny values
    b = np.nextafter(m, np.float32(2)).astype(np.float32)
    blocks.append(np.concatenate([[1.0], b, np.nextafter(m, np.float32(-2)), np.zeros(64 - 31)]).astype(np.float32))
    return np.concatenate(blocks)


@pytest.mark.parametrize("case", ["normal", "adversarial", "rows688", "odd"])
def test_quantize_bit_equal_to_oracle(case):
    L = _lib()
    rng = np.random.default_rng(1)
    if case == "normal":
        w = rng.standard_normal(64 * 3000, dtype=np.float32) * np.float32(0.02)
    elif case == "adversarial":
        w = _adversarial()
    elif case == "rows688":   # a [256, 688] down projection: blocks straddle rows
        w = (rng.standard_normal((256, 688), dtype=np.float32) * np.float32(0.02)).reshape(-1)
    else:
        w = rng.standard_normal(64 * 5 + 37, dtype=np.float32)
    codes, absmax = L.lsn_nf4_quantize(w)
    oc, oa = onf4.quantize(w)
    assert np.array_equal(codes, oc)
    assert np.array_equal(absmax.view(np.uint32), oa.view(np.uint32))
    d = L.lsn_nf4_dequantize(codes, absmax, w.size)
    od = onf4.dequantize(oc, oa, w.size)
    assert np.array_equal(d.view(np.uint32), od.view(np.uint32))


def test_quantize_large_multithreaded_matches_oracle():
    L = _lib()
    w = np.random.default_rng(2).standard_normal(64 * 40000, dtype=np.float32)
    codes, absmax = L.lsn_nf4_quantize(w)
    oc, oa = onf4.quantize(w)
    assert np.array_equal(codes, oc) and np.array_equal(absmax, oa)


def test_quantize_rejects_non_finite():
    L = _lib()
    w = np.zeros(128, np.float32)
    w[77] = np.inf
    with pytest.raises(L.LsnError) as e:
        L.lsn_nf4_quantize(w)
    assert e.value.status == L.LSN_ERR_INVALID


def test_workspace_and_preflight_refusal():
    import synth
    from layer_streamed_nf4_double_amd import trainer
    L = _lib()
    shape = dict(synth.WORKLOADS["tiny"], n_layers=6)
    cfg = trainer.make_config(shape, "stream_host")
    need = L.lsn_workspace_bytes(cfg)
    cfg_res = trainer.make_config(shape, "resident")
    need_res = L.lsn_workspace_bytes(cfg_res)
    assert need_res > need        # resident keeps every record, streaming two slots
    # a workspace that is too small is refused before any device work
    with pytest.raises(L.LsnError) as e:
        L.lsn_create(cfg, 0x1000, need - 1, 0)
    assert e.value.status == L.LSN_ERR_NOFIT
    assert f"needs {need} bytes" in str(e.value), str(e.value)
    cfg.vram_budget = need - 1
    with pytest.raises(L.LsnError) as e:
        L.lsn_create(cfg, 0x1000, need, 0)
    assert e.value.status == L.LSN_ERR_NOFIT


def test_invalid_configs_rejected():
    import synth
    from layer_streamed_nf4_double_amd import trainer
    L = _lib()
    for field, val in [("lora_rank", 17), ("n_kv_heads", 3), ("head_dim", 60), ("vocab", 1001),
                       ("max_seq_len", 10 ** 6)]:
        cfg = trainer.make_config(synth.WORKLOADS["tiny"], "stream_host")
        setattr(cfg, field, val)
        with pytest.raises(L.LsnError) as e:
            L.lsn_workspace_bytes(cfg)
        assert e.value.status == L.LSN_ERR_INVALID, field
    # the reason travels with the error (calls without a context keep it per thread)
    assert "max_seq_len" in str(e.value), str(e.value)


def test_head_on_host_workspace():
    """With head_on_host the embedding and LM-head tables leave the workspace
    (2 V H bf16 for an untied head, V H for a tied one); the option needs a
    streamed base."""
    import synth
    from layer_streamed_nf4_double_amd import trainer
    L = _lib()
    for name in ("llama3.1-8b-shaped", "qwen2.5-3b-shaped", "tiny"):
        w = dict(synth.WORKLOADS[name], n_layers=4)
        dev = L.lsn_workspace_bytes(trainer.make_config(w, "stream_host"))
        host = L.lsn_workspace_bytes(trainer.make_config(w, "stream_host", head_on_host=True))
        tables = (1 if w["tied"] else 2) * w["vocab"] * w["hidden"] * 2
        # the smaller LM-head chunk (one slot of W_lm rows) also shrinks its buffers
        assert tables <= dev - host <= tables + 6 * w["seq_len"] * w["n_seq"] * 65536, name
        cfg = trainer.make_config(w, "resident", head_on_host=True)
        with pytest.raises(L.LsnError) as e:
            L.lsn_workspace_bytes(cfg)
        assert e.value.status == L.LSN_ERR_INVALID


def test_record_sizes_match_layout():
    """Per-layer record = NF4 codes (P/2) + absmax (P/16) + norms, 4 KiB aligned."""
    import synth
    from layer_streamed_nf4_double_amd import trainer
    L = _lib()
    for name, want in [("tiny", 444672), ("llama3.1-8b-shaped", 122683392),
                       ("qwen2.5-3b-shaped", 43352064)]:
        w = dict(synth.WORKLOADS[name], n_layers=4)
        P = sum(np.prod(synth.proj_shape(w, p)) for p in synth.PROJ)
        assert P // 2 + P // 16 == want
        cfg = trainer.make_config(w, "stream_host")
        ws_stream = L.lsn_workspace_bytes(cfg)
        cfg.mode = L.LSN_RESIDENT
        ws_res = L.lsn_workspace_bytes(cfg)
        rec = (ws_res - ws_stream) // (w["n_layers"] - 2)
        assert want <= rec <= want + 4096 + 256 * 4 + 4 * w["hidden"]


def test_one_hip_runtime_in_the_process():
    """The library binds to PyTorch's HIP runtime: loading the binding maps a
    single libamdhip64 into the process (a second runtime would not see the
    GPU once torch holds it)."""
    _lib()
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_host_id_check():
    """trainer.check_ids: token ids in [0, vocab), targets in [0, vocab) or
    -1; anything else is refused on the host before a batch reaches the
    device."""
    from layer_streamed_nf4_double_amd.trainer import check_ids
    tok = np.array([[0, 5, 1023]], np.int32)
    check_ids(tok, np.array([5, 1023, -1], np.int32), 1024)
    for bad_tok, bad_tgt in [([[0, 1024, 3]], [1, 2, -1]), ([[-1, 2, 3]], [1, 2, -1]),
                             ([[0, 1, 2]], [1, 1024, -1]), ([[0, 1, 2]], [1, -2, -1])]:
        with pytest.raises(ValueError):
            check_ids(np.array(bad_tok, np.int32), np.array(bad_tgt, np.int32), 1024)


def test_config_checks_without_a_gpu():
    """Configuration errors come back as LSN_ERR_INVALID from the sizing
    calls (no device needed): the slot count, and an LM-head chunk that
    cannot fit a layer slot when the head streams through the slots."""
    L = _lib()
    import synth
    from layer_streamed_nf4_double_amd.trainer import make_config
    w = synth.WORKLOADS["tiny"]
    base = L.lsn_workspace_bytes(make_config(w, "stream_host"))
    assert L.lsn_workspace_bytes(make_config(w, "stream_host", n_slots=2)) == base
    rec = L.lsn_config_record_bytes(make_config(w, "stream_host"))
    assert L.lsn_workspace_bytes(make_config(w, "stream_host", n_slots=4)) == base + 2 * rec
    assert L.lsn_workspace_bytes(make_config(w, "resident", n_slots=4)) == \
        L.lsn_workspace_bytes(make_config(w, "resident"))
    for n in (1, 5, -1):
        with pytest.raises(L.LsnError) as e:
            L.lsn_workspace_bytes(make_config(w, "stream_host", n_slots=n))
        assert e.value.status == L.LSN_ERR_INVALID
    # an explicit head chunk larger than a slot of W_lm rows
    rows = rec // (2 * w["hidden"]) // 8 * 8 + 8
    with pytest.raises(L.LsnError):
        L.lsn_workspace_bytes(make_config(w, "stream_host", head_on_host=True,
                                          head_chunk_rows=rows))
    # the automatic head chunk of a tiny slot stays inside it: a 1-layer,
    # 64-wide stack whose slot holds fewer than 256 W_lm rows
    small = dict(w, hidden=64, n_heads=1, n_kv_heads=1, head_dim=64, ffn=64, vocab=4096)
    L.lsn_workspace_bytes(make_config(small, "stream_host", head_on_host=True))


def test_sequence_groups_workspace_without_a_gpu():
    """layer_tokens sizes the layer buffers for one group of whole sequences
    and leaves the LM head's at max_tokens: a two-sequence (DPO pair)
    workspace with layer_tokens = seq_len lies strictly between the
    one-sequence workspace and the ungrouped two-sequence one, at least the
    head's per-token buffers above the former; a single-sequence
    config, or layer_tokens at or above max_tokens, changes nothing; a
    negative value is refused."""
    L = _lib()
    import synth
    from layer_streamed_nf4_double_amd.trainer import make_config
    for name in ("tiny", "llama3.1-8b-shaped", "qwen2.5-3b-shaped"):
        w = synth.WORKLOADS[name]
        S = w["seq_len"]
        one = L.lsn_workspace_bytes(make_config(w, "stream_host", S, S))
        pair = L.lsn_workspace_bytes(make_config(w, "stream_host", 2 * S, S))
        grouped = L.lsn_workspace_bytes(make_config(w, "stream_host", 2 * S, S, layer_tokens=S))
        assert one < grouped < pair, (name, one, grouped, pair)
        assert L.lsn_workspace_bytes(make_config(w, "stream_host", S, S, layer_tokens=S)) == one
        assert L.lsn_workspace_bytes(make_config(w, "stream_host", 2 * S, S,
                                                 layer_tokens=4 * S)) == pair
        # below one sequence: still one sequence per group
        assert L.lsn_workspace_bytes(make_config(w, "stream_host", 2 * S, S,
                                                 layer_tokens=8)) == grouped
        # the LM head's buffers (final norm bf16 + fp32 gradient, five fp32
        # per-token scalars, its logits chunk and split-k scratch) keep all
        # 2 S tokens
        H = w["hidden"]
        assert grouped - one >= S * (2 * H + 4 * H + 5 * 4), name
    with pytest.raises(L.LsnError) as e:
        L.lsn_workspace_bytes(make_config(synth.WORKLOADS["tiny"], "stream_host",
                                          layer_tokens=-1))
    assert e.value.status == L.LSN_ERR_INVALID
