"""Adapter files and run planning (host side, no GPU)."""
import numpy as np
import pytest

from layer_streamed_nf4_double_amd import adapter as ad

SHAPES = {"q": (64, 32), "v": (16, 32)}


def _adapters(seed=0, layers=2, r=4):
    rng = np.random.default_rng(seed)
    out = {}
    for layer in range(layers):
        for p, (N, K) in SHAPES.items():
            out[(layer, p)] = (rng.standard_normal((K, r)).astype(np.float32),
                               rng.standard_normal((r, N)).astype(np.float32))
    return out


def test_keys_are_plain_and_round_trip_bitwise():
    a = _adapters()
    sd = ad.adapter_state_dict(a)
    assert all(".inner." not in k for k in sd)
    assert "base_model.model.model.layers.1.self_attn.v_proj.lora_B.weight" in sd
    assert sd["base_model.model.model.layers.0.self_attn.q_proj.lora_A.weight"].shape == (4, 32)
    assert sd["base_model.model.model.layers.0.self_attn.q_proj.lora_B.weight"].shape == (64, 4)
    back = ad.adapters_from_state_dict(sd, 2, ("q", "v"), SHAPES, 4)
    for k, (A, B) in a.items():
        assert np.array_equal(back[k][0], A) and np.array_equal(back[k][1], B)


def test_wrapper_segment_is_rejected_not_ignored():
    sd = ad.adapter_state_dict(_adapters())
    bad = {k.replace(".self_attn.", ".inner.self_attn."): v for k, v in sd.items()}
    with pytest.raises(ValueError):
        ad.adapters_from_state_dict(bad, 2, ("q", "v"), SHAPES, 4)
    missing = dict(sd)
    missing.pop(next(iter(missing)))
    with pytest.raises(ValueError):
        ad.adapters_from_state_dict(missing, 2, ("q", "v"), SHAPES, 4)
    wrong = dict(sd)
    k = "base_model.model.model.layers.0.self_attn.q_proj.lora_A.weight"
    wrong[k] = wrong[k][:, :16]
    with pytest.raises(ValueError):
        ad.adapters_from_state_dict(wrong, 2, ("q", "v"), SHAPES, 4)


def test_file_round_trip_with_safetensors(tmp_path):
    from safetensors.numpy import load_file, save_file
    sd = ad.adapter_state_dict(_adapters(3))
    save_file(sd, str(tmp_path / "a.safetensors"))
    back = load_file(str(tmp_path / "a.safetensors"))
    assert set(back) == set(sd)
    for k in sd:
        assert np.array_equal(back[k], sd[k])


def test_plan_run_source_and_preflight():
    rec = 122_699_776
    # 8B-shaped stack (32 records, 3.9 GB): RAM when it fits with the reserve
    assert ad.plan_run(32, rec, 3 << 30, 200 << 30, 64 << 30) == "stream_host"
    assert ad.plan_run(32, rec, 3 << 30, 200 << 30, 10 << 30) == "stream_file"
    assert ad.plan_run(32, rec, 3 << 30, 200 << 30, 10 << 30, source="stream_host") == "stream_host"
    with pytest.raises(ad.NoFit):
        ad.plan_run(32, rec, 5 << 30, 4 << 30, 64 << 30)
    assert ad.host_bytes_available() > 0
