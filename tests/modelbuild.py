"""Test helpers: the same seeded model built twice, once for the oracle (its
own NF4 quantizer, numpy arrays) and once for the GPU library (the library's
host quantizer, loaded through the C ABI).  Nothing computed by the GPU path
feeds the oracle."""
import numpy as np

import synth
from oracle import model as om
from oracle import nf4 as onf4

BF16_ONE = 0x3F80


def oracle_config(w, lora_targets=("q", "v")):
    return om.Config(n_layers=w["n_layers"], hidden=w["hidden"], n_heads=w["n_heads"],
                     n_kv_heads=w["n_kv_heads"], head_dim=w["head_dim"], ffn=w["ffn"],
                     vocab=w["vocab"], rms_eps=w["rms_eps"], rope_theta=w["rope_theta"],
                     lora_rank=w["lora_rank"], lora_alpha=w["lora_alpha"],
                     lora_targets=lora_targets, tied=w["tied"])


def oracle_layer(w, layer, dtype=np.float64):
    lw = {}
    for p in synth.PROJ:
        W = synth.layer_weights_f32(w, layer, p)
        c, a = onf4.quantize(W)
        lw[p] = onf4.dequantize(c, a, W.size).reshape(W.shape).astype(dtype)
    lw["attn_norm"] = np.ones(w["hidden"], dtype)
    lw["mlp_norm"] = np.ones(w["hidden"], dtype)
    return lw


def oracle_lora(w, b_zero, lora_targets=("q", "v"), dtype=np.float64):
    out = []
    for layer in range(w["n_layers"]):
        d = {}
        for p in lora_targets:
            A, B = synth.lora_init(w, layer, p, b_zero)
            d[p] = (A.astype(dtype), B.astype(dtype))
        out.append(d)
    return out


def oracle_head(w, dtype=np.float64):
    emb, lm, _ = synth.head_tables(w)
    return dict(embed=synth.bf16_to_f32(emb).astype(dtype),
                lm_head=synth.bf16_to_f32(lm).astype(dtype),
                final_norm=np.ones(w["hidden"], dtype))


def oracle_model(w, b_zero, lora_targets=("q", "v"), dtype=np.float64):
    cfg = oracle_config(w, lora_targets)
    layers = [oracle_layer(w, i, dtype) for i in range(w["n_layers"])]
    return cfg, layers, oracle_lora(w, b_zero, lora_targets, dtype), oracle_head(w, dtype)


def gpu_model(w, mode, b_zero, lora_targets=("q", "v"), store_path=None, max_tokens=None,
              max_seq_len=None, head_on_host=False, head_chunk_rows=0):
    from layer_streamed_nf4_double_amd import _lib as L
    from layer_streamed_nf4_double_amd.trainer import LayerStreamedLoRA
    m = LayerStreamedLoRA(w, mode, max_tokens=max_tokens, max_seq_len=max_seq_len,
                          head_on_host=head_on_host, head_chunk_rows=head_chunk_rows,
                          lora_targets=lora_targets, store_path=store_path)
    ones = np.full(w["hidden"], BF16_ONE, np.uint16)
    for layer in range(w["n_layers"]):
        codes, absmax = [], []
        for p in synth.PROJ:
            c, a = L.lsn_nf4_quantize(synth.layer_weights_f32(w, layer, p))
            codes.append(c)
            absmax.append(a)
        m.load_layer(layer, codes, absmax, ones, ones)
        for p in lora_targets:
            A, B = synth.lora_init(w, layer, p, b_zero)
            m.set_lora(layer, p, A, B)
    emb, lm, _ = synth.head_tables(w)
    m.load_head(emb, lm, ones)
    return m


def rel(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    den = np.linalg.norm(o)
    return float(np.linalg.norm(g - o) / (den if den > 0 else 1.0))


def assert_close(g, o, tol, what):
    """Norm-relative error <= tol (the bar), and every element within
    tol * (|o| + rms(o) * sqrt(2 ln n)): the absolute floor is the largest
    of n Gaussian errors whose norm sits at the bar, so an element fails only
    if it is an outlier the norm alone would hide.  Prints the errors."""
    g = np.asarray(g, np.float64).reshape(-1)
    o = np.asarray(o, np.float64).reshape(-1)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU values"
    r = rel(g, o)
    rms = np.sqrt(np.mean(o * o)) if o.size else 0.0
    worst = float(np.max(np.abs(g - o))) if o.size else 0.0
    print(f"  [{what}] rel L2 {r:.2e}, worst |diff| {worst:.2e} (rms {rms:.2e})", flush=True)
    assert r <= tol, f"{what}: relative L2 error {r:.3e} > {tol}"
    floor = rms * np.sqrt(2.0 * np.log(max(o.size, 2)))
    bad = np.abs(g - o) > tol * (np.abs(o) + floor)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {o.size} elements off, worst "
                           f"{np.max(np.abs(g - o)):.3e} (rms {rms:.3e})")
    return r
