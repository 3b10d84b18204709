"""LoRA adapter files and run planning (host side).

Adapter files.  Only the adapter trains, so the adapter is the artifact of
a run ("Soup: Fine-Tune an 8B Model on a 4 GB GPU", section "Why Layer
Streaming Matters Beyond the Laptop").  The pages report a release whose
streamed adapters were saved under keys with an extra ``.inner.`` segment,
so every loader silently returned the untuned base ("Show HN: Fine-tune an
8B model on a 4 GB laptop GPU", third paragraph; axbrief.com article, "Beyond
Memory: The Layer Streaming Breakthrough").  Files written here use the plain
key names of a causal-LM LoRA checkpoint, and the loader rejects any unknown
or missing key instead of ignoring it:

    base_model.model.model.layers.{i}.self_attn.{q,k,v,o}_proj.lora_A.weight  [r, in]
    base_model.model.model.layers.{i}.self_attn.{q,k,v,o}_proj.lora_B.weight  [out, r]
    base_model.model.model.layers.{i}.mlp.{gate,up,down}_proj.lora_{A,B}.weight

With y = x W + s (x A) B and A [in, r], B [r, out] inside the library, the
file holds A^T and B^T (the [r, in] / [out, r] orientation of a linear layer).

Run planning.  ``stream_source: auto`` keeps the base in RAM when it fits and
on NVMe when it does not, and a pre-flight refuses a run that will not fit
("Soup: Fine-Tune an 8B Model on a 4 GB GPU", sections "The Core Idea: Layer
Streaming" and "A Practical Quick Start").
"""
import json
import os

import numpy as np

PROJ = ("q", "k", "v", "o", "gate", "up", "down")
_MODULE = {"q": "self_attn.q_proj", "k": "self_attn.k_proj", "v": "self_attn.v_proj",
           "o": "self_attn.o_proj", "gate": "mlp.gate_proj", "up": "mlp.up_proj",
           "down": "mlp.down_proj"}


def adapter_key(layer, proj, which):
    """Checkpoint key of lora_A / lora_B of ``proj`` in ``layer``."""
    return f"base_model.model.model.layers.{layer}.{_MODULE[proj]}.lora_{which}.weight"


def adapter_state_dict(adapters):
    """{(layer, proj): (A [in, r], B [r, out])} -> {key: array} in file layout."""
    out = {}
    for (layer, proj), (A, B) in sorted(adapters.items()):
        out[adapter_key(layer, proj, "A")] = np.ascontiguousarray(np.asarray(A, np.float32).T)
        out[adapter_key(layer, proj, "B")] = np.ascontiguousarray(np.asarray(B, np.float32).T)
    return out


def adapters_from_state_dict(sd, n_layers, targets, shapes, rank):
    """Inverse of ``adapter_state_dict``.  Every expected key must be present
    with its exact shape and no other key may exist (a wrapper segment such as
    ``.inner.`` is an error, not a silently ignored entry)."""
    want = {}
    for layer in range(n_layers):
        for p in targets:
            N, K = shapes[p]
            want[adapter_key(layer, p, "A")] = (rank, K)
            want[adapter_key(layer, p, "B")] = (N, rank)
    extra = sorted(set(sd) - set(want))
    missing = sorted(set(want) - set(sd))
    if extra or missing:
        raise ValueError(f"adapter keys do not match: {len(missing)} missing "
                         f"(e.g. {missing[:2]}), {len(extra)} unexpected (e.g. {extra[:2]})")
    out = {}
    for layer in range(n_layers):
        for p in targets:
            a = np.asarray(sd[adapter_key(layer, p, "A")], np.float32)
            b = np.asarray(sd[adapter_key(layer, p, "B")], np.float32)
            if a.shape != want[adapter_key(layer, p, "A")] or b.shape != want[adapter_key(layer, p, "B")]:
                raise ValueError(f"adapter shape mismatch at layer {layer} {p}")
            out[(layer, p)] = (np.ascontiguousarray(a.T), np.ascontiguousarray(b.T))
    return out


def save_adapter(model, directory):
    """Write ``adapter_model.safetensors`` and ``adapter_config.json`` for a
    LayerStreamedLoRA model."""
    from safetensors.numpy import save_file
    os.makedirs(directory, exist_ok=True)
    adapters = {}
    for layer in range(model.cfg.n_layers):
        for p in model.lora_targets:
            A, B, _, _ = model.get_lora(layer, p)
            adapters[(layer, p)] = (A, B)
    save_file(adapter_state_dict(adapters), os.path.join(directory, "adapter_model.safetensors"))
    cfg = {"peft_type": "LORA", "r": int(model.cfg.lora_rank),
           "lora_alpha": float(model.cfg.lora_alpha), "lora_dropout": 0.0, "bias": "none",
           "target_modules": [_MODULE[p].split(".")[1] for p in model.lora_targets],
           "task_type": "CAUSAL_LM"}
    with open(os.path.join(directory, "adapter_config.json"), "w") as f:
        json.dump(cfg, f, indent=1)


def load_adapter(model, directory):
    """Load a file written by ``save_adapter`` (or any file with the same keys)
    into a LayerStreamedLoRA model."""
    from safetensors.numpy import load_file
    with open(os.path.join(directory, "adapter_config.json")) as f:
        cfg = json.load(f)
    if int(cfg["r"]) != model.cfg.lora_rank or abs(float(cfg["lora_alpha"]) - model.cfg.lora_alpha) > 0:
        raise ValueError("adapter rank / alpha differ from the model's")
    sd = load_file(os.path.join(directory, "adapter_model.safetensors"))
    shapes = {p: model.proj_shape(p) for p in model.lora_targets}
    ad = adapters_from_state_dict(sd, model.cfg.n_layers, model.lora_targets, shapes,
                                  model.cfg.lora_rank)
    for (layer, p), (A, B) in ad.items():
        model.set_lora(layer, p, A, B)


# ---------------------------------------------------------------------------
# run planning: stream source and pre-flight
# ---------------------------------------------------------------------------
class NoFit(RuntimeError):
    """The run needs more device memory than the GPU (or the budget) offers."""


def host_bytes_available():
    """MemAvailable of the host, in bytes."""
    with open("/proc/meminfo") as f:
        for line in f:
            if line.startswith("MemAvailable:"):
                return int(line.split()[1]) * 1024
    raise OSError("MemAvailable not found")


def plan_run(n_layers, record_bytes, workspace_bytes, device_free, host_available,
             host_reserve=8 << 30, source="auto"):
    """Where the base lives and whether the run fits.

    source 'auto': pinned host RAM when n_layers * record_bytes leaves
    host_reserve bytes free, else the file source.  Raises NoFit when the
    device workspace does not fit in device_free.  Returns the mode name."""
    if workspace_bytes > device_free:
        raise NoFit(f"device workspace {workspace_bytes / 1e9:.2f} GB exceeds the "
                    f"{device_free / 1e9:.2f} GB available")
    if source != "auto":
        return source
    store = n_layers * record_bytes
    return "stream_host" if store + host_reserve <= host_available else "stream_file"
