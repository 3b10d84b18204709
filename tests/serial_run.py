"""Two streamed SFT steps and two streamed DPO steps (fused reference pass)
of the tiny decoder with 5 layers and B != 0, every result as a flat list of
arrays: losses (DPO: loss, z, pc, pr, rc, rr), log-probs, and A, B, dA, dB
of every adapter after each step.  Run in-process by
tests/test_gpu_bitexact.py and, as a script, in a child process whose HIP
runtime serializes every kernel and copy (python tests/serial_run.py OUT.npz)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def run():
    import torch

    import synth
    from tests.modelbuild import gpu_model
    from layer_streamed_nf4_double_amd.trainer import device_batch, sft_targets
    w = dict(synth.WORKLOADS["tiny"], n_layers=5)
    S = w["seq_len"]
    out = []

    def adapters(m):
        for layer in range(w["n_layers"]):
            for p in ("q", "v"):
                out.extend(np.asarray(x, np.float32).ravel() for x in m.get_lora(layer, p))

    tokens = synth.sft_tokens(w)
    tok, tgt = device_batch(tokens, sft_targets(tokens), w["vocab"])
    m = gpu_model(w, "stream_host", b_zero=False)
    for _ in range(2):
        loss = m.sft_step(tok, tgt, 1, S, 0.1)
        m.sync()
        out.append(loss[:1].cpu().numpy().copy())
        out.append(m.logp[:S].cpu().numpy().copy())
        adapters(m)
    m.close()
    P = S // 4
    pr = synth.tokens((P,), w["vocab"], 89, synth.TID_PROMPT)
    ch = np.concatenate([pr, synth.tokens((S - P,), w["vocab"], 89, synth.TID_CHOSEN)])
    rj = np.concatenate([pr, synth.tokens((S - P,), w["vocab"], 89, synth.TID_REJECTED)])
    pair = np.stack([ch, rj])
    tok, tgt = device_batch(pair, sft_targets(pair), w["vocab"])
    m = gpu_model(w, "stream_host", b_zero=False, max_tokens=2 * S)
    for _ in range(2):
        o = m.dpo_step(tok, tgt, S, P, 0.1, 0.1, fused=True)
        m.sync()
        out.append(o[:6].cpu().numpy().copy())
        out.append(m.logp[:2 * S].cpu().numpy().copy())
        out.append(m.logp_ref[:2 * S].cpu().numpy().copy())
        adapters(m)
    m.close()
    return out


if __name__ == "__main__":
    res = run()
    np.savez(sys.argv[1], *res)
    print(f"serial_run: {len(res)} arrays, serialize kernel "
          f"{os.environ.get('AMD_SERIALIZE_KERNEL')} copy {os.environ.get('AMD_SERIALIZE_COPY')}",
          flush=True)
