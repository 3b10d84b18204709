#!/usr/bin/env python3
"""Benchmark of layer-streamed NF4-LoRA training on one MI355X.

Default workload: a Llama-3.1-8B-shaped decoder (32 layers, hidden 4096,
32 q / 8 kv heads of 128, SwiGLU 14336, vocab 128256, RoPE theta 5e5), random
N(0, 0.02) base quantized to NF4 (block-64 absmax) and held in pinned host
RAM, LoRA r=16 (alpha 32) on q and v, one sequence of 512 uniform random
tokens.  A step is one streamed SFT step: forward over the stack (each layer
record copied host->device into one of two slots on a side stream while the
previous layer computes), LM-head log-probs, loss, LM-head backward, backward
over the stack (records streamed again, layer recomputed from its saved
input), SGD on the adapter.  The same model then runs streamed DPO steps on
one preference pair (2 x 512 tokens, 128 shared prompt tokens, beta 0.1).

Prints ONE JSON line (rank 0, N = 1).  Timing: W warm-up steps, then K steps
between two device synchronizations.  Inputs are resident before the clock
starts (the base in pinned host memory, tokens on the device).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

_T_START = time.perf_counter()
METRIC = "train tokens/sec (streamed NF4-LoRA SFT & DPO, 1 GPU); peak VRAM; % roofline"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3.1-8b-shaped")
    ap.add_argument("--mode", default="stream_host", choices=["stream_host", "resident"])
    ap.add_argument("--dpo-steps", type=int, default=5)
    ap.add_argument("--file-steps", type=int, default=2,
                    help="timed SFT steps with the base streamed from a store file (0: skip)")
    ap.add_argument("--second-workload", default="qwen2.5-3b-shaped",
                    help="a second streamed SFT + DPO leg ('' or 'none': skip)")
    ap.add_argument("--second-steps", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the projection, dequant and resident measurements")
    ap.add_argument("--link-mb", type=int, default=256)
    ap.add_argument("--projection-only", action="store_true",
                    help="only time the single projection and the standalone dequantization "
                         "(for counter profiles of those kernels)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run device-to-device copies of this size (counter calibration)")
    return ap.parse_args()


def copy_probe(mb, reps=5):
    """Plain device copies of known size: FETCH_SIZE / WRITE_SIZE of these
    dispatches calibrate the HBM traffic counters."""
    import torch
    n = mb << 20
    src = torch.empty(n // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n, "reps": reps}), flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(workload, mode):
    """HBM bytes per launch of the fused NF4 GEMM from the committed
    rocprofv3 FETCH_SIZE + WRITE_SIZE runs of the default workload (the
    8B-shaped streamed step), if the GEMM source is unchanged since they were
    taken; None for any other workload or a changed kernel."""
    import hashlib
    if workload != "llama3.1-8b-shaped" or mode != "stream_host":
        return None
    prof = os.path.join(ROOT, "profiles", "nf4f_gemm_llama8b_sft_traffic.md")
    src = os.path.join(ROOT, "layer_streamed_nf4_double_amd", "csrc", "gemm_nf4f.hip")
    try:
        kv = dict(l.split(": ", 1) for l in open(prof).read().splitlines() if ": " in l and
                  l.split(": ", 1)[0] in ("traffic_bytes_per_launch", "gemm_source_sha256"))
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if kv.get("gemm_source_sha256", "").strip() != digest:
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


# ---------------------------------------------------------------------------
# model construction (off the clock)
# ---------------------------------------------------------------------------
def quantized_layers(w):
    """Seeded fp32 weights -> NF4 records with the library's host codec."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import synth
    from layer_streamed_nf4_double_amd import _lib as L

    def one(layer):
        codes, absmax = [], []
        for p in synth.PROJ:
            c, a = L.lsn_nf4_quantize(synth.layer_weights_f32(w, layer, p))
            codes.append(c)
            absmax.append(a)
        return codes, absmax

    ones = np.full(w["hidden"], 0x3F80, np.uint16)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for layer, (codes, absmax) in enumerate(ex.map(one, range(w["n_layers"]))):
            if layer % 8 == 0:
                log(f"[bench] quantized layer {layer}/{w['n_layers']}")
            yield layer, codes, absmax, ones, ones


def build_model(w, mode, max_tokens, max_seq_len, layers, head, store_path=None,
                head_on_host=False, n_slots=0, layer_tokens=0):
    import numpy as np

    import synth
    from layer_streamed_nf4_double_amd.trainer import LayerStreamedLoRA
    m = LayerStreamedLoRA(w, mode, max_tokens=max_tokens, max_seq_len=max_seq_len,
                          store_path=store_path, head_on_host=head_on_host, n_slots=n_slots,
                          layer_tokens=layer_tokens)
    for layer, codes, absmax, g1, g2 in layers:
        m.load_layer(layer, codes, absmax, g1, g2)
    for layer in range(w["n_layers"]):
        for p in ("q", "v"):
            A, B = synth.lora_init(w, layer, p, b_zero=True)
            m.set_lora(layer, p, A, B)
    emb, lm, ones = head
    m.load_head(emb, lm, ones)
    return m


def storage_read_bandwidth(path, request):
    """Sequential O_DIRECT read of the whole file at path in requests of
    `request` bytes (the record size, as the file source issues them) into a
    page-aligned buffer: GB/s, or None when the file system refuses O_DIRECT."""
    import mmap
    try:
        fd = os.open(path, os.O_RDONLY | os.O_DIRECT)
    except OSError:
        return None
    buf = mmap.mmap(-1, request)
    try:
        done, t0 = 0, time.perf_counter()
        while True:
            n = os.preadv(fd, [buf], done)
            if n <= 0:
                break
            done += n
        dt = time.perf_counter() - t0
    finally:
        os.close(fd)
        buf.close()
    return done / dt / 1e9


def mount_of(path):
    """(device, file system type) of the mount holding path, from /proc/mounts."""
    path = os.path.realpath(path)
    best = ("?", "?", "")
    try:
        with open("/proc/mounts") as f:
            for line in f:
                dev, mnt, fstype = line.split()[:3]
                if (path == mnt or path.startswith(mnt.rstrip("/") + "/")) and len(mnt) > len(best[2]):
                    best = (dev, fstype, mnt)
    except OSError:
        pass
    return best[0], best[1]


def file_source_leg(torch, L, w, S, layers, head, tok, tgt, rec_bytes, steps):
    """The SFT step with the base streamed from a store file on local storage
    (records read with O_DIRECT into pinned bounce buffers, then copied to the
    slots).  The roofline is the storage read rate, probed on the same file."""
    import shutil
    import tempfile
    d = tempfile.mkdtemp(prefix="lsn_store_")
    path = os.path.join(d, "store.bin")
    try:
        torch.cuda.reset_peak_memory_stats()
        mf = build_model(w, "stream_file", S, S, layers, head, store_path=path)
        direct = L.lsn_file_direct_io(mf.ctx)
        fd = os.open(path, os.O_RDONLY)
        os.fsync(fd)
        os.close(fd)
        # two passes: the virtual disk's backing store caches on its host side,
        # so the second pass shows the rate the streamed steps see
        probes = [storage_read_bandwidth(path, rec_bytes) for _ in range(2)]
        disk = None if probes[0] is None else max(probes)
        log(f"[bench] store file on {mount_of(path)}: O_DIRECT {direct}, "
            f"probe reads {[p if p is None else round(p, 2) for p in probes]} GB/s")
        mf.sft_step(tok, tgt, 1, S, 1e-4)
        mf.sync()
        l0, b0, _ = mf.stats()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            mf.sft_step(tok, tgt, 1, S, 1e-4)
            torch.cuda.synchronize()
            log(f"[bench] file source step {i + 1}/{steps}")
        fdt = (time.perf_counter() - t0) / steps
        l1, b1, _ = mf.stats()
        fpeak = torch.cuda.max_memory_allocated()
        floss = float(mf.loss[0].item())
        mf.close()
        del mf
        torch.cuda.empty_cache()
    finally:
        shutil.rmtree(d, ignore_errors=True)
    gbps = (b1 - b0) / steps / fdt / 1e9
    dev, fstype = mount_of(d)
    out = {"tokens_per_s": round(S / fdt, 2), "ms_per_step": round(fdt * 1e3, 1),
           "steps": steps, "loss": floss, "direct_io": bool(direct),
           "storage": f"{dev} ({fstype})", "layer_loads_per_step": (l1 - l0) / steps,
           "achieved_GBps": round(gbps, 2),
           "bound": "storage read", "probe_read_GBps": None if disk is None else round(disk, 2),
           "probe_passes_GBps": [p if p is None else round(p, 2) for p in probes],
           "frac": None if not disk else round(gbps / disk, 4),
           "pinned_host_bytes": 2 * int(rec_bytes), "peak_vram_bytes": int(fpeak)}
    log(f"[bench] file source {fdt * 1e3:.0f} ms/step, {S / fdt:.1f} tok/s, {gbps:.2f} GB/s")
    return out


def head_on_host_leg(torch, L, w, S, layers, head, tok, tgt, steps, link_best):
    """The streamed SFT step with the embedding and LM-head tables in pinned
    host memory: W_lm streams through the layer slots each step, and the
    device holds the slots, the adapters and one layer's activations."""
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    m = build_model(w, "stream_host", S, S, layers, head, head_on_host=True)
    m.sft_step(tok, tgt, 1, S, 1e-4)
    m.sync()
    l0, b0, _ = m.stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        m.sft_step(tok, tgt, 1, S, 1e-4)
    torch.cuda.synchronize()
    hdt = (time.perf_counter() - t0) / steps
    l1, b1, _ = m.stats()
    peak = torch.cuda.max_memory_allocated()
    loss = float(m.loss[0].item())
    m.close()
    del m
    torch.cuda.empty_cache()
    gbps = (b1 - b0) / steps / hdt / 1e9
    out = {"tokens_per_s": round(S / hdt, 2), "ms_per_step": round(hdt * 1e3, 2), "steps": steps,
           "loss": loss, "peak_vram_bytes": int(peak),
           "layer_loads_per_step": (l1 - l0) / steps,
           "h2d_bytes_per_step": int((b1 - b0) / steps), "achieved_GBps": round(gbps, 2),
           "link_frac": round(gbps / link_best, 4),
           "note": "embedding and LM head in pinned host memory; W_lm streamed through the "
                   "layer slots each step"}
    log(f"[bench] head on host: {hdt * 1e3:.1f} ms/step, {S / hdt:.1f} tok/s, "
        f"peak {peak / 1e9:.2f} GB, {gbps:.1f} GB/s")
    return out


def algorithmic_bytes(w, rec_bytes, dpo=False):
    """Host-link bytes of one step as the method defines them (every decoder
    record streamed per pass, the LM head table streamed once per head pass):
    SFT 2 L records + 1 W_lm; DPO with a separate reference forward 3 L
    records + 2 W_lm."""
    wlm = w["vocab"] * w["hidden"] * 2
    L = w["n_layers"]
    return (3 * L * rec_bytes + 2 * wlm) if dpo else (2 * L * rec_bytes + wlm)


def sft_leg(torch, w, layers, head, tok, tgt, steps, warmup, n_slots=0, mode="stream_host"):
    """Streamed (or resident) SFT steps: ms/step, tokens/s, record loads and
    host->device bytes per step, peak device memory, final loss."""
    S = w["seq_len"]
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    m = build_model(w, mode, S, S, layers, head, n_slots=n_slots)
    for _ in range(warmup):
        m.sft_step(tok, tgt, 1, S, 1e-4)
    m.sync()
    l0, b0, _ = m.stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        m.sft_step(tok, tgt, 1, S, 1e-4)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    l1, b1, _ = m.stats()
    out = {"tokens_per_s": round(S / dt, 2), "ms_per_step": round(dt * 1e3, 2), "steps": steps,
           "peak_vram_bytes": int(torch.cuda.max_memory_allocated()),
           "layer_loads_per_step": (l1 - l0) / steps, "h2d_bytes_per_step": int((b1 - b0) / steps),
           "loss": float(m.loss[0].item())}
    m.close()
    del m
    torch.cuda.empty_cache()
    return out, dt


def dpo_leg(torch, w, layers, head, steps, warmup, sft_peak, sft_loads, link_best, rec_bytes,
            n_slots=0, layer_tokens=0):
    """Streamed DPO steps on one preference pair (fused reference pass).
    layer_tokens = seq_len: each layer runs the chosen and then the rejected
    sequence on its record (half the activation workspace, same copies)."""
    import numpy as np

    import synth
    from layer_streamed_nf4_double_amd.trainer import device_batch, sft_targets
    S = w["seq_len"]
    ch, rj = synth.dpo_pair(w)
    dtok = np.stack([ch, rj])
    d_tok, d_tgt = device_batch(dtok, sft_targets(dtok), w["vocab"])
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    md = build_model(w, "stream_host", 2 * S, S, layers, head, n_slots=n_slots,
                     layer_tokens=layer_tokens)
    P, beta = synth.dpo_prompt_len(w), synth.DPO_PAIR["beta"]
    for _ in range(max(1, warmup)):
        md.dpo_step(d_tok, d_tgt, S, P, beta, 1e-4)
    md.sync()
    l0, b0, _ = md.stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        md.dpo_step(d_tok, d_tgt, S, P, beta, 1e-4)
    torch.cuda.synchronize()
    ddt = (time.perf_counter() - t0) / steps
    l1, b1, _ = md.stats()
    dpeak = torch.cuda.max_memory_allocated()
    out = md.loss[:2].cpu().numpy()
    md.close()
    del md
    torch.cuda.empty_cache()
    alg = algorithmic_bytes(w, rec_bytes, dpo=True)
    return {"tokens_per_s": round(2 * S / ddt, 2), "ms_per_step": round(ddt * 1e3, 2),
            "n_slots": n_slots or 2,
            "layer_groups": ("one sequence per layer launch group (chosen, then rejected)"
                             if layer_tokens else "the pair as one 2 x seq_len batch"),
            "reference_pass": "fused with the policy forward (one record copy per layer)",
            "tokens_per_step": 2 * S, "loss": float(out[0]),
            "layer_loads_per_step": (l1 - l0) / steps,
            "layer_loads_ratio_vs_sft": round((l1 - l0) / steps / max(sft_loads, 1e-9), 3),
            "h2d_GBps": round((b1 - b0) / steps / ddt / 1e9, 2),
            "link_frac": round((b1 - b0) / steps / ddt / 1e9 / link_best, 4),
            "algorithmic_bytes_per_step": int(alg),
            "link_frac_algorithmic": round(alg / ddt / 1e9 / link_best, 4),
            "peak_vram_bytes": int(dpeak),
            "peak_vram_ratio_vs_sft": round(dpeak / sft_peak, 3)}


def link_bandwidth(torch, mb, reps=20):
    """Pinned host -> device copies of mb MiB on one stream (GB/s, best and median)."""
    n = mb << 20
    src = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    times = []
    with torch.cuda.stream(s):
        for _ in range(3):
            dst.copy_(src, non_blocking=True)
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            dst.copy_(src, non_blocking=True)
            e1.record(s)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) / 1e3)
    times.sort()
    return n / times[0] / 1e9, n / times[len(times) // 2] / 1e9


# ---------------------------------------------------------------------------
# the single projection (512 x 4096 -> 14336, rank-16 adapter) and the
# standalone dequantization, timed with events on the stream they run on
def projection_kernels(torch, reps=20):
    import numpy as np

    import synth
    from layer_streamed_nf4_double_amd import _lib as L
    p = synth.PROJECTION
    M, K, N, r, sc = p["M"], p["K"], p["N"], p["r"], p["scale"]
    wid = p["wid"]
    W = synth.normal((N, K), wid, 0, 0)
    c, a = L.lsn_nf4_quantize(W)
    cd, ad = torch.from_numpy(c).cuda(), torch.from_numpy(a).cuda()
    X = torch.from_numpy(synth.bf16_bits(synth.normal((M, K), wid, 0, synth.TID_X, std=1.0))).cuda()
    dY = torch.from_numpy(synth.bf16_bits(synth.normal((M, N), wid, 0, synth.TID_DY, std=1.0))).cuda()
    A = torch.from_numpy(synth.normal((K, r), wid, 0, 10)).cuda()
    B = torch.from_numpy(synth.normal((r, N), wid, 0, 11)).cuda()
    Y = torch.empty(M, N, device="cuda")
    dX = torch.empty(M, K, device="cuda")
    dA = torch.empty(K, r, device="cuda")
    dB = torch.empty(r, N, device="cuda")
    Wb = torch.empty(N * K, dtype=torch.int16, device="cuda")
    sb = L.lsn_nf4_linear_scratch_bytes(M, K, N, r)
    scr = torch.empty(sb, dtype=torch.uint8, device="cuda")

    def timed(fn):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3  # us

    fwd = timed(lambda: L.lsn_nf4_linear_fwd(cd, ad, M, K, N, X, A, B, r, sc, Y, scr, sb))
    bwd = timed(lambda: L.lsn_nf4_linear_bwd(cd, ad, M, K, N, X, A, B, r, sc, dY, dX, dA, dB,
                                             scr, sb))
    deq = timed(lambda: L.lsn_nf4_dequant(cd, ad, N * K, Wb, 1))
    gemm = 2.0 * M * N * K
    lora_f = 2.0 * M * r * (K + N)          # x A and (s t) B
    lora_b = 2.0 * M * r * (N + 2 * K + N)  # dY B^T, u A^T, x^T u, t^T dY
    deq_bytes = N * K // 2 + N * K // 16 + 2 * N * K

    def mf(flops, us):
        t = flops / (us * 1e-6) / 1e12
        return {"us": round(us, 2), "tflops": round(t, 1), "frac": round(t / MFMA_BF16_PEAK_TFLOPS, 4)}
    gbps = deq_bytes / (deq * 1e-6) / 1e9
    return {"shape": f"X [{M},{K}] bf16 . NF4 W [{K},{N}] + rank-{r} adapter",
            "fwd": mf(gemm + lora_f, fwd), "bwd_dx_da_db": mf(gemm + lora_b, bwd),
            "note": "end to end through lsn_nf4_linear_fwd / _bwd: adapter products, "
                    "split-k reduction and NF4 GEMM; flops = 2MNK + adapter products",
            "dequant_bf16": {"us": round(deq, 2), "bytes": deq_bytes, "GBps": round(gbps, 1),
                             "frac": round(gbps / HBM_PEAK_GBPS, 4), "bound": "hbm"}}


def library_bf16_context(torch, w, T, reps=30):
    """The step's forward NF4 GEMM launches (per layer: q|k|v, o and gate|up
    twice, in the forward and the backward's recompute, and down once) run as
    plain bf16 GEMMs of the same shapes in the ROCm BLAS library
    (torch.matmul, x [T, K] times W^T with W stored [N, K], the layout the NF4
    kernel reads its weights in).  Context for the roofline fraction: the
    library gets no dequantization to do.  Not part of the path."""
    H, F = w["hidden"], w["ffn"]
    d, nq, nkv = w["head_dim"], w["n_heads"], w["n_kv_heads"]
    shapes = {"q|k|v": (H, (nq + 2 * nkv) * d, 2), "o": (nq * d, H, 2),
              "gate|up": (H, 2 * F, 2), "down": (F, H, 1)}
    g = torch.Generator(device="cuda").manual_seed(0)
    out, tot_us, tot_fl, n = {}, 0.0, 0.0, 0
    for name, (K, N, per_layer) in shapes.items():
        x = torch.randn(T, K, device="cuda", dtype=torch.bfloat16, generator=g)
        wt = torch.randn(N, K, device="cuda", dtype=torch.bfloat16, generator=g)
        for _ in range(5):
            x @ wt.t()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            x @ wt.t()
        e1.record()
        e1.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        fl = 2.0 * T * K * N
        out[name] = {"us": round(us, 2), "frac": round(fl / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        tot_us += per_layer * us
        tot_fl += per_layer * fl
        n += per_layer
        del x, wt
    torch.cuda.empty_cache()
    return {"what": "torch.matmul bf16 (ROCm BLAS library), same shapes and launch mix",
            "avg_us": round(tot_us / n, 2),
            "frac": round(tot_fl / (tot_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "per_shape": out}


def step_flops(w, T, n_seq):
    """Algorithmic flops of one SFT step: each projection 3 times (forward,
    recompute, dX), the LM head twice (log-probs, dX), attention scores and
    values in the forward, the recompute and twice in the backward."""
    H, F, L = w["hidden"], w["ffn"], w["n_layers"]
    d, nq, nkv = w["head_dim"], w["n_heads"], w["n_kv_heads"]
    params = H * (nq * d) + 2 * H * (nkv * d) + (nq * d) * H + 3 * H * F
    S = T // n_seq
    attn = 2 * 2 * n_seq * S * S * d * nq
    return 3 * 2 * T * params * L + 2 * 2 * T * w["vocab"] * H + 4 * attn * L


def environment(torch, w, rec_bytes):
    import platform
    props = torch.cuda.get_device_properties(0)
    env = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
           "gpu": torch.cuda.get_device_name(0), "gpu_arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count, "gpu_memory_bytes": props.total_memory,
           "seed": 0, "pinned_store_bytes": int(rec_bytes) * w["n_layers"],
           "python": platform.python_version(), "host_threads": os.cpu_count(),
           "elapsed_s": round(time.perf_counter() - _T_START, 1)}
    # the installed HIP headers' version (read from the header rather than by
    # running hipcc: a child process of this one would start a second GPU
    # runtime under a profiler's preloaded library)
    try:
        import re
        with open("/opt/rocm/include/hip/hip_version.h") as f:
            d = dict(re.findall(r"#define HIP_VERSION_(MAJOR|MINOR|PATCH|GITHASH)\s+\"?(\w+)", f.read()))
        env["hipcc"] = f"HIP version: {d['MAJOR']}.{d['MINOR']}.{d['PATCH']}-{d['GITHASH']}"
    except (OSError, KeyError):
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            env["host_cpu"] = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
        with open("/proc/meminfo") as f:
            env["host_ram_bytes"] = int(next(l.split()[1] for l in f if l.startswith("MemTotal"))) * 1024
    except (OSError, StopIteration):
        pass
    return env


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample
# ---------------------------------------------------------------------------
def cpu_baseline(w, tokens):
    """Times the float32 oracle on one decoder layer (dequantize + forward, and
    dequantize + recomputed forward + backward) and on the LM head (forward +
    backward) at the real shape and 512 tokens, then scales to a full step:
    L x layer + head."""
    import numpy as np

    import synth
    from oracle import model as om
    from oracle import nf4 as onf4
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cfg = om.Config(n_layers=w["n_layers"], hidden=w["hidden"], n_heads=w["n_heads"],
                    n_kv_heads=w["n_kv_heads"], head_dim=w["head_dim"], ffn=w["ffn"],
                    vocab=w["vocab"], rms_eps=w["rms_eps"], rope_theta=w["rope_theta"],
                    lora_rank=w["lora_rank"], lora_alpha=w["lora_alpha"], tied=w["tied"])
    # off the clock: NF4 quantization of one layer (oracle codec), head tables
    rec = {}
    for p in synth.PROJ:
        W = synth.layer_weights_f32(w, 0, p)
        rec[p] = onf4.quantize(W) + (W.shape,)
    lora = {p: synth.lora_init(w, 0, p, b_zero=True) for p in ("q", "v")}
    emb, lm, _ = synth.head_tables(w)
    head = dict(embed=synth.bf16_to_f32(emb), lm_head=synth.bf16_to_f32(lm),
                final_norm=np.ones(w["hidden"], np.float32))
    h = head["embed"][tokens.reshape(-1)]
    targets = om.sft_targets(tokens)

    def deq():
        lw = {p: onf4.dequantize(c, a, int(np.prod(s))).reshape(s) for p, (c, a, s) in rec.items()}
        lw["attn_norm"] = np.ones(w["hidden"], np.float32)
        lw["mlp_norm"] = np.ones(w["hidden"], np.float32)
        return lw

    t0 = time.perf_counter()
    lw = deq()
    out, _ = om.layer_forward(cfg, lw, lora, h, 1)
    t1 = time.perf_counter()
    lw = deq()
    _, cache = om.layer_forward(cfg, lw, lora, h, 1)
    om.layer_backward(cfg, lw, lora, cache, out)
    t2 = time.perf_counter()
    logp, hc = om.head_logprobs(cfg, head, out, targets)
    _, dlogp = om.sft_loss(logp, targets)
    om.head_backward(cfg, head, hc, dlogp)
    t3 = time.perf_counter()
    step = w["n_layers"] * ((t1 - t0) + (t2 - t1)) + (t3 - t2)
    T = tokens.size
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
    except Exception:
        pass
    out = {"value": T / step, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "extrapolated": True, "blas": blas,
           "sample": (f"float32 numpy oracle, one {w['hidden']}-wide decoder layer "
                      f"(dequantize+forward {t1 - t0:.2f} s; dequantize+recompute+backward "
                      f"{t2 - t1:.2f} s) and the LM head fwd+bwd ({t3 - t2:.2f} s) at "
                      f"{T} tokens; the full step is extrapolated as {w['n_layers']} x the "
                      f"layer + the head: {step:.1f} s/step")}
    out["projection"] = cpu_projection(threads)
    return out


def cpu_projection(threads):
    """The oracle's forward NF4 projection with a rank-16 adapter at
    512 x 4096 -> 14336 (dequantize W, then x W + s (x A) B in float32), on
    all BLAS threads and on one."""
    import numpy as np

    import synth
    from oracle import model as om
    from oracle import nf4 as onf4
    p = synth.PROJECTION
    M, K, N, r, sc, wid = p["M"], p["K"], p["N"], p["r"], p["scale"], p["wid"]
    c, a = onf4.quantize(synth.normal((N, K), wid, 0, 0))
    x = synth.bf16_to_f32(synth.bf16_bits(synth.normal((M, K), wid, 0, synth.TID_X, std=1.0)))
    A = synth.normal((K, r), wid, 0, 10)
    B = synth.normal((r, N), wid, 0, 11)

    def run():
        t0 = time.perf_counter()
        Wt = onf4.dequantize(c, a, N * K).reshape(N, K)
        om.lora_linear(x, Wt, A, B, sc)
        return time.perf_counter() - t0

    res = {"shape": f"[{M},{K}] x NF4 [{K},{N}] + rank-{r} adapter, float32",
           "flops": 2.0 * M * N * K}
    res["seconds_all_threads"] = round(min(run() for _ in range(2)), 3)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            res["seconds_one_thread"] = round(run(), 3)
    except Exception:
        res["seconds_one_thread"] = None
    res["threads"] = int(threads)
    return res


# ---------------------------------------------------------------------------
def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on exactly one GPU (no collectives, no sharding); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mb:
        copy_probe(args.copy_probe_mb)
        return
    if args.projection_only:
        import torch
        print(json.dumps(projection_kernels(torch, reps=5)), flush=True)
        return
    import numpy as np
    import torch

    import synth
    from layer_streamed_nf4_double_amd import _lib as L
    from layer_streamed_nf4_double_amd.trainer import device_batch, sft_targets

    torch.cuda.set_device(0)
    w = synth.WORKLOADS[args.workload]
    S = w["seq_len"]
    log(f"[bench] workload {args.workload} mode {args.mode}")

    # ---- off the clock: weights, head tables, tokens ----
    t_setup = time.perf_counter()
    layers = list(quantized_layers(w))
    head = synth.head_tables(w)
    tokens = synth.sft_tokens(w)
    tok = torch.from_numpy(tokens.reshape(-1).astype(np.int32)).cuda()
    tgt = torch.from_numpy(sft_targets(tokens)).cuda()
    log(f"[bench] setup {time.perf_counter() - t_setup:.1f} s")

    link_best, link_med = link_bandwidth(torch, args.link_mb)
    log(f"[bench] host->device link: best {link_best:.1f} GB/s, median {link_med:.1f} GB/s")

    # ---- SFT ----
    torch.cuda.reset_peak_memory_stats()
    m = build_model(w, args.mode, S, S, layers, head)
    rec_bytes = L.lsn_record_bytes(m.ctx)
    for _ in range(args.warmup):
        m.sft_step(tok, tgt, 1, S, 1e-4)
    m.sync()
    loads0, bytes0, ws = m.stats()
    L.lsn_set_profiling(m.ctx, 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        m.sft_step(tok, tgt, 1, S, 1e-4)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dt = (t1 - t0) / args.steps
    loads1, bytes1, _ = m.stats()
    peak = torch.cuda.max_memory_allocated()
    loss = float(m.loss[0].item())
    n_gemm, flops, ms = L.lsn_profile_query(m.ctx, 0, 0, 2, 3)   # NF4 fwd GEMM, 256x256 kernel
    # the copies' own rate, from event pairs around each record copy in one
    # more (untimed) step: those events add packets between the copies, so
    # the timed steps record GEMM launches only
    L.lsn_set_profiling(m.ctx, 2)
    m.sft_step(tok, tgt, 1, S, 1e-4)
    n_cp, cp_bytes, cp_ms = L.lsn_profile_query(m.ctx, 1)
    L.lsn_set_profiling(m.ctx, 0)
    m.close()
    del m
    torch.cuda.empty_cache()
    h2d_per_step = (bytes1 - bytes0) / args.steps
    loads_per_step = (loads1 - loads0) / args.steps
    sft_tok_s = S / dt
    log(f"[bench] SFT {dt * 1e3:.1f} ms/step, {sft_tok_s:.1f} tok/s, loss {loss:.4f}, "
        f"{loads_per_step:.1f} loads/step, peak {peak / 1e9:.2f} GB")

    achieved = flops / (ms / 1e3) / 1e12 if ms > 0 else 0.0
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(args.workload, args.mode),
                "kernel": "nf4f_kernel (fused NF4-dequant MFMA GEMM, 256x256 or 256x128 tile)",
                "launches": int(n_gemm), "avg_us": round(ms / max(n_gemm, 1) * 1e3, 2),
                "flop_per_launch": flops / max(n_gemm, 1)}
    copy_gbps = cp_bytes / (cp_ms / 1e3) / 1e9 if cp_ms > 0 else 0.0
    alg = algorithmic_bytes(w, rec_bytes)
    link = {"bound": "host-link", "measured_peak_GBps": round(link_best, 2),
            "measured_median_GBps": round(link_med, 2),
            "h2d_bytes_per_step": int(h2d_per_step), "record_bytes": int(rec_bytes),
            "layer_loads_per_step": loads_per_step,
            "achieved_GBps": round(h2d_per_step / dt / 1e9, 2),
            "frac": round(h2d_per_step / dt / 1e9 / link_best, 4),
            "algorithmic_bytes_per_step": int(alg),
            "frac_algorithmic": round(alg / dt / 1e9 / link_best, 4),
            "note": "frac: bytes actually copied (2L - 4 records; the embedding and LM head stay "
                    "in device memory). frac_algorithmic: the method's bytes (2L records + one "
                    "W_lm pass) over the same step time; above 1 because the head stays "
                    "resident and 4 records are reused",
            "copy_engine_GBps_while_copying": round(copy_gbps, 2)}

    # ---- DPO on the same streamed base ----
    dpo = None
    if args.dpo_steps > 0:
        dpo = dpo_leg(torch, w, layers, head, args.dpo_steps, args.warmup, peak, loads_per_step,
                      link_best, rec_bytes)
        log(f"[bench] DPO {dpo['ms_per_step']:.1f} ms/step, {dpo['tokens_per_s']:.1f} tok/s, "
            f"loss {dpo['loss']:.4f}")
        if not args.no_extras:
            dpo["seq_groups"] = dpo_leg(torch, w, layers, head, max(1, args.dpo_steps // 2),
                                        args.warmup, peak, loads_per_step, link_best, rec_bytes,
                                        layer_tokens=S)
            log(f"[bench] DPO, one sequence per layer group: "
                f"{dpo['seq_groups']['ms_per_step']:.1f} ms/step, peak "
                f"{dpo['seq_groups']['peak_vram_bytes'] / 1e9:.2f} GB")

    # ---- three device slots (one more record resident: two fewer copies per step) ----
    slots3 = None
    if args.mode == "stream_host" and not args.no_extras:
        slots3, _ = sft_leg(torch, w, layers, head, tok, tgt, max(1, args.steps // 2),
                            args.warmup, n_slots=3)
        slots3["n_slots"] = 3
        slots3["link_frac"] = round(slots3["h2d_bytes_per_step"] / (slots3["ms_per_step"] / 1e3)
                                    / 1e9 / link_best, 4)
        log(f"[bench] 3 slots: {slots3['ms_per_step']:.1f} ms/step, "
            f"{slots3['layer_loads_per_step']} loads/step, peak {slots3['peak_vram_bytes'] / 1e9:.2f} GB")
        if dpo is not None:
            slots3["dpo"] = dpo_leg(torch, w, layers, head, max(1, args.dpo_steps // 2), args.warmup,
                                    slots3["peak_vram_bytes"], slots3["layer_loads_per_step"],
                                    link_best, rec_bytes, n_slots=3)
            log(f"[bench] 3 slots: DPO {slots3['dpo']['ms_per_step']:.1f} ms/step")

    # ---- the same step with the base resident on the device (peak VRAM side by side) ----
    resident = projection = file_src = head_host = None
    if not args.no_extras:
        if args.mode == "stream_host":
            torch.cuda.reset_peak_memory_stats()
            mr = build_model(w, "resident", S, S, layers, head)
            for _ in range(args.warmup):
                mr.sft_step(tok, tgt, 1, S, 1e-4)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                mr.sft_step(tok, tgt, 1, S, 1e-4)
            torch.cuda.synchronize()
            rdt = (time.perf_counter() - t0) / args.steps
            resident = {"tokens_per_s": round(S / rdt, 2), "ms_per_step": round(rdt * 1e3, 2),
                        "peak_vram_bytes": int(torch.cuda.max_memory_allocated()),
                        "compute_frac": round(step_flops(w, S, 1) / rdt / 1e12
                                              / MFMA_BF16_PEAK_TFLOPS, 4)}
            mr.close()
            del mr
            torch.cuda.empty_cache()
            log(f"[bench] resident SFT {rdt * 1e3:.1f} ms/step, peak "
                f"{resident['peak_vram_bytes'] / 1e9:.2f} GB")
        if args.mode == "stream_host":
            head_host = head_on_host_leg(torch, L, w, S, layers, head, tok, tgt,
                                         max(1, args.steps // 2), link_best)
        if args.mode == "stream_host" and args.file_steps > 0:
            file_src = file_source_leg(torch, L, w, S, layers, head, tok, tgt, rec_bytes,
                                       args.file_steps)
        projection = projection_kernels(torch)
        log(f"[bench] projection fwd {projection['fwd']['us']} us, bwd "
            f"{projection['bwd_dx_da_db']['us']} us, dequant {projection['dequant_bf16']['us']} us")

    # ---- a second workload: streamed SFT and DPO at its own shape ----
    second = None
    if args.second_workload not in ("", "none") and args.second_workload != args.workload:
        w2 = synth.WORKLOADS[args.second_workload]
        log(f"[bench] second workload {args.second_workload}")
        layers2 = list(quantized_layers(w2))
        head2 = synth.head_tables(w2)
        tokens2 = synth.sft_tokens(w2)
        tok2, tgt2 = device_batch(tokens2, sft_targets(tokens2), w2["vocab"])
        sft2, dt2 = sft_leg(torch, w2, layers2, head2, tok2, tgt2, args.second_steps,
                            args.warmup)
        from layer_streamed_nf4_double_amd.trainer import make_config
        rec2 = L.lsn_config_record_bytes(make_config(w2, "stream_host"))
        alg2 = algorithmic_bytes(w2, rec2)
        sft2.update({"record_bytes": int(rec2),
                     "link_frac": round(sft2["h2d_bytes_per_step"] / dt2 / 1e9 / link_best, 4),
                     "algorithmic_bytes_per_step": int(alg2),
                     "link_frac_algorithmic": round(alg2 / dt2 / 1e9 / link_best, 4)})
        dpo2 = dpo_leg(torch, w2, layers2, head2, max(1, args.second_steps // 2), args.warmup,
                       sft2["peak_vram_bytes"], sft2["layer_loads_per_step"], link_best, rec2)
        dpo2_3 = dpo_leg(torch, w2, layers2, head2, max(1, args.second_steps // 2), args.warmup,
                         sft2["peak_vram_bytes"], sft2["layer_loads_per_step"], link_best, rec2,
                         n_slots=3)
        dpo2["seq_groups"] = dpo_leg(torch, w2, layers2, head2, max(1, args.second_steps // 2),
                                     args.warmup, sft2["peak_vram_bytes"],
                                     sft2["layer_loads_per_step"], link_best, rec2,
                                     layer_tokens=w2["seq_len"])
        second = {"workload": f"{args.second_workload} streamed LoRA-SFT step (seq "
                              f"{w2['seq_len']}) and DPO step (2 x {w2['seq_len']})",
                  "n_layers": w2["n_layers"], "hidden": w2["hidden"], "vocab": w2["vocab"],
                  "tied": bool(w2["tied"]), "sft": sft2, "dpo": dpo2, "dpo_slots3": dpo2_3,
                  "link_note": "no record is copied while the LM head runs (both slots hold the "
                               "backward's first records); the copies themselves start 20-60 us "
                               "apart"}
        log(f"[bench] {args.second_workload}: SFT {sft2['tokens_per_s']} tok/s, DPO "
            f"{dpo2['tokens_per_s']} tok/s, DPO with 3 slots {dpo2_3['tokens_per_s']} tok/s")
        del layers2

    cpu = None
    # last of the GPU legs: the BLAS library keeps a workspace allocated, which
    # would count in the later legs' peak memory
    if not args.no_extras:
        library = library_bf16_context(torch, w, S)
        roofline["library_bf16_same_launches"] = library
        log(f"[bench] bf16 library GEMMs, same launch mix: {library['avg_us']} us per launch, "
            f"frac {library['frac']}")
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle sample)")
        cpu = cpu_baseline(w, tokens)
        log(f"[bench] oracle {cpu['value']:.3f} tok/s on {cpu['cores']} threads")

    line = {"metric": METRIC, "value": round(sft_tok_s, 2), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 3),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,0.02) NF4 base, uniform random tokens)",
            "config": {"workload": f"{args.workload} streamed LoRA-SFT step",
                       "n_layers": w["n_layers"], "hidden": w["hidden"], "ffn": w["ffn"],
                       "vocab": w["vocab"], "heads": f"{w['n_heads']}q/{w['n_kv_heads']}kv",
                       "global_batch": 1, "seq_len": S, "lora": "r16 a32 q,v",
                       "base": "NF4 block-64, pinned host RAM" if args.mode == "stream_host"
                       else "NF4 block-64, device resident",
                       "head": "embedding and LM head (bf16) resident in device memory; the "
                               "decoder layers stream (head_on_host: the head_on_host leg)",
                       "slots": 2,
                       "parallelism": "none (1 GPU)"},
            "peak_vram_bytes": int(peak), "loss": loss,
            "roofline": roofline, "link": link,
            "compute_utilization": {"flops_per_step": step_flops(w, S, 1),
                                    "frac": round(step_flops(w, S, 1) / dt / 1e12
                                                  / MFMA_BF16_PEAK_TFLOPS, 4)},
            "dpo": dpo, "slots3": slots3, "resident": resident, "head_on_host": head_host,
            "file_source": file_src, "second_workload": second,
            "projection": projection,
            "env": environment(torch, w, rec_bytes), "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
