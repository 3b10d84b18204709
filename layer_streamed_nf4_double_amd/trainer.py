"""SFT / DPO step loops over liblsn.  Orchestration only: every computation is
a call into the C ABI; PyTorch provides device memory and the stream.

One SFT step (page "Soup: Fine-Tune an 8B Model on a 4 GB GPU", "The Core Idea:
Layer Streaming"): forward over the streamed stack keeping each layer's input,
LM-head log-probs, loss, LM-head backward, backward over the stack in reverse
(each layer re-streamed and recomputed from its saved input), SGD on the
adapter.  One DPO step (page "Show HN: Fine-tune an 8B model on a 4 GB laptop
GPU", first paragraph): a reference forward with the adapter switched off,
then the policy forward with it on, both over the same streamed base, then
the DPO loss and the backward of the policy pass.  By default both forwards
run on one copy of each layer record (lsn_forward_layer_pair), so a DPO step
streams the stack twice, like SFT, instead of three times.
"""
import contextlib
import os

import numpy as np

from . import _lib as L
from ._lib import (LSN_PASS_BWD, LSN_PASS_FWD, LSN_RESIDENT, LSN_STREAM_FILE,
                   LSN_STREAM_HOST, PROJ, PROJ_ID)

MODES = {"resident": LSN_RESIDENT, "stream_host": LSN_STREAM_HOST, "stream_file": LSN_STREAM_FILE}
PREF_LOSSES = {"dpo": L.LSN_LOSS_DPO, "simpo": L.LSN_LOSS_SIMPO, "orpo": L.LSN_LOSS_ORPO,
               "kto": L.LSN_LOSS_KTO}


def make_config(shape, mode="stream_host", max_tokens=None, max_seq_len=None,
                lora_targets=("q", "v"), store_path=None, vram_budget=0, head_on_host=False,
                head_chunk_rows=0, n_slots=0, layer_tokens=0):
    """lsn_config from a shape dict (n_layers, hidden, n_heads, n_kv_heads,
    head_dim, ffn, vocab, rms_eps, rope_theta, lora_rank, lora_alpha, tied)."""
    cfg = L.lsn_config()
    cfg.n_layers = shape["n_layers"]
    cfg.hidden = shape["hidden"]
    cfg.n_heads = shape["n_heads"]
    cfg.n_kv_heads = shape["n_kv_heads"]
    cfg.head_dim = shape["head_dim"]
    cfg.ffn = shape["ffn"]
    cfg.vocab = shape["vocab"]
    cfg.tied_embeddings = int(bool(shape["tied"]))
    cfg.rms_eps = shape["rms_eps"]
    cfg.rope_theta = shape["rope_theta"]
    cfg.lora_rank = shape["lora_rank"]
    cfg.lora_alpha = shape["lora_alpha"]
    cfg.lora_targets = sum(1 << PROJ_ID[p] for p in lora_targets)
    cfg.max_seq_len = max_seq_len or shape["seq_len"]
    cfg.max_tokens = max_tokens or shape["n_seq"] * shape["seq_len"]
    cfg.mode = MODES[mode]
    cfg.store_path = store_path.encode() if store_path else None
    cfg.vram_budget = vram_budget
    cfg.head_on_host = int(bool(head_on_host))
    cfg.head_chunk_rows = head_chunk_rows
    cfg.n_slots = n_slots
    cfg.layer_tokens = layer_tokens
    return cfg


class LayerStreamedLoRA:
    """A context plus the activation tensors of one step."""

    def __init__(self, shape, mode="stream_host", max_tokens=None, max_seq_len=None,
                 lora_targets=("q", "v"), store_path=None, device="cuda:0", stream=None,
                 head_on_host=False, head_chunk_rows=0, n_slots=0, vram_budget=0,
                 layer_tokens=0):
        """mode: resident | stream_host | stream_file | auto.  'auto' keeps the
        base in pinned RAM when it fits and in a file (store_path, or a file
        in $TMPDIR) when it does not; every mode is pre-flighted against the
        free device memory (adapter.NoFit).  head_on_host (streamed modes):
        the embedding and LM-head tables stay in pinned host memory and W_lm
        streams through the layer slots.  n_slots: device slots of the layer
        stream (0: two).  vram_budget: lsn_create refuses a workspace larger
        than this many bytes (0: no limit).  layer_tokens: tokens of one layer
        launch group (0: the whole pass); a DPO pair with layer_tokens =
        seq_len runs the chosen and the rejected sequence one after the other
        on each record, with half the activation workspace."""
        import tempfile

        import torch

        from . import adapter
        self.torch = torch
        self.shape = dict(shape)
        self.device = torch.device(device)
        # sizes only (a streamed file store needs no path for them)
        probe = make_config(shape, "stream_host" if mode in ("auto", "stream_file") else mode,
                            max_tokens, max_seq_len, lora_targets, store_path,
                            head_on_host=head_on_host, head_chunk_rows=head_chunk_rows,
                            n_slots=n_slots, layer_tokens=layer_tokens)
        free, _ = torch.cuda.mem_get_info(self.device)
        mode = adapter.plan_run(shape["n_layers"], L.lsn_config_record_bytes(probe),
                                L.lsn_workspace_bytes(probe), free,
                                adapter.host_bytes_available(),
                                source="auto" if mode == "auto" else mode)
        self._own_store = None  # a store file this object created, removed by close()
        if mode == "stream_file" and not store_path:
            store_path = os.path.join(tempfile.gettempdir(), f"lsn_store_{os.getpid()}_{id(self)}.bin")
            self._own_store = store_path
        self.mode = mode
        self.cfg = make_config(shape, mode, max_tokens, max_seq_len, lora_targets, store_path,
                               vram_budget=vram_budget, head_on_host=head_on_host,
                               head_chunk_rows=head_chunk_rows, n_slots=n_slots,
                               layer_tokens=layer_tokens)
        self.lora_targets = tuple(lora_targets)
        self.ws_bytes = L.lsn_workspace_bytes(self.cfg)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        # The caller's current stream by default.  When another stream is
        # given, the step methods order it against the caller's current
        # stream on entry and exit.
        self.stream = stream or torch.cuda.current_stream(self.device)
        self.ctx = L.lsn_create(self.cfg, self.ws, self.ws_bytes, self.stream.cuda_stream)
        T, H, nl = self.cfg.max_tokens, self.cfg.hidden, self.cfg.n_layers
        f32 = dict(dtype=torch.float32, device=self.device)
        self.hs = [torch.empty(T, H, **f32) for _ in range(nl + 1)]
        self.href = [torch.empty(T, H, **f32) for _ in range(2)]  # fused DPO reference
        self.dh = torch.empty(T, H, **f32)
        self.logp = torch.empty(T, **f32)
        self.logp_ref = torch.empty(T, **f32)
        self.dlogp = torch.empty(T, **f32)
        self.loss = torch.zeros(8, **f32)

    def close(self):
        if self.ctx:
            self.stream.synchronize()
            L.lsn_destroy(self.ctx)
            self.ctx = None
        if getattr(self, "_own_store", None):
            try:
                os.remove(self._own_store)
            except OSError:
                pass
            self._own_store = None

    @contextlib.contextmanager
    def _ordered(self):
        """Runs a step on the context's stream after the caller's pending
        work, and makes the caller's stream wait for the step."""
        cur = self.torch.cuda.current_stream(self.device)
        if cur != self.stream:
            self.stream.wait_stream(cur)
        try:
            yield
        finally:
            if cur != self.stream:
                cur.wait_stream(self.stream)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---------------------------------------------------------------- weights
    def load_layer(self, layer, codes, absmax, attn_norm_bf16, mlp_norm_bf16):
        L.lsn_load_layer_nf4(self.ctx, layer, codes, absmax, attn_norm_bf16, mlp_norm_bf16)

    def load_head(self, embed_bf16, lm_head_bf16, final_norm_bf16):
        L.lsn_load_head(self.ctx, embed_bf16, None if self.cfg.tied_embeddings else lm_head_bf16,
                        final_norm_bf16)

    def proj_shape(self, proj):
        H, F = self.cfg.hidden, self.cfg.ffn
        qd = self.cfg.n_heads * self.cfg.head_dim
        kvd = self.cfg.n_kv_heads * self.cfg.head_dim
        return {"q": (qd, H), "k": (kvd, H), "v": (kvd, H), "o": (H, qd),
                "gate": (F, H), "up": (F, H), "down": (H, F)}[proj]

    def set_lora(self, layer, proj, A, B):
        L.lsn_set_lora(self.ctx, layer, PROJ_ID[proj], A, B)

    def get_lora(self, layer, proj):
        N, K = self.proj_shape(proj)
        return L.lsn_get_lora(self.ctx, layer, PROJ_ID[proj], K, N, self.cfg.lora_rank)

    def stats(self):
        return L.lsn_stats(self.ctx)

    def sync(self):
        L.lsn_sync(self.ctx)

    # ---------------------------------------------------------------- steps
    def _forward(self, tokens, n_seq, seq_len, save=True):
        T = n_seq * seq_len
        L.lsn_begin_pass(self.ctx, LSN_PASS_FWD, n_seq, seq_len)
        hs = [h[:T] for h in self.hs]
        L.lsn_embed(self.ctx, tokens, hs[0])
        nl = self.cfg.n_layers
        for i in range(nl):
            if save:
                L.lsn_forward_layer(self.ctx, i, hs[i], hs[i + 1])
            else:  # ping-pong between two buffers, nothing kept
                L.lsn_forward_layer(self.ctx, i, hs[i % 2], hs[(i + 1) % 2])
        return hs[nl] if save else hs[nl % 2]

    def _backward(self, n_seq, seq_len):
        T = n_seq * seq_len
        dh = self.dh[:T]
        L.lsn_zero_grads(self.ctx)
        L.lsn_begin_pass(self.ctx, LSN_PASS_BWD, n_seq, seq_len)
        for i in reversed(range(self.cfg.n_layers)):
            L.lsn_backward_layer(self.ctx, i, self.hs[i][:T], dh, dh)

    def sft_step(self, tokens, targets, n_seq, seq_len, lr):
        """tokens, targets: device int32 [n_seq*seq_len].  Returns the device
        loss tensor (loss[0]); logp of the step stays in self.logp."""
        with self._ordered():
            T = n_seq * seq_len
            hL = self._forward(tokens, n_seq, seq_len, save=True)
            L.lsn_lm_head_logprobs(self.ctx, hL, targets, self.logp[:T], 1)
            L.lsn_sft_loss(self.ctx, self.logp[:T], targets, T, self.loss, self.dlogp[:T])
            L.lsn_lm_head_backward(self.ctx, hL, targets, self.dlogp[:T], self.dh[:T])
            self._backward(n_seq, seq_len)
            if lr is not None:
                L.lsn_sgd_step(self.ctx, lr)
            return self.loss

    def _forward_pair(self, tokens, n_seq, seq_len):
        """Reference (adapter off) and policy forward sharing every layer
        record; the policy inputs are kept.  Returns (h_ref_L, h_L)."""
        T = n_seq * seq_len
        L.lsn_begin_pass(self.ctx, LSN_PASS_FWD, n_seq, seq_len)
        hs = [h[:T] for h in self.hs]
        hr = [h[:T] for h in self.href]
        L.lsn_embed(self.ctx, tokens, hs[0])
        L.lsn_embed(self.ctx, tokens, hr[0])
        for i in range(self.cfg.n_layers):
            L.lsn_forward_layer_pair(self.ctx, i, hr[i % 2], hr[(i + 1) % 2], hs[i], hs[i + 1])
        return hr[self.cfg.n_layers % 2], hs[self.cfg.n_layers]

    def dpo_step(self, tokens, targets, seq_len, prompt_len, beta, lr, fused=True):
        """tokens, targets: device int32 [2*seq_len] (chosen then rejected).
        loss[0..5] = loss, z, pc, pr, rc, rr.  fused: the reference forward
        runs on the same record copy as the policy forward (2L record loads
        per step instead of 3L); the results are the same bits."""
        with self._ordered():
            T = 2 * seq_len
            if fused:
                L.lsn_set_adapter_enabled(self.ctx, 1)
                h_ref, hL = self._forward_pair(tokens, 2, seq_len)
                L.lsn_lm_head_logprobs(self.ctx, h_ref, targets, self.logp_ref[:T], 0)
            else:
                L.lsn_set_adapter_enabled(self.ctx, 0)
                h_ref = self._forward(tokens, 2, seq_len, save=False)
                L.lsn_lm_head_logprobs(self.ctx, h_ref, targets, self.logp_ref[:T], 0)
                L.lsn_set_adapter_enabled(self.ctx, 1)
                hL = self._forward(tokens, 2, seq_len, save=True)
            L.lsn_lm_head_logprobs(self.ctx, hL, targets, self.logp[:T], 1)
            L.lsn_dpo_loss(self.ctx, self.logp[:T], self.logp_ref[:T], seq_len, prompt_len, beta,
                           self.loss, self.dlogp[:T])
            L.lsn_lm_head_backward(self.ctx, hL, targets, self.dlogp[:T], self.dh[:T])
            self._backward(2, seq_len)
            if lr is not None:
                L.lsn_sgd_step(self.ctx, lr)
            return self.loss


    def pref_step(self, kind, tokens, targets, seq_len, prompt_len, beta, param, lr):
        """One preference step on a pair with the loss ``kind`` (dpo, simpo, orpo,
        kto).  Losses with a reference (dpo, kto) run the adapter-off forward on
        the same record copies as the policy forward; reference-free ones
        (simpo, orpo) stream the stack once forward, like SFT."""
        with self._ordered():
            T = 2 * seq_len
            k = PREF_LOSSES[kind]
            L.lsn_set_adapter_enabled(self.ctx, 1)
            ref = None
            if k in (L.LSN_LOSS_DPO, L.LSN_LOSS_KTO):
                h_ref, hL = self._forward_pair(tokens, 2, seq_len)
                L.lsn_lm_head_logprobs(self.ctx, h_ref, targets, self.logp_ref[:T], 0)
                ref = self.logp_ref[:T]
            else:
                hL = self._forward(tokens, 2, seq_len, save=True)
            L.lsn_lm_head_logprobs(self.ctx, hL, targets, self.logp[:T], 1)
            L.lsn_pref_loss(self.ctx, k, self.logp[:T], ref, seq_len, prompt_len, beta, param,
                            self.loss, self.dlogp[:T])
            L.lsn_lm_head_backward(self.ctx, hL, targets, self.dlogp[:T], self.dh[:T])
            self._backward(2, seq_len)
            if lr is not None:
                L.lsn_sgd_step(self.ctx, lr)
            return self.loss


def check_ids(tokens, targets, vocab):
    """Host-side range check of a batch before it goes to the device: every
    token id in [0, vocab), every target in [0, vocab) or -1 (no target).
    The kernels stay in bounds for any id (an out-of-range token embeds as a
    NaN row, an out-of-range target gives a NaN log-prob), so this turns a
    bad batch into an error instead of a NaN loss."""
    tokens = np.asarray(tokens)
    targets = np.asarray(targets)
    if tokens.size and (tokens.min() < 0 or tokens.max() >= vocab):
        raise ValueError(f"token ids must lie in [0, {vocab})")
    if targets.size and (targets.min() < -1 or targets.max() >= vocab):
        raise ValueError(f"targets must lie in [0, {vocab}) or be -1")


def device_batch(tokens, targets, vocab, device="cuda"):
    """Checked int32 device copies of host tokens and targets (flattened)."""
    import torch
    tokens = np.ascontiguousarray(np.asarray(tokens).reshape(-1), dtype=np.int32)
    targets = np.ascontiguousarray(np.asarray(targets).reshape(-1), dtype=np.int32)
    check_ids(tokens, targets, vocab)
    return (torch.from_numpy(tokens).to(device), torch.from_numpy(targets).to(device))


def sft_targets(tokens):
    """Next-token targets: position t predicts token t+1; the last position of
    each sequence has none (-1)."""
    tokens = np.asarray(tokens)
    t = np.full(tokens.shape, -1, dtype=np.int32)
    t[:, :-1] = tokens[:, 1:]
    return t.reshape(-1)
