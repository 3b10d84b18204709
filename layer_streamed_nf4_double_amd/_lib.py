"""ctypes binding of liblsn (include/lsn.h): argument marshalling only.

Every function keeps the C name.  Device pointers may be given as torch
tensors (their data_ptr()) or plain integers; host arrays as numpy arrays.
A missing library raises at import time: there is no fallback path.
"""
import ctypes
import os

import numpy as np
# PyTorch ships its own HIP runtime (libamdhip64.so, soname libamdhip64.so.7)
# and the library links the system one under that soname.  With torch loaded
# first the library binds to torch's runtime; loaded first itself, it would
# bring in a second runtime that does not see the GPU once torch has taken it.
import torch  # noqa: F401  (load order only)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblsn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"liblsn.so not built ({LIB_PATH}); run "
                      "python -m layer_streamed_nf4_double_amd.build")
_lib = ctypes.CDLL(LIB_PATH)

LSN_OK, LSN_ERR_INVALID, LSN_ERR_NOFIT, LSN_ERR_HIP, LSN_ERR_IO, LSN_ERR_STATE = range(6)
STATUS_NAMES = {0: "LSN_OK", 1: "LSN_ERR_INVALID", 2: "LSN_ERR_NOFIT", 3: "LSN_ERR_HIP",
                4: "LSN_ERR_IO", 5: "LSN_ERR_STATE"}
LSN_RESIDENT, LSN_STREAM_HOST, LSN_STREAM_FILE = 0, 1, 2
LSN_PASS_FWD, LSN_PASS_BWD = 0, 1
PROJ = ("q", "k", "v", "o", "gate", "up", "down")
PROJ_ID = {p: i for i, p in enumerate(PROJ)}


class LsnError(RuntimeError):
    def __init__(self, status, msg=""):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")


class lsn_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("tied_embeddings", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("lora_rank", ctypes.c_int32), ("lora_alpha", ctypes.c_float),
                ("lora_targets", ctypes.c_uint32), ("max_tokens", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("store_path", ctypes.c_char_p), ("vram_budget", ctypes.c_uint64),
                ("head_on_host", ctypes.c_int32), ("head_chunk_rows", ctypes.c_int32),
                ("n_slots", ctypes.c_int32), ("layer_tokens", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32, _U32, _U64, _F = ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float
_CFG = ctypes.POINTER(lsn_config)
_SIGS = {
    "lsn_nf4_codebook": [_P],
    "lsn_nf4_quantize": [_P, _U64, _P, _P],
    "lsn_nf4_dequantize": [_P, _P, _U64, _P],
    "lsn_nf4_dequant": [_P, _P, _U64, _P, _I32, _P],
    "lsn_nf4_linear_scratch_bytes": [_I32, _I32, _I32, _I32, ctypes.POINTER(_U64)],
    "lsn_nf4_linear_fwd": [_P, _P, _I32, _I32, _I32, _P, _P, _P, _I32, _F, _P, _P, _U64, _P],
    "lsn_nf4_linear_bwd": [_P, _P, _I32, _I32, _I32, _P, _P, _P, _I32, _F, _P, _P, _P, _P, _P,
                           _U64, _P],
    "lsn_nf4_linear_fwd_noalloc": [_P, _P, _I32, _I32, _I32, _P, _P, _P, _I32, _F, _P, _P],
    "lsn_workspace_bytes": [_CFG, ctypes.POINTER(_U64)],
    "lsn_config_record_bytes": [_CFG, ctypes.POINTER(_U64)],
    "lsn_create": [_CFG, _P, _U64, _P, ctypes.POINTER(_P)],
    "lsn_destroy": [_P],
    "lsn_last_error": [_P],
    "lsn_sync": [_P],
    "lsn_record_bytes": [_P, ctypes.POINTER(_U64)],
    "lsn_file_direct_io": [_P, ctypes.POINTER(_I32)],
    "lsn_load_layer_nf4": [_P, _I32, ctypes.POINTER(_P), ctypes.POINTER(_P), _P, _P],
    "lsn_load_head": [_P, _P, _P, _P],
    "lsn_set_lora": [_P, _I32, _I32, _P, _P],
    "lsn_get_lora": [_P, _I32, _I32, _P, _P, _P, _P],
    "lsn_set_adapter_enabled": [_P, _I32],
    "lsn_zero_grads": [_P],
    "lsn_sgd_step": [_P, _F],
    "lsn_begin_pass": [_P, _I32, _I32, _I32],
    "lsn_embed": [_P, _P, _P],
    "lsn_forward_layer": [_P, _I32, _P, _P],
    "lsn_forward_layer_pair": [_P, _I32, _P, _P, _P, _P],
    "lsn_backward_layer": [_P, _I32, _P, _P, _P],
    "lsn_lm_head_logprobs": [_P, _P, _P, _P, _I32],
    "lsn_lm_head_backward": [_P, _P, _P, _P, _P],
    "lsn_sft_loss": [_P, _P, _P, _I32, _P, _P],
    "lsn_dpo_loss": [_P, _P, _P, _I32, _I32, _F, _P, _P],
    "lsn_pref_loss": [_P, _I32, _P, _P, _I32, _I32, _F, _F, _P, _P],
    "lsn_stats": [_P, ctypes.POINTER(_U64), ctypes.POINTER(_U64), ctypes.POINTER(_U64)],
    "lsn_copy_stream": [_P, ctypes.POINTER(_P)],
    "lsn_set_fault_injection": [_P, _I32, _I32, _I32],
    "lsn_set_profiling": [_P, _I32],
    "lsn_profile_query": [_P, _I32, _I32, _I32, _I32, ctypes.POINTER(_U64),
                          ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_lib.lsn_destroy.restype = None
_lib.lsn_last_error.restype = ctypes.c_char_p
EXPORTED = tuple(_SIGS)


def _ptr(x):
    """Device or host address of a torch tensor, numpy array, int or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        assert x.flags["C_CONTIGUOUS"], "host arrays must be contiguous"
        return x.ctypes.data
    if hasattr(x, "data_ptr"):
        assert x.is_contiguous(), "tensors must be contiguous"
        return x.data_ptr()
    raise TypeError(f"cannot take the address of {type(x)}")


def _check(st, ctx=None, what=""):
    if st != LSN_OK:
        # without a context the library keeps the thread's last message
        m = _lib.lsn_last_error(ctx if ctx else None)
        msg = f"{what}: {m.decode() if m else ''}"
        raise LsnError(st, msg)


# ---------------------------------------------------------------------------
# codec
# ---------------------------------------------------------------------------
def lsn_nf4_codebook():
    out = np.zeros(16, np.float32)
    _check(_lib.lsn_nf4_codebook(_ptr(out)), what="lsn_nf4_codebook")
    return out


def lsn_nf4_quantize(w):
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    n = w.size
    codes = np.zeros((n + 1) // 2, np.uint8)
    absmax = np.zeros((n + 63) // 64, np.float32)
    _check(_lib.lsn_nf4_quantize(_ptr(w), n, _ptr(codes), _ptr(absmax)), what="lsn_nf4_quantize")
    return codes, absmax


def lsn_nf4_dequantize(codes, absmax, n):
    out = np.zeros(n, np.float32)
    _check(_lib.lsn_nf4_dequantize(_ptr(np.ascontiguousarray(codes)),
                                        _ptr(np.ascontiguousarray(absmax)), n, _ptr(out)),
           what="lsn_nf4_dequantize")
    return out


def lsn_nf4_dequant(codes, absmax, n, out, out_bf16, stream=0):
    _check(_lib.lsn_nf4_dequant(_ptr(codes), _ptr(absmax), n, _ptr(out), int(out_bf16),
                                _ptr(stream)), what="lsn_nf4_dequant")


def lsn_nf4_linear_scratch_bytes(M, K, N, r):
    b = _U64(0)
    _check(_lib.lsn_nf4_linear_scratch_bytes(M, K, N, r, ctypes.byref(b)),
           what="lsn_nf4_linear_scratch_bytes")
    return b.value


def lsn_nf4_linear_fwd(codes, absmax, M, K, N, X, A, B, r, s, Y, scratch, scratch_bytes,
                       stream=0):
    _check(_lib.lsn_nf4_linear_fwd(_ptr(codes), _ptr(absmax), M, K, N, _ptr(X), _ptr(A), _ptr(B),
                                   r, s, _ptr(Y), _ptr(scratch), scratch_bytes, _ptr(stream)),
           what="lsn_nf4_linear_fwd")


def lsn_nf4_linear_fwd_noalloc(codes, absmax, M, K, N, X, A, B, r, s, Y, stream=0):
    _check(_lib.lsn_nf4_linear_fwd_noalloc(_ptr(codes), _ptr(absmax), M, K, N, _ptr(X), _ptr(A),
                                           _ptr(B), r, s, _ptr(Y), _ptr(stream)),
           what="lsn_nf4_linear_fwd_noalloc")


def lsn_nf4_linear_bwd(codes, absmax, M, K, N, X, A, B, r, s, dY, dX, dA, dB, scratch,
                       scratch_bytes, stream=0):
    _check(_lib.lsn_nf4_linear_bwd(_ptr(codes), _ptr(absmax), M, K, N, _ptr(X), _ptr(A), _ptr(B),
                                   r, s, _ptr(dY), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(scratch),
                                   scratch_bytes, _ptr(stream)), what="lsn_nf4_linear_bwd")


# ---------------------------------------------------------------------------
# context
# ---------------------------------------------------------------------------
def lsn_workspace_bytes(cfg):
    b = _U64(0)
    _check(_lib.lsn_workspace_bytes(ctypes.byref(cfg), ctypes.byref(b)), what="lsn_workspace_bytes")
    return b.value


def lsn_config_record_bytes(cfg):
    b = _U64(0)
    _check(_lib.lsn_config_record_bytes(ctypes.byref(cfg), ctypes.byref(b)),
           what="lsn_config_record_bytes")
    return b.value


def lsn_create(cfg, dev_ws, ws_bytes, stream=0):
    out = _P(None)
    _check(_lib.lsn_create(ctypes.byref(cfg), _ptr(dev_ws), ws_bytes, _ptr(stream),
                           ctypes.byref(out)), what="lsn_create")
    return out.value


def lsn_destroy(ctx):
    _lib.lsn_destroy(ctx)


def lsn_last_error(ctx):
    m = _lib.lsn_last_error(ctx)
    return m.decode() if m else ""


def lsn_sync(ctx):
    _check(_lib.lsn_sync(ctx), ctx, "lsn_sync")


def lsn_record_bytes(ctx):
    b = _U64(0)
    _check(_lib.lsn_record_bytes(ctx, ctypes.byref(b)), ctx, "lsn_record_bytes")
    return b.value


def lsn_file_direct_io(ctx):
    d = _I32(0)
    _check(_lib.lsn_file_direct_io(ctx, ctypes.byref(d)), ctx, "lsn_file_direct_io")
    return bool(d.value)


def lsn_load_layer_nf4(ctx, layer, codes, absmax, attn_norm_bf16, mlp_norm_bf16):
    """codes/absmax: sequences of 7 host arrays in projection order."""
    cs = [np.ascontiguousarray(c, dtype=np.uint8) for c in codes]
    am = [np.ascontiguousarray(a, dtype=np.float32) for a in absmax]
    cp = (_P * 7)(*[_ptr(c) for c in cs])
    ap = (_P * 7)(*[_ptr(a) for a in am])
    g1 = np.ascontiguousarray(attn_norm_bf16, dtype=np.uint16)
    g2 = np.ascontiguousarray(mlp_norm_bf16, dtype=np.uint16)
    _check(_lib.lsn_load_layer_nf4(ctx, layer, cp, ap, _ptr(g1), _ptr(g2)), ctx,
           "lsn_load_layer_nf4")


def lsn_load_head(ctx, embed_bf16, lm_head_bf16, final_norm_bf16):
    e = np.ascontiguousarray(embed_bf16, dtype=np.uint16)
    lm = None if lm_head_bf16 is None else np.ascontiguousarray(lm_head_bf16, dtype=np.uint16)
    f = np.ascontiguousarray(final_norm_bf16, dtype=np.uint16)
    _check(_lib.lsn_load_head(ctx, _ptr(e), _ptr(lm), _ptr(f)), ctx, "lsn_load_head")


def lsn_set_lora(ctx, layer, proj, A=None, B=None):
    A = None if A is None else np.ascontiguousarray(A, dtype=np.float32)
    B = None if B is None else np.ascontiguousarray(B, dtype=np.float32)
    _check(_lib.lsn_set_lora(ctx, layer, proj, _ptr(A), _ptr(B)), ctx, "lsn_set_lora")


def lsn_get_lora(ctx, layer, proj, K, N, r):
    A = np.zeros((K, r), np.float32)
    B = np.zeros((r, N), np.float32)
    dA = np.zeros((K, r), np.float32)
    dB = np.zeros((r, N), np.float32)
    _check(_lib.lsn_get_lora(ctx, layer, proj, _ptr(A), _ptr(B), _ptr(dA), _ptr(dB)), ctx,
           "lsn_get_lora")
    return A, B, dA, dB


def lsn_set_adapter_enabled(ctx, enabled):
    _check(_lib.lsn_set_adapter_enabled(ctx, int(enabled)), ctx, "lsn_set_adapter_enabled")


def lsn_zero_grads(ctx):
    _check(_lib.lsn_zero_grads(ctx), ctx, "lsn_zero_grads")


def lsn_sgd_step(ctx, lr):
    _check(_lib.lsn_sgd_step(ctx, lr), ctx, "lsn_sgd_step")


def lsn_begin_pass(ctx, kind, n_seq, seq_len):
    _check(_lib.lsn_begin_pass(ctx, kind, n_seq, seq_len), ctx, "lsn_begin_pass")


def lsn_embed(ctx, tokens, h0):
    _check(_lib.lsn_embed(ctx, _ptr(tokens), _ptr(h0)), ctx, "lsn_embed")


def lsn_forward_layer(ctx, layer, h_in, h_out):
    _check(_lib.lsn_forward_layer(ctx, layer, _ptr(h_in), _ptr(h_out)), ctx, "lsn_forward_layer")


def lsn_forward_layer_pair(ctx, layer, h_ref_in, h_ref_out, h_in, h_out):
    _check(_lib.lsn_forward_layer_pair(ctx, layer, _ptr(h_ref_in), _ptr(h_ref_out), _ptr(h_in),
                                       _ptr(h_out)), ctx, "lsn_forward_layer_pair")


def lsn_backward_layer(ctx, layer, h_in, dh_out, dh_in):
    _check(_lib.lsn_backward_layer(ctx, layer, _ptr(h_in), _ptr(dh_out), _ptr(dh_in)), ctx,
           "lsn_backward_layer")


def lsn_lm_head_logprobs(ctx, h, targets, logp, want_grad_state):
    _check(_lib.lsn_lm_head_logprobs(ctx, _ptr(h), _ptr(targets), _ptr(logp), int(want_grad_state)),
           ctx, "lsn_lm_head_logprobs")


def lsn_lm_head_backward(ctx, h, targets, dlogp, dh):
    _check(_lib.lsn_lm_head_backward(ctx, _ptr(h), _ptr(targets), _ptr(dlogp), _ptr(dh)), ctx,
           "lsn_lm_head_backward")


def lsn_sft_loss(ctx, logp, targets, n, loss, dlogp):
    _check(_lib.lsn_sft_loss(ctx, _ptr(logp), _ptr(targets), n, _ptr(loss), _ptr(dlogp)), ctx,
           "lsn_sft_loss")


def lsn_dpo_loss(ctx, logp_pol, logp_ref, seq_len, prompt_len, beta, out6, dlogp_pol):
    _check(_lib.lsn_dpo_loss(ctx, _ptr(logp_pol), _ptr(logp_ref), seq_len, prompt_len, beta,
                             _ptr(out6), _ptr(dlogp_pol)), ctx, "lsn_dpo_loss")


LSN_LOSS_DPO, LSN_LOSS_SIMPO, LSN_LOSS_ORPO, LSN_LOSS_KTO = 0, 1, 2, 3


def lsn_pref_loss(ctx, kind, logp_pol, logp_ref, seq_len, prompt_len, beta, param, out6,
                  dlogp_pol):
    _check(_lib.lsn_pref_loss(ctx, kind, _ptr(logp_pol), _ptr(logp_ref), seq_len, prompt_len,
                              beta, param, _ptr(out6), _ptr(dlogp_pol)), ctx, "lsn_pref_loss")


def lsn_stats(ctx):
    a, b, c = _U64(0), _U64(0), _U64(0)
    _check(_lib.lsn_stats(ctx, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), ctx,
           "lsn_stats")
    return a.value, b.value, c.value


def lsn_copy_stream(ctx):
    s = _P(None)
    _check(_lib.lsn_copy_stream(ctx, ctypes.byref(s)), ctx, "lsn_copy_stream")
    return s.value or 0


def lsn_set_fault_injection(ctx, copy_delay_us=0, compute_delay_us=0, poison_slots=False):
    _check(_lib.lsn_set_fault_injection(ctx, int(copy_delay_us), int(compute_delay_us),
                                        int(bool(poison_slots))), ctx, "lsn_set_fault_injection")


def lsn_set_profiling(ctx, on):
    _check(_lib.lsn_set_profiling(ctx, int(on)), ctx, "lsn_set_profiling")


def lsn_profile_query(ctx, what, a=0, b=0, tile=-1):
    """(launches, work, ms) over the recorded events (see lsn.h)."""
    n, w, t = _U64(0), ctypes.c_double(0), ctypes.c_double(0)
    _check(_lib.lsn_profile_query(ctx, what, a, b, tile, ctypes.byref(n), ctypes.byref(w),
                                  ctypes.byref(t)), ctx, "lsn_profile_query")
    return n.value, w.value, t.value
