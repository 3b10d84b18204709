"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
benchmark.  Holds no arithmetic of the method: only random draws, the named
workload shapes and bfloat16 storage rounding of input tables.

Every tensor has its own counter-addressed stream,
``PCG64(SeedSequence([seed, workload_id, layer, tensor_id]))``, so any layer
can be regenerated on its own, in any order and in parallel.

Weights: float32 standard normal times float32(0.02).  RMSNorm gains: 1.
Tokens: integers uniform in [0, vocab).
"""
import numpy as np

SEED = 0

# tensor ids inside a layer (stored as W^T = [out, in])
PROJ = ("q", "k", "v", "o", "gate", "up", "down")
TID = {name: i for i, name in enumerate(PROJ)}
TID_LORA = {("q", "A"): 10, ("q", "B"): 11, ("v", "A"): 12, ("v", "B"): 13,
            ("k", "A"): 14, ("k", "B"): 15, ("o", "A"): 16, ("o", "B"): 17,
            ("gate", "A"): 18, ("gate", "B"): 19, ("up", "A"): 20,
            ("up", "B"): 21, ("down", "A"): 22, ("down", "B"): 23}
TID_EMBED, TID_LM_HEAD = 100, 101
TID_TOKENS, TID_PROMPT, TID_CHOSEN, TID_REJECTED = 200, 201, 202, 203
TID_X, TID_DY = 300, 301

# named workloads: decoder shapes (no trained weights exist; shapes only)
WORKLOADS = {
    "tiny": dict(wid=0, n_layers=2, hidden=256, n_heads=4, n_kv_heads=4,
                 head_dim=64, ffn=688, vocab=1024, rms_eps=1e-5,
                 rope_theta=1e4, lora_rank=8, lora_alpha=16.0, tied=False,
                 n_seq=1, seq_len=64),
    "qwen2.5-3b-shaped": dict(wid=2, n_layers=36, hidden=2048, n_heads=16,
                              n_kv_heads=2, head_dim=128, ffn=11008,
                              vocab=151936, rms_eps=1e-6, rope_theta=1e6,
                              lora_rank=16, lora_alpha=32.0, tied=True,
                              n_seq=1, seq_len=512),
    "llama3.1-8b-shaped": dict(wid=3, n_layers=32, hidden=4096, n_heads=32,
                               n_kv_heads=8, head_dim=128, ffn=14336,
                               vocab=128256, rms_eps=1e-5, rope_theta=5e5,
                               lora_rank=16, lora_alpha=32.0, tied=False,
                               n_seq=1, seq_len=512),
}
# single NF4 projection with a rank-16 adapter
PROJECTION = dict(wid=1, M=512, K=4096, N=14336, r=16, scale=2.0)
# one DPO pair on the 8B shape: 128 shared prompt tokens, 384 response tokens
DPO_PAIR = dict(wid=4, prompt_len=128, seq_len=512, beta=0.1)


def rng(wid, layer, tid, seed=SEED):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(seed), int(wid), int(layer), int(tid)])))


def normal(shape, wid, layer, tid, std=0.02, seed=SEED):
    """float32 standard normal * float32(std) from its own stream."""
    z = rng(wid, layer, tid, seed).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    return z


def tokens(shape, vocab, wid, tid=TID_TOKENS, layer=0, seed=SEED):
    return rng(wid, layer, tid, seed).integers(0, vocab, size=shape, dtype=np.int32)


def bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + (((b >> 16) & 1) + np.uint32(0x7FFF))
    return (b >> 16).astype(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x):
    """float32 values that are exactly representable in bfloat16 (RNE)."""
    return bf16_to_f32(bf16_bits(x))


def layer_weights_f32(w, layer, proj):
    """Frozen base projection ``proj`` of ``layer`` as float32 W^T [out, in]."""
    N, K = proj_shape(w, proj)
    return normal((N, K), w["wid"], layer, TID[proj])


def proj_shape(w, proj):
    H, F = w["hidden"], w["ffn"]
    qd = w["n_heads"] * w["head_dim"]
    kvd = w["n_kv_heads"] * w["head_dim"]
    return {"q": (qd, H), "k": (kvd, H), "v": (kvd, H), "o": (H, qd),
            "gate": (F, H), "up": (F, H), "down": (H, F)}[proj]


def lora_init(w, layer, proj, b_zero):
    """(A [K, r], B [r, N]) float32; A ~ N(0, 0.02); B = 0 or ~ N(0, 0.02)."""
    N, K = proj_shape(w, proj)
    r = w["lora_rank"]
    A = normal((K, r), w["wid"], layer, TID_LORA[(proj, "A")])
    if b_zero:
        B = np.zeros((r, N), np.float32)
    else:
        B = normal((r, N), w["wid"], layer, TID_LORA[(proj, "B")])
    return A, B


def head_tables(w):
    """bfloat16 embedding and LM head tables (bit patterns) and the final norm
    gain (ones).  A tied model returns the same array for both."""
    V, H = w["vocab"], w["hidden"]
    emb = bf16_bits(normal((V, H), w["wid"], 0, TID_EMBED))
    lm = emb if w["tied"] else bf16_bits(normal((V, H), w["wid"], 0, TID_LM_HEAD))
    return emb, lm, np.ones(H, np.float32)


def sft_tokens(w):
    return tokens((w["n_seq"], w["seq_len"]), w["vocab"], w["wid"])


def dpo_prompt_len(w, pair=DPO_PAIR):
    """128 shared prompt tokens at seq 512; a quarter of shorter sequences."""
    return min(pair["prompt_len"], w["seq_len"] // 4)


def dpo_pair(w, pair=DPO_PAIR):
    """(chosen [S], rejected [S]) at the workload's sequence length: a shared
    random prompt, then independent random responses."""
    S, P, V = w["seq_len"], dpo_prompt_len(w, pair), w["vocab"]
    prompt = tokens((P,), V, pair["wid"], TID_PROMPT)
    ch = tokens((S - P,), V, pair["wid"], TID_CHOSEN)
    rj = tokens((S - P,), V, pair["wid"], TID_REJECTED)
    return np.concatenate([prompt, ch]), np.concatenate([prompt, rj])
