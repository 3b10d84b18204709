"""NF4 blockwise codec (oracle).

Test infrastructure only; see ``oracle/__init__.py``.

The pages name the format only: the streamed base is optionally quantized to
NF4, which shrinks the stored weights about fourfold ("Soup: Fine-Tune an 8B
Model on a 4 GB GPU", section "The Core Idea: Layer Streaming", and the
``quantization: 4bit  # NF4`` key of its example config).  They print no code
table.  Readings taken here (plainest construction of "4-bit NormalFloat"):

* codebook: 16 values. Positive side = standard-normal quantiles at the first
  8 of 9 evenly spaced probabilities from 1-delta down to 1/2; negative side =
  minus the quantiles at the first 7 of 8 evenly spaced probabilities over the
  same range; plus an exact 0; sorted and divided by the largest value, so the
  table spans [-1, 1]. delta = (1/32 + 1/30) / 2. Computed in float64, then
  each value rounded to float32.
* blocks: 64 consecutive elements of the flattened weight (stored [out, in]
  row-major, as a causal-LM linear layer stores it); one float32 absmax per
  block; a partial last block is allowed.
* code of an element: x = fl32(w / absmax) (IEEE float32 division), code =
  number of float32 midpoints m_j = fl32((c_j + c_{j+1}) / 2) with x > m_j.
  Exact ties therefore go to the lower code.  An all-zero block stores absmax
  0 and code 7 (the exact zero) everywhere.  NaN / Inf inputs are rejected.
* packing: byte i holds element 2i in its low nibble and element 2i+1 in its
  high nibble; an odd length pads a zero high nibble.
* dequantize: w' = fl32(c[code] * absmax), one float32 multiply.
"""
import numpy as np
from scipy.stats import norm

BLOCK = 64


def codebook_f64():
    """The 16 NF4 levels in float64, before rounding (construction above)."""
    delta = 0.5 * (1.0 / 32.0 + 1.0 / 30.0)
    top = 1.0 - delta
    positive = norm.ppf(np.linspace(top, 0.5, 9)[:-1])     # 8 values > 0
    negative = -norm.ppf(np.linspace(top, 0.5, 8)[:-1])    # 7 values < 0
    levels = np.sort(np.concatenate([negative, [0.0], positive]))
    return levels / levels.max()


def codebook():
    """float32 codebook c_0 < ... < c_15 with c_0 = -1, c_7 = 0, c_15 = 1."""
    return codebook_f64().astype(np.float32)


def midpoints():
    """float32 decision thresholds m_j = fl32((c_j + c_{j+1}) / 2), j = 0..14,
    taken from the float64 levels."""
    c = codebook_f64()
    return ((c[:-1] + c[1:]) / 2.0).astype(np.float32)


def quantize(w):
    """Quantize a float32 array (any shape; flattened row-major).

    Returns (codes uint8 [ceil(n/2)], absmax float32 [ceil(n/64)]).
    Blocks are processed in batches, each element exactly as stated above.
    """
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    if not np.all(np.isfinite(w)):
        raise ValueError("NF4 quantize: non-finite input")
    n = w.size
    nblocks = (n + BLOCK - 1) // BLOCK
    mids = midpoints()
    padded = np.zeros(nblocks * BLOCK, np.float32)
    padded[:n] = w
    blocks = padded.reshape(nblocks, BLOCK)
    absmax = np.max(np.abs(blocks), axis=1).astype(np.float32)
    codes = np.empty((nblocks, BLOCK), dtype=np.uint8)
    step = 8192
    for b0 in range(0, nblocks, step):
        blk = blocks[b0:b0 + step]
        a = absmax[b0:b0 + step]
        safe = np.where(a == 0, np.float32(1), a)
        x = (blk / safe[:, None]).astype(np.float32)      # float32 / float32
        c = np.zeros(blk.shape, dtype=np.uint8)
        for m in mids:                                     # count thresholds below x
            c += (x > m)
        c[a == 0] = 7                                      # all-zero block: exact zero
        codes[b0:b0 + step] = c
    return pack(codes.reshape(-1)[:n]), absmax


def pack(codes):
    """Pack 4-bit codes two per byte, even element in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if codes.size % 2:
        codes = np.concatenate([codes, np.zeros(1, np.uint8)])
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)


def unpack(packed, n):
    """Inverse of ``pack``: the first n 4-bit codes."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed & 0x0F
    out[1::2] = packed >> 4
    return out[:n]


def dequantize(packed, absmax, n):
    """w'_e = fl32(c[code_e] * absmax[e // 64]) as a float32 vector of length n."""
    c = codebook()
    codes = unpack(packed, n)
    scale = np.repeat(np.asarray(absmax, dtype=np.float32), BLOCK)[:n]
    return (c[codes] * scale).astype(np.float32)
