"""GPU parity of the NF4 kernels through the C ABI: device dequantization
(bit-exact) and the NF4 + LoRA projection forward/backward against the
float64 oracle (bf16 compute: outputs within 2e-2, LoRA gradients within
5e-2, relative)."""
import sys

import numpy as np
import pytest

import synth
from oracle import nf4 as onf4
from tests.modelbuild import assert_close

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need a GPU"
    return t


@pytest.fixture(scope="module")
def L():
    from layer_streamed_nf4_double_amd import _lib
    return _lib


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("shape", [(256, 688), (1024, 4096), (7, 64 * 3)])
def test_dequant_bit_exact(torch, L, shape):
    say(f"[dequant] shape={shape}")
    W = synth.normal(shape, 9, 0, 1)
    codes, absmax = onf4.quantize(W)
    n = W.size
    want = onf4.dequantize(codes, absmax, n)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    L.lsn_nf4_dequant(_dev(torch, codes), _dev(torch, absmax), n, out, 0)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))
    outb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    L.lsn_nf4_dequant(_dev(torch, codes), _dev(torch, absmax), n, outb, 1)
    torch.cuda.synchronize()
    got = outb.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, synth.bf16_bits(want))


def _linear_case(M, K, N, r, seed):
    wid = 50 + seed
    X = synth.bf16_round(synth.normal((M, K), wid, 0, synth.TID_X, std=1.0))
    W = synth.normal((N, K), wid, 0, 0)                # stored W^T [N, K]
    A = synth.normal((K, r), wid, 0, 10) if r else None
    B = synth.normal((r, N), wid, 0, 11) if r else None
    dY = synth.bf16_round(synth.normal((M, N), wid, 0, synth.TID_DY, std=1.0))
    return X, W, A, B, dY


def _oracle_linear(X, Wd, A, B, s, dY):
    """float64: y = x W + s (x A) B and its backward (W = Wd^T frozen)."""
    from oracle import model as om
    X, Wd, dY = (np.asarray(v, np.float64) for v in (X, Wd, dY))
    if A is None:
        return X @ Wd.T, dY @ Wd, None, None
    A, B = np.asarray(A, np.float64), np.asarray(B, np.float64)
    y = om.lora_linear(X, Wd, A, B, s)
    dx, dA, dB = om.lora_linear_backward(X, Wd, A, B, s, dY)
    return y, dx, dA, dB


def _gpu_linear(torch, L, X, W, A, B, r, s, dY):
    M, K = X.shape
    N = W.shape[0]
    codes, absmax = L.lsn_nf4_quantize(W)
    cd, ad = _dev(torch, codes), _dev(torch, absmax)
    Xd = _dev(torch, synth.bf16_bits(X))
    dYd = _dev(torch, synth.bf16_bits(dY))
    Ad = _dev(torch, A) if r else None
    Bd = _dev(torch, B) if r else None
    sb = L.lsn_nf4_linear_scratch_bytes(M, K, N, r)
    scr = torch.empty(max(sb, 1), dtype=torch.uint8, device="cuda")
    # outputs start as NaN: every element must be written, none accumulated into
    nan = float("nan")
    Y = torch.full((M, N), nan, dtype=torch.float32, device="cuda")
    dX = torch.full((M, K), nan, dtype=torch.float32, device="cuda")
    dA = torch.full((K, max(r, 1)), nan, dtype=torch.float32, device="cuda")
    dB = torch.full((max(r, 1), N), nan, dtype=torch.float32, device="cuda")
    L.lsn_nf4_linear_fwd(cd, ad, M, K, N, Xd, Ad, Bd, r, s, Y, scr, sb)
    L.lsn_nf4_linear_bwd(cd, ad, M, K, N, Xd, Ad, Bd, r, s, dYd, dX, dA if r else None,
                         dB if r else None, scr, sb)
    torch.cuda.synchronize()
    return (Y.cpu().numpy(), dX.cpu().numpy(), dA.cpu().numpy() if r else None,
            dB.cpu().numpy() if r else None, codes, absmax)


# M >= 256 with K a multiple of 64 takes the 256 x 256 forward kernel:
# (256, 64, 256) one slice; (256, 832, 256) k range split 5/5/3; (512, 4096,
# 256) split 8 x 8 slices; (257, 128, 296) one-row M tail and a ragged N
# tile; (300, 1024, 2056) ragged M and N with the rank-16 extension.
# M >= 256 with N a multiple of 64 and K a multiple of 64 (K >= 128) takes the
# 256 x 256 input-gradient kernel: (256, 832, 256) a last column tile with one
# of four waves inside; (512, 4096, 256) 32 tiles of 4 slices; (300, 384,
# 1024) ragged M, half a column tile, split 4 and the rank-16 extension;
# (512, 640, 2048) split 8 x 4 slices.
# The low-rank down projection t = x A splits k over up to 8 workgroups per
# 16 rows: (40, 4096, 512, 8) takes 8 splits with a ragged last row block
# and rank 8 (columns 8-15 of every fragment masked).
@pytest.mark.parametrize("M,K,N,r", [(200, 688, 264, 8), (64, 256, 256, 16), (1, 16, 8, 4),
                                     (300, 1024, 2056, 16), (96, 512, 640, 0),
                                     (256, 64, 256, 0), (256, 832, 256, 16),
                                     (512, 4096, 256, 0), (257, 128, 296, 8),
                                     (300, 384, 1024, 16), (512, 640, 2048, 0),
                                     (40, 4096, 512, 8)])
def test_linear_parity_small(torch, L, M, K, N, r):
    say(f"[linear] M={M} K={K} N={N} r={r}")
    s = 2.0
    X, W, A, B, dY = _linear_case(M, K, N, r, seed=M % 7)
    Y, dX, dA, dB, codes, absmax = _gpu_linear(torch, L, X, W, A, B, r, s, dY)
    oc, oa = onf4.quantize(W)
    assert np.array_equal(codes, oc) and np.array_equal(absmax, oa)
    Wd = onf4.dequantize(oc, oa, W.size).reshape(W.shape)
    y, dx, da, db = _oracle_linear(X, Wd, A, B, s, dY)
    assert_close(Y, y, 2e-2, "Y")
    assert_close(dX, dx, 2e-2, "dX")
    if r:
        assert_close(dA, da, 5e-2, "dA")
        assert_close(dB, db, 5e-2, "dB")


def test_linear_parity_full_projection(torch, L):
    """The 512 x 4096 -> 14336 projection with a rank-16 adapter, full size."""
    p = synth.PROJECTION
    M, K, N, r, s = p["M"], p["K"], p["N"], p["r"], p["scale"]
    say(f"[linear-full] M={M} K={K} N={N} r={r}")
    wid = p["wid"]
    X = synth.bf16_round(synth.normal((M, K), wid, 0, synth.TID_X, std=1.0))
    W = synth.normal((N, K), wid, 0, 0)
    A = synth.normal((K, r), wid, 0, 10)
    B = synth.normal((r, N), wid, 0, 11)
    dY = synth.bf16_round(synth.normal((M, N), wid, 0, synth.TID_DY, std=1.0))
    Y, dX, dA, dB, codes, absmax = _gpu_linear(torch, L, X, W, A, B, r, s, dY)
    oc, oa = onf4.quantize(W)
    assert np.array_equal(codes, oc) and np.array_equal(absmax, oa)
    Wd = onf4.dequantize(oc, oa, W.size).reshape(W.shape)
    y, dx, da, db = _oracle_linear(X, Wd, A, B, s, dY)
    assert_close(Y, y, 2e-2, "Y")
    assert_close(dX, dx, 2e-2, "dX")
    assert_close(dA, da, 5e-2, "dA")
    assert_close(dB, db, 5e-2, "dB")


def test_b_zero_equals_no_adapter_bitwise_and_deterministic(torch, L):
    say("[linear] B=0 vs no adapter")
    M, K, N, r = 128, 512, 384, 16
    X, W, A, B, dY = _linear_case(M, K, N, r, seed=3)
    B0 = np.zeros_like(B)
    Y0 = _gpu_linear(torch, L, X, W, A, B0, r, 2.0, dY)[0]
    Yn = _gpu_linear(torch, L, X, W, None, None, 0, 2.0, dY)[0]
    assert np.array_equal(Y0.view(np.uint32), Yn.view(np.uint32))
    a = _gpu_linear(torch, L, X, W, A, B, r, 2.0, dY)
    b = _gpu_linear(torch, L, X, W, A, B, r, 2.0, dY)
    for u, v in zip(a[:4], b[:4]):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32))


def test_linear_invalid_shapes_rejected(torch, L):
    z = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.LsnError) as e:
        L.lsn_nf4_linear_fwd(z, z, 4, 24, 8, z, None, None, 0, 1.0, z, None, 0)  # K % 16
    assert e.value.status == L.LSN_ERR_INVALID
    with pytest.raises(L.LsnError) as e:
        L.lsn_nf4_linear_fwd(z, z, 4, 16, 8, z, z, z, 4, 1.0, z, None, 0)  # no scratch
    assert e.value.status == L.LSN_ERR_INVALID
    # an empty batch is a no-op
    L.lsn_nf4_linear_fwd(z, z, 0, 16, 8, z, None, None, 0, 1.0, z, None, 0)


def test_linear_empty_batch_zero_grads(torch, L):
    """M = 0: the backward writes zero adapter gradients and nothing else."""
    say("[linear] M=0 backward")
    K, N, r = 64, 32, 4
    codes, absmax = L.lsn_nf4_quantize(synth.normal((N, K), 5, 0, 0))
    cd, ad = _dev(torch, codes), _dev(torch, absmax)
    x = torch.zeros(8, dtype=torch.int16, device="cuda")  # never read or written at M = 0
    A = torch.zeros(K, r, device="cuda")
    B = torch.zeros(r, N, device="cuda")
    dA = torch.full((K, r), float("nan"), device="cuda")
    dB = torch.full((r, N), float("nan"), device="cuda")
    sb = L.lsn_nf4_linear_scratch_bytes(0, K, N, r)
    scr = torch.empty(max(sb, 1), dtype=torch.uint8, device="cuda")
    L.lsn_nf4_linear_bwd(cd, ad, 0, K, N, x, A, B, r, 2.0, x, x, dA, dB, scr, sb)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dA).item() == 0 and torch.count_nonzero(dB).item() == 0
