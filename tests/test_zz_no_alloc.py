"""The allocation-free forward projection (lsn_nf4_linear_fwd_noalloc,
scratch in a fixed device array inside the library) against the
scratch-taking lsn_nf4_linear_fwd, through the C ABI: two calls in a row,
the second smaller (so it reads a scratch array the first call left full),
each bit for bit equal to the scratch-taking call on the same inputs; and a
shape whose scratch exceeds the array is refused."""
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _case(torch, L, M, K, N, r, s, wid):
    W = synth.normal((N, K), wid, 0, 0)
    c, a = L.lsn_nf4_quantize(W)
    cd, ad = torch.from_numpy(c).cuda(), torch.from_numpy(a).cuda()
    X = torch.from_numpy(synth.bf16_bits(synth.normal((M, K), wid, 0, synth.TID_X, std=1.0))).cuda()
    A = torch.from_numpy(synth.normal((K, r), wid, 0, 10)).cuda() if r else None
    B = torch.from_numpy(synth.normal((r, N), wid, 0, 11)).cuda() if r else None
    return cd, ad, X, A, B


def test_noalloc_forward_equals_scratch_forward():
    import torch
    from layer_streamed_nf4_double_amd import _lib as L
    assert torch.cuda.is_available()
    # the projection the bench times, then a smaller, ragged one
    for (M, K, N, r, s, wid) in ((512, 4096, 14336, 16, 2.0, 1), (300, 2048, 4104, 8, 0.5, 6)):
        say(f"[noalloc] {M} x {K} -> {N}, rank {r}")
        cd, ad, X, A, B = _case(torch, L, M, K, N, r, s, wid)
        sb = L.lsn_nf4_linear_scratch_bytes(M, K, N, r)
        scr = torch.empty(sb, dtype=torch.uint8, device="cuda")
        Y0 = torch.full((M, N), float("nan"), device="cuda")
        Y1 = torch.full((M, N), float("nan"), device="cuda")
        L.lsn_nf4_linear_fwd(cd, ad, M, K, N, X, A, B, r, s, Y0, scr, sb)
        L.lsn_nf4_linear_fwd_noalloc(cd, ad, M, K, N, X, A, B, r, s, Y1)
        torch.cuda.synchronize()
        y0, y1 = Y0.cpu().numpy(), Y1.cpu().numpy()
        assert np.all(np.isfinite(y1))
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
        del scr


def test_noalloc_refuses_oversized_scratch():
    import torch
    from layer_streamed_nf4_double_amd import _lib as L
    M, K, N = 256, 4096, 8192  # 32 tiles: split 8 x 8 MiB partial sums > 64 MiB
    cd, ad, X, A, B = _case(torch, L, M, K, N, 16, 2.0, 7)
    Y = torch.empty(M, N, device="cuda")
    with pytest.raises(L.LsnError) as e:
        L.lsn_nf4_linear_fwd_noalloc(cd, ad, M, K, N, X, A, B, 16, 2.0, Y)
    assert e.value.status == L.LSN_ERR_INVALID
    assert "scratch" in str(e.value)
