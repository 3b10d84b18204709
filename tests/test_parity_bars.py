"""The parity bar helper itself (CPU): assert_close must fail on the kind of
mistake a GEMM makes, one wrong output tile, which the global norm bar
alone averages away at the full sizes."""
import numpy as np
import pytest

from tests.modelbuild import assert_close


def _ref(shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def test_global_noise_at_the_bar_passes():
    o = _ref((2048, 1024))
    g = o + 0.5e-2 * _ref(o.shape, 1)
    assert_close(g, o, 2e-2, "noise")


def test_one_wrong_tile_fails_though_the_norm_passes():
    o = _ref((2048, 4096))  # 128 tiles of 256 x 256
    g = o.copy()
    g[256:512, 1024:1280] *= 1.10  # 10% off in one tile
    rel = np.linalg.norm(g - o) / np.linalg.norm(o)
    assert rel < 2e-2  # the global bar alone would pass it
    with pytest.raises(AssertionError, match="tile"):
        assert_close(g, o, 2e-2, "one tile")


def test_one_wrong_chunk_of_a_vector_fails():
    o = _ref(1 << 20)
    g = o.copy()
    g[65536:131072] += 0.06 * np.sqrt(np.mean(o * o))
    with pytest.raises(AssertionError, match="tile"):
        assert_close(g, o, 2e-2, "one chunk")


def test_small_tiles_use_the_average_scale():
    """A tile whose reference values are near zero (a cancelling DPO gradient
    region) is held to the average scale, not to its own tiny norm."""
    o = _ref((512, 512))
    o[:256, :256] *= 1e-6
    g = o + 1e-3 * _ref(o.shape, 2)
    assert_close(g, o, 2e-2, "small tile")
