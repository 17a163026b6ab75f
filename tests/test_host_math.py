"""Host-side integer identities the kernels rely on."""
import numpy as np


def test_small_division_by_multiplier():
    """For 0 <= t < 2^16 and 2 <= G < 2^16, the high 32 bits of
    t * ceil(2^32 / G) equal t // G (used to split a row index into token
    and head-in-group without a hardware divide)."""
    t = np.arange(1 << 16, dtype=np.uint64)
    Gs = list(range(2, 1025)) + list(np.random.default_rng(0).integers(1025, 1 << 16, 300))
    for G in Gs:
        G = int(G)
        M = np.uint64(((1 << 32) + G - 1) // G)
        assert M < (1 << 32)
        q = (t * M) >> np.uint64(32)
        assert np.array_equal(q, t // np.uint64(G)), G
