"""Host logic of the cross-attention inputs: packed sample spans."""
import numpy as np

import workloads as W


def test_cross_lengths_ranges():
    totals = []
    for seed in range(5):
        t, im = W.cross_lengths(32, seed)
        assert len(t) == len(im) == 32
        assert all(100 <= x < 200 for x in t)
        assert all(1200 <= x <= 3000 for x in im)
        totals.append(sum(t))
        assert W.cross_lengths(32, seed) == (t, im)   # seeded
    # no parity adjustment: odd text totals occur (any S is accepted)
    assert any(x % 2 for x in totals)


def test_cross_bounds_are_each_samples_image_span():
    text, image = [3, 1, 4], [5, 9, 2]
    lo, hi = W.cross_bounds(text, image)
    assert lo.dtype == np.int32 and hi.dtype == np.int32
    assert lo.tolist() == [0, 0, 0, 5, 14, 14, 14, 14]
    assert hi.tolist() == [5, 5, 5, 14, 16, 16, 16, 16]
    assert np.all(np.diff(lo) >= 0) and np.all(np.diff(hi) >= 0) and np.all(hi > lo)


def test_cross_tensors_shapes_and_seeding():
    q, k, v = W.cross_tensors(2, 6, 10, 4, 2, 8, seed=3)
    assert tuple(q.shape) == (2, 6, 4, 8) and tuple(k.shape) == (2, 10, 2, 8)
    assert tuple(v.shape) == tuple(k.shape)
    q2, _, _ = W.cross_tensors(2, 6, 10, 4, 2, 8, seed=3)
    assert bool((q == q2).all())
