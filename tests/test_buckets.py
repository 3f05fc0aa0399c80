"""Pins of the relative-distance bucket rule (oracle.buckets)."""
import numpy as np
import pytest

from oracle.buckets import bucket, bucket_np


def octave_table(mbits, nb, max_delta):
    """Independent construction: one bucket per distance below 2^m, then each
    octave [2^e, 2^(e+1)) cut into 2^m equal-width ranges, ids handed out in
    increasing order, clamped to nb-1."""
    s = 1 << mbits
    tab = np.zeros(max_delta + 1, dtype=np.int64)
    nxt = 0
    for dlt in range(min(s, max_delta + 1)):
        tab[dlt] = nxt
        nxt += 1
    e = mbits
    while (1 << e) <= max_delta:
        width = 1 << (e - mbits)
        for k in range(s):
            lo = (1 << e) + k * width
            hi = min(lo + width, max_delta + 1)
            if lo <= max_delta:
                tab[lo:hi] = nxt
            nxt += 1
        e += 1
    return np.minimum(tab, nb - 1)


def test_hand_values_m3_nb32():
    # m = 3: distances 0..15 map to themselves; [16,32) in steps of 2;
    # [32,64) in steps of 4; 64 and beyond clamp at 31.
    exp = {0: 0, 1: 1, 7: 7, 8: 8, 15: 15, 16: 16, 17: 16, 18: 17, 31: 23,
           32: 24, 35: 24, 36: 25, 63: 31, 64: 31, 1000: 31}
    for dlt, b in exp.items():
        assert bucket(dlt, 3, 32) == b, dlt
    assert bucket(-5, 3, 32) == 0


def test_hand_values_m4_nb256():
    # m = 4: [256, 512) has width 16 -> bucket 16*(8-4+1) + (d>>4) - 16.
    assert bucket(255, 4, 256) == 16 * 4 + (255 >> 3) - 16
    assert bucket(256, 4, 256) == 80
    assert bucket(271, 4, 256) == 80
    assert bucket(272, 4, 256) == 81
    assert bucket(16447, 4, 256) == 16 * 11 + (16447 >> 10) - 16


@pytest.mark.parametrize("mbits,nb,maxd", [(3, 32, 200), (3, 128, 5000), (4, 256, 40000), (2, 64, 300000), (0, 8, 100)])
def test_matches_octave_table(mbits, nb, maxd):
    tab = octave_table(mbits, nb, maxd)
    got = bucket_np(np.arange(maxd + 1), mbits, nb)
    assert np.array_equal(got, tab)
    for dlt in list(range(0, min(maxd, 600))) + [maxd]:
        assert bucket(dlt, mbits, nb) == tab[dlt]


@pytest.mark.parametrize("mbits", [1, 2, 3, 4, 5])
def test_monotone_and_unit_steps(mbits):
    b = bucket_np(np.arange(1 << 20), mbits, 1 << 30)
    steps = np.diff(b)
    assert np.all((steps == 0) | (steps == 1))
    # every octave above 2^m uses exactly 2^m buckets
    e = mbits + 5
    seg = b[(1 << e):(1 << (e + 1))]
    assert len(np.unique(seg)) == 1 << mbits


def test_large_and_negative_deltas():
    d = np.array([-10, -1, 0, 2**31, 2**40], dtype=np.int64)
    got = bucket_np(d, 2, 64)
    assert list(got) == [0, 0, 0, 63, 63]
