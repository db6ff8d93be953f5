"""Host logic of the full-grid parity check (no GPU): which output rows the
oracle compares so that every tile of a launch grid is covered."""
import numpy as np

from tests import parity


def test_band_rows_cover_every_tile_band():
    r = parity.band_rows(30000, 256)
    assert len(r) == 2 * 118
    assert {0, 255, 256, 511, 29952, 29999} <= set(r.tolist())
    # every band [256b, 256b + 256) holds its first and last row
    for b in range(118):
        lo, hi = 256 * b, min(256 * b + 256, 30000) - 1
        assert lo in r and hi in r


def test_band_rows_with_extra_and_small_m():
    assert parity.band_rows(5, 16).tolist() == [0, 4]
    assert parity.band_rows(4096, 192, [7, 7, 4000]).tolist()[:4] == [0, 7, 191, 192]
    assert len(parity.band_rows(4096, 192)) == 44


def test_path_of():
    assert parity.path_of({"kind": "i8", "fmt": None}) == 0
    assert parity.path_of({"kind": "f8", "fmt": None}) == 1
    assert parity.path_of({"kind": "mx", "fmt": "e4m3"}) == 2
    assert parity.path_of({"kind": "mx", "fmt": "e2m1"}) == 3
    assert parity.path_of({"kind": "f8b", "fmt": None}) == 4
    assert parity.path_of({"kind": "mx", "fmt": "e4m3/e2m1"}) == 5
    assert parity.path_of({"kind": "mx", "fmt": "e2m1/e4m3"}) == 8
