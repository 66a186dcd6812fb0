"""Host-side checks of the evidence harness's L2 panel model (no GPU)."""

import pytest

from fp4_post_quantization_amd.evidence import panel_fetch


def test_one_partial_tile_fetches_its_rows_once():
    # one 256 x 256 tile holding 100 x 60 outputs: 100 rows of A and 60 of B
    assert panel_fetch(100, 60, 1000, 256, 256) == (100 + 60) * 1000


def test_rounds_split_over_xcds_by_hand():
    # 8 x 4 tiles of 256 on 8 XCDs: 4 tiles each, numbers 4x .. 4x + 3 of one group of 8 tile
    # rows walked column by column, i.e. 4 tile rows of one tile column: 4 A + 1 B panels per XCD
    assert panel_fetch(8 * 256, 4 * 256, 10, 256, 256) == 8 * (4 + 1) * 256 * 10


def test_resident_rounds_do_not_share_panels():
    # one XCD, 2 resident tiles, a 2 x 2 grid: the first pair = tile rows 0, 1 of column 0 (2 A + 1 B),
    # the second pair = the same rows of column 1 (2 A again + 1 B)
    assert panel_fetch(512, 512, 1, 256, 256, resident=2, xcds=1) == (2 + 1 + 2 + 1) * 256


@pytest.mark.parametrize("m,n", [(8192, 4096), (8192, 14336), (1000, 3000)])
def test_every_tile_is_fetched_at_least_once(m, n):
    # never less than reading A and B once, never more than every tile reading its own panels
    tiles = (-(-m // 256)) * (-(-n // 256))
    got = panel_fetch(m, n, 1, 256, 256)
    assert m + n <= got <= tiles * 512
