"""The split plan's column rule, as the GPU plan test states it, checked on the CPU
against brute force: cutting the axis of tiles (each sequence preceded by 3
start-up units) into columns of ceil(U / C) units gives every sequence one piece
per column its tiles meet, every column at most one piece per sequence, and at
most C + B - 1 pieces in all (no GPU needed)."""

import numpy as np
import pytest

START_UNITS = 3


def closed_form(n_keys, C):
    tiles = -(-n_keys // 32)
    units_end = np.cumsum(tiles + START_UNITS)
    first_tile = units_end - tiles
    U = int(units_end[-1])
    width = -(-U // C)
    return (units_end - 1) // width - first_tile // width + 1, first_tile, units_end, width


def brute_force(first_tile, units_end, width, U):
    """Pieces per sequence by walking every column and every tile unit."""
    pieces = np.zeros(len(first_tile), dtype=np.int64)
    n_cols = -(-U // width)
    for j in range(n_cols):
        lo, hi = j * width, min((j + 1) * width, U)
        for b, (f, e) in enumerate(zip(first_tile, units_end)):
            if max(lo, f) < min(hi, e):
                pieces[b] += 1
    return pieces


@pytest.mark.parametrize("seed", range(12))
def test_column_rule_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    n_keys = rng.integers(1, 20000, size=B) if seed % 3 else rng.integers(1, 200, size=B)
    C = int(rng.integers(1, 300))
    pieces, first_tile, units_end, width = closed_form(n_keys, C)
    U = int(units_end[-1])
    assert np.array_equal(pieces, brute_force(first_tile, units_end, width, U))
    assert pieces.min() >= 1
    assert pieces.sum() <= C + B - 1
    # every column's work: its tile units plus the start-up units it holds
    n_cols = -(-U // width)
    assert n_cols <= C


def test_one_sequence_gets_equal_columns():
    """A single 185,016-key sequence over 32 columns: columns of 181 units, the
    first holding the 3 start-up units and 178 tiles, the critical path 181 tiles."""
    pieces, first_tile, units_end, width = closed_form(np.array([185016]), 32)
    assert width == 181 and pieces[0] == 32
