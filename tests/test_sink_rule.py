"""The sink-row rule the GPU parity tests apply (tests/parity_util.py), pinned on the
CPU: racing tombstoned stores leave each chunk of the store's vector width whole
from one tombstoned source row; every other byte must equal the oracle's."""
import numpy as np
import pytest

import oracle
import ukv_workloads as W
from parity_util import assert_bytes_equal_with_sinks, copy_unit, ospecs, round8


def _pool():
    w = W.tiny_mha(seed=0)
    specs = ospecs(w.shapes)
    n = round8(int(oracle.plan(specs, w.page_size).required_bytes))
    return oracle.OraclePool(specs, w.page_size, W.fill_pattern_host(3, 0, n).copy())


def _setup(unit):
    orc = _pool()
    rb = orc.row_bytes(0)
    g = np.random.default_rng(11)
    cands = [g.integers(0, 256, rb, dtype=np.uint8) for _ in range(3)]
    off = orc.view_base(0, 1, 0)
    got = orc.raw.copy()
    # chunk i of the sink row from candidate i % 3
    for i in range(rb // unit):
        got[off + i * unit: off + (i + 1) * unit] = cands[i % 3][i * unit: (i + 1) * unit]
    return orc, rb, cands, off, got


def test_copy_unit_is_the_widest_common_power_of_two():
    assert copy_unit(2048, 0, 1 << 20) == 16
    assert copy_unit(2048, 8) == 8
    assert copy_unit(1152, 16, 2) == 2
    assert copy_unit(34) == 2
    assert copy_unit(7) == 1


@pytest.mark.parametrize("unit", [16, 4])
def test_whole_chunks_from_the_candidates_pass(unit):
    orc, rb, cands, off, got = _setup(unit)
    assert_bytes_equal_with_sinks(got, orc, {(0, 1, 0): (unit, cands)})


def test_a_torn_chunk_fails_at_its_width_only():
    """Half of one 16-byte chunk from another candidate: whole 4- and 8-byte pieces
    still each come from one row, a 16-byte chunk does not."""
    orc, rb, cands, off, got = _setup(16)
    got[off + 8: off + 16] = cands[1][8:16]  # chunk 0 is candidate 0's
    with pytest.raises(AssertionError, match="16-byte chunks"):
        assert_bytes_equal_with_sinks(got, orc, {(0, 1, 0): (16, cands)})
    assert_bytes_equal_with_sinks(got, orc, {(0, 1, 0): (8, cands)})
    assert_bytes_equal_with_sinks(got, orc, {(0, 1, 0): (4, cands)})


def test_a_chunk_from_no_candidate_fails():
    orc, rb, cands, off, got = _setup(4)
    got[off + 4 * 7] ^= 1
    with pytest.raises(AssertionError, match="from no tombstoned row"):
        assert_bytes_equal_with_sinks(got, orc, {(0, 1, 0): (4, cands)})


def test_bytes_off_the_sink_rows_must_match():
    orc, rb, cands, off, got = _setup(16)
    got[off + rb] ^= 1  # row 1 of the view: not a sink row
    with pytest.raises(AssertionError, match="bytes differ"):
        assert_bytes_equal_with_sinks(got, orc, {(0, 1, 0): (16, cands)})
    got = orc.raw.copy()
    got[off] ^= 1  # a sink row with no recorded store
    with pytest.raises(AssertionError, match="bytes differ"):
        assert_bytes_equal_with_sinks(got, orc, {})
