"""The tile scheduler's program -> (batch, split, tile row, tile column) map,
evaluated on the host by the same code the kernels run (dg_schedule_map).

The map must be a bijection onto every (b, s, pid_m, pid_n) with ceil-div
tile counts ("Skill: Write a Triton GEMM Kernel", Correctness requirements
and Common failure modes).  Without the XCD remap it must be the grouped
order of "GEMM Kernel Optimization", L2 Cache Grouping: bands of G tile
rows, each walked column by column.  That order is checked against a list
built by plain enumeration (nested loops over bands, columns and rows, no
index arithmetic shared with the library), and its purpose, fewer distinct
A and B panels per run of consecutive programs than row-major order, is
checked directly."""
import itertools

import numpy as np
import pytest

import dense_gemm_10_amd as dg


def _grouped_order(num_pid_m, num_pid_n, group):
    """The grouped tile order as an explicit list of (tile row, tile column),
    built by enumeration: bands of `group` tile rows from the top, each band
    column by column from the left, each column top to bottom."""
    order = []
    for first in range(0, num_pid_m, group):
        rows = range(first, min(first + group, num_pid_m))
        for col in range(num_pid_n):
            for row in rows:
                order.append((row, col))
    return order


def _is_bijection(m, batch, splits, npm, npn):
    P = batch * splits * npm * npn
    if m.shape != (P, 4):
        return False
    ok = ((m[:, 0] >= 0) & (m[:, 0] < batch) & (m[:, 1] >= 0) & (m[:, 1] < splits) &
          (m[:, 2] >= 0) & (m[:, 2] < npm) & (m[:, 3] >= 0) & (m[:, 3] < npn)).all()
    key = ((m[:, 0].astype(np.int64) * splits + m[:, 1]) * npm + m[:, 2]) * npn + m[:, 3]
    return bool(ok) and np.unique(key).size == P


def test_bijection_exhaustive_small_grids():
    for npm, npn in itertools.product(range(1, 41), range(1, 41)):
        for g in (1, 2, 3, 5, 8, 9):
            for remap in (0, -1):
                m = dg.dg_schedule_map(npm, npn, 1, 1, 1, 1, g, remap)
                assert _is_bijection(m, 1, 1, npm, npn), (npm, npn, g, remap)


@pytest.mark.parametrize("batch,splits", [(1, 2), (3, 1), (2, 3), (32, 1), (1, 8), (32, 8)])
def test_bijection_with_batch_and_splits(batch, splits):
    for npm, npn in [(1, 1), (3, 7), (16, 17), (4, 4)]:
        for remap in (0, -1):
            m = dg.dg_schedule_map(npm, npn, batch, splits, 1, 1, 8, remap)
            assert _is_bijection(m, batch, splits, npm, npn)


@pytest.mark.parametrize("M,N,bm,bn", [(4096, 4096, 256, 256), (4096, 4096, 128, 128),
                                       (4095, 4097, 256, 256), (4095, 4097, 128, 128),
                                       (256, 256, 128, 128), (1000, 1, 64, 64)])
def test_real_grids_use_ceil_div(M, N, bm, bn):
    npm, npn = -(-M // bm), -(-N // bn)
    for remap in (0, -1):
        m = dg.dg_schedule_map(M, N, 1, 1, bm, bn, 8, remap)
        assert _is_bijection(m, 1, 1, npm, npn)
        # the last, partial tile row and column are present
        assert (m[:, 2] == npm - 1).any() and (m[:, 3] == npn - 1).any()


def test_without_remap_equals_enumerated_order():
    for npm, npn, g in itertools.product([1, 2, 7, 16, 33], [1, 3, 16, 17], [1, 3, 4, 8, 16]):
        m = dg.dg_schedule_map(npm, npn, 1, 1, 1, 1, g, -1)
        want = _grouped_order(npm, npn, g)
        assert [tuple(r) for r in m[:, 2:].tolist()] == want, (npm, npn, g)


def _panels_per_window(coords, window):
    """Mean number of distinct A row panels plus B column panels over the
    aligned runs of `window` consecutive programs (the contiguous runs the
    XCD remap hands to one L2)."""
    counts = []
    for s in range(0, len(coords), window):
        run = coords[s:s + window]
        counts.append(len({r for r, _ in run}) + len({c for _, c in run}))
    return sum(counts) / len(counts)


@pytest.mark.parametrize("npm,npn,g,window", [(16, 16, 8, 32), (32, 32, 8, 64), (17, 17, 8, 32),
                                              (16, 16, 4, 16)])
def test_grouping_reuses_panels(npm, npn, g, window):
    """A window of consecutive programs the size of one wave share of an
    L2 (e.g. 32 tiles of one XCD) loads fewer panels in grouped order than
    in row-major order, and every band of the grouped order touches only
    its own g tile rows."""
    grouped = [tuple(r) for r in dg.dg_schedule_map(npm, npn, 1, 1, 1, 1, g, -1)[:, 2:].tolist()]
    rowmajor = [tuple(r) for r in dg.dg_schedule_map(npm, npn, 1, 1, 1, 1, 1, -1)[:, 2:].tolist()]
    assert _panels_per_window(grouped, window) < _panels_per_window(rowmajor, window)
    for band in range(0, npm, g):
        lo, hi = band * npn, min(band + g, npm) * npn
        assert {r for r, _ in grouped[lo:hi]} == set(range(band, min(band + g, npm)))


def test_group_one_is_row_major():
    m = dg.dg_schedule_map(5, 7, 1, 1, 1, 1, 1, -1)
    pid = np.arange(35)
    assert np.array_equal(m[:, 2], pid // 7)
    assert np.array_equal(m[:, 3], pid % 7)


def test_grid_beyond_31_bits_is_refused():
    # the decode is 32-bit: 2^31 - 1 programs pass the size check (and fail
    # only for want of an output array), 2^31 and more are refused
    lib = dg._load()
    assert lib.dg_schedule_map(2**31 - 1, 1, 1, 1, 1, 1, 0, 0, None, 0) == dg.DG_ERROR_INVALID_VALUE
    assert lib.dg_schedule_map(2**31, 1, 1, 1, 1, 1, 0, 0, None, 0) == dg.DG_ERROR_NOT_SUPPORTED
    assert lib.dg_schedule_map(1 << 20, 1 << 20, 4, 1, 1, 1, 0, 0, None, 0) == dg.DG_ERROR_NOT_SUPPORTED
    assert lib.dg_schedule_map(1 << 40, 1 << 40, 1 << 40, 8, 1, 1, 0, 0, None, 0) == dg.DG_ERROR_NOT_SUPPORTED


def test_batch_and_split_decode_order():
    # without remap: tiles of one (b, s) are consecutive, then split, then batch
    m = dg.dg_schedule_map(2, 3, 4, 5, 1, 1, 8, -1)
    T = 6
    pid = np.arange(4 * 5 * T)
    assert np.array_equal(m[:, 1], (pid // T) % 5)
    assert np.array_equal(m[:, 0], pid // (T * 5))


@pytest.mark.parametrize("P_grid", [(16, 16), (32, 33), (3, 5), (17, 1)])
def test_xcd_remap_gives_each_xcd_a_contiguous_run(P_grid):
    """Programs p with p mod 8 == x (the ones the hardware places on XCD x)
    must cover one contiguous run of the un-remapped (grouped) order."""
    npm, npn = P_grid
    P = npm * npn
    plain = dg.dg_schedule_map(npm, npn, 1, 1, 1, 1, 8, -1)
    remapped = dg.dg_schedule_map(npm, npn, 1, 1, 1, 1, 8, 0)
    logical = {tuple(r): i for i, r in enumerate(plain.tolist())}
    ids = np.array([logical[tuple(r)] for r in remapped.tolist()])
    assert np.unique(ids).size == P
    starts = []
    for x in range(8):
        mine = np.sort(ids[x::8])
        if mine.size == 0:
            continue
        assert np.array_equal(mine, np.arange(mine[0], mine[0] + mine.size))
        starts.append(mine[0])
    # and XCD x's run precedes XCD x+1's
    assert starts == sorted(starts)


def test_group_of_8_tiles_on_one_xcd_form_a_block():
    # 4096^2 with 256^2 tiles: XCD 0 gets logical 0..31 = 8 tile rows x 4 columns
    m = dg.dg_schedule_map(4096, 4096, 1, 1, 256, 256, 8, 0)
    x0 = m[0::8]
    assert set(x0[:, 2].tolist()) == set(range(8))
    assert set(x0[:, 3].tolist()) == set(range(4))
