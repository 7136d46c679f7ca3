"""The row selection of the full-size parity tests (``gpu_util.covering_rows``).

At the benchmark sizes the oracle checks a chosen subset of tokens. The subset
must hold, for the routing the GPU ran, a row of every unit of work: every
128-row piece of every GEMM-tiled expert (ragged tails included), every 16-row
streamed chunk, every row piece of the shared expert. This checks the selection
against units re-derived here with plain loops, on routings with skewed and
empty experts, for each path's unit sizes.
"""
import numpy as np
import pytest

from gpu_util import covering_rows, resolved_path


def _units(ids, E, path):
    """Token sets of every unit, from a plain walk over the pairs in order."""
    T, k = ids.shape
    slots = {e: [] for e in range(E)}
    for t in range(T):
        for j in range(k):
            slots[int(ids[t, j])].append(t)  # pairs ascending: the dispatch order
    units = []
    for e in range(E):
        n = len(slots[e])
        size = 16 if path == "decode" or (path == "hybrid" and n <= 32) else 128
        for i in range(0, n, size):
            units.append(set(slots[e][i:i + size]))
    shared = 16 if path == "decode" else 128
    for i in range(0, T, shared):
        units.append(set(range(i, min(i + shared, T))))
    return units


def _routing(T, E, k, skew, seed):
    rng = np.random.default_rng(seed)
    p = np.arange(1, E + 1, dtype=np.float64) ** -skew
    p /= p.sum()
    ids = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        ids[t] = rng.choice(E, size=k, replace=False, p=p)
    return ids


CASES = [
    (16, 16, 1, 0.0, "decode"),
    (900, 16, 1, 0.0, "prefill_wide"),
    (900, 16, 1, 0.0, "prefill"),
    (1000, 64, 1, 1.1, "hybrid"),   # a few GEMM experts, many streamed, some empty
    (700, 40, 4, 0.5, "hybrid"),
    (1500, 24, 3, 0.3, "prefill_wide"),
]


@pytest.mark.parametrize("T,E,k,skew,path", CASES)
def test_every_unit_has_a_checked_row(T, E, k, skew, path):
    ids = _routing(T, E, k, skew, seed=T + E)
    cov = covering_rows(ids, E, path)
    rows = set(cov.rows.tolist())
    units = _units(ids, E, path)
    assert cov.units == len(units)
    missed = [i for i, u in enumerate(units) if not (u & rows)]
    assert not missed, f"{len(missed)} units without a checked row"
    touched = set(ids.ravel().tolist())
    assert touched <= set(ids[cov.rows].ravel().tolist())
    assert len(rows) <= len(units)


def test_extra_rows_kept_and_counted():
    ids = _routing(600, 12, 2, 0.2, seed=3)
    extra = np.array([0, 599, 123])
    cov = covering_rows(ids, 12, "prefill_wide", extra=extra)
    assert set(extra.tolist()) <= set(cov.rows.tolist())


def test_resolved_path_follows_the_documented_rule():
    assert resolved_path(16, 16, 1) == "decode"
    assert resolved_path(64, 4, 1) == "decode"
    assert resolved_path(65, 4, 1) == "hybrid"
    assert resolved_path(4096, 128, 1) == "hybrid"      # 32 pairs per expert on average
    assert resolved_path(8192, 16, 1) == "prefill_wide"
    assert resolved_path(16384, 128, 8) == "prefill_wide"
    assert resolved_path(8192, 16, 1, "prefill") == "prefill"
