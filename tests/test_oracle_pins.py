"""The fp64 oracle against its pins (CPU only)."""

import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


@pytest.mark.parametrize("Sk, ns, expect", [
    # reading R8: L = ceil(Sk / ns); chunk c = [cL, min((c+1)L, Sk)); chunks past the end are empty
    (10, 4, [(0, 3), (3, 6), (6, 9), (9, 10)]),
    (10, 6, [(0, 2), (2, 4), (4, 6), (6, 8), (8, 10), (10, 10)]),
    (7, 7, [(i, i + 1) for i in range(7)]),
    (8, 3, [(0, 3), (3, 6), (6, 8)]),
    (0, 1, [(0, 0)]),
    (5, 1, [(0, 5)]),
])
def test_split_bounds_hand_cases(Sk, ns, expect):
    assert oracle.split_bounds(Sk, ns) == expect


@pytest.mark.parametrize("Sk, ns", [(1, 1), (100, 7), (4097, 64), (70000, 70000), (1000, 300), (33, 32)])
def test_split_bounds_partition(Sk, ns):
    """The chunks are ns consecutive, disjoint ranges that cover [0, Sk) in
    order, every non-empty one but the last holding exactly ceil(Sk/ns) keys."""
    b = oracle.split_bounds(Sk, ns)
    L = -(-Sk // ns)
    assert len(b) == ns
    assert b[0][0] == 0 and b[-1][1] == Sk
    for (lo0, hi0), (lo1, hi1) in zip(b, b[1:]):
        assert hi0 == lo1 and lo0 <= hi0
    sizes = [hi - lo for lo, hi in b]
    nonempty = [s for s in sizes if s > 0]
    assert sum(sizes) == Sk
    assert all(s == L for s in nonempty[:-1]) and 0 < nonempty[-1] <= L
