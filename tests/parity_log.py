"""Totals of whole-output parity checks, printed in the test session's summary (tests/conftest.py)."""
from collections import OrderedDict

_totals = OrderedDict()   # label -> [elements, bit-exact elements, outputs]


def record(label: str, elements: int, exact: int, outputs: int):
    t = _totals.setdefault(label, [0, 0, 0])
    t[0] += elements
    t[1] += exact
    t[2] += outputs


def lines():
    return [f"{label}: {exact:,} of {n:,} elements bit-exact against the oracle ({outs} outputs)"
            for label, (n, exact, outs) in _totals.items()]
