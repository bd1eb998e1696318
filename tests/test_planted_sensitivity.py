"""The planted window-edge inputs (tests/planted.py) can see a routing
mistake at the edge: moving the window by one in the oracle (so that the pair
at distance w0 - 1 turns remote, or the pair at distance w0 turns local)
changes the planted rows' outputs by far more than the bf16 tolerance.  The
GPU tests that use these inputs would therefore fail on such a mistake."""
import numpy as np
import pytest

import oracle
from zero_shot_rope_bifocal_amd import workloads as W

import planted


def _prefill(inp, wp, w0, theta, rows):
    L = inp["lens"][0]
    q = W.as_f64(inp["q"][rows], inp["dtype"])
    o, _ = oracle.bifocal_sequence(q, W.as_f64(inp["k"], inp["dtype"]), W.as_f64(inp["v"], inp["dtype"]),
                                   np.asarray(rows), L, wp, w0, theta)
    return o


@pytest.mark.parametrize("dt,d,w0", [("bf16", 128, 100), ("bf16", 64, 64), ("f32", 128, 37), ("bf16", 128, 1)])
def test_edge_prefill_sees_off_by_one(dt, d, w0):
    L, wp, theta = 1100, 256, 1e4
    inp, rows = planted.edge_prefill(L, 4, 2, d, dt, wp, w0, theta, seed=61)
    assert len(rows) >= 10
    good = _prefill(inp, wp, w0, theta, rows)
    # at w0 = 1 the local edge key is the diagonal, the same in both branches
    for shifted in ((w0 + 1,) if w0 == 1 else (w0 - 1, w0 + 1)):
        moved = _prefill(inp, wp, shifted, theta, rows)
        per_row = np.max(np.abs(moved - good), axis=(1, 2))
        assert np.min(per_row) > 0.2, (shifted, per_row)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_edge_decode_sees_off_by_one(dt):
    seq_L, wp, w0, theta = [1500, 900, 1234, 777], 128, 100, 1e4
    inp, planted_b = planted.edge_decode(seq_L, 1500, 8, 2, 128, dt, wp, w0, theta, seed=62)
    assert planted_b == [0, 1, 2, 3]
    args = (W.as_f64(inp["q"], dt), W.as_f64(inp["k"], dt), W.as_f64(inp["v"], dt), inp["seq_L"], wp)
    good, _ = oracle.bifocal_decode(*args, w0, theta)
    for shifted in (w0 - 1, w0 + 1):
        moved, _ = oracle.bifocal_decode(*args, shifted, theta)
        per_seq = np.max(np.abs(moved - good), axis=(1, 2))
        assert np.min(per_seq) > 0.2, (shifted, per_seq)
