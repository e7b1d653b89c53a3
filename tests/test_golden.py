"""The oracle reproduces its stored regression fixture bit for bit."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _load():
    o, s = {}, {}
    with open(os.path.join(HERE, "golden", "tiny_round0.txt")) as f:
        for line in f:
            if line.startswith("#"):
                continue
            tag, idx, *words = line.split()
            arr = np.array([int(w, 16) for w in words], np.uint32).view(np.float32)
            (o if tag == "o" else s)[int(idx)] = arr
    return o, s


def test_tiny_round0_fixture():
    import sys
    sys.path.insert(0, os.path.join(HERE, "golden"))
    import make_golden
    o_ref, s_ref = _load()
    o, srows = make_golden.compute()
    assert len(o_ref) == 8 and len(s_ref) == 3
    for t, row in o_ref.items():
        assert np.array_equal(o[t].view(np.uint32), row.view(np.uint32))
    for n, i in enumerate(make_golden.STATE_ROWS):
        assert np.array_equal(srows[n].view(np.uint32), s_ref[i].view(np.uint32))
