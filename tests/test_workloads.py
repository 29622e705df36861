"""The workload shapes agree with what the pages print (tests/golden/onetrans_shapes.json)."""
import json
import os

from onetrans_inputs import ALL, ONETRANS_L, ONETRANS_S, pyramid_schedule

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "onetrans_shapes.json")))


def test_shapes_match_pages():
    for wl, key in ((ONETRANS_S, "onetrans_s"), (ONETRANS_L, "onetrans_l")):
        g = GOLDEN[key]
        assert wl.n_layers == g["n_layers"] and wl.d_model == g["d_model"]
        assert wl.q_sched[0] == g["q_first"] and wl.q_sched[-1] == g["q_last"]
        if "n_heads" in g:
            assert wl.n_heads == g["n_heads"]


def test_pyramid_interior_rounded_and_non_increasing():
    m = GOLDEN["pyramid_round_multiple"]
    for wl in ALL.values():
        q = wl.q_sched
        assert len(q) == wl.n_layers and q[0] <= wl.s_len
        assert all(a >= b >= 1 for a, b in zip(q, q[1:]))
        assert all(x % m == 0 for x in q[1:-1])
    assert pyramid_schedule(1500, 16, 8) == (1500, 1280, 1088, 864, 640, 448, 224, 16)
    assert pyramid_schedule(1190, 12, 6) == (1190, 960, 704, 480, 256, 12)
