"""Host-side check of the per-workgroup timeline summary (no GPU): stamps are 100 MHz counter
values, a zero stamp means the workgroup never reached that point and must be left out of the
statistics, and the workgroup count of each point says how many reached it."""
import numpy as np

from sparse_attention_15_amd import timeline as T


def _row(lines, name):
    return next(l for l in lines if l.startswith(f"| {name} |")).strip("|").split("|")


def test_unreached_points_are_left_out():
    raw = np.array([[1000, 1200, 0],
                    [1100, 0, 0],
                    [1300, 1500, 1700]], dtype=np.uint64)
    lines = T._table("k", ["a", "b", "c"], raw, 1000)
    assert lines[0].startswith("**k** (3 workgroups)")
    a, b, c = _row(lines, "a"), _row(lines, "b"), _row(lines, "c")
    assert int(a[1]) == 3 and float(a[2]) == 0.0 and float(a[6]) == 3.0      # 0, 1, 3 us
    assert int(b[1]) == 2 and float(b[2]) == 2.0 and float(b[6]) == 5.0      # 2 and 5 us
    assert int(c[1]) == 1 and float(c[4]) == 7.0                              # only the third
    assert all(float(v) >= 0 for r in (a, b, c) for v in r[2:])


def test_a_point_nobody_reached_is_marked():
    raw = np.array([[500, 0], [600, 0]], dtype=np.uint64)
    lines = T._table("k", ["start", "end"], raw, 500)
    assert _row(lines, "end")[1:] == [" 0 ", " - ", " - ", " - ", " - ", " - "]
