"""Host logic of the per-work-group timeline summary (no GPU): a hand-made timestamp
array whose start, duration and end figures are known."""
import numpy as np

from bit_quantized_routed_amd import timeline as tl


def test_summary_figures():
    buf = np.zeros((2, tl.MAX_WG, tl.SLOTS), dtype=np.uint64)
    base = 10_000
    # gate/up (kind 1): two routed work-groups (prologues 5 and 7 us), one shared-expert
    # work-group, one with no work; XCC ids 0, 1, 1, 2
    for b, (t0, t1, t2, role, xcc) in enumerate([(0, 500, 2000, 0, 0), (100, 800, 2600, 0, 1),
                                                  (50, 0, 2400, 1, 1), (20, 0, 120, 2, 2)]):
        buf[1, b, 0], buf[1, b, 1], buf[1, b, 2] = base + t0, base + t1, base + t2
        buf[1, b, 3], buf[1, b, 4] = xcc, role
    # down (kind 0): one routed work-group starting 1 us after the gate/up launch's end
    buf[0, 0, 0], buf[0, 0, 1], buf[0, 0, 2] = base + 2700, base + 2900, base + 4700
    text = "\n".join(tl.summarise(buf))
    assert "gate/up launch: 4 work-groups, last end 26.00 us" in text
    assert "routed   n=    2  start p50/p90/max 0.50/0.90/1.00  duration 22.50/24.50/25.00  end 23.00/25.40/26.00" \
           "  prologue 6.00/6.80/7.00" in text
    assert "shared   n=    1" in text and "no work  n=    1" in text
    assert "last end per XCC: 20.0 26.0 1.2 - - - - -" in text
    assert "down launch: 1 work-groups, last end 20.00 us" in text
    assert "gate/up last end -> down first start 1.00 us; gate/up first start -> down last end 47.00 us" in text
