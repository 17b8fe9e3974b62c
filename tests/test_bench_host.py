"""Host logic of the benchmark script: the per-(layer, loop range) (c, G) plan."""
import pytest

import bench
from oracle import loopvq_oracle as O
from synth import workloads as W


def test_plan_parse_and_bits():
    wl = W.DEEP_8K
    plan = bench.parse_plan("8:4x4,24:8x4/32:8x2/32:4x8/32:8x4", wl)
    assert plan == [[(8, 4, 4), (24, 8, 4)], [(32, 8, 2)], [(32, 4, 8)], [(32, 8, 4)]]
    want = (8 * O.bits_per_elem(8, 4, 4) + 24 * O.bits_per_elem(8, 8, 4) + 32 * O.bits_per_elem(8, 8, 2)
            + 32 * O.bits_per_elem(8, 4, 8) + 32 * O.bits_per_elem(8, 8, 4)) / (4 * 32)
    assert bench.plan_bits_per_elem(plan, 8) == pytest.approx(want, rel=1e-15)
    # one layer entry applies to every layer
    assert bench.parse_plan("32:4x4", wl) == [[(32, 4, 4)]] * wl.layers
    assert bench.plan_bits_per_elem(bench.parse_plan("32:4x4", wl), 8) == 0.5


@pytest.mark.parametrize("bad", ["16:4x4", "30:4x4,2:8x2/32:4x4/32:4x4/32:4x4", "32:4x4/32:4x4", "12:4x8,20:4x4"])
def test_plan_rejects(bad):
    with pytest.raises(ValueError):
        bench.parse_plan(bad, W.DEEP_8K)
