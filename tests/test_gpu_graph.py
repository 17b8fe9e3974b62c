"""A decode step (every decode launch of the stack plus the eviction) captured in a HIP graph
replays to the eager result, bit for bit (needs an MI355X).  The decode is deterministic: its
value histogram adds integers, so the order of the atomics does not matter."""
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from synth import workloads as W  # noqa: E402


def test_decode_step_graph_replays_match_eager():
    import bench
    print("graph capture of a decode step", flush=True)
    sys.stdout.flush()
    wl = W.LAYER_4K.with_(name="graph_small", batch=4, context=1024)
    b = bench.Bench(wl)
    b.reps, b.replicas, b.rep_i = b.reps[:1], 1, 0   # one cache copy: eager and graph read the same bytes
    # the first step's eviction rewrites one VQ position; from the second step on every step
    # reads the same cache and its eviction rewrites the same bytes
    b.step()
    b.step()
    torch.cuda.synchronize()
    ref = b.out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.step()
    for _ in range(3):
        b.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(b.out, ref), "graph replay differs from the eager step"
        b.out.fill_(float("nan"))
        b.step()                      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(b.out, ref), "eager step after a replay differs"
    del g, b
    torch.cuda.empty_cache()
