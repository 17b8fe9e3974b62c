"""GPU parity of the bf16 window rows of decode attention (needs an MI355X).

The window rows are the exact bf16 prefix and recent tokens of a sequence.  These cases make
the window large: a recent window that covers the whole context (the uncompressed-cache
comparison, no vector-quantized rows), a wide window beside vector-quantized rows, and the
32K stack with the recent window equal to the whole context at its full shape (sampled queries,
launched as the benchmark's comparison mode launches it).
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("lvq_harness")

from oracle import loopvq_oracle as O  # noqa: E402
from synth import workloads as W  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# recent window >= context: every row is a bf16 window row
ALL_BF16 = W.LAYER_4K.with_(name="layer_bf16_small", batch=3, q_heads=4, kv_heads=2, context=1500, recent=1492)
# a 600-token recent window beside vector-quantized rows
WIDE = W.LAYER_4K.with_(name="layer_wide_recent", batch=3, q_heads=4, kv_heads=2, context=1500, recent=600)


@pytest.mark.parametrize("splits", [0, 1, 4, 7])
def test_whole_context_window(splits):
    _say(f"whole-context bf16 window, splits={splits}")
    wl = ALL_BF16
    case = H.Case(wl, 0, 1, [1500, 1, 999])
    assert int(case.n_vq.sum()) == 0
    empty = np.zeros((0, wl.groups), np.int64)
    o_ref, lse_ref = case.oracle_decode(lambda k, b, h: empty)
    case.gpu_setup()
    o, lse = case.gpu_decode(num_splits=splits)
    _say(f"  rel/max={H.check_attention(o, o_ref, lse, lse_ref)}")


@pytest.mark.parametrize("scale", [64.0, 4096.0])
def test_whole_context_window_peaked(scale):
    """Queries scaled by 2^6 and 2^12 (exact in bf16): scores span hundreds of log2 units, so the
    softmax reference of the window steps moves many times (each time a score passes it by 8)."""
    from synth import gen
    _say(f"whole-context bf16 window, queries x{scale}")
    wl = ALL_BF16
    case = H.Case(wl, 0, 3, [1500, 700, 999])
    case.q = gen.to_bf16_bits(gen.bf16_to_f64(case.q) * scale)
    empty = np.zeros((0, wl.groups), np.int64)
    o_ref, lse_ref = case.oracle_decode(lambda k, b, h: empty)
    case.gpu_setup()
    o, lse = case.gpu_decode(num_splits=0)
    _say(f"  rel/max={H.check_attention(o, o_ref, lse, lse_ref)}")


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_wide_window_beside_vq_rows(splits):
    _say(f"600-row recent window + vector-quantized rows, splits={splits}")
    wl = WIDE
    case = H.Case(wl, 0, 2, [1500, 650, 1])
    exp = case.oracle_encode()
    case.gpu_setup()
    pool_ref = case.oracle_pool(lambda k, b, h: exp[k, b, h][0])
    case.d_pool.copy_(torch.from_numpy(pool_ref.reshape(-1)).to(H.DEV))
    o_ref, lse_ref = case.oracle_decode(lambda k, b, h: exp[k, b, h][0])
    o, lse = case.gpu_decode(num_splits=splits)
    _say(f"  rel/max={H.check_attention(o, o_ref, lse, lse_ref)}")


def test_stack32k_uncompressed_cache_sampled():
    """The 32K stack with the recent window = context - prefix (the comparison launch of the
    benchmark: same kernel, split plan and shapes), checked on sampled queries."""
    import bench
    _say("32K stack, bf16 cache, full shape")
    bb = bench.Bf16Bench(W.STACK_32K)
    wl = bb.wl
    assert wl.n_vq == 0
    l, t = 3, 2
    bb.out.fill_(float("nan"))
    bb.decode(l, t)
    torch.cuda.synchronize()
    out = bb.out.cpu().numpy().astype(np.float64)
    assert np.isfinite(out).all()
    zero_cb = np.zeros((wl.groups, wl.codewords, wl.chans * wl.loop_group))
    empty = np.zeros((0, wl.groups), np.int64)
    samples = [(0, 0), (17, 5), (40, 11), (63, 15)]
    o_ref = np.zeros((len(samples), wl.head_dim))
    for i, (b, hq) in enumerate(samples):
        h = hq // (wl.q_heads // wl.kv_heads)
        win = [H.f64(a.cpu().numpy().view(np.uint16)) for a in (bb.pre[0, b, h], bb.pre[1, b, h],
                                                                 bb.rec[0, b, h], bb.rec[1, b, h])]
        q = H.f64(bb.q[l, t, b, hq].cpu().numpy().view(np.uint16))
        o_ref[i], _ = O.decode_query(q, win[0], win[1], empty, empty, zero_cb, zero_cb, win[2], win[3], t % wl.loop_group,
                                     wl.chans, 1.0 / np.sqrt(wl.head_dim))
    got = np.stack([out[b, hq] for b, hq in samples])
    _say(f"  rel/max={H.check_attention(got, o_ref)}")
    del bb
    torch.cuda.empty_cache()
