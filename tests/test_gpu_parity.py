"""GPU parity of the LoopVQ HIP library against the CPU oracle (needs an MI355X).

Small cases run the whole chain (encode -> packed pages -> decode) and compare
every index, every page byte and every attention output; full-size cases run
the workload's decode launch (same shapes and split plan the benchmark times)
and compare sampled queries.
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


def _chain(case, decode_splits=(0,), scale=None):
    """Encode both kinds on the GPU, compare indices and pages, then decode and compare."""
    wl = case.wl
    exp = case.oracle_encode()
    case.gpu_setup()
    excused = 0
    for kind in (0, 1):
        gidx, rows, n_rerank = case.gpu_encode(kind)
        C_of = case.cbk if kind == 0 else case.cbv
        for h in range(wl.kv_heads):
            C = H.codebooks_f64(C_of, case.l, case.jc, h)
            for b in range(wl.batch):
                sel = [r for r, (bb, _) in enumerate(rows) if bb == b]
                if not sel:
                    continue
                idx, d1, d2, x = exp[kind, b, h]
                for g in range(wl.groups):
                    excused += H.check_indices(gidx[sel, h, g], idx[:, g], d1[:, g], d2[:, g], x[:, g], C[g])
    # page bytes: the GPU pool equals the oracle's packing of the oracle's indices
    pool_ref = case.oracle_pool(lambda k, b, h: exp[k, b, h][0])
    pool_gpu = case.d_pool.cpu().numpy().reshape(pool_ref.shape)
    if excused == 0:
        assert np.array_equal(pool_gpu, pool_ref), "packed pages differ"
    else:
        assert (pool_gpu != pool_ref).sum() <= excused
    # decode over the oracle's pages (uploaded), then over the GPU-encoded pages
    o_ref, lse_ref = case.oracle_decode(lambda k, b, h: exp[k, b, h][0], scale=scale)
    gpu_pool = case.d_pool.clone()
    case.d_pool.copy_(torch.from_numpy(pool_ref.reshape(-1)).to(H.DEV))
    res = []
    for S in decode_splits:
        o, lse = case.gpu_decode(num_splits=S, scale=scale or 0.0)
        res.append(H.check_attention(o, o_ref, lse, lse_ref))
    case.d_pool.copy_(gpu_pool)
    if excused == 0:
        o, lse = case.gpu_decode(num_splits=decode_splits[0], scale=scale or 0.0)
        H.check_attention(o, o_ref, lse, lse_ref)
    return excused, res


@pytest.mark.parametrize("loop", [0, 1, 2, 3])
def test_tiny_chain(loop):
    _say(f"tiny chain loop={loop}")
    case = H.Case(W.TINY, 0, loop, [W.TINY.context])
    excused, res = _chain(case, decode_splits=(0, 1, 3))
    _say(f"  excused={excused} rel/max={res}")


SMALL = W.LAYER_4K.with_(batch=6, q_heads=4, kv_heads=4, context=700)


@pytest.mark.parametrize("splits", [(0, 1), (3, 7)])
def test_small_ragged_chain(splits):
    lens = [700, 1, 72, 73, 137, 391]           # edge cases: one token, no VQ rows, one VQ row, ragged tails
    _say(f"small ragged chain splits={splits}")
    case = H.Case(SMALL, 0, 2, lens, seed=1)
    _chain(case, decode_splits=splits)


@pytest.mark.parametrize("c,lens", [(4, [2147, 2819, 4451, 4771]), (8, [2179, 3011, 4227, 4867])])
def test_tile_count_sweep_chain(c, lens):
    """One split, with lengths chosen so that the waves' tile counts run through 4..10: the tile loop
    keeps four tiles in flight, and these counts reach every remainder of its steady state, each
    sequence with a ragged last tile (c=4: 32-token tiles over 16 waves, 65/86/137/147 tiles;
    c=8: 64-token tiles over 8 waves, 33/46/65/75 tiles)."""
    if c == 4:
        wl = SMALL.with_(batch=4, q_heads=2, kv_heads=1, context=4800)
    else:
        wl = W.QUARTER_16K.with_(layers=1, batch=4, q_heads=2, kv_heads=1, context=4900)
    _say(f"tile-count sweep c={c} lens={lens}")
    _chain(H.Case(wl, 0, 1, lens, seed=11), decode_splits=(1, 0))


def test_gqa_chain():
    wl = SMALL.with_(batch=2, q_heads=8, kv_heads=2, context=600)
    _say("gqa chain")
    _chain(H.Case(wl, 0, 1, [600, 333], seed=2), decode_splits=(0, 2))


def test_quarter_bit_rotated_chain():
    wl = W.QUARTER_16K.with_(layers=2, batch=3, q_heads=2, kv_heads=2, context=900)
    _say("quarter-bit rotated chain")
    _chain(H.Case(wl, 1, 3, [900, 301, 73], seed=3), decode_splits=(0, 2))


def test_per_loop_group_codebooks_chain():
    wl = SMALL.with_(loops=8, batch=2, q_heads=2, kv_heads=2, context=500, codebook_per_loop_group=True)
    _say("per-loop-group codebooks chain")
    _chain(H.Case(wl, 0, 5, [500, 250], seed=4), decode_splits=(0,))


@pytest.mark.parametrize("c,G,loop", [(8, 2, 3), (4, 8, 13)])
def test_other_loop_group_sizes_chain(c, G, loop):
    """0.5 bit as 8 channels x 2 loop steps, and 0.25 bit as 4 channels x 8 loop steps."""
    wl = SMALL.with_(loops=16, loop_group=G, chans=c, batch=3, q_heads=4, kv_heads=2, context=600)
    _say(f"chain c={c} G={G} loop={loop}")
    _chain(H.Case(wl, 0, loop, [600, 73, 333], seed=9), decode_splits=(0, 3))


def test_d64_page128_chain():
    wl = W.TINY.with_(batch=3, q_heads=2, kv_heads=2, context=800, page_tokens=128)
    _say("d64 page128 chain")
    _chain(H.Case(wl, 0, 3, [800, 200, 450], seed=5), decode_splits=(0, 4))


def test_d128_page256_chain():
    """d=128 (32 channel groups) with 256-token pages: eight 32-token decode tiles per page."""
    wl = W.LAYER_4K.with_(batch=3, q_heads=2, kv_heads=2, context=1100, page_tokens=256)
    _say("d128 page256 chain")
    _chain(H.Case(wl, 0, 2, [1100, 300, 713], seed=8), decode_splits=(0, 3))


def test_large_scores_take_exact_maximum_path():
    """Scores far above the first tile's maximum (scale 50x) force the split's exact-maximum redo."""
    wl = SMALL.with_(batch=2, q_heads=2, kv_heads=2, context=1500)
    _say("large-score redo path")
    case = H.Case(wl, 0, 0, [1500, 900], seed=6)
    _chain(case, decode_splits=(0, 1), scale=50.0 / np.sqrt(wl.head_dim))


def test_no_vq_rows_is_plain_attention():
    wl = SMALL.with_(batch=4, q_heads=2, kv_heads=2, context=72)
    _say("no VQ rows")
    case = H.Case(wl, 0, 1, [72, 1, 9, 40], seed=7)
    case.gpu_setup()
    exp = {(k, b, h): np.zeros((0, wl.groups), np.int64) for k in (0, 1) for b in range(4) for h in range(2)}
    o_ref, lse_ref = case.oracle_decode(lambda k, b, h: exp[k, b, h])
    o, lse = case.gpu_decode()
    H.check_attention(o, o_ref, lse, lse_ref)


@pytest.mark.parametrize("splits", [0, 3])
def test_decode_is_bitwise_reproducible(splits):
    """Two runs on the same inputs give identical bits: the value histograms are integer sums and
    every other reduction has a fixed order."""
    case = H.Case(SMALL.with_(batch=2, q_heads=2, kv_heads=2), 0, 1, [700, 650], seed=8)
    exp = case.oracle_encode()
    case.gpu_setup()
    pool_ref = case.oracle_pool(lambda k, b, h: exp[k, b, h][0])
    case.d_pool.copy_(torch.from_numpy(pool_ref.reshape(-1)).to(H.DEV))
    o1, l1 = case.gpu_decode(num_splits=splits)
    o2, l2 = case.gpu_decode(num_splits=splits)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------------------------
# Full-size launches, sampled queries
# ---------------------------------------------------------------------------------
FULL = [
    (W.LAYER_4K, 0, 3),
    (W.STACK_32K, 17, 2),
    (W.QUARTER_16K, 9, 1),
    (W.DEEP_8K, 2, 29),
    (W.DEEP_8K.with_(codebook_per_loop_group=True), 3, 21),
    # the other built (c, G) shapes at the deep workload's full size: 8 channels x 2 loop steps
    # (0.5 bit, 16 groups) and 4 channels x 8 loop steps (0.25 bit, 32 groups)
    (W.DEEP_8K.with_(chans=8, loop_group=2), 1, 13),
    (W.DEEP_8K.with_(loop_group=8), 2, 30),
]


@pytest.mark.parametrize("wl,layer,loop", FULL, ids=[w.name + ("_cbj" if w.codebook_per_loop_group else "")
                                                     + (f"_c{w.chans}g{w.loop_group}" if (w.chans, w.loop_group)
                                                        != (4, 4) else "") for w, _, _ in FULL])
def test_full_size_decode_sampled(wl, layer, loop):
    rng = np.random.default_rng(wl.wid)
    samples = [(int(rng.integers(wl.batch)), int(rng.integers(wl.q_heads))) for _ in range(6)]
    samples += [(0, 0), (wl.batch - 1, wl.q_heads - 1)]
    _say(f"full-size {wl.name} layer={layer} loop={loop} samples={samples}")
    fc = H.FullCase(wl, layer, loop, samples)
    fc.upload()
    o, lse = fc.gpu_decode()
    for b, hq in samples:
        o_ref, lse_ref = fc.oracle(b, hq)
        H.check_attention(o[b, hq][None], o_ref[None], np.array([lse[b, hq]]), np.array([lse_ref]))
    _say("  ok")


def test_full_size_ragged_decode_sampled():
    wl = W.LAYER_4K
    lens = np.random.default_rng(11).integers(1, wl.context + 1, wl.batch)
    lens[:4] = [wl.context, 1, 72, 73]
    samples = [(b, hq) for b in range(8) for hq in (0, 15)]
    _say("full-size ragged layer decode")
    fc = H.FullCase(wl, 0, 1, samples, lens=lens)
    fc.upload()
    o, lse = fc.gpu_decode()
    for b, hq in samples:
        o_ref, lse_ref = fc.oracle(b, hq)
        H.check_attention(o[b, hq][None], o_ref[None], np.array([lse[b, hq]]), np.array([lse_ref]))


@pytest.mark.parametrize("wl,loop", [(W.LAYER_4K, 2), (W.DEEP_8K, 17)], ids=["layer4k", "deep8k"])
def test_full_launch_every_query(wl, loop):
    """Every query of a full-size decode launch (512 queries of 4K or 8K tokens) against the oracle,
    with the automatic split plan and with 3 splits."""
    samples = [(b, hq) for b in range(wl.batch) for hq in range(wl.q_heads)]
    _say(f"every query of {wl.name} loop={loop}")
    fc = H.FullCase(wl, 0, loop, samples, seed=16)
    fc.upload()
    o_ref = np.zeros((wl.batch, wl.q_heads, wl.head_dim))
    lse_ref = np.zeros((wl.batch, wl.q_heads))
    for b, hq in samples:
        o_ref[b, hq], lse_ref[b, hq] = fc.oracle(b, hq)
    for S in (0, 3):
        o, lse = fc.gpu_decode(num_splits=S)
        rel, mx = H.check_attention(o, o_ref, lse, lse_ref)
        _say(f"  splits {S}: rel-L2 {rel:.2e}, max-abs {mx:.2e}")
