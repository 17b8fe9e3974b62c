"""loopvq_decode_attn_noalloc against loopvq_decode_attn on the GPU (needs an MI355X).

The allocation-free entry point runs the same kernels with the split partials in the
library's static per-GPU array instead of a caller workspace, so its outputs must equal the
workspace entry point's bit for bit.  Two calls in a row, the second on a smaller input (the
array keeps the first call's partials), then the first shape again; split plans with S > 1
(explicit and automatic), so that the array is really used, and S = 1.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("lvq_harness")

import sub_bit_loop_loopvq_amd as lvq  # noqa: E402
from synth import workloads as W  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _setup(wl, lens):
    case = H.Case(wl, 0, 1, lens)
    exp = case.oracle_encode()
    case.gpu_setup()
    pool_ref = case.oracle_pool(lambda k, b, h: exp[k, b, h][0])
    case.d_pool.copy_(torch.from_numpy(pool_ref.reshape(-1)).to(H.DEV))
    torch.cuda.synchronize()
    return case


def _noalloc(case, num_splits):
    wl = case.wl
    out = torch.full((wl.batch, wl.q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device=H.DEV)
    lse = torch.full((wl.batch, wl.q_heads), float("nan"), dtype=torch.float32, device=H.DEV)
    lvq.loopvq_decode_attn_noalloc(case.cfg, layer=case.l, loop=case.t, batch=wl.batch, q=case.d_q,
                                   seq_lens=case.d_lens, max_seq_len=int(case.lens.max()), out=out,
                                   block_table=case.d_bt, pool=case.pool_base(),
                                   max_pages_per_seq=case.paging.max_pages, num_pages=case.paging.num_pages,
                                   cb_k_prep=case.d_prep[0], cb_v_prep=case.d_prep[1], k_prefix=case.d_win[0],
                                   v_prefix=case.d_win[1], k_recent=case.d_win[2], v_recent=case.d_win[3],
                                   rot=case.d_rot, lse=lse, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


BIG = W.LAYER_4K.with_(batch=6, q_heads=4, kv_heads=2, context=900)
SMALL = W.LAYER_4K.with_(batch=2, q_heads=2, kv_heads=2, context=400)


@pytest.mark.parametrize("splits_big,splits_small", [(7, 3), (0, 0), (1, 5)])
def test_noalloc_equals_workspace_entry_point(splits_big, splits_small):
    _say(f"noalloc splits {splits_big} then {splits_small}")
    big = _setup(BIG, [900, 1, 73, 300, 650, 899])
    small = _setup(SMALL, [400, 150])
    for case, S in ((big, splits_big), (small, splits_small), (big, splits_big)):
        o_ref, lse_ref = case.gpu_decode(num_splits=S)
        o, lse = _noalloc(case, S)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        assert np.array_equal(o, o_ref), f"output differs (batch {case.wl.batch}, splits {S})"
        assert np.array_equal(lse, lse_ref), f"lse differs (batch {case.wl.batch}, splits {S})"
    _say("  ok")



def test_noalloc_replays_under_graph_capture():
    """Captured in a HIP graph (the use the entry point is for), the allocation-free decode replays
    to its eager result bit for bit, three times, with eager calls of the same entry point (on
    another input) between the replays; 7 splits, so the static partials array is used."""
    _say("noalloc under graph capture")
    case = _setup(BIG, [900, 1, 73, 300, 650, 899])
    other = _setup(SMALL, [400, 150])
    o_ref, lse_ref = _noalloc(case, 7)
    wl = case.wl
    out = torch.full((wl.batch, wl.q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device=H.DEV)
    lse = torch.full((wl.batch, wl.q_heads), float("nan"), dtype=torch.float32, device=H.DEV)

    def call():
        lvq.loopvq_decode_attn_noalloc(case.cfg, layer=case.l, loop=case.t, batch=wl.batch, q=case.d_q,
                                       seq_lens=case.d_lens, max_seq_len=int(case.lens.max()), out=out,
                                       block_table=case.d_bt, pool=case.pool_base(),
                                       max_pages_per_seq=case.paging.max_pages, num_pages=case.paging.num_pages,
                                       cb_k_prep=case.d_prep[0], cb_v_prep=case.d_prep[1], k_prefix=case.d_win[0],
                                       v_prefix=case.d_win[1], k_recent=case.d_win[2], v_recent=case.d_win[3],
                                       rot=case.d_rot, lse=lse, num_splits=7)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                        # warm-up on the capture's stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().astype(np.float64), o_ref), "graph replay output differs"
        assert np.array_equal(lse.cpu().numpy().astype(np.float64), lse_ref), "graph replay lse differs"
        _noalloc(other, 3)            # an eager call between replays rewrites the static array
    del g
    torch.cuda.empty_cache()
    _say("  ok")
