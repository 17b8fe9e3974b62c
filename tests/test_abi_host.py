"""C-ABI checks that need no GPU: the library loads, exports every declared entry point,
and rejects bad calls on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import sub_bit_loop_loopvq_amd as lvq
from oracle import loopvq_oracle as O
from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_entry_points():
    text = open(os.path.join(ROOT, "include", "loopvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(loopvq_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_entry_points()
    assert set(names) == set(lvq.EXPORTS)
    L = lvq.lib()
    for n in names:
        assert hasattr(L, n), n
    # symbols are plain C (unmangled) exports
    raw = ctypes.CDLL(lvq.LIB_PATH)
    for n in names:
        ctypes.cast(getattr(raw, n), ctypes.c_void_p)


def test_struct_sizes_match_header_layout():
    # int32 x12 config; layout 9 int64 + 1 double
    assert ctypes.sizeof(lvq.loopvq_config) == 48
    assert ctypes.sizeof(lvq.loopvq_layout) == 80
    assert ctypes.sizeof(lvq.loopvq_encode_args) == 4 * 4 + 8 + 3 * 8 + 3 * 8 + 4 + 4 + 8 + 5 * 8
    assert ctypes.sizeof(lvq.loopvq_decode_args) == 6 * 4 + 8 + 10 * 8 + 8 + 8 + 8 + 8
    assert ctypes.sizeof(lvq.loopvq_evict_args) == 4 + 4 + 8 + 12 * 8
    assert ctypes.sizeof(lvq.loopvq_extend_args) == 6 * 4 + 8 + 14 * 8 + 8 + 8 + 8
    assert ctypes.sizeof(lvq.loopvq_lloyd_args) == 3 * 4 + 4 + 8 + 3 * 8 + 7 * 8 + 8 + 8


@pytest.mark.parametrize("wl", W.ALL, ids=[w.name for w in W.ALL])
def test_config_check_and_bits_per_elem(wl):
    cfg = lvq.make_config(wl)
    assert lvq.loopvq_config_check(cfg) == 0
    assert lvq.loopvq_bits_per_elem(cfg) == O.bits_per_elem(wl.index_bits, wl.chans, wl.loop_group)


def test_config_rules_agree_with_oracle():
    base = dict(T=4, G=4, Hq=16, Hkv=16, d=128, c=4, b=8)
    for bad in [{}, dict(T=6), dict(d=130), dict(Hq=3, Hkv=2), dict(b=17), dict(b=0), dict(d=24, c=4),
                dict(c=8), dict(c=2, d=64), dict(G=2), dict(Hq=32)]:
        kw = dict(base, **bad)
        try:
            O.check_config(**kw)
            oracle_ok = True
        except ValueError:
            oracle_ok = False
        cfg = lvq.make_config(num_layers=1, num_loops=kw["T"], loop_group=kw["G"], num_q_heads=kw["Hq"],
                              num_kv_heads=kw["Hkv"], head_dim=kw["d"], chans_per_group=kw["c"],
                              index_bits=kw["b"], prefix_tokens=8, recent_tokens=64, page_tokens=64,
                              codebook_per_loop_group=0)
        assert (lvq.loopvq_config_check(cfg) == 0) == oracle_ok, kw


def test_config_rejections_and_messages():
    good = lvq.make_config(W.STACK_32K)
    for field, val in [("num_loops", 6), ("page_tokens", 96), ("page_tokens", 32), ("prefix_tokens", -1),
                       ("codebook_per_loop_group", 2), ("num_layers", 0), ("index_bits", 0)]:
        cfg = lvq.make_config(W.STACK_32K)
        setattr(cfg, field, val)
        assert lvq.loopvq_config_check(cfg) == lvq.LOOPVQ_ERR_INVALID_ARG, field
        assert lvq.loopvq_last_error() != ""
        assert lvq.loopvq_bits_per_elem(cfg) == -1.0
    assert lvq.loopvq_config_check(good) == 0 and lvq.loopvq_last_error() == ""


@pytest.mark.parametrize("wl", W.ALL, ids=[w.name for w in W.ALL])
def test_layout_query_closed_forms(wl):
    cfg = lvq.make_config(wl)
    num_pages = 1000
    lay = lvq.loopvq_layout_query(cfg, wl.batch, num_pages)
    ref = O.page_layout(wl.page_tokens, wl.groups, wl.index_bits)
    assert lay.page_bytes == ref["page_bytes"] and lay.kind_bytes == ref["kind_bytes"]
    assert lay.tile_bytes == 2 * wl.index_bits
    assert lay.pool_head_stride_bytes == num_pages * lay.page_bytes
    assert lay.pool_bytes == wl.layers * wl.loop_groups * wl.kv_heads * num_pages * lay.page_bytes
    assert lay.codebook_elems == wl.layers * wl.cb_loop_groups * wl.kv_heads * wl.groups * wl.codewords * wl.sub_len
    assert lay.norms_elems == wl.layers * wl.cb_loop_groups * wl.kv_heads * wl.groups * wl.codewords
    assert lay.prefix_elems == wl.batch * wl.kv_heads * wl.prefix * wl.head_dim
    assert lay.recent_elems == wl.batch * wl.kv_heads * wl.recent * wl.head_dim
    assert lay.bits_per_elem == O.bits_per_elem(wl.index_bits, wl.chans, wl.loop_group)
    # index bytes of one sequence's VQ rows: n_vq * (d/c) * b/8 per kind, padded to whole pages
    n_pages = -(-wl.n_vq // wl.page_tokens)
    assert n_pages * lay.kind_bytes >= wl.n_vq * wl.groups * wl.index_bits // 8


def test_layout_query_rejects():
    cfg = lvq.make_config(W.TINY)
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_layout_query(cfg, 0, 10)
    assert e.value.status == lvq.LOOPVQ_ERR_INVALID_ARG
    with pytest.raises(lvq.LoopVQError):
        lvq.loopvq_layout_query(cfg, 1, 0)


FAKE = 1 << 20   # never dereferenced: every call below fails validation first


def _decode_kw(wl, **over):
    kw = dict(layer=0, loop=0, batch=wl.batch, q=FAKE, seq_lens=FAKE, max_seq_len=wl.context, out=FAKE,
              block_table=FAKE, pool=FAKE, max_pages_per_seq=600, num_pages=10, cb_k_prep=FAKE, cb_v_prep=FAKE,
              k_prefix=FAKE, v_prefix=FAKE, k_recent=FAKE, v_recent=FAKE, workspace=None, workspace_bytes=0,
              stream=0)
    kw.update(over)
    return kw


@pytest.mark.parametrize("over,status", [
    (dict(layer=24), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(loop=4), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(batch=0), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(q=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(pool=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(k_recent=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(num_splits=300), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(max_pages_per_seq=2 ** 25), lvq.LOOPVQ_ERR_INVALID_ARG),     # 2^25 pages x 64 tokens = 2^31
    (dict(pool=FAKE + 8), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(k_prefix=FAKE + 2), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(out=FAKE + 2), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(num_splits=4), lvq.LOOPVQ_ERR_WORKSPACE),
])
def test_decode_rejects_before_launch(over, status):
    wl = W.STACK_32K
    cfg = lvq.make_config(wl)
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_decode_attn(cfg, **_decode_kw(wl, **over))
    assert e.value.status == status


def test_decode_auto_split_workspace_is_checked():
    wl = W.TINY                                     # 1 query: the plan splits long contexts
    cfg = lvq.make_config(wl.with_(context=60000))
    need = lvq.loopvq_decode_attn_workspace(cfg, 1, 60000)
    assert need > 0
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_decode_attn(cfg, **_decode_kw(wl, batch=1, max_seq_len=60000, workspace_bytes=need - 1,
                                                 workspace=FAKE, max_pages_per_seq=1000))
    assert e.value.status == lvq.LOOPVQ_ERR_WORKSPACE


def test_decode_rejects_a_block_table_shorter_than_the_context():
    """max_seq_len - P - R vector-quantized rows need that many page slots per sequence."""
    wl = W.STACK_32K
    cfg = lvq.make_config(wl)
    need = -(-(wl.context - wl.prefix - wl.recent) // wl.page_tokens)   # 511 pages of 64 tokens
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_decode_attn(cfg, **_decode_kw(wl, max_pages_per_seq=need - 1))
    assert e.value.status == lvq.LOOPVQ_ERR_INVALID_ARG
    assert "max_pages_per_seq" in lvq.loopvq_last_error()
    # exactly enough pages passes every check up to the workspace, the last one before a launch
    # (one sequence: the plan splits it, so the empty workspace is refused)
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_decode_attn(cfg, **_decode_kw(wl, batch=1, max_pages_per_seq=need))
    assert e.value.status == lvq.LOOPVQ_ERR_WORKSPACE


def test_decode_rejects_too_few_splits_for_the_histogram_bound():
    """One split holds at most 65,536 vector-quantized rows (its 64-bit value histogram and the page
    ids a wave keeps); an explicit split count below that is refused before any launch."""
    wl = W.TINY.with_(context=2 * 65536 + 200)
    cfg = lvq.make_config(wl)
    kw = _decode_kw(wl, batch=1, max_seq_len=wl.context, max_pages_per_seq=4096, workspace=FAKE,
                    workspace_bytes=1 << 30)
    for S in (1, 2):
        with pytest.raises(lvq.LoopVQError) as e:
            lvq.loopvq_decode_attn(cfg, **dict(kw, num_splits=S))
        assert e.value.status == lvq.LOOPVQ_ERR_INVALID_ARG
        assert "splits" in lvq.loopvq_last_error()
    # three splits are enough: the call then stops at the workspace, the last check before a launch
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_decode_attn(cfg, **dict(kw, num_splits=3, workspace_bytes=16))
    assert e.value.status == lvq.LOOPVQ_ERR_WORKSPACE


def test_decode_rejects_a_page_region_of_2_gib():
    """Index tiles are read with 32-bit buffer offsets over one kv-head's page region, so
    num_pages * page_bytes must stay below 2 GiB."""
    wl = W.STACK_32K
    cfg = lvq.make_config(wl)
    page_bytes = lvq.loopvq_layout_query(cfg, 1, 1).page_bytes
    too_many = (2 ** 31 - 1) // page_bytes + 1      # the first count whose region reaches 2^31 bytes
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_decode_attn(cfg, **_decode_kw(wl, num_pages=too_many))
    assert e.value.status == lvq.LOOPVQ_ERR_UNSUPPORTED
    with pytest.raises(lvq.LoopVQError) as e:   # one page fewer passes, up to the workspace check
        lvq.loopvq_decode_attn(cfg, **_decode_kw(wl, batch=1, num_pages=too_many - 1))
    assert e.value.status == lvq.LOOPVQ_ERR_WORKSPACE



def test_decode_noalloc_refuses_a_plan_beyond_the_static_array():
    """The allocation-free decode refuses, before any HIP call, a split plan whose partials exceed
    its static per-GPU array; up to that size it checks exactly what the workspace entry point checks."""
    wl = W.LAYER_4K.with_(batch=128)
    cfg = lvq.make_config(wl)
    assert 256 * wl.batch * wl.q_heads * (wl.head_dim + 4) * 4 > 16 << 20
    kw = _decode_kw(wl, num_splits=256, max_pages_per_seq=64)
    kw.pop("workspace"), kw.pop("workspace_bytes")
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_decode_attn_noalloc(cfg, **kw)
    assert e.value.status == lvq.LOOPVQ_ERR_WORKSPACE
    assert "static scratch" in lvq.loopvq_last_error()
    for over, status in ((dict(layer=1), lvq.LOOPVQ_ERR_INVALID_ARG), (dict(pool=FAKE + 8), lvq.LOOPVQ_ERR_MISALIGNED),
                         (dict(num_splits=300), lvq.LOOPVQ_ERR_INVALID_ARG)):
        with pytest.raises(lvq.LoopVQError) as e:
            lvq.loopvq_decode_attn_noalloc(cfg, **dict(kw, **over))
        assert e.value.status == status

def test_unsupported_variants_rejected():
    for over in [dict(index_bits=9), dict(loop_group=2, num_loops=4), dict(chans_per_group=8, head_dim=256),
                 dict(loop_group=8, num_loops=8, chans_per_group=8)]:
        cfg = lvq.make_config(W.LAYER_4K)
        for k, v in over.items():
            setattr(cfg, k, v)
        assert lvq.loopvq_config_check(cfg) == 0
        with pytest.raises(lvq.LoopVQError) as e:
            lvq.loopvq_decode_attn(cfg, **_decode_kw(W.LAYER_4K))
        assert e.value.status == lvq.LOOPVQ_ERR_UNSUPPORTED


def _encode_kw(**over):
    kw = dict(layer=0, loop_group=0, kind=0, n_tokens=10, src=FAKE, stride_loop=4096, stride_token=2048,
              stride_head=128, seq_id=FAKE, vq_pos=FAKE, block_table=FAKE, batch=2, max_pages_per_seq=4,
              num_pages=8, cb=FAKE, cb_norms=FAKE, pool=FAKE, stream=0)
    kw.update(over)
    return kw


@pytest.mark.parametrize("over,status", [
    (dict(kind=2), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(loop_group=1), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(n_tokens=-1), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(cb_norms=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(batch=0), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(src=FAKE + 4), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(stride_token=2050), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(cb=FAKE + 8), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(seq_id=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(block_table=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(pool=None), lvq.LOOPVQ_ERR_INVALID_ARG),                 # no pool and no out_idx
    (dict(pool=None, out_idx=FAKE + 2), lvq.LOOPVQ_ERR_MISALIGNED),   # assignment only: out_idx checked
])
def test_encode_rejects_before_launch(over, status):
    cfg = lvq.make_config(W.LAYER_4K)
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_encode(cfg, **_encode_kw(**over))
    assert e.value.status == status


def _evict_kw(**over):
    kw = dict(batch=2, max_pages_per_seq=4, num_pages=8, k_ring=FAKE, v_ring=FAKE, ring_slot=FAKE, vq_pos=FAKE,
              block_table=FAKE, cb_k=FAKE, cb_v=FAKE, norms_k=FAKE, norms_v=FAKE, pool=FAKE, stream=0)
    kw.update(over)
    return kw


@pytest.mark.parametrize("over,status", [
    (dict(batch=0), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(num_pages=0), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(ring_slot=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(norms_v=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(v_ring=FAKE + 8), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(cb_k=FAKE + 2), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(out_idx=FAKE + 2), lvq.LOOPVQ_ERR_MISALIGNED),
])
def test_evict_rejects_before_launch(over, status):
    cfg = lvq.make_config(W.LAYER_4K)
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_evict(cfg, **_evict_kw(**over))
    assert e.value.status == status


def test_evict_needs_a_recent_window_and_a_built_variant():
    cfg = lvq.make_config(W.LAYER_4K)
    cfg.recent_tokens = 0
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_evict(cfg, **_evict_kw())
    assert e.value.status == lvq.LOOPVQ_ERR_INVALID_ARG
    cfg = lvq.make_config(W.LAYER_4K)
    cfg.index_bits = 9
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_evict(cfg, **_evict_kw())
    assert e.value.status == lvq.LOOPVQ_ERR_UNSUPPORTED


def _extend_kw(**over):
    kw = dict(layer=0, loop=0, batch=2, chunk=16, q=FAKE, k_new=FAKE, v_new=FAKE, seq_lens=FAKE, max_seq_len=500,
              out=FAKE, block_table=FAKE, pool=FAKE, max_pages_per_seq=8, num_pages=16, cb_k_grp=FAKE,
              cb_v_grp=FAKE, k_prefix=FAKE, v_prefix=FAKE, k_recent=FAKE, v_recent=FAKE, stream=0)
    kw.update(over)
    return kw


@pytest.mark.parametrize("over,status", [
    (dict(chunk=0), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(loop=4), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(k_new=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(pool=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(k_recent=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(max_pages_per_seq=2 ** 25), lvq.LOOPVQ_ERR_INVALID_ARG),     # 2^25 pages x 64 tokens = 2^31
    (dict(max_pages_per_seq=6), lvq.LOOPVQ_ERR_INVALID_ARG),           # 428 VQ rows need 7 pages of 64
    (dict(q=FAKE + 8), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(out=FAKE + 4), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(v_new=FAKE + 2), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(lse=FAKE + 2), lvq.LOOPVQ_ERR_MISALIGNED),
])
def test_extend_rejects_before_launch(over, status):
    cfg = lvq.make_config(W.LAYER_4K)
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_extend_attn(cfg, **_extend_kw(**over))
    assert e.value.status == status


def _lloyd_kw(**over):
    kw = dict(layer=0, cb_set=0, n_samples=1000, src=FAKE, stride_loop=1000 * 16 * 128, stride_token=16 * 128,
              stride_head=128, weight=FAKE, cb=FAKE, cb_norms=FAKE, assign=FAKE, workspace=FAKE,
              workspace_bytes=1 << 40, stream=0)
    kw.update(over)
    return kw


@pytest.mark.parametrize("over,status", [
    (dict(layer=1), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(cb_set=1), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(n_samples=-1), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(weight=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(assign=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(workspace=None), lvq.LOOPVQ_ERR_INVALID_ARG),
    (dict(src=FAKE + 8), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(stride_token=16 * 128 + 4), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(weight=FAKE + 8), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(distortion=FAKE + 4), lvq.LOOPVQ_ERR_MISALIGNED),
    (dict(workspace_bytes=64), lvq.LOOPVQ_ERR_WORKSPACE),
])
def test_lloyd_rejects_before_launch(over, status):
    cfg = lvq.make_config(W.LAYER_4K)
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_lloyd_step(cfg, **_lloyd_kw(**over))
    assert e.value.status == status
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_lloyd_update(cfg, **_lloyd_kw(**over))
    assert e.value.status == status


def test_lloyd_workspace_sizes():
    cfg = lvq.make_config(W.LAYER_4K)
    wl = W.LAYER_4K
    sizes = [lvq.loopvq_lloyd_workspace(cfg, n) for n in (0, 1, 5000, 100_000, 10_000_000)]
    assert all(s % 16 == 0 and s > 0 for s in sizes)
    assert sizes == sorted(sizes) and sizes[-1] == sizes[-2], "partials are capped by the workgroup count"
    # at least one set of partial sums: every (kv-head, loop step, channel, codeword) in fp64
    assert sizes[0] >= wl.kv_heads * wl.loop_group * wl.head_dim * wl.codewords * 8
    with pytest.raises(lvq.LoopVQError):
        lvq.loopvq_lloyd_workspace(cfg, -1)
    # per-group codebooks: cb_set ranges over the loop groups [0, J)
    pg = lvq.make_config(W.DEEP_8K)
    pg.codebook_per_loop_group = 1
    for bad in (W.DEEP_8K.loop_groups, -1):
        with pytest.raises(lvq.LoopVQError) as e:
            lvq.loopvq_lloyd_step(pg, **_lloyd_kw(cb_set=bad, stride_loop=1000 * 32 * 128, stride_token=32 * 128))
        assert e.value.status == lvq.LOOPVQ_ERR_INVALID_ARG


def test_codebook_prepare_groups_rejects():
    cfg = lvq.make_config(W.TINY)
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_codebook_prepare_groups(cfg, None, FAKE, stream=0)
    assert e.value.status == lvq.LOOPVQ_ERR_INVALID_ARG
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_codebook_prepare_groups(cfg, FAKE, FAKE + 2, stream=0)
    assert e.value.status == lvq.LOOPVQ_ERR_MISALIGNED


def test_codebook_prepare_rejects():
    cfg = lvq.make_config(W.TINY)
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_codebook_prepare(cfg, None, FAKE, None, stream=0)
    assert e.value.status == lvq.LOOPVQ_ERR_INVALID_ARG
    with pytest.raises(lvq.LoopVQError) as e:
        lvq.loopvq_codebook_prepare(cfg, FAKE + 2, FAKE, None, stream=0)
    assert e.value.status == lvq.LOOPVQ_ERR_MISALIGNED


def test_status_strings():
    for s, txt in [(0, "ok"), (-1, "invalid argument"), (-2, "unsupported variant"), (-3, "misaligned pointer"),
                   (-4, "workspace too small"), (-5, "HIP error"), (7, "unknown status")]:
        assert lvq.loopvq_status_string(s) == txt


# ---------------------------------------------------------------------------------
# The plain-C caller (tests/c_abi/decode_c.c): links against loopvq.h and the library
# with gcc, and its host-side steps run without a GPU
# ---------------------------------------------------------------------------------
C_CALLER = os.path.join(ROOT, "tests", "c_abi", "decode_c")


def _c_caller():
    if not os.path.exists(C_CALLER):
        import __graft_entry__
        __graft_entry__.build_c_caller()
    return C_CALLER


def _write_c_args(path, cfg, **extra):
    with open(os.path.join(path, "args.txt"), "w") as f:
        for name, _ in cfg._fields_:
            f.write(f"{name} {getattr(cfg, name)}\n")
        for k, v in extra.items():
            f.write(f"{k} {v}\n")


C_EXTRA = dict(layer=0, loop=1, batch=2, max_pages_per_seq=4, max_seq_len=500, num_splits=0, num_pages=8,
               pool_offset=0, pool_slice_bytes=0, softmax_scale=0.0, has_rot=0)


def test_c_caller_rejects_bad_config_before_any_hip_call(tmp_path):
    import subprocess
    cfg = lvq.make_config(W.TINY.with_(loop_group=3))
    _write_c_args(str(tmp_path), cfg, **C_EXTRA)
    r = subprocess.run([_c_caller(), str(tmp_path)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1
    assert "loopvq_config_check" in r.stderr and "returned invalid argument" in r.stderr
    assert "multiple of loop_group" in r.stderr


def test_c_caller_sizes_buffers_from_layout_query(tmp_path):
    import subprocess
    cfg = lvq.make_config(W.TINY)
    _write_c_args(str(tmp_path), cfg, **C_EXTRA)
    r = subprocess.run([_c_caller(), str(tmp_path)], capture_output=True, text=True, timeout=60)
    lay = lvq.loopvq_layout_query(cfg, C_EXTRA["batch"], C_EXTRA["num_pages"])
    assert r.returncode == 1 and "cannot open" in r.stderr and "q.bin" in r.stderr
    assert f"0.500 bits per element, pool {lay.pool_bytes} bytes, page {lay.page_bytes} bytes" in r.stdout
