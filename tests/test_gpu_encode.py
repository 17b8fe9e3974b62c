"""GPU encode at full size (bulk quantization of 65536 tokens) and the device generator twin."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("lvq_harness")

import sub_bit_loop_loopvq_amd as lvq  # noqa: E402
from oracle import loopvq_oracle as O  # noqa: E402
from synth import gen, workloads as W  # noqa: E402
from synth.device import DeviceGen  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("wl,kind,layer", [(W.TINY, 1, 0), (W.QUARTER_16K, 0, 7), (W.DEEP_8K, 0, 3),
                                           (W.LAYER_4K, 0, 0)])
def test_device_generator_matches_host(wl, kind, layer):
    _say(f"device generator {wl.name} kind={kind}")
    dg = DeviceGen(wl)
    b0, nb, h0, nh = wl.batch - 1 if wl.batch > 1 else 0, 1, 0, min(2, wl.kv_heads)
    n0, nn = 5, 70
    t0, nt = (wl.loops - 4, 4)
    d = wl.head_dim
    out = torch.zeros((nt, nb, nh, nn, d), dtype=torch.int16, device="cuda")
    dg.kv(out, kind=kind, layer=layer, b0=b0, nb=nb, h0=h0, nh=nh, n0=n0, nn=nn, t0=t0, nt=nt,
          s_loop=nb * nh * nn * d, s_b=nh * nn * d, s_h=nn * d, s_n=d)
    got = out.cpu().numpy().view(np.uint16)
    for h in range(nh):
        want = gen.kv_tokens(wl, kind, layer, b0, h0 + h, n0, n0 + nn, t0, t0 + nt)     # [nn][nt][d]
        assert np.array_equal(got[:, 0, h], want.transpose(1, 0, 2))


@pytest.mark.parametrize("c,G", [(4, 4), (8, 2), (4, 8)], ids=["c4g4", "c8g2", "c4g8"])
def test_full_size_encode_sampled(c, G):
    """65536 tokens x 32 kv-heads x all groups of one (layer, loop group), keys and values, at the
    deep workload's (c, G) = (4, 4) and at the other built shapes (8, 2) and (4, 8)."""
    wl = W.DEEP_8K.with_(chans=c, loop_group=G)
    layer, j = 1, min(5, wl.loop_groups - 1)
    per_seq = wl.encode_tokens // wl.batch          # 4096 tokens per sequence
    rows = wl.encode_tokens
    Hkv, d, G, P = wl.kv_heads, wl.head_dim, wl.loop_group, wl.prefix
    cfg = lvq.make_config(wl)
    paging = H.Paging([per_seq] * wl.batch, wl.page_tokens, seed=3, spare=0)
    lay = lvq.loopvq_layout_query(cfg, wl.batch, paging.num_pages)
    dg = DeviceGen(wl)
    src = torch.empty((G, rows, Hkv, d), dtype=torch.int16, device="cuda")
    seq = torch.arange(rows, dtype=torch.int32, device="cuda") // per_seq
    pos = torch.arange(rows, dtype=torch.int32, device="cuda") % per_seq
    bt = H.dev_i32(paging.table)
    slice_bytes = Hkv * lay.pool_head_stride_bytes
    pool = torch.zeros(slice_bytes, dtype=torch.uint8, device="cuda")
    shift = (layer * wl.loop_groups + j) * slice_bytes
    rng = np.random.default_rng(5)
    samp_r = rng.integers(0, rows, 48)
    samp_r[:2] = [0, rows - 1]
    samp_h = rng.integers(0, Hkv, 48)
    sc = gen.scales(wl)
    for kind in (0, 1):
        _say(f"full-size encode kind={kind}")
        for b in range(wl.batch):
            dg.kv(src[:, b * per_seq:], kind=kind, layer=layer, b0=b, nb=1, h0=0, nh=Hkv, n0=P, nn=per_seq,
                  t0=j * G, nt=G, s_loop=rows * Hkv * d, s_b=0, s_h=d, s_n=Hkv * d)
        cb = gen.codebooks(wl, kind, sc, layers=[layer])
        d_cb = H.dev_u16(cb)
        d_prep = torch.empty_like(d_cb)
        d_norm = torch.empty(lay.norms_elems, dtype=torch.float32, device="cuda")
        lvq.loopvq_codebook_prepare(cfg, d_cb, d_prep, d_norm)
        out_idx = torch.full((rows, Hkv, wl.groups), -1, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
        lvq.loopvq_encode(cfg, layer=layer, loop_group=j, kind=kind, n_tokens=rows, src=src,
                          stride_loop=rows * Hkv * d, stride_token=Hkv * d, stride_head=d, seq_id=seq, vq_pos=pos,
                          block_table=bt, batch=wl.batch, max_pages_per_seq=paging.max_pages,
                          num_pages=paging.num_pages, cb=d_cb, cb_norms=d_norm, pool=pool.data_ptr() - shift,
                          out_idx=out_idx, rerank_count=cnt)
        torch.cuda.synchronize()
        _say(f"  re-ranked sub-vectors: {int(cnt.item())} of {rows * Hkv * wl.groups}")
        assert (out_idx >= 0).all().item()
        src_s = src[:, torch.from_numpy(samp_r).cuda(), torch.from_numpy(samp_h).cuda()].cpu().numpy().view(np.uint16)
        idx_s = out_idx[torch.from_numpy(samp_r).cuda(), torch.from_numpy(samp_h).cuda()].cpu().numpy()
        pool_np = pool.cpu().numpy().reshape(Hkv, paging.num_pages, lay.page_bytes)
        excused = 0
        for i, (r, h) in enumerate(zip(samp_r, samp_h)):
            b, u = divmod(int(r), per_seq)
            host = gen.kv_tokens(wl, kind, layer, b, int(h), P + u, P + u + 1, j * G, j * G + G, sc)[0]   # [G][d]
            assert np.array_equal(src_s[:, i], host), "device generator differs from host generator"
            x = O.subvectors(H.f64(host)[:, None, :], wl.chans)[0]          # [NG][E]
            C = H.codebooks_f64(cb, layer, 0, int(h))
            for g in range(wl.groups):
                k, d1, d2 = O.encode(x[g][None], C[g])
                excused += H.check_indices(idx_s[i, g:g + 1], k, d1, d2, x[g][None], C[g])
                if idx_s[i, g] == k[0]:
                    # the index byte in its page (oracle page layout)
                    page = paging.table[b, u // wl.page_tokens]
                    w = u % wl.page_tokens
                    tile = (w // 4) * (wl.groups // 4) + g // 4
                    off = kind * (lay.page_bytes // 2) + tile * 16 + (w % 4) * 4 + (g % 4)
                    assert pool_np[h, page, off] == k[0]
        _say(f"  sampled 48 rows x {wl.groups} groups, excused near-ties: {excused}")
        del d_cb, d_prep, d_norm, out_idx
