"""GPU extend (chunked prefill) attention over the packed cache against the oracle.

The cache is the small encode/decode case of the harness (host generator values, oracle
brute-force indices packed by the oracle); the chunk's keys / values are the next tokens of
each sequence from the same generator, its queries seeded normals in bf16.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("lvq_harness")

import sub_bit_loop_loopvq_amd as lvq  # noqa: E402
from oracle import loopvq_oracle as O  # noqa: E402
from synth import gen, workloads as W  # noqa: E402

CASES = {
    # d=64, c=4, GQA 2:1; empty cache, prefix only, no VQ rows, one VQ row, VQ tiles with a tail;
    # a chunk of 70 rows with per-sequence lengths
    "d64_gqa": (W.TINY.with_(batch=5, q_heads=4, kv_heads=2, context=520), 0, 1, [0, 5, 72, 73, 300], 70,
                [70, 1, 64, 65, 33]),
    # d=128, c=4: two row blocks per (sequence, head), explicit chunk of 130
    "d128": (W.LAYER_4K.with_(batch=3, q_heads=4, kv_heads=4, context=800), 0, 2, [600, 200, 80], 130, None),
    # d=128, c=8, rotated keys (q' = R^T q on the GPU)
    "c8_rot": (W.QUARTER_16K.with_(layers=1, batch=2, q_heads=2, kv_heads=2, context=500), 0, 3, [400, 150], 40,
               None),
    # c=8 without a rotation (16 groups: half of the threads idle in index staging), 300 chunk rows
    # of GQA 4:1 = 1200 query rows: five 256-row workgroups per (sequence, kv-head), the last ragged
    "c8_gqa": (W.QUARTER_16K.with_(layers=1, batch=2, q_heads=8, kv_heads=2, context=700, rotate_keys=False), 0, 2,
               [650, 100], 300, [300, 77]),
    # c=4 over G=8 loop steps (0.25 bit), loop step 6 of its group
    "c4_g8": (W.LAYER_4K.with_(loops=8, loop_group=8, batch=2, q_heads=4, kv_heads=2, context=400), 0, 6, [300, 90],
              50, None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_extend_matches_oracle(name):
    wl, layer, loop, lens, M, clens = CASES[name]
    case = H.Case(wl, layer, loop, lens, seed=4)
    enc = case.oracle_encode()
    idx_of = lambda kind, b, h: enc[kind, b, h][0]   # noqa: E731
    case.gpu_setup()
    case.d_pool.copy_(torch.from_numpy(case.oracle_pool(idx_of).reshape(-1)).to(H.DEV))
    B, Hq, Hkv, d = wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim
    grp = Hq // Hkv
    kn = np.zeros((B, Hkv, M, d), np.uint16)
    vn = np.zeros((B, Hkv, M, d), np.uint16)
    for b in range(B):
        for h in range(Hkv):
            kn[b, h] = gen.kv_tokens(wl, 0, layer, b, h, lens[b], lens[b] + M, loop, loop + 1, case.sc)[:, 0]
            vn[b, h] = gen.kv_tokens(wl, 1, layer, b, h, lens[b], lens[b] + M, loop, loop + 1, case.sc)[:, 0]
    q = gen.to_bf16_bits(np.random.default_rng(21).normal(size=(B, M, Hq, d)))
    out = torch.full((B, M, Hq, d), float("nan"), dtype=torch.float32, device=H.DEV)
    print(f"extend {name}: lens {lens}, chunk {M}", flush=True)
    lvq.loopvq_extend_attn(case.cfg, layer=layer, loop=loop, batch=B, chunk=M, q=H.dev_u16(q), k_new=H.dev_u16(kn),
                           v_new=H.dev_u16(vn), seq_lens=case.d_lens, max_seq_len=int(max(lens)), out=out,
                           chunk_lens=H.dev_i32(clens) if clens is not None else None, block_table=case.d_bt,
                           pool=case.pool_base(), max_pages_per_seq=case.paging.max_pages,
                           num_pages=case.paging.num_pages, cb_k_grp=case.d_grp[0], cb_v_grp=case.d_grp[1],
                           k_prefix=case.d_win[0], v_prefix=case.d_win[1], k_recent=case.d_win[2],
                           v_recent=case.d_win[3], rot=case.d_rot)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    scale = 1.0 / np.sqrt(d)
    checked, worst = 0, (0.0, 0.0)
    for b in range(B):
        n_pre, n_vq, n_rec = case.split[b]
        Mb = M if clens is None else clens[b]
        assert np.isnan(got[b, Mb:]).all(), "rows past the chunk length must stay untouched"
        for hq in range(Hq):
            h = hq // grp
            o_ref, _ = O.extend_attention(
                H.f64(q[b, :Mb, hq]), H.f64(case.kp[b, h, :n_pre]), H.f64(case.vp[b, h, :n_pre]), idx_of(0, b, h),
                idx_of(1, b, h), H.codebooks_f64(case.cbk, layer, case.jc, h),
                H.codebooks_f64(case.cbv, layer, case.jc, h), H.f64(case.kr[b, h, :n_rec]),
                H.f64(case.vr[b, h, :n_rec]), H.f64(kn[b, h, :Mb]), H.f64(vn[b, h, :Mb]), case.tau, wl.chans, scale,
                case.rot)
            rel, mx = H.check_attention(got[b, :Mb, hq], o_ref)
            worst = (max(worst[0], rel), max(worst[1], mx))
            checked += Mb
    print(f"  {checked} rows checked; worst rel-L2 {worst[0]:.2e}, max-abs {worst[1]:.2e}", flush=True)


@pytest.mark.parametrize("c,G,d", [(4, 4, 128), (8, 2, 128), (4, 8, 64)])
def test_group_major_codebooks_layout(c, G, d):
    """loopvq_codebook_prepare_groups writes [L][Jcb][Hkv][G][NG][K][c]: the canonical rows
    [..][NG][K][G*c] with each row split into its G loop slices, moved in front of the groups."""
    wl = W.TINY.with_(layers=2, loops=2 * G, loop_group=G, chans=c, head_dim=d, kv_heads=2, q_heads=2,
                      codebook_per_loop_group=True)
    cfg = lvq.make_config(wl)
    L, Jcb, Hkv, NG, K = wl.layers, wl.cb_loop_groups, wl.kv_heads, wl.groups, wl.codewords
    bits = np.random.default_rng(12).integers(0, 1 << 16, size=(L, Jcb, Hkv, NG, K, G * c)).astype(np.uint16)
    d_cb = H.dev_u16(bits)
    d_grp = torch.empty_like(d_cb)
    lvq.loopvq_codebook_prepare_groups(cfg, d_cb, d_grp)
    torch.cuda.synchronize()
    want = bits.reshape(L, Jcb, Hkv, NG, K, G, c).transpose(0, 1, 2, 5, 3, 4, 6)
    got = d_grp.cpu().numpy().view(np.uint16).reshape(want.shape)
    assert np.array_equal(got, want)
