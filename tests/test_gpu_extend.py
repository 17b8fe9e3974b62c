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
    # d=128 with 256-token pages: four 64-token key tiles per page, the last page partly used
    "d128_page256": (W.LAYER_4K.with_(batch=2, q_heads=4, kv_heads=2, context=900, page_tokens=256), 0, 1, [900, 333],
                     100, [100, 37]),
}


def _run_extend(name, mutate=None, abs_scale=1.0):
    """One extend launch of CASES[name] checked row by row against the oracle; mutate(case, kn, vn)
    may change the host values before they are uploaded."""
    _run_extend_case(name, *CASES[name], mutate=mutate, abs_scale=abs_scale)


def _run_extend_case(name, wl, layer, loop, lens, M, clens, mutate=None, abs_scale=1.0, seed=4):
    case = H.Case(wl, layer, loop, lens, seed=seed)
    B, Hq, Hkv, d = wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim
    grp = Hq // Hkv
    kn = np.zeros((B, Hkv, M, d), np.uint16)
    vn = np.zeros((B, Hkv, M, d), np.uint16)
    for b in range(B):
        for h in range(Hkv):
            kn[b, h] = gen.kv_tokens(wl, 0, layer, b, h, lens[b], lens[b] + M, loop, loop + 1, case.sc)[:, 0]
            vn[b, h] = gen.kv_tokens(wl, 1, layer, b, h, lens[b], lens[b] + M, loop, loop + 1, case.sc)[:, 0]
    if mutate is not None:
        mutate(case, kn, vn)
    enc = case.oracle_encode()
    idx_of = lambda kind, b, h: enc[kind, b, h][0]   # noqa: E731
    case.gpu_setup()
    case.d_pool.copy_(torch.from_numpy(case.oracle_pool(idx_of).reshape(-1)).to(H.DEV))
    q = gen.to_bf16_bits(np.random.default_rng(21).normal(size=(B, M, Hq, d)))
    out = torch.full((B, M, Hq, d), float("nan"), dtype=torch.float32, device=H.DEV)
    lse = torch.full((B, M, Hq), float("nan"), dtype=torch.float32, device=H.DEV)
    print(f"extend {name}: lens {lens}, chunk {M}", flush=True)
    lvq.loopvq_extend_attn(case.cfg, layer=layer, loop=loop, batch=B, chunk=M, q=H.dev_u16(q), k_new=H.dev_u16(kn),
                           v_new=H.dev_u16(vn), seq_lens=case.d_lens, max_seq_len=int(max(lens)), out=out, lse=lse,
                           chunk_lens=H.dev_i32(clens) if clens is not None else None, block_table=case.d_bt,
                           pool=case.pool_base(), max_pages_per_seq=case.paging.max_pages,
                           num_pages=case.paging.num_pages, cb_k_grp=case.d_grp[0], cb_v_grp=case.d_grp[1],
                           k_prefix=case.d_win[0], v_prefix=case.d_win[1], k_recent=case.d_win[2],
                           v_recent=case.d_win[3], rot=case.d_rot)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    got_lse = lse.cpu().numpy().astype(np.float64)
    scale = 1.0 / np.sqrt(d)
    checked, worst = 0, (0.0, 0.0)
    for b in range(B):
        n_pre, n_vq, n_rec = case.split[b]
        Mb = M if clens is None else clens[b]
        assert np.isnan(got[b, Mb:]).all(), "rows past the chunk length must stay untouched"
        assert np.isnan(got_lse[b, Mb:]).all(), "lse of rows past the chunk length must stay untouched"
        if Mb == 0:
            continue
        for hq in range(Hq):
            h = hq // grp
            o_ref, lse_ref = O.extend_attention(
                H.f64(q[b, :Mb, hq]), H.f64(case.kp[b, h, :n_pre]), H.f64(case.vp[b, h, :n_pre]), idx_of(0, b, h),
                idx_of(1, b, h), H.codebooks_f64(case.cbk, layer, case.jc, h),
                H.codebooks_f64(case.cbv, layer, case.jc, h), H.f64(case.kr[b, h, :n_rec]),
                H.f64(case.vr[b, h, :n_rec]), H.f64(kn[b, h, :Mb]), H.f64(vn[b, h, :Mb]), case.tau, wl.chans, scale,
                case.rot)
            # (abs_scale: the max-abs bound in units of the largest value magnitude, for values far from 1)
            rel, mx = H.check_attention(got[b, :Mb, hq] / abs_scale, o_ref / abs_scale, got_lse[b, :Mb, hq], lse_ref)
            worst = (max(worst[0], rel), max(worst[1], mx))
            checked += Mb
    print(f"  {checked} rows checked; worst rel-L2 {worst[0]:.2e}, max-abs {worst[1]:.2e}", flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_extend_matches_oracle(name):
    _run_extend(name)


def _scaled(bits, factor):
    """bf16 bits times a power of two (exact for the normal values the generator makes)."""
    return gen.to_bf16_bits(H.f64(bits) * factor)


def _huge_recent(case, kn, vn):
    # one value of 2^17 (beyond fp16) in the longest sequence's recent window: its workgroups switch
    # to the bf16 value product after the prefix and vector-quantized tiles
    b = int(np.argmax(case.lens))
    assert case.split[b][2] > 5
    case.vr[b, 0, 5, 3] = _scaled(np.array([0x3f80], np.uint16), 2.0 ** 17)[0]


def _huge_chunk_tail(case, kn, vn):
    # 2^16 (the first magnitude outside fp16) in the last chunk token of sequence 1
    vn[1, 1, -1, 7] = _scaled(np.array([0x3f80], np.uint16), 2.0 ** 16)[0]


def _tiny_values(case, kn, vn):
    # every value (windows, chunk, the value rows of the cache and their codebooks) times 2^-20:
    # below fp16's exact range, so every tile takes the bf16 product; the indices do not change
    for arr in (case.vp, case.vr, vn):
        arr[...] = _scaled(arr, 2.0 ** -20)
    case.cbv = _scaled(case.cbv, 2.0 ** -20)
    for key in list(case.kv):
        if key[0] == 1:
            case.kv[key] = _scaled(case.kv[key], 2.0 ** -20)


def _huge_codebook(case, kn, vn):
    # the vector-quantized values (the value codebooks and the rows they encode) times 2^16: the
    # codebook slice fails the per-workgroup check, and every tile takes the bf16 product
    case.cbv = _scaled(case.cbv, 2.0 ** 16)
    for key in list(case.kv):
        if key[0] == 1:
            case.kv[key] = _scaled(case.kv[key], 2.0 ** 16)


@pytest.mark.parametrize("name,mode", [("d128", "huge_recent"), ("d128", "huge_chunk_tail"), ("d128", "tiny"),
                                       ("c8_gqa", "tiny"), ("d64_gqa", "huge_recent"), ("d128", "huge_codebook"),
                                       ("c8_rot", "huge_recent"), ("c8_rot", "huge_codebook")])
def test_extend_values_outside_fp16(name, mode):
    """Value tiles are multiplied in fp16 when all their values convert exactly; a tile with a value
    of magnitude >= 2^16 (or non-finite) or a nonzero one below 2^-17 sends the rest of the
    workgroup's tiles to the bf16 product, and so does such a value anywhere in the kv-head's value
    codebook slice (checked once, before the first tile).  Same tolerance as every extend case; for values of
    2^17 the max-abs bound is taken relative to that magnitude."""
    mut = {"huge_recent": _huge_recent, "huge_chunk_tail": _huge_chunk_tail, "tiny": _tiny_values,
           "huge_codebook": _huge_codebook}[mode]
    _run_extend(name, mut, abs_scale=2.0 ** 17 if mode.startswith("huge") else 1.0)


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


FULL_EXTEND = [
    # (workload, chunk, sampled (sequence, q-head) pairs, sampled chunk rows)
    (W.LAYER_4K, 512, [(0, 0), (17, 9), (31, 15)], [0, 37, 255, 256, 300]),   # both 256-row workgroups
    (W.STACK_32K, 256, [(0, 0), (63, 15)], [0, 100, 255]),
    (W.QUARTER_16K, 256, [(5, 3), (127, 15)], [0, 64, 255]),                   # rotated keys, c=8
]


@pytest.mark.parametrize("wl,M,samples,rows", FULL_EXTEND, ids=[w.name for w, _, _, _ in FULL_EXTEND])
def test_extend_full_size_sampled(wl, M, samples, rows):
    """An extend workload at its full shape (the launch bench.py --extend times for it), checked on
    sampled rows of a few (sequence, head) pairs against the oracle.  The sampled pairs hold
    generator indices packed by the oracle and generator windows and chunk rows; the other
    sequences' pages are zero and their chunk rows plain normals (computed, not checked)."""
    layer, loop = 0, 1
    fc = H.FullCase(wl, layer, loop, samples)
    fc.upload()
    B, Hq, Hkv, d = wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim
    N = int(wl.context)
    d_grp = []
    for cb in (fc.cbk, fc.cbv):
        d_cb = H.dev_u16(cb)
        g = torch.empty_like(d_cb)
        lvq.loopvq_codebook_prepare_groups(fc.cfg, d_cb, g)
        d_grp.append(g)
        del d_cb
    rng = np.random.default_rng(77)
    q = gen.to_bf16_bits(rng.normal(size=(B, M, Hq, d)))
    kn = gen.to_bf16_bits(rng.normal(size=(B, Hkv, M, d)))
    vn = gen.to_bf16_bits(rng.normal(size=(B, Hkv, M, d)))
    for b, h in fc.pairs:
        kn[b, h] = gen.kv_tokens(wl, 0, layer, b, h, N, N + M, loop, loop + 1, fc.sc)[:, 0]
        vn[b, h] = gen.kv_tokens(wl, 1, layer, b, h, N, N + M, loop, loop + 1, fc.sc)[:, 0]
    out = torch.full((B, M, Hq, d), float("nan"), dtype=torch.float32, device=H.DEV)
    lse = torch.full((B, M, Hq), float("nan"), dtype=torch.float32, device=H.DEV)
    print(f"extend full size {wl.name}: {B} x {Hq} heads, cache {N}, chunk {M}", flush=True)
    lvq.loopvq_extend_attn(fc.cfg, layer=layer, loop=loop, batch=B, chunk=M, q=H.dev_u16(q), k_new=H.dev_u16(kn),
                           v_new=H.dev_u16(vn), seq_lens=fc.d_lens, max_seq_len=N, out=out, lse=lse,
                           block_table=fc.d_bt,
                           pool=fc.d_pool.data_ptr() - fc.pool_shift, max_pages_per_seq=fc.paging.max_pages,
                           num_pages=fc.paging.num_pages, cb_k_grp=d_grp[0], cb_v_grp=d_grp[1],
                           k_prefix=fc.d_win[0], v_prefix=fc.d_win[1], k_recent=fc.d_win[2], v_recent=fc.d_win[3],
                           rot=fc.d_rot)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item(), "every row of the chunk is computed"
    assert not torch.isnan(lse).any().item(), "every row's lse is written"
    got = out.cpu().numpy().astype(np.float64)
    got_lse = lse.cpu().numpy().astype(np.float64)
    del out, lse
    grp = Hq // Hkv
    worst = 0.0
    i_max = max(rows)
    for b, hq in samples:
        h = hq // grp
        n_pre, _, n_rec = fc.split[b]
        o_ref, lse_ref = O.extend_attention(
            H.f64(q[b, :i_max + 1, hq]), H.f64(fc.kp[b, h, :n_pre]), H.f64(fc.vp[b, h, :n_pre]), fc.idx[0, b, h],
            fc.idx[1, b, h], H.codebooks_f64(fc.cbk, fc.l, fc.jc, h), H.codebooks_f64(fc.cbv, fc.l, fc.jc, h),
            H.f64(fc.kr[b, h, :n_rec]), H.f64(fc.vr[b, h, :n_rec]), H.f64(kn[b, h, :i_max + 1]),
            H.f64(vn[b, h, :i_max + 1]), fc.tau, wl.chans, 1.0 / np.sqrt(d), fc.rot)
        rel, _ = H.check_attention(got[b, rows, hq], o_ref[rows], got_lse[b, rows, hq], lse_ref[rows])
        worst = max(worst, rel)
    print(f"  {len(samples) * len(rows)} sampled rows; worst rel-L2 {worst:.2e}", flush=True)
