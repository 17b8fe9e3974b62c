"""GPU parity at the limits the host checks allow (needs an MI355X).

- The top of the largest page region: a kv-head's pages may span up to 2^31 - 1 bytes (the
  kernels address a region with 32-bit buffer offsets).  Every sequence's pages are taken from
  the top of a region of that size, for two kv-heads (the second region starts 2 GiB into the
  pool); encode writes them, then decode and extend read them.
- The longest split: one split may hold 65,536 vector-quantized rows (128 tiles per wave, the
  page ids a wave keeps in registers), at 32 and at 16 channel groups, with one split, the
  largest split count (256) and the automatic plan.
- The widest weights a split accepts without its exact-maximum redo: every row after the first
  tiles scores 16.5 (log2 units) above the reference and all of them add to one value-histogram
  bucket, 65,024 x 2^16.5 x 2^30 (about 2^62.5), close to the 64-bit limit.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("lvq_harness")

import sub_bit_loop_loopvq_amd as lvq  # noqa: E402
from oracle import loopvq_oracle as O  # noqa: E402
from synth import gen, workloads as W  # noqa: E402

INT32_MAX = 2 ** 31 - 1


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class TopPaging:
    """Block tables whose page ids are the top ones of a region of num_pages pages, shuffled."""

    def __init__(self, n_vq_per_seq, PT: int, num_pages: int, seed: int):
        need = [max(1, -(-int(n) // PT)) for n in n_vq_per_seq]
        self.PT = PT
        self.max_pages = max(need)
        self.num_pages = num_pages
        self.total = sum(need)
        ids = num_pages - 1 - np.random.default_rng(seed).permutation(self.total)
        self.table = np.zeros((len(need), self.max_pages), dtype=np.int32)
        pos = 0
        for b, k in enumerate(need):
            self.table[b, :k] = ids[pos:pos + k]
            pos += k


TOP_CASES = {
    # c=4, d=128: 4 KB pages, 524,287 of them per kv-head
    "c4_d128": (W.LAYER_4K.with_(batch=2, q_heads=4, kv_heads=2, context=700), 1, [700, 333], 40),
    # c=8, d=128, rotated keys: 2 KB pages, 1,048,575 per kv-head
    "c8_rot": (W.QUARTER_16K.with_(layers=1, batch=2, q_heads=2, kv_heads=2, context=600), 2, [600, 150], 30),
}


@pytest.mark.parametrize("name", list(TOP_CASES))
def test_top_of_largest_page_region(name):
    wl, loop, lens, M = TOP_CASES[name]
    B, Hq, Hkv, d = wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim
    lay = O.page_layout(wl.page_tokens, wl.groups, wl.index_bits)
    pb = lay["page_bytes"]
    num_pages = INT32_MAX // pb
    _say(f"top of region {name}: {num_pages} pages of {pb} B per kv-head, lens {lens}")
    case = H.Case(wl, 0, loop, lens, seed=13)
    case.paging = TopPaging(case.n_vq, wl.page_tokens, num_pages, seed=13)
    exp = case.oracle_encode()
    idx_of = lambda k, b, h: exp[k, b, h][0]  # noqa: E731
    case.gpu_setup()
    assert case.d_pool.numel() == Hkv * num_pages * pb and case.pool_shift == 0

    # encode both kinds into the top pages: every index, then every used page byte
    for kind in (0, 1):
        _say(f"  encode kind {kind}")
        gidx, rows, _ = case.gpu_encode(kind)
        C_of = case.cbk if kind == 0 else case.cbv
        for h in range(Hkv):
            C = H.codebooks_f64(C_of, 0, case.jc, h)
            for b in range(B):
                sel = [r for r, (bb, _) in enumerate(rows) if bb == b]
                idx, d1, d2, x = exp[kind, b, h]
                for g in range(wl.groups):
                    assert H.check_indices(gidx[sel, h, g], idx[:, g], d1[:, g], d2[:, g], x[:, g], C[g]) == 0
    pool = case.d_pool.view(Hkv, num_pages, pb)
    for b in range(B):
        if case.n_vq[b] == 0:
            continue
        for h in range(Hkv):
            pages = O.pack_sequence(idx_of(0, b, h), idx_of(1, b, h), wl.page_tokens, wl.index_bits)
            for p in range(pages.shape[0]):
                got = pool[h, int(case.paging.table[b, p])].cpu().numpy()
                assert np.array_equal(got, pages[p]), f"page {p} of sequence {b}, kv-head {h}"
    lowest = num_pages - case.paging.total
    for h in range(Hkv):
        assert int(pool[h, lowest - 1].count_nonzero()) == 0 and int(pool[h, 0].count_nonzero()) == 0

    # decode over the encoded pages
    _say("  decode")
    o_ref, lse_ref = case.oracle_decode(idx_of)
    for S in (0, 3):
        o, lse = case.gpu_decode(num_splits=S)
        H.check_attention(o, o_ref, lse, lse_ref)

    # extend over the same pages
    _say(f"  extend, chunk {M}")
    kn = np.zeros((B, Hkv, M, d), np.uint16)
    vn = np.zeros((B, Hkv, M, d), np.uint16)
    for b in range(B):
        for h in range(Hkv):
            kn[b, h] = gen.kv_tokens(wl, 0, 0, b, h, lens[b], lens[b] + M, loop, loop + 1, case.sc)[:, 0]
            vn[b, h] = gen.kv_tokens(wl, 1, 0, b, h, lens[b], lens[b] + M, loop, loop + 1, case.sc)[:, 0]
    q = gen.to_bf16_bits(np.random.default_rng(22).normal(size=(B, M, Hq, d)))
    out = torch.full((B, M, Hq, d), float("nan"), dtype=torch.float32, device=H.DEV)
    lvq.loopvq_extend_attn(case.cfg, layer=0, loop=loop, batch=B, chunk=M, q=H.dev_u16(q), k_new=H.dev_u16(kn),
                           v_new=H.dev_u16(vn), seq_lens=case.d_lens, max_seq_len=int(max(lens)), out=out,
                           block_table=case.d_bt, pool=case.pool_base(), max_pages_per_seq=case.paging.max_pages,
                           num_pages=num_pages, cb_k_grp=case.d_grp[0], cb_v_grp=case.d_grp[1],
                           k_prefix=case.d_win[0], v_prefix=case.d_win[1], k_recent=case.d_win[2],
                           v_recent=case.d_win[3], rot=case.d_rot)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    grp = Hq // Hkv
    for b in range(B):
        n_pre, _, n_rec = case.split[b]
        for hq in range(Hq):
            h = hq // grp
            o_ref, _ = O.extend_attention(
                H.f64(q[b, :, hq]), H.f64(case.kp[b, h, :n_pre]), H.f64(case.vp[b, h, :n_pre]), idx_of(0, b, h),
                idx_of(1, b, h), H.codebooks_f64(case.cbk, 0, case.jc, h), H.codebooks_f64(case.cbv, 0, case.jc, h),
                H.f64(case.kr[b, h, :n_rec]), H.f64(case.vr[b, h, :n_rec]), H.f64(kn[b, h]), H.f64(vn[b, h]),
                case.tau, wl.chans, 1.0 / np.sqrt(d), case.rot)
            H.check_attention(got[b, :, hq], o_ref)
    del pool, case
    torch.cuda.empty_cache()
    _say("  ok")


# 65,536 vector-quantized rows: the most one split holds
LONGEST = 65536 + 72
LONG_CASES = {
    "ng32": W.LAYER_4K.with_(batch=3, q_heads=2, kv_heads=2, context=LONGEST),
    "ng16": W.QUARTER_16K.with_(layers=1, batch=3, q_heads=2, kv_heads=1, context=LONGEST, rotate_keys=False),
}


@pytest.mark.parametrize("name", list(LONG_CASES))
def test_longest_split(name):
    wl = LONG_CASES[name]
    lens = [LONGEST, LONGEST - 1, 40001]
    samples = [(b, hq) for b in range(wl.batch) for hq in range(wl.q_heads)]
    _say(f"longest split {name}: lens {lens}")
    fc = H.FullCase(wl, 0, 1, samples, lens=lens, seed=14)
    fc.upload()
    refs = {(b, hq): fc.oracle(b, hq) for b, hq in samples}
    for S in (1, 256, 0):
        _say(f"  splits {S}")
        o, lse = fc.gpu_decode(num_splits=S)
        for b, hq in samples:
            o_ref, lse_ref = refs[b, hq]
            H.check_attention(o[b, hq][None], o_ref[None], np.array([lse[b, hq]]), np.array([lse_ref]))
    _say("  ok")


@pytest.mark.parametrize("name", list(LONG_CASES))
def test_widest_weights_in_one_bucket(name):
    """Rows [0, 512) (the first tile of every wave) take, per group, the codeword with the lowest
    q.codeword product and rows [512, 65536) the highest; the softmax scale makes the gap 16.5 in
    log2 units, just under the redo threshold, and every later row's value index is the same
    codeword, so one histogram bucket per group receives 65,024 weights of 2^16.5."""
    wl = LONG_CASES[name].with_(batch=1, q_heads=1, kv_heads=1)
    fc = H.FullCase(wl, 0, 2, [(0, 0)], lens=[LONGEST], seed=15)
    n_vq = int(fc.n_vq[0])
    assert n_vq == 65536
    cbk = H.codebooks_f64(fc.cbk, 0, fc.jc, 0)              # [NG][K][c*G]
    c, tau = wl.chans, fc.tau
    q = H.f64(fc.q[0, 0])
    lut = np.stack([cbk[g][:, tau * c:(tau + 1) * c] @ q[g * c:(g + 1) * c] for g in range(wl.groups)])  # [NG][K]
    lo, hi = lut.argmin(axis=1), lut.argmax(axis=1)
    gap = float((lut.max(axis=1) - lut.min(axis=1)).sum())
    scale = 16.5 / (gap * np.log2(np.e))
    first = 512
    idx_k = np.empty((n_vq, wl.groups), np.int64)
    idx_k[:first] = lo
    idx_k[first:] = hi
    idx_v = np.empty((n_vq, wl.groups), np.int64)
    idx_v[:first] = 3
    idx_v[first:] = 200
    fc.idx[0, 0, 0] = idx_k
    fc.idx[1, 0, 0] = idx_v
    _say(f"widest weights {name}: score gap {gap:.3f}, scale {scale:.5f}")
    fc.upload()
    o_ref, lse_ref = fc.oracle(0, 0, scale=scale)
    o, lse = fc.gpu_decode(num_splits=1, scale=scale)
    rel, mx = H.check_attention(o[0, 0][None], o_ref[None], np.array([lse[0, 0]]), np.array([lse_ref]))
    _say(f"  ok: rel-L2 {rel:.2e}, max-abs {mx:.2e}")
