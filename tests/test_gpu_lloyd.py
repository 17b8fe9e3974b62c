"""GPU Lloyd step (one weighted k-means iteration of codebook learning) against the oracle.

Samples are the seeded synthetic K/V planes of the host generator, weights the seeded
stand-ins for Fisher information (one in 16 is zero), the initial codebooks the seeded
codebooks.  Per (kv-head, group):
  * the assignment equals the oracle's brute-force encode, exactly;
  * every codeword equals the oracle's weighted mean rounded to bf16, exactly, except where
    that mean lies within 1e-12 (relative) of a bf16 rounding midpoint: both sides sum in
    fp64 in different orders, so there the neighbouring bf16 is accepted and counted;
  * codewords without weight keep their value; the cluster weights (sums of multiples of
    2^-23, exact in fp64 in any order) equal numpy's bincount exactly; the distortion is
    within 1e-9 (relative) of the oracle's; the norms equal what codebook_prepare writes;
  * codebook sets other than the one stepped are untouched.
Two iterations run; the second starts from the GPU's first codebook on both sides.  The
oracle checks every group of three kv-heads in the first iteration and one in the second.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("lvq_harness")

import sub_bit_loop_loopvq_amd as lvq  # noqa: E402
from oracle import loopvq_oracle as O  # noqa: E402
from synth import gen  # noqa: E402
from synth import workloads as W  # noqa: E402
from synth.device import DeviceGen  # noqa: E402
from synth.workloads import Workload  # noqa: E402

MID_REL = 1e-12
DIST_REL = 1e-9


def _say(msg):
    print(msg, flush=True)


def _wl(c, d, Hkv, L=1, T=4, per_group=False, G=4):
    return Workload(name=f"lloyd_c{c}_g{G}_d{d}_h{Hkv}", layers=L, loops=T, loop_group=G, q_heads=Hkv, kv_heads=Hkv,
                    head_dim=d, chans=c, index_bits=8, batch=1, context=8192, outlier_channels=2,
                    codebook_per_loop_group=per_group, wid=11)


def check_codewords(got_bits, mean, old):
    """got_bits: GPU bf16 bits [K][E]; mean: oracle fp64 update (mean for hit codewords, old value
    otherwise).  Returns the number of excused near-midpoint elements."""
    want = O.round_to_bf16(mean)
    got = H.f64(got_bits)
    bad = got != want
    if not bad.any():
        return 0
    m, gv, wv = mean[bad], got[bad], want[bad]
    gb = got_bits[bad].astype(np.int64)
    wb = gen.to_bf16_bits(wv).astype(np.int64)        # wv is a bf16 value: exact round trip
    assert (np.abs(gb - wb) == 1).all(), f"codewords differ by more than one bf16 step: {gv[:4]} vs {wv[:4]}"
    mid = (gv + wv) / 2
    assert (np.abs(m - mid) <= MID_REL * np.abs(m)).all(), f"non-midpoint codeword mismatch: {m[:4]} {gv[:4]} {wv[:4]}"
    return int(bad.sum())


def run_step(cfg, wl, d_src, strides, n, d_w, d_cb, d_norm, layer, cb_set):
    NG, Hkv = wl.groups, wl.kv_heads
    assign = torch.full((max(n, 1), Hkv, NG), -1, dtype=torch.int32, device="cuda")
    cw = torch.full((Hkv, NG, wl.codewords), -1.0, dtype=torch.float64, device="cuda")
    dist = torch.full((Hkv, NG), -1.0, dtype=torch.float64, device="cuda")
    ws = torch.empty(lvq.loopvq_lloyd_workspace(cfg, n), dtype=torch.uint8, device="cuda")
    lvq.loopvq_lloyd_step(cfg, layer=layer, cb_set=cb_set, n_samples=n, src=d_src, stride_loop=strides[0],
                          stride_token=strides[1], stride_head=strides[2], weight=d_w, cb=d_cb, cb_norms=d_norm,
                          assign=assign, workspace=ws, cluster_weight=cw, distortion=dist)
    torch.cuda.synchronize()
    return assign[:n].cpu().numpy(), cw.cpu().numpy(), dist.cpu().numpy()


CASES = {
    # c=4, d=64: small-batch assignment path, padded rows
    "c4_d64": (4, 64, 2, 2999, 8, 1, 4, False, 0, 0),
    # c=4, d=128: staged bulk assignment path (n * Hkv >= 16384), several row chunks
    "c4_d128_bulk": (4, 128, 8, 2053, 0, 1, 4, False, 0, 0),
    # c=8, d=128, per-loop-group codebooks: set (layer 1, loop group 1) of 2 x 2
    "c8_d128_sets": (8, 128, 2, 3001, 16, 2, 8, True, 1, 1),
}
# other loop-group sizes (G in the last field), staged bulk assignment path
CASES_G = {
    "c8_g2_bulk": (8, 128, 4, 4111, 0, 1, 4, True, 0, 1, 2),
    "c4_g8_bulk": (4, 128, 4, 4100, 8, 1, 8, False, 0, 0, 8),
}


@pytest.mark.parametrize("name", list(CASES) + list(CASES_G))
def test_lloyd_matches_oracle(name):
    if name in CASES:
        c, d, Hkv, n, pad, L, T, per_group, layer, cb_set = CASES[name]
        G = 4
    else:
        c, d, Hkv, n, pad, L, T, per_group, layer, cb_set, G = CASES_G[name]
    wl = _wl(c, d, Hkv, L, T, per_group, G)
    NG, G, K = wl.groups, wl.loop_group, wl.codewords
    cfg = lvq.make_config(wl)
    sc = gen.scales(wl)
    # sample planes [G][n][Hkv][d + pad]: loop steps jG..jG+G-1 of sequence 0, tokens 0..n-1
    src = np.zeros((G, n, Hkv, d + pad), np.uint16)
    for h in range(Hkv):
        src[:, :, h, :d] = gen.kv_tokens(wl, 0, layer, 0, h, 0, n, cb_set * G, cb_set * G + G, sc).transpose(1, 0, 2)
    strides = (n * Hkv * (d + pad), Hkv * (d + pad), d + pad)
    w = gen.sample_weights(wl, n)
    cb0 = gen.codebooks(wl, 0, sc)                                 # [L][Jcb][Hkv][NG][K][E]
    lay = lvq.loopvq_layout_query(cfg, 1, 1)
    d_cb = H.dev_u16(cb0)
    d_norm = torch.empty(lay.norms_elems, dtype=torch.float32, device="cuda")
    lvq.loopvq_codebook_prepare(cfg, d_cb, torch.empty_like(d_cb), d_norm)
    norms0 = d_norm.cpu().numpy().reshape(cb0.shape[:-1])
    d_src, d_w = H.dev_u16(src), H.dev_f32(w)
    x = {h: O.subvectors(H.f64(src[:, :, h, :d]), c) for h in {0, Hkv // 2, Hkv - 1}}   # [n][NG][E]
    cur = cb0[layer, cb_set].copy()                                # [Hkv][NG][K][E] bits
    excused = 0
    for it in range(2):
        _say(f"lloyd {name}: iteration {it}, n={n}")
        a_gpu, cw_gpu, dist_gpu = run_step(cfg, wl, d_src, strides, n, d_w, d_cb, d_norm, layer, cb_set)
        cb_now = d_cb.cpu().numpy().view(np.uint16).reshape(cb0.shape)
        # the oracle checks every group of a few kv-heads (first and last included)
        heads = sorted({0, Hkv // 2, Hkv - 1}) if it == 0 else [Hkv - 1]
        for h in heads:
            for g in range(NG):
                C = H.f64(cur[h, g])
                a, mean, dist = O.lloyd_step(x[h][:, g], w[:, h, g].astype(np.float64), C, to_bf16=False)
                assert np.array_equal(a_gpu[:, h, g], a), (it, h, g)
                excused += check_codewords(cb_now[layer, cb_set, h, g], mean, C)
                wsum = np.bincount(a, weights=w[:, h, g].astype(np.float64), minlength=K)
                assert np.array_equal(cw_gpu[h, g], wsum), (it, h, g)
                empty = wsum == 0
                assert np.array_equal(cb_now[layer, cb_set, h, g][empty], cur[h, g][empty])
                assert abs(dist_gpu[h, g] - dist) <= DIST_REL * abs(dist), (it, h, g, dist_gpu[h, g], dist)
        # norms: what codebook_prepare writes for the updated codebooks
        ref = torch.empty_like(d_norm)
        lvq.loopvq_codebook_prepare(cfg, d_cb, torch.empty_like(d_cb), ref)
        torch.cuda.synchronize()
        assert torch.equal(d_norm, ref)
        # every other set untouched
        others = np.ones(cb0.shape[:2], bool)
        others[layer, cb_set] = False
        assert np.array_equal(cb_now[others], cb0[others])
        assert np.array_equal(d_norm.cpu().numpy().reshape(norms0.shape)[others], norms0[others])
        cur = cb_now[layer, cb_set].copy()
    _say(f"  near-midpoint codeword elements excused: {excused}")


def test_lloyd_without_samples_keeps_the_codebook():
    wl = _wl(4, 128, 2)
    cfg = lvq.make_config(wl)
    cb0 = gen.codebooks(wl, 0, gen.scales(wl))
    lay = lvq.loopvq_layout_query(cfg, 1, 1)
    d_cb = H.dev_u16(cb0)
    d_norm = torch.empty(lay.norms_elems, dtype=torch.float32, device="cuda")
    lvq.loopvq_codebook_prepare(cfg, d_cb, torch.empty_like(d_cb), d_norm)
    want_norm = d_norm.clone()
    d_norm.fill_(-1.0)
    src = torch.zeros(64, dtype=torch.int16, device="cuda")
    d_w = torch.zeros(16, dtype=torch.float32, device="cuda")
    a, cw, dist = run_step(cfg, wl, src, (0, 0, 0), 0, d_w, d_cb, d_norm, 0, 0)
    assert np.array_equal(d_cb.cpu().numpy().view(np.uint16).reshape(cb0.shape), cb0)
    assert torch.equal(d_norm, want_norm)
    assert (cw == 0).all() and (dist == 0).all()


def test_full_size_lloyd_sampled():
    """65536 samples x 32 kv-heads x 32 groups (the deep-recurrence encode shape), keys of
    (layer 1, loop group 5); four (kv-head, group) pairs checked in full against the oracle."""
    wl = W.DEEP_8K
    layer, j = 1, 5
    n, Hkv, d, G, NG, K = wl.encode_tokens, wl.kv_heads, wl.head_dim, wl.loop_group, wl.groups, wl.codewords
    per_seq = n // wl.batch
    cfg = lvq.make_config(wl)
    sc = gen.scales(wl)
    dg = DeviceGen(wl)
    src = torch.empty((G, n, Hkv, d), dtype=torch.int16, device="cuda")
    for b in range(wl.batch):
        dg.kv(src[:, b * per_seq:], kind=0, layer=layer, b0=b, nb=1, h0=0, nh=Hkv, n0=wl.prefix, nn=per_seq,
              t0=j * G, nt=G, s_loop=n * Hkv * d, s_b=0, s_h=d, s_n=Hkv * d)
    w = gen.sample_weights(wl, n, salt=3)
    cb0 = gen.codebooks(wl, 0, sc, layers=[layer])
    jc = j if wl.codebook_per_loop_group else 0
    lay = lvq.loopvq_layout_query(cfg, 1, 1)
    d_cb = H.dev_u16(cb0)
    d_norm = torch.empty(lay.norms_elems, dtype=torch.float32, device="cuda")
    lvq.loopvq_codebook_prepare(cfg, d_cb, torch.empty_like(d_cb), d_norm)
    _say(f"full-size lloyd: {n} samples x {Hkv} heads x {NG} groups")
    a_gpu, cw_gpu, dist_gpu = run_step(cfg, wl, src, (n * Hkv * d, Hkv * d, d), n, H.dev_f32(w), d_cb, d_norm, layer,
                                       jc)
    cb_now = d_cb.cpu().numpy().view(np.uint16).reshape(cb0.shape)
    assert ((a_gpu >= 0) & (a_gpu < K)).all()
    assert (dist_gpu > 0).all()
    excused = 0
    for h, g in [(0, 0), (7, 13), (20, 31), (Hkv - 1, 5)]:
        planes = src[:, :, h].cpu().numpy().view(np.uint16)             # [G][n][d]
        for r in (0, per_seq + 17, n - 1):
            b, u = divmod(r, per_seq)
            host = gen.kv_tokens(wl, 0, layer, b, h, wl.prefix + u, wl.prefix + u + 1, j * G, j * G + G, sc)[0]
            assert np.array_equal(planes[:, r], host), "device generator differs from host generator"
        xg = O.subvectors(H.f64(planes), wl.chans)[:, g]
        C = H.codebooks_f64(cb0, layer, jc, h)[g]
        a, mean, dist = O.lloyd_step(xg, w[:, h, g].astype(np.float64), C, to_bf16=False)
        assert np.array_equal(a_gpu[:, h, g], a), (h, g)
        excused += check_codewords(cb_now[layer, jc, h, g], mean, C)
        assert np.array_equal(cw_gpu[h, g], np.bincount(a, weights=w[:, h, g].astype(np.float64), minlength=K))
        assert abs(dist_gpu[h, g] - dist) <= DIST_REL * abs(dist), (h, g)
    _say(f"  near-midpoint codeword elements excused: {excused}")


def test_update_after_poolless_encode_equals_step():
    """loopvq_encode without a pool (assignment only) followed by loopvq_lloyd_update gives what
    loopvq_lloyd_step gives, bit for bit."""
    wl = _wl(4, 128, 4)
    n = 4500                                   # n * Hkv >= 16384: the staged assignment path
    cfg = lvq.make_config(wl)
    sc = gen.scales(wl)
    src = np.zeros((4, n, 4, 128), np.uint16)
    for h in range(4):
        src[:, :, h] = gen.kv_tokens(wl, 1, 0, 0, h, 0, n, 0, 4, sc).transpose(1, 0, 2)
    d_src, d_w = H.dev_u16(src), H.dev_f32(gen.sample_weights(wl, n, salt=5))
    strides = dict(stride_loop=n * 4 * 128, stride_token=4 * 128, stride_head=128)
    cb0 = gen.codebooks(wl, 1, sc)
    lay = lvq.loopvq_layout_query(cfg, 1, 1)
    outs = []
    for split in (False, True):
        d_cb = H.dev_u16(cb0)
        d_norm = torch.empty(lay.norms_elems, dtype=torch.float32, device="cuda")
        lvq.loopvq_codebook_prepare(cfg, d_cb, torch.empty_like(d_cb), d_norm)
        assign = torch.full((n, 4, wl.groups), -1, dtype=torch.int32, device="cuda")
        ws = torch.empty(lvq.loopvq_lloyd_workspace(cfg, n), dtype=torch.uint8, device="cuda")
        kw = dict(layer=0, cb_set=0, n_samples=n, src=d_src, weight=d_w, cb=d_cb, cb_norms=d_norm, assign=assign,
                  workspace=ws, **strides)
        _say(f"lloyd split={split}")
        if split:
            lvq.loopvq_encode(cfg, layer=0, loop_group=0, kind=1, n_tokens=n, src=d_src, seq_id=None, vq_pos=None,
                              block_table=None, batch=1, max_pages_per_seq=1, num_pages=1, cb=d_cb, cb_norms=d_norm,
                              pool=None, out_idx=assign, **strides)
            lvq.loopvq_lloyd_update(cfg, **kw)
        else:
            lvq.loopvq_lloyd_step(cfg, **kw)
        torch.cuda.synchronize()
        outs.append((assign.cpu().numpy(), d_cb.cpu().numpy(), d_norm.cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    assert not np.array_equal(outs[0][1], cb0.view(np.int16)), "the step changed the codebook"
