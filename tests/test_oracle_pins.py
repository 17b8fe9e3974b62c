"""Pins of the CPU oracle against things other than itself.

Every check here compares the oracle with a library routine, brute force, a
closed form, a hand-worked example under tests/golden/, or an identity that a
dropped term, a wrong sign, a wrong index or a transposed operand would break.
"""
import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.spatial.distance import cdist
from scipy.special import softmax

from oracle import loopvq_oracle as O
from synth import gen, workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# Encode: brute force vs scipy vs an exhaustive loop; hand example
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(6))
def test_encode_matches_cdist_and_exhaustive_loop(seed):
    r = _rng(seed)
    K, E, n = int(r.integers(1, 40)), int(r.integers(1, 9)), 50
    C = np.round(r.normal(size=(K, E)) * 4) / 4          # coarse grid -> real ties
    if K > 3:
        C[K - 1] = C[1]                                   # duplicated codeword
    x = np.round(r.normal(size=(n, E)) * 4) / 4
    idx, d1, d2 = O.encode(x, C, chunk=7)
    ref = cdist(x, C, "sqeuclidean")
    assert np.array_equal(idx, ref.argmin(axis=1))       # argmin: first occurrence
    for i in range(n):
        best_k, best_d = 0, None
        for k in range(K):
            dk = sum((float(x[i, e]) - float(C[k, e])) ** 2 for e in range(E))
            if best_d is None or dk < best_d:
                best_k, best_d = k, dk
        assert idx[i] == best_k
        assert d1[i] == pytest.approx(best_d, abs=1e-12)
        others = sorted(ref[i, k] for k in range(K) if k != best_k)
        if others:
            assert d2[i] == pytest.approx(others[0], abs=1e-12)


def test_encode_duplicated_codeword_picks_lowest():
    C = np.array([[1.0, 2.0], [3.0, 4.0], [1.0, 2.0], [3.0, 4.0]])
    idx, d1, d2 = O.encode(np.array([[1.0, 2.0], [3.0, 4.1]]), C)
    assert list(idx) == [0, 1]
    assert d1[0] == 0.0 and d2[0] == 0.0
    assert O.near_tie(d1, d2).tolist() == [True, True]


def test_encode_hand_example():
    g = json.load(open(os.path.join(GOLD, "hand_encode.json")))
    C = np.array(g["codebook"], dtype=np.float64)
    for case in g["cases"]:
        x = np.array([case["x"]], dtype=np.float64)
        assert np.array_equal(O.sq_dists(x, C)[0], np.array(case["dist"]))
        idx, d1, _ = O.encode(x, C)
        assert idx[0] == case["idx"]
        assert d1[0] == min(case["dist"])


def test_encode_single_codeword():
    idx, d1, d2 = O.encode(_rng(1).normal(size=(9, 5)), np.zeros((1, 5)))
    assert (idx == 0).all() and np.isinf(d2).all()


# ---------------------------------------------------------------------------
# Bits per element (closed form) and page sizes
# ---------------------------------------------------------------------------
def test_bits_per_elem_closed_form():
    assert O.bits_per_elem(2, 1, 2) == 1.0                 # K=4, c=1, G=2
    expect = {"tiny_d64_n512": 0.5, "layer16h_d128_b32_n4k": 0.5, "stack24x4_h16_d128_b64_n32k": 0.5,
              "stack24x4_c8_rot_b128_n16k": 0.25, "deep4x32_h32_d128_b16_n8k": 0.5}
    for wl in W.ALL:
        assert O.bits_per_elem(wl.index_bits, wl.chans, wl.loop_group) == expect[wl.name]
        assert np.log2(wl.codewords) / (wl.chans * wl.loop_group) == expect[wl.name]


@pytest.mark.parametrize("b,PT,NG", [(8, 64, 32), (8, 64, 16), (3, 16, 8), (9, 128, 4)])
def test_page_bytes_closed_form(b, PT, NG):
    lay = O.page_layout(PT, NG, b)
    # index bits of PT tokens x NG groups x 2 kinds, in bytes
    assert lay["page_bytes"] * 8 == 2 * PT * NG * b
    n = 3 * PT - 5
    r = _rng(b)
    ik = r.integers(0, 1 << b, (n, NG))
    iv = r.integers(0, 1 << b, (n, NG))
    pages = O.pack_sequence(ik, iv, PT, b)
    assert pages.shape == (3, lay["page_bytes"])


def test_config_checks():
    O.check_config(4, 4, 16, 16, 128, 4, 8)
    for bad in [dict(T=6, G=4), dict(d=130, c=4), dict(Hq=3, Hkv=2), dict(b=17), dict(b=0), dict(d=24, c=4)]:
        kw = dict(T=4, G=4, Hq=16, Hkv=16, d=128, c=4, b=8)
        kw.update(bad)
        with pytest.raises(ValueError):
            O.check_config(**kw)


# ---------------------------------------------------------------------------
# Packing: hand-worked bytes, independent big-integer formulation, round trips
# ---------------------------------------------------------------------------
def test_pack_tile_hand_examples():
    g = json.load(open(os.path.join(GOLD, "pack_tiles.json")))
    for case in g["cases"]:
        b, vals, want = case["b"], case["vals"], bytes.fromhex(case["bytes"])
        assert O.pack_tile(vals, b) == want
        assert O.unpack_tile(want, b) == vals
        assert O.pack_tiles(np.array([vals]), b).tobytes() == want
        assert O.unpack_tiles(np.frombuffer(want, dtype=np.uint8)[None], b)[0].tolist() == vals


@settings(max_examples=200, deadline=None)
@given(b=st.integers(1, 16), data=st.data())
def test_pack_roundtrip_and_bigint(b, data):
    vals = data.draw(st.lists(st.integers(0, (1 << b) - 1), min_size=16, max_size=16))
    packed = O.pack_tile(vals, b)
    as_int = sum(v << (e * b) for e, v in enumerate(vals))   # little-endian integer view
    assert packed == as_int.to_bytes(2 * b, "little")
    assert O.unpack_tile(packed, b) == vals
    assert O.unpack_tiles(O.pack_tiles(np.array([vals]), b), b)[0].tolist() == vals


def test_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.pack_tile([256] + [0] * 15, 8)
    with pytest.raises(ValueError):
        O.pack_tiles(np.full((1, 16), -1), 4)


@pytest.mark.parametrize("b,PT,NG,n", [(8, 64, 32, 201), (8, 64, 16, 64), (5, 16, 8, 33), (9, 32, 4, 1), (8, 64, 32, 0)])
def test_sequence_roundtrip_layout_and_padding(b, PT, NG, n):
    r = _rng(n + b)
    ik = r.integers(0, 1 << b, (n, NG))
    iv = r.integers(0, 1 << b, (n, NG))
    pages = O.pack_sequence(ik, iv, PT, b)
    k2, v2 = O.unpack_sequence(pages, n, NG, PT, b)
    assert np.array_equal(k2, ik) and np.array_equal(v2, iv)
    lay = O.page_layout(PT, NG, b)
    # location of one index, written out from the layout description
    for (u, g, kind) in [(0, 0, 0), (n - 1, NG - 1, 1), (n // 2, NG // 3, 0)] if n else []:
        page, w = divmod(u, PT)
        Q, i = divmod(w, 4)
        uq, rr = divmod(g, 4)
        tile_off = kind * lay["kind_bytes"] + (Q * (NG // 4) + uq) * lay["tile_bytes"]
        tile = pages[page, tile_off:tile_off + lay["tile_bytes"]].tobytes()
        e = 4 * i + rr
        as_int = int.from_bytes(tile, "little")
        want = (ik if kind == 0 else iv)[u, g]
        assert (as_int >> (e * b)) & ((1 << b) - 1) == want
    # padding tokens of the last page are zero bits
    if n % PT:
        k_pad, v_pad = O.unpack_sequence(pages, pages.shape[0] * PT, NG, PT, b)
        assert (k_pad[n:] == 0).all() and (v_pad[n:] == 0).all()


# ---------------------------------------------------------------------------
# Sub-vectors and dequantization
# ---------------------------------------------------------------------------
def test_subvector_order_written_out():
    G, n, d, c = 4, 3, 16, 4
    planes = np.arange(G * n * d, dtype=np.float64).reshape(G, n, d)
    x = O.subvectors(planes, c)
    for tok, g, tau, i in itertools.product(range(n), range(d // c), range(G), range(c)):
        assert x[tok, g, tau * c + i] == planes[tau, tok, g * c + i]


def test_generator_codebook_rows_are_subvectors_of_fresh_tokens():
    wl = W.TINY
    cb = gen.codebooks(wl, 0)                      # [L][Jcb][H][NG][K][E]
    tok = gen.codebook_tokens(wl, 0, 0, 0)         # [K][T][d]
    planes = gen.bf16_to_f64(tok[:, :wl.loop_group, :]).transpose(1, 0, 2)   # [G][K][d]
    x = O.subvectors(planes, wl.chans)             # [K][NG][E]
    assert np.array_equal(gen.bf16_to_f64(cb[0, 0, 0]), x.transpose(1, 0, 2))


def test_dequantize_inverts_exact_codebook_encode():
    r = _rng(3)
    G, n, d, c = 4, 40, 32, 4
    planes = r.normal(size=(G, n, d))
    x = O.subvectors(planes, c)
    NG = d // c
    # codebook per group = the data sub-vectors in a shuffled order, plus far fillers
    C = np.empty((NG, 64, c * G))
    for g in range(NG):
        C[g, :n] = x[r.permutation(n), g]
        C[g, n:] = 100 + r.normal(size=(64 - n, c * G))
    idx = np.stack([O.encode(x[:, g], C[g])[0] for g in range(NG)], axis=1)
    for tau in range(G):
        assert np.array_equal(O.dequantize(idx, C, tau, c), planes[tau])


# ---------------------------------------------------------------------------
# Attention: textbook softmax, exact codebook, special cases, invariants
# ---------------------------------------------------------------------------
def _plain_attention(q, keys, vals, scale):
    p = softmax(scale * (keys @ q))
    return p @ vals, np.log(np.exp(scale * (keys @ q)).sum())


def test_attention_matches_scipy_softmax():
    r = _rng(5)
    q, keys, vals = r.normal(size=16), r.normal(size=(37, 16)), r.normal(size=(37, 16))
    o, lse = O.attention(q, keys, vals, 0.25)
    o2, lse2 = _plain_attention(q, keys, vals, 0.25)
    assert np.allclose(o, o2, rtol=1e-13, atol=1e-14)
    assert lse == pytest.approx(lse2, rel=1e-13)


def _exact_codebook_case(b, seed, P=3, R=5, n_vq=20, d=16, c=4, G=4):
    """Cache whose vector-quantized rows are all codewords: VQ attention == plain bf16 attention."""
    r = _rng(seed)
    K = 1 << b
    NG = d // c
    tau = int(r.integers(0, G))
    planes = gen.bf16_to_f64(gen.to_bf16_bits(r.normal(size=(G, n_vq, d))))
    x = O.subvectors(planes, c)
    C = np.empty((NG, K, c * G))
    slot = r.permutation(K)[:n_vq]
    for g in range(NG):
        C[g] = gen.bf16_to_f64(gen.to_bf16_bits(r.normal(size=(K, c * G)) * 50 + 200))
        C[g, slot] = x[:, g]
    idx_k = np.stack([O.encode(x[:, g], C[g])[0] for g in range(NG)], axis=1)
    # pack and unpack through the page format on the way
    pages = O.pack_sequence(idx_k, idx_k, 8, b)
    idx_k2, _ = O.unpack_sequence(pages, n_vq, NG, 8, b)
    kp, vp = r.normal(size=(P, d)), r.normal(size=(P, d))
    kr, vr = r.normal(size=(R, d)), r.normal(size=(R, d))
    q = r.normal(size=d)
    vals_tau = planes[tau] * 0.5 - 1.0
    # values: use a second exact codebook built the same way
    xv = O.subvectors(planes * 0.5 - 1.0, c)
    Cv = C.copy()
    for g in range(NG):
        Cv[g, slot] = xv[:, g]
    idx_v = np.stack([O.encode(xv[:, g], Cv[g])[0] for g in range(NG)], axis=1)
    return dict(q=q, kp=kp, vp=vp, kr=kr, vr=vr, planes=planes, vals_tau=vals_tau, tau=tau,
                idx_k=idx_k2, idx_v=idx_v, C=C, Cv=Cv, c=c)


@pytest.mark.parametrize("b,seed", [(8, 0), (8, 1), (9, 2), (6, 3)])
def test_exact_codebook_reproduces_plain_attention(b, seed):
    e = _exact_codebook_case(b, seed)
    assert np.array_equal(O.dequantize(e["idx_k"], e["C"], e["tau"], e["c"]), e["planes"][e["tau"]])
    o, lse = O.decode_query(e["q"], e["kp"], e["vp"], e["idx_k"], e["idx_v"], e["C"], e["Cv"],
                            e["kr"], e["vr"], e["tau"], e["c"], 0.3)
    keys = np.concatenate([e["kp"], e["planes"][e["tau"]], e["kr"]])
    vals = np.concatenate([e["vp"], e["vals_tau"], e["vr"]])
    o2, lse2 = _plain_attention(e["q"], keys, vals, 0.3)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-12)
    assert lse == pytest.approx(lse2, rel=1e-12)


def test_context_split():
    assert O.split_context(512, 8, 64) == (8, 440, 64)
    assert O.split_context(72, 8, 64) == (8, 0, 64)
    assert O.split_context(73, 8, 64) == (8, 1, 64)
    assert O.split_context(5, 8, 64) == (5, 0, 0)
    assert O.split_context(1, 8, 64) == (1, 0, 0)
    assert O.split_context(40, 8, 64) == (8, 0, 32)


def test_no_vq_tokens_is_plain_attention():
    r = _rng(7)
    d = 8
    kp, vp, kr, vr = r.normal(size=(8, d)), r.normal(size=(8, d)), r.normal(size=(20, d)), r.normal(size=(20, d))
    q = r.normal(size=d)
    empty = np.zeros((0, 2), dtype=np.int64)
    C = r.normal(size=(2, 4, 16))
    o, _ = O.decode_query(q, kp, vp, empty, empty, C, C, kr, vr, 1, 4, 0.5)
    o2, _ = _plain_attention(q, np.concatenate([kp, kr]), np.concatenate([vp, vr]), 0.5)
    assert np.allclose(o, o2, rtol=1e-13, atol=1e-14)


def test_zero_query_gives_mean_of_values():
    r = _rng(8)
    d, c, G, NG, K = 16, 4, 4, 4, 16
    C, Cv = r.normal(size=(NG, K, c * G)), r.normal(size=(NG, K, c * G))
    ik, iv = r.integers(0, K, (30, NG)), r.integers(0, K, (30, NG))
    kp, vp, kr, vr = (r.normal(size=(8, d)), r.normal(size=(8, d)),
                      r.normal(size=(11, d)), r.normal(size=(11, d)))
    o, lse = O.decode_query(np.zeros(d), kp, vp, ik, iv, C, Cv, kr, vr, 2, c, 0.1)
    vals = np.concatenate([vp, O.dequantize(iv, Cv, 2, c), vr])
    assert np.allclose(o, vals.mean(axis=0), rtol=1e-13, atol=1e-14)
    assert lse == pytest.approx(np.log(49), rel=1e-14)


def test_single_token_gives_its_value_row():
    r = _rng(9)
    d = 8
    empty = np.zeros((0, 2), dtype=np.int64)
    C = r.normal(size=(2, 4, 16))
    kp, vp = r.normal(size=(1, d)), r.normal(size=(1, d))
    o, lse = O.decode_query(r.normal(size=d), kp, vp, empty, empty, C, C,
                            np.zeros((0, d)), np.zeros((0, d)), 0, 4, 1.0)
    assert np.array_equal(o, vp[0])


def test_rotation_identity_and_orthogonal_invariance():
    r = _rng(10)
    d = 32
    q, keys, vals = r.normal(size=d), r.normal(size=(25, d)), r.normal(size=(25, d))
    o0, l0 = O.attention(q, keys, vals, 0.2)
    o1, l1 = O.attention(q, keys, vals, 0.2, rot=np.eye(d))
    assert np.array_equal(o0, o1) and l0 == l1
    Qm, Rm = np.linalg.qr(r.normal(size=(d, d)))
    Qm = Qm * np.sign(np.diag(Rm))                  # Haar-distributed orthogonal matrix
    o2, l2 = O.attention(q, keys @ Qm, vals, 0.2, rot=Qm)   # keys stored as Q^T k (row form k Q)
    assert np.allclose(o2, o0, rtol=1e-12, atol=1e-13)
    assert l2 == pytest.approx(l0, rel=1e-12)
    # a wrongly transposed rotation breaks it
    o3, _ = O.attention(q, keys @ Qm, vals, 0.2, rot=Qm.T)
    assert not np.allclose(o3, o0, rtol=1e-6)


def test_generator_rotation_is_orthogonal_and_matches_dense_form():
    wl = W.QUARTER_16K.with_(head_dim=16, chans=4, layers=1, kv_heads=1, batch=1, context=10)
    R = gen.rotation_matrix_f32(wl).astype(np.float64)
    assert np.allclose(R @ R.T, np.eye(16), atol=1e-6)
    # keys generated rotated equal R^T applied to the unrotated keys (up to bf16 rounding)
    k_rot = gen.bf16_to_f64(gen.kv_tokens(wl, 0, 0, 0, 0, 0, 10, 0, 4))
    k_raw = gen.bf16_to_f64(gen.kv_tokens(wl.with_(rotate_keys=False), 0, 0, 0, 0, 0, 10, 0, 4))
    want = k_raw @ R                                   # row form of R^T k
    assert np.allclose(k_rot, want, rtol=2e-2, atol=2e-2 * np.abs(want).max())


@pytest.mark.parametrize("seed", range(3))
def test_permutation_and_window_order_invariance(seed):
    r = _rng(20 + seed)
    d, c, G, NG, K, n = 16, 4, 4, 4, 32, 50
    C, Cv = r.normal(size=(NG, K, c * G)), r.normal(size=(NG, K, c * G))
    ik, iv = r.integers(0, K, (n, NG)), r.integers(0, K, (n, NG))
    kp, vp, kr, vr = (r.normal(size=(8, d)), r.normal(size=(8, d)),
                      r.normal(size=(13, d)), r.normal(size=(13, d)))
    q = r.normal(size=d)
    o, lse = O.decode_query(q, kp, vp, ik, iv, C, Cv, kr, vr, 3, c, 0.3)
    p, w = r.permutation(n), r.permutation(13)
    o2, lse2 = O.decode_query(q, kp, vp, ik[p], iv[p], C, Cv, kr[w], vr[w], 3, c, 0.3)
    assert np.allclose(o2, o, rtol=1e-14, atol=1e-14)
    assert lse2 == pytest.approx(lse, rel=1e-14)
    # permuting key indices without their value indices is a different cache
    o3, _ = O.decode_query(q, kp, vp, ik[p], iv, C, Cv, kr, vr, 3, c, 0.3)
    assert not np.allclose(o3, o, rtol=1e-6)


def test_lut_score_equals_dequantized_dot_product():
    """Score of a VQ token as a sum over groups of (q-slice . codeword-slice) lookups."""
    r = _rng(30)
    d, c, G, NG, K, n, tau = 32, 4, 4, 8, 64, 40, 2
    C = r.normal(size=(NG, K, c * G))
    idx = r.integers(0, K, (n, NG))
    q = r.normal(size=d)
    lut = np.array([[q[g * c:(g + 1) * c] @ C[g, k, tau * c:(tau + 1) * c] for g in range(NG)]
                    for k in range(K)])                 # [K][NG]
    s_lut = np.array([sum(lut[idx[m, g], g] for g in range(NG)) for m in range(n)])
    s_deq = O.dequantize(idx, C, tau, c) @ q
    assert np.allclose(s_lut, s_deq, rtol=1e-12, atol=1e-12)


def test_indices_in_range_after_encode():
    r = _rng(31)
    C = r.normal(size=(16, 8))
    idx, _, _ = O.encode(r.normal(size=(100, 8)), C)
    assert idx.min() >= 0 and idx.max() < 16


def test_near_tie_rule():
    d1 = np.array([1.0, 1.0, 0.0, 2.0])
    d2 = np.array([1.0 + 5e-7, 1.0 + 2e-6, 0.0, 3.0])
    assert O.near_tie(d1, d2).tolist() == [True, False, True, False]


# ---------------------------------------------------------------------------
# Extend (chunked prefill) over the cache
# ---------------------------------------------------------------------------
def _extend_case(seed, n_vq=23, P=3, R=5, M=9, d=16, c=4, K=16):
    r = _rng(seed)
    NG = d // c
    C, Cv = r.normal(size=(NG, K, c * 4)), r.normal(size=(NG, K, c * 4))
    ik, iv = r.integers(0, K, (n_vq, NG)), r.integers(0, K, (n_vq, NG))
    win = [r.normal(size=(n, d)) for n in (P, P, R, R)]
    kc, vc = r.normal(size=(M, d)), r.normal(size=(M, d))
    q = r.normal(size=(M, d))
    return dict(q=q, kp=win[0], vp=win[1], kr=win[2], vr=win[3], ik=ik, iv=iv, C=C, Cv=Cv, kc=kc, vc=vc, c=c)


def test_extend_matches_masked_softmax_over_the_explicit_cache():
    """Row i of the chunk == softmax over [all cache rows, chunk rows 0..i] written as one masked
    score matrix (scipy softmax over a dense mask, an independent formulation)."""
    e = _extend_case(11)
    tau, scale = 3, 0.35
    o, lse = O.extend_attention(e["q"], e["kp"], e["vp"], e["ik"], e["iv"], e["C"], e["Cv"], e["kr"], e["vr"],
                                e["kc"], e["vc"], tau, e["c"], scale)
    # cache keys written out directly from the codebooks (no dequantize helper)
    NG = e["C"].shape[0]
    kq = np.concatenate([e["C"][g][e["ik"][:, g], tau * 4:tau * 4 + 4] for g in range(NG)], axis=1)
    vq = np.concatenate([e["Cv"][g][e["iv"][:, g], tau * 4:tau * 4 + 4] for g in range(NG)], axis=1)
    keys = np.concatenate([e["kp"], kq, e["kr"], e["kc"]])
    vals = np.concatenate([e["vp"], vq, e["vr"], e["vc"]])
    n_cache = len(keys) - len(e["kc"])
    M = len(e["q"])
    mask = np.zeros((M, len(keys)), dtype=bool)
    mask[:, :n_cache] = True
    for i in range(M):
        mask[i, n_cache:n_cache + i + 1] = True
    S = np.where(mask, scale * (e["q"] @ keys.T), -np.inf)
    Pm = softmax(S, axis=1)
    assert np.allclose(o, Pm @ vals, rtol=1e-12, atol=1e-13)
    from scipy.special import logsumexp
    assert np.allclose(lse, logsumexp(S, axis=1), rtol=1e-12)


def test_extend_is_causal_inside_the_chunk():
    e = _extend_case(12)
    o, _ = O.extend_attention(e["q"], e["kp"], e["vp"], e["ik"], e["iv"], e["C"], e["Cv"], e["kr"], e["vr"],
                              e["kc"], e["vc"], 1, e["c"], 0.3)
    kc2, vc2 = e["kc"].copy(), e["vc"].copy()
    kc2[5:] += 3.0
    vc2[5:] -= 7.0
    o2, _ = O.extend_attention(e["q"], e["kp"], e["vp"], e["ik"], e["iv"], e["C"], e["Cv"], e["kr"], e["vr"],
                               kc2, vc2, 1, e["c"], 0.3)
    assert np.array_equal(o[:5], o2[:5])
    assert not np.allclose(o[5:], o2[5:])


def test_extend_closed_forms():
    e = _extend_case(13, n_vq=0, P=0, R=0)
    empty = np.zeros((0, 4), dtype=np.int64)
    d = e["q"].shape[1]
    none = np.zeros((0, d))
    # empty cache: the first chunk row sees only itself
    o, lse = O.extend_attention(e["q"], none, none, empty, empty, e["C"], e["Cv"], none, none, e["kc"], e["vc"], 0,
                                e["c"], 0.5)
    assert np.array_equal(o[0], e["vc"][0])
    assert lse[0] == pytest.approx(0.5 * e["q"][0] @ e["kc"][0], rel=1e-14)
    # a zero query averages every visible value row
    f = _extend_case(14)
    q0 = np.zeros_like(f["q"])
    o, lse = O.extend_attention(q0, f["kp"], f["vp"], f["ik"], f["iv"], f["C"], f["Cv"], f["kr"], f["vr"],
                                f["kc"], f["vc"], 2, f["c"], 0.2)
    base = np.concatenate([f["vp"], O.dequantize(f["iv"], f["Cv"], 2, f["c"]), f["vr"]])
    for i in range(len(q0)):
        vis = np.concatenate([base, f["vc"][:i + 1]])
        assert np.allclose(o[i], vis.mean(axis=0), rtol=1e-13, atol=1e-14)
        assert lse[i] == pytest.approx(np.log(len(vis)), rel=1e-14)


# ---------------------------------------------------------------------------
# Weighted Lloyd iteration (codebook learning)
# ---------------------------------------------------------------------------
def test_round_to_bf16_matches_the_bit_level_rounding():
    r = _rng(30)
    v = np.concatenate([r.normal(size=2000) * 10.0 ** r.integers(-8, 8, 2000), [1.0, 1.00390625, 1.01171875, -3.5]])
    # bit level: fp64 -> fp32 is exact for these (they are made exact in fp32 first), then the
    # bf16 round-half-even on the fp32 bits
    v32 = v.astype(np.float32).astype(np.float64)
    u = v32.astype(np.float32).view(np.uint32).astype(np.uint64)
    bits = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint32)
    ref = (bits << np.uint32(16)).view(np.float32).astype(np.float64)
    assert np.array_equal(O.round_to_bf16(v32), ref)
    # ties go to the even significand: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7
    assert O.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert O.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def _all_finite_bf16():
    """Every finite non-negative bf16 value, in increasing order, from its bit patterns (an fp32
    whose low 16 bits are zero is exactly one bf16)."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << np.uint32(16)
    return bits, bits.view(np.float32).astype(np.float64)


def test_round_to_bf16_over_the_whole_format():
    """Brute force over all 32,640 finite non-negative bf16 values (subnormals included): each
    is kept, each gap's midpoint goes to the neighbour with the even pattern, and values just
    inside a gap go to the nearer end; past the largest finite value the result overflows to
    infinity exactly from the rounding threshold on.  The sign is symmetric."""
    bits, vals = _all_finite_bf16()
    a, b = vals[:-1], vals[1:]
    mid = (a + b) / 2.0                              # exact in fp64
    eps = (b - a) * 2.0 ** -20
    assert np.array_equal(O.round_to_bf16(vals), vals)
    assert np.array_equal(O.round_to_bf16(-vals), -vals)
    assert np.array_equal(O.round_to_bf16(mid - eps), a)
    assert np.array_equal(O.round_to_bf16(mid + eps), b)
    even_lo = ((bits[:-1] >> np.uint32(16)) & np.uint32(1)) == 0
    assert np.array_equal(O.round_to_bf16(mid), np.where(even_lo, a, b))
    assert np.array_equal(O.round_to_bf16(-mid), -np.where(even_lo, a, b))
    top = vals[-1]                                   # largest finite bf16, pattern 0x7F7F
    assert bits[-1] == 0x7F7F << 16 and top == O.BF16_MAX
    step = 2.0 ** (127 - 7)
    thr = top + step / 2                             # halfway to 2^128: rounds up, to even
    assert O.round_to_bf16(np.array([thr - step * 2.0 ** -20]))[0] == top
    assert O.round_to_bf16(np.array([thr, 1e39, 1e300]))[0] == np.inf
    assert np.all(np.isinf(O.round_to_bf16(np.array([thr, 1e39, 1e300]))))
    assert O.round_to_bf16(np.array([-thr]))[0] == -np.inf
    # far below the smallest subnormal 2^-133: zero; half of it ties to zero (even)
    assert np.array_equal(O.round_to_bf16(np.array([1e-300, 2.0 ** -134, 2.0 ** -134 * 1.0000001])),
                          np.array([0.0, 0.0, 2.0 ** -133]))


def test_pool_offset_is_the_row_major_pool_index():
    """pool_offset against numpy's own row-major indexing of [L][J][Hkv][num_pages][page_bytes]."""
    L, J, Hkv, num_pages, page_bytes = 3, 2, 5, 7, 16
    pool = np.arange(L * J * Hkv * num_pages * page_bytes).reshape(L, J, Hkv, num_pages, page_bytes)
    for l, j, h, pg in itertools.product(range(L), range(J), range(Hkv), range(num_pages)):
        assert O.pool_offset(l, j, h, pg, J, Hkv, num_pages, page_bytes) == pool[l, j, h, pg, 0]
    # a transposed pair of indices (kv-head and loop group swapped) is caught
    assert O.pool_offset(0, 1, 0, 0, J, Hkv, num_pages, page_bytes) != O.pool_offset(0, 0, 1, 0, J, Hkv, num_pages,
                                                                                       page_bytes)


def test_empty_context_is_zero_output_and_minus_infinite_lse():
    """N = 0: an empty softmax (sum of no terms); N < 0 is not a context."""
    d = 8
    z = np.zeros((0, d))
    cb = [np.zeros((4, 4))] * (d // 4)
    o, lse = O.decode_query(np.ones(d), z, z, np.zeros((0, d // 4), int), np.zeros((0, d // 4), int), cb, cb,
                            z, z, 0, 4, 1.0)
    assert np.array_equal(o, np.zeros(d)) and lse == -np.inf
    assert O.split_context(0, 8, 64) == (0, 0, 0)
    with pytest.raises(ValueError):
        O.split_context(-1, 8, 64)
    # one token more: its value row, lse = its score (the N = 1 closed form still holds)
    k1, v1 = np.ones((1, d)), np.arange(d, dtype=float)[None]
    o, lse = O.decode_query(np.ones(d), k1, v1, np.zeros((0, d // 4), int), np.zeros((0, d // 4), int), cb, cb,
                            z, z, 0, 4, 0.5)
    assert np.array_equal(o, v1[0]) and lse == pytest.approx(0.5 * d, rel=1e-15)


def test_lloyd_hand_example():
    x = np.array([[0.0], [1.0], [10.0], [11.0]])
    w = np.array([1.0, 3.0, 1.0, 1.0])
    C = np.array([[0.0], [10.0]])
    a, C1, dist = O.lloyd_step(x, w, C)
    assert list(a) == [0, 0, 1, 1]
    assert np.array_equal(C1, np.array([[0.75], [10.5]]))
    assert dist == pytest.approx(3.0 + 1.0)


def test_lloyd_single_codeword_is_the_weighted_mean():
    r = _rng(31)
    x, w = r.normal(size=(500, 16)), r.uniform(0.1, 3.0, 500)
    _, C1, _ = O.lloyd_step(x, w, np.zeros((1, 16)), to_bf16=False)
    assert np.allclose(C1[0], np.average(x, axis=0, weights=w), rtol=1e-13, atol=1e-15)


def test_lloyd_matches_sklearn_weighted_kmeans_iteration():
    from sklearn.cluster import KMeans
    r = _rng(32)
    K, E = 12, 16
    centers = r.normal(size=(K, E)) * 4
    x = np.concatenate([centers[k] + r.normal(size=(40, E)) for k in range(K)])
    w = r.uniform(0.2, 2.0, len(x))
    C0 = centers + r.normal(size=(K, E)) * 0.5
    _, C1, _ = O.lloyd_step(x, w, C0, to_bf16=False)
    km = KMeans(n_clusters=K, init=C0, n_init=1, max_iter=1, algorithm="lloyd", tol=0.0).fit(x, sample_weight=w)
    assert np.allclose(C1, km.cluster_centers_, rtol=1e-10, atol=1e-12)


def test_lloyd_keeps_empty_codewords_and_decreases_the_objective():
    r = _rng(33)
    x, w = r.normal(size=(300, 8)), r.uniform(0.5, 1.5, 300)
    C = np.concatenate([r.normal(size=(6, 8)), np.full((1, 8), 1e3)])   # the far codeword gets nothing
    prev = np.inf
    for _ in range(6):
        a, C_new, dist = O.lloyd_step(x, w, C, to_bf16=False)
        assert not (a == 6).any() and np.array_equal(C_new[6], C[6])
        assert dist <= prev * (1 + 1e-12)
        prev, C = dist, C_new
