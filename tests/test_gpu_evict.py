"""GPU eviction (the token leaving the bf16 recent window, every layer / loop group / kind in one
launch) against the oracle's brute-force encode and page layout, byte for byte."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("lvq_harness")

import sub_bit_loop_loopvq_amd as lvq  # noqa: E402
from oracle import loopvq_oracle as O  # noqa: E402
from synth import gen  # noqa: E402
from synth.workloads import Workload  # noqa: E402


def _wl(c, d, per_group, G=4):
    return Workload(name=f"evict_c{c}_g{G}_d{d}_cb{int(per_group)}", layers=2, loops=8, loop_group=G, q_heads=4,
                    kv_heads=2, head_dim=d, chans=c, index_bits=8, batch=5, context=600, prefix=2, recent=8,
                    outlier_channels=4, codebook_per_loop_group=per_group, wid=7)


@pytest.mark.parametrize("c,d,per_group,G", [(4, 64, False, 4), (4, 128, True, 4), (8, 128, False, 4),
                                              (8, 128, True, 2), (4, 64, False, 8)])
def test_evict_matches_oracle(c, d, per_group, G):
    wl = _wl(c, d, per_group, G)
    L, T, G, J, B, Hkv, R, NG = wl.layers, wl.loops, wl.loop_group, wl.loop_groups, wl.batch, wl.kv_heads, \
        wl.recent, wl.groups
    Jcb = J if per_group else 1
    sc = gen.scales(wl)
    rng = np.random.default_rng(3)
    # rings [kind][L][T][B][Hkv][R][d]: slot s of sequence b holds token 100 + 7*b + s
    ring = np.zeros((2, L, T, B, Hkv, R, d), dtype=np.uint16)
    for kind in (0, 1):
        for l in range(L):
            for b in range(B):
                for h in range(Hkv):
                    tok = gen.kv_tokens(wl, kind, l, b, h, 100 + 7 * b, 100 + 7 * b + R, 0, T, sc)   # [R][T][d]
                    ring[kind, l, :, b, h] = tok.transpose(1, 0, 2)
    cbs = [gen.codebooks(wl, kind, sc) for kind in (0, 1)]                                 # [L][Jcb][H][NG][K][E]
    per_seq = 130
    paging = H.Paging([per_seq] * B, wl.page_tokens, seed=9)
    slot = rng.integers(0, R, size=B).astype(np.int32)
    vq = rng.integers(0, per_seq, size=B).astype(np.int32)
    slot[1] = R          # out of the ring: skipped
    vq[3] = -1           # not evicted: skipped
    cfg = lvq.make_config(wl)
    lay = lvq.loopvq_layout_query(cfg, B, paging.num_pages)
    d_cb, d_norm = [], []
    for kind in (0, 1):
        t = H.dev_u16(cbs[kind])
        n = torch.empty(lay.norms_elems, dtype=torch.float32, device="cuda")
        lvq.loopvq_codebook_prepare(cfg, t, torch.empty_like(t), n)
        d_cb.append(t)
        d_norm.append(n)
    pool = torch.zeros(lay.pool_bytes, dtype=torch.uint8, device="cuda")
    out_idx = torch.full((L, J, 2, B, Hkv, NG), -7, dtype=torch.int32, device="cuda")
    print(f"evict {wl.name}", flush=True)
    lvq.loopvq_evict(cfg, batch=B, max_pages_per_seq=paging.max_pages, num_pages=paging.num_pages,
                     k_ring=H.dev_u16(ring[0]), v_ring=H.dev_u16(ring[1]), ring_slot=H.dev_i32(slot),
                     vq_pos=H.dev_i32(vq), block_table=H.dev_i32(paging.table), cb_k=d_cb[0], cb_v=d_cb[1],
                     norms_k=d_norm[0], norms_v=d_norm[1], pool=pool, out_idx=out_idx)
    torch.cuda.synchronize()
    got_pool = pool.cpu().numpy().reshape(L, J, Hkv, paging.num_pages, lay.page_bytes)
    got_idx = out_idx.cpu().numpy()
    want_pool = np.zeros_like(got_pool)
    kind_bytes = lay.page_bytes // 2
    for l in range(L):
        for j in range(J):
            jc = j if per_group else 0
            for kind in (0, 1):
                for b in range(B):
                    if not (0 <= slot[b] < R) or vq[b] < 0:
                        continue
                    page = paging.table[b, vq[b] // wl.page_tokens]
                    w = vq[b] % wl.page_tokens
                    for h in range(Hkv):
                        planes = H.f64(ring[kind, l, j * G:(j + 1) * G, b, h, slot[b]])[:, None, :]   # [G][1][d]
                        x = O.subvectors(planes, c)[0]                                            # [NG][E]
                        C = H.codebooks_f64(cbs[kind], l, jc, h)
                        for g in range(NG):
                            k, _, _ = O.encode(x[g][None], C[g])
                            assert got_idx[l, j, kind, b, h, g] == k[0], (l, j, kind, b, h, g)
                            off = kind * kind_bytes + ((w // 4) * (NG // 4) + g // 4) * 16 + (w % 4) * 4 + g % 4
                            want_pool[l, j, h, page, off] = k[0]
    assert np.array_equal(got_pool, want_pool)
    assert Jcb in (1, J)


def test_full_size_evict_sampled():
    """The eviction launch of the 32K decode step at its full shape (24 layers x 1 loop group x 2
    kinds x 64 sequences x 16 kv-heads x 32 groups, the launch bench.py times in every step).  The
    rings stay zero except the leaving slot of three sampled sequences, which holds generator
    tokens; every index and every pool byte is checked: the sampled rows against the oracle's
    brute-force encode, the zero rows against the codeword of smallest norm (lowest index on ties),
    which is what the encode definition gives for x = 0."""
    from synth import workloads as W
    wl = W.STACK_32K
    L, T, G, J, B, Hkv, R, NG, d, c = (wl.layers, wl.loops, wl.loop_group, wl.loop_groups, wl.batch, wl.kv_heads,
                                       wl.recent, wl.groups, wl.head_dim, wl.chans)
    sc = gen.scales(wl)
    rng = np.random.default_rng(21)
    per_seq = 130
    paging = H.Paging([per_seq] * B, wl.page_tokens, seed=9)
    slot = rng.integers(0, R, size=B).astype(np.int32)
    vq = rng.integers(0, per_seq, size=B).astype(np.int32)
    sampled = [0, 29, B - 1]
    cfg = lvq.make_config(wl)
    lay = lvq.loopvq_layout_query(cfg, B, paging.num_pages)
    cbs = [gen.codebooks(wl, kind, sc) for kind in (0, 1)]                 # [L][1][H][NG][K][E]
    d_cb, d_norm = [], []
    for kind in (0, 1):
        t = H.dev_u16(cbs[kind])
        n = torch.empty(lay.norms_elems, dtype=torch.float32, device="cuda")
        lvq.loopvq_codebook_prepare(cfg, t, torch.empty_like(t), n)
        d_cb.append(t)
        d_norm.append(n)
    rings = [torch.zeros((L, T, B, Hkv, R, d), dtype=torch.int16, device="cuda") for _ in (0, 1)]
    rows = {}
    for kind in (0, 1):
        for l in range(L):
            for b in sampled:
                for h in range(Hkv):
                    tok = gen.kv_tokens(wl, kind, l, b, h, 5000 + b, 5001 + b, 0, T, sc)[0]   # [T][d]
                    rows[kind, l, b, h] = tok
                    rings[kind][l, :, b, h, slot[b]] = torch.from_numpy(tok.view(np.int16)).to("cuda")
    pool = torch.zeros(lay.pool_bytes, dtype=torch.uint8, device="cuda")
    out_idx = torch.full((L, J, 2, B, Hkv, NG), -7, dtype=torch.int32, device="cuda")
    print(f"full-size evict {wl.name}", flush=True)
    lvq.loopvq_evict(cfg, batch=B, max_pages_per_seq=paging.max_pages, num_pages=paging.num_pages,
                     k_ring=rings[0], v_ring=rings[1], ring_slot=H.dev_i32(slot), vq_pos=H.dev_i32(vq),
                     block_table=H.dev_i32(paging.table), cb_k=d_cb[0], cb_v=d_cb[1], norms_k=d_norm[0],
                     norms_v=d_norm[1], pool=pool, out_idx=out_idx)
    torch.cuda.synchronize()
    got_idx = out_idx.cpu().numpy()
    got_pool = pool.cpu().numpy().reshape(L, J, Hkv, paging.num_pages, lay.page_bytes)
    want_idx = np.empty_like(got_idx)
    for l in range(L):
        for kind in (0, 1):
            for h in range(Hkv):
                C = H.codebooks_f64(cbs[kind], l, 0, h)                      # [NG][K][E]
                zero_best = np.argmin((C * C).sum(-1), axis=1)              # first minimum = lowest index
                want_idx[l, 0, kind, :, h, :] = zero_best[None, :]
                for b in sampled:
                    x = O.subvectors(H.f64(rows[kind, l, b, h])[:, None, :], c)[0]    # [NG][E]
                    for g in range(NG):
                        want_idx[l, 0, kind, b, h, g] = O.encode(x[g][None], C[g])[0][0]
    assert np.array_equal(got_idx, want_idx)
    want_pool = np.zeros_like(got_pool)
    kind_bytes = lay.page_bytes // 2
    for b in range(B):
        page = paging.table[b, vq[b] // wl.page_tokens]
        w = vq[b] % wl.page_tokens
        for kind in (0, 1):
            for g in range(NG):
                off = kind * kind_bytes + ((w // 4) * (NG // 4) + g // 4) * 16 + (w % 4) * 4 + g % 4
                want_pool[:, 0, :, page, off] = want_idx[:, 0, kind, b, :, g]
    assert np.array_equal(got_pool, want_pool)
    print(f"  {L * 2 * B * Hkv * NG} indices and the pool checked", flush=True)
