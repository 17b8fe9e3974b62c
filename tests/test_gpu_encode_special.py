"""GPU encode on extreme bf16 values: every index must equal the oracle's brute force.

Rows and codewords mix exact zeros, bf16 subnormals (down to 2^-133), tiny normals (2^-120
scale), ordinary values and large values (2^56 scale: sums of squares up to about 2^125), with
exact hits (rows equal to a codeword) and a zero codeword.  The screen's fp32 arithmetic cannot
resolve anything below 2^-126 (subnormal products underflow), so rows of those scales must be
settled by the exact fp64 re-rank; the 2^56 rows put the relative error bound near the top of
the fp32 range.  Both the small-batch and the staged bulk paths run, at c=4 and c=8.  No
near-tie is excused.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("lvq_harness")

import sub_bit_loop_loopvq_amd as lvq  # noqa: E402
from oracle import loopvq_oracle as O  # noqa: E402
from synth import gen  # noqa: E402
from synth.workloads import Workload  # noqa: E402

SCALES = [0.0, 2.0 ** -133, 2.0 ** -120, 1.0, 2.0 ** 56]


def _bf16_exact(a):
    return gen.bf16_to_f64(gen.to_bf16_bits(a))


def _values(E: int, NG: int, n: int, seed: int):
    rng = np.random.default_rng(seed)
    # codewords: per group 51 of each nonzero scale family, plus a zero codeword
    C = np.zeros((NG, 256, E))
    for f, s in enumerate(SCALES[1:]):
        if s == 2.0 ** -133:
            v = rng.integers(-7, 8, size=(NG, 51, E)) * s       # subnormal multiples of 2^-133
        else:
            v = rng.standard_normal((NG, 51, E)) * s
        C[:, 1 + 51 * f:1 + 51 * (f + 1)] = v
    C[:, 205:] = rng.standard_normal((NG, 51, E)) * np.array([1.0, 2.0 ** 56])[rng.integers(0, 2, size=(NG, 51, 1))]
    C = _bf16_exact(C)
    # rows: families by row index; one row in 8 is an exact codeword hit
    fam = rng.integers(0, len(SCALES), size=(n, NG))
    x = np.zeros((n, NG, E))
    for f, s in enumerate(SCALES):
        sel = fam == f
        cnt = int(sel.sum())
        if s == 0.0:
            continue
        if s == 2.0 ** -133:
            x[sel] = rng.integers(-7, 8, size=(cnt, E)) * s
        else:
            x[sel] = rng.standard_normal((cnt, E)) * s
    hit = rng.random((n, NG)) < 0.125
    k = rng.integers(0, 256, size=(n, NG))
    gidx = np.broadcast_to(np.arange(NG)[None, :], (n, NG))
    x[hit] = C[gidx[hit], k[hit]]
    return _bf16_exact(x), C


@pytest.mark.parametrize("c,d,n", [(4, 64, 300), (4, 64, 16500), (8, 128, 260), (8, 128, 16450)])
def test_extreme_values_match_oracle(c, d, n):
    G, NG, E = 4, d // c, 4 * c
    B = 4
    wl = Workload(name=f"special_c{c}", layers=1, loops=G, loop_group=G, q_heads=1, kv_heads=1, head_dim=d,
                  chans=c, index_bits=8, batch=B, context=n + 72, wid=0)
    x, C = _values(E, NG, n, seed=3 + c + n)
    src = x.reshape(n, NG, G, c).transpose(2, 0, 1, 3).reshape(G, n, 1, d)
    src_bits = gen.to_bf16_bits(src)
    assert np.array_equal(gen.bf16_to_f64(src_bits), src)
    cb_bits = gen.to_bf16_bits(C)[None, None, None]
    per_seq = -(-n // B)
    seq = np.arange(n) // per_seq
    pos = np.arange(n) % per_seq
    paging = H.Paging([per_seq] * B, wl.page_tokens, seed=7)
    cfg = lvq.make_config(wl)
    lay = lvq.loopvq_layout_query(cfg, B, paging.num_pages)
    d_cb = H.dev_u16(cb_bits)
    d_norm = torch.empty(lay.norms_elems, dtype=torch.float32, device="cuda")
    lvq.loopvq_codebook_prepare(cfg, d_cb, torch.empty_like(d_cb), d_norm)
    pool = torch.zeros(lay.pool_bytes, dtype=torch.uint8, device="cuda")
    out_idx = torch.full((n, 1, NG), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    print(f"extreme values c={c} d={d} rows={n}", flush=True)
    lvq.loopvq_encode(cfg, layer=0, loop_group=0, kind=0, n_tokens=n, src=H.dev_u16(src_bits), stride_loop=n * d,
                      stride_token=d, stride_head=d, seq_id=H.dev_i32(seq), vq_pos=H.dev_i32(pos),
                      block_table=H.dev_i32(paging.table), batch=B, max_pages_per_seq=paging.max_pages,
                      num_pages=paging.num_pages, cb=d_cb, cb_norms=d_norm, pool=pool, out_idx=out_idx,
                      rerank_count=cnt)
    torch.cuda.synchronize()
    got = out_idx[:, 0].cpu().numpy()
    want = np.stack([O.encode(x[:, g], C[g])[0] for g in range(NG)], axis=1)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} indices differ, first at (row, group) {tuple(bad[0])}"
    print(f"  re-ranked {int(cnt.item())} of {n * NG}", flush=True)
