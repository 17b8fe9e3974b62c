"""GPU encode on planted exact and sub-fp32 near ties: every index must equal the oracle's.

Each group's codebook holds, for 16 anchor vectors A_m, the codewords
  A_m + e0 + 2^-15 e1   (distance 1 + 2^-30 from A_m: loses by less than fp32 can resolve),
  A_m + e1              (distance 1: the lowest index among the minimisers),
  A_m + e0              (distance 1: an exact tie, higher index),
  a duplicate of A_m + e1, and 12 farther codewords,
and every row is one of the anchors.  All values are exact in bf16.  A screen that settles
such rows in fp32 picks the first codeword; the brute-force definition (lowest index among the
exact minimisers, the oracle) picks the second.  Both the small-batch and the staged bulk paths
run, at 0.5 bit (c=4) and 0.25 bit (c=8).  No near-tie is excused here.
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


def _planted(E: int, NG: int, n: int, seed: int):
    rng = np.random.default_rng(seed)
    A = np.zeros((NG, 16, E))
    A[:, :, 2:] = rng.integers(-8, 9, size=(NG, 16, E - 2))
    A[:, :, 2] = 16 * np.arange(16)[None, :] - 128          # anchors at least 16 apart
    C = np.repeat(A, 16, axis=1).reshape(NG, 16, 16, E).copy()
    C[:, :, 0, 0] += 1.0
    C[:, :, 0, 1] += 2.0 ** -15
    C[:, :, 1, 1] += 1.0
    C[:, :, 2, 0] += 1.0
    C[:, :, 3, 1] += 1.0
    far = rng.integers(-3, 4, size=(NG, 16, 12, E)).astype(np.float64)
    far[..., 3] = 3.0                                           # squared distance >= 9
    C[:, :, 4:] += far
    C = C.reshape(NG, 256, E)
    m = rng.integers(0, 16, size=(n, NG))
    x = A[np.arange(NG)[None, :], m]                           # [n][NG][E]
    return x, C


@pytest.mark.parametrize("c,d,n", [(4, 64, 100), (4, 64, 16461), (8, 128, 90), (8, 128, 16411)])
def test_planted_ties_match_oracle(c, d, n):
    G, NG, E = 4, d // c, 4 * c
    B = 4
    wl = Workload(name=f"ties_c{c}", layers=1, loops=G, loop_group=G, q_heads=1, kv_heads=1, head_dim=d, chans=c,
                  index_bits=8, batch=B, context=n + 72, wid=0)
    x, C = _planted(E, NG, n, seed=11 + c + n)
    # rows -> the G loop-step planes: src[tau][r][0][g*c + i] = x[r][g][tau*c + i]
    src = x.reshape(n, NG, G, c).transpose(2, 0, 1, 3).reshape(G, n, 1, d)
    src_bits = gen.to_bf16_bits(src)
    assert np.array_equal(gen.bf16_to_f64(src_bits), src), "planted values must be exact in bf16"
    cb_bits = gen.to_bf16_bits(C)[None, None, None]               # [L=1][Jcb=1][Hkv=1][NG][K][E]
    assert np.array_equal(gen.bf16_to_f64(cb_bits[0, 0, 0]), C)
    per_seq = -(-n // B)
    seq = np.arange(n) // per_seq
    pos = np.arange(n) % per_seq
    paging = H.Paging([per_seq] * B, wl.page_tokens, seed=5)
    cfg = lvq.make_config(wl)
    lay = lvq.loopvq_layout_query(cfg, B, paging.num_pages)
    d_cb = H.dev_u16(cb_bits)
    d_norm = torch.empty(lay.norms_elems, dtype=torch.float32, device="cuda")
    lvq.loopvq_codebook_prepare(cfg, d_cb, torch.empty_like(d_cb), d_norm)
    pool = torch.zeros(lay.pool_bytes, dtype=torch.uint8, device="cuda")
    out_idx = torch.full((n, 1, NG), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    print(f"planted ties c={c} d={d} rows={n}", flush=True)
    lvq.loopvq_encode(cfg, layer=0, loop_group=0, kind=1, n_tokens=n, src=H.dev_u16(src_bits), stride_loop=n * d,
                      stride_token=d, stride_head=d, seq_id=H.dev_i32(seq), vq_pos=H.dev_i32(pos),
                      block_table=H.dev_i32(paging.table), batch=B, max_pages_per_seq=paging.max_pages,
                      num_pages=paging.num_pages, cb=d_cb, cb_norms=d_norm, pool=pool, out_idx=out_idx,
                      rerank_count=cnt)
    torch.cuda.synchronize()
    got = out_idx[:, 0].cpu().numpy()
    want = np.stack([O.encode(x[:, g], C[g])[0] for g in range(NG)], axis=1)
    assert np.array_equal(want % 16, np.ones_like(want)), "oracle: the lowest exact minimiser is slot 1"
    assert np.array_equal(got, want)
    assert int(cnt.item()) == n * NG, "every planted row needs the exact re-rank"
    # the index bytes in their pages (oracle layout)
    pool_np = pool.cpu().numpy().reshape(paging.num_pages, lay.page_bytes)
    kind_bytes = lay.page_bytes // 2
    for r in range(0, n, max(1, n // 64)):
        page = paging.table[seq[r], pos[r] // wl.page_tokens]
        w = pos[r] % wl.page_tokens
        for g in range(NG):
            off = kind_bytes + ((w // 4) * (NG // 4) + g // 4) * 16 + (w % 4) * 4 + (g % 4)
            assert pool_np[page, off] == want[r, g]
