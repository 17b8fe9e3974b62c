"""Shared helpers of the GPU parity tests: build a seeded case, run the library, run the oracle.

Inputs come from synth/ (host generator, or its device twin for large buffers).
Expected values come from oracle/ only; GPU outputs are compared with them and
never fed back into the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import sub_bit_loop_loopvq_amd as lvq
from oracle import loopvq_oracle as O
from synth import gen
from synth.workloads import Workload

DEV = "cuda"
REL_L2 = 1e-3     # attention output tolerance: relative L2 per query
MAX_ABS = 1e-2    # and max absolute error


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(DEV)


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32))).to(DEV)


def f64(bits: np.ndarray) -> np.ndarray:
    return gen.bf16_to_f64(bits)


class Paging:
    """Block tables with shuffled page ids (exercises the indirection)."""

    def __init__(self, n_vq_per_seq, PT: int, seed: int = 0, spare: int = 3):
        self.PT = PT
        need = [max(1, -(-int(n) // PT)) for n in n_vq_per_seq]
        self.max_pages = max(need)
        self.num_pages = sum(need) + spare
        perm = np.random.default_rng(seed).permutation(self.num_pages)
        self.table = np.zeros((len(need), self.max_pages), dtype=np.int32)
        pos = 0
        for b, k in enumerate(need):
            self.table[b, :k] = perm[pos:pos + k]
            pos += k


def codebooks_f64(cb_bits: np.ndarray, l: int, jc: int, h: int) -> np.ndarray:
    return f64(cb_bits[l, jc, h])             # [NG][K][E]


class Case:
    """One (layer, loop step) decode launch plus the encode of its loop group, small enough for the oracle."""

    def __init__(self, wl: Workload, layer: int, loop: int, lens, seed: int = 0):
        self.wl, self.l, self.t = wl, layer, loop
        self.j, self.tau = loop // wl.loop_group, loop % wl.loop_group
        self.jc = self.j if wl.codebook_per_loop_group else 0
        self.lens = np.asarray(lens, dtype=np.int32)
        B, H, d, P, R, G = wl.batch, wl.kv_heads, wl.head_dim, wl.prefix, wl.recent, wl.loop_group
        assert len(self.lens) == B
        self.sc = gen.scales(wl)
        self.cbk = gen.codebooks(wl, 0, self.sc)
        self.cbv = gen.codebooks(wl, 1, self.sc)
        self.q = gen.queries(wl, layer, loop)
        self.rot = gen.rotation_matrix_f32(wl) if wl.rotate_keys else None
        self.split = [O.split_context(int(n), P, R) for n in self.lens]
        self.n_vq = np.array([s[1] for s in self.split], dtype=np.int64)
        # cache values of the loop group, per (b, h): [N_b][G][d] bf16 bits, K and V
        self.kv = {}
        for b in range(B):
            for h in range(H):
                for kind in (0, 1):
                    self.kv[kind, b, h] = gen.kv_tokens(wl, kind, layer, b, h, 0, int(self.lens[b]),
                                                        self.j * G, self.j * G + G, self.sc)
        self.kp = np.zeros((B, H, P, d), np.uint16)
        self.vp = np.zeros((B, H, P, d), np.uint16)
        self.kr = np.zeros((B, H, R, d), np.uint16)
        self.vr = np.zeros((B, H, R, d), np.uint16)
        for b in range(B):
            n_pre, n_vq, n_rec = self.split[b]
            N = int(self.lens[b])
            for h in range(H):
                self.kp[b, h, :n_pre] = self.kv[0, b, h][:n_pre, self.tau]
                self.vp[b, h, :n_pre] = self.kv[1, b, h][:n_pre, self.tau]
                self.kr[b, h, :n_rec] = self.kv[0, b, h][N - n_rec:N, self.tau]
                self.vr[b, h, :n_rec] = self.kv[1, b, h][N - n_rec:N, self.tau]
        self.paging = Paging(self.n_vq, wl.page_tokens, seed)

    # ---------------- oracle side ----------------
    def oracle_encode(self):
        """idx[kind][b][h] -> [n_vq][NG] plus (d1, d2) for the near-tie rule."""
        wl = self.wl
        out = {}
        for (kind, b, h), vals in self.kv.items():
            n_pre, n_vq, _ = self.split[b]
            planes = f64(vals[n_pre:n_pre + n_vq]).transpose(1, 0, 2)        # [G][n_vq][d]
            x = O.subvectors(planes, wl.chans)                                # [n_vq][NG][E]
            C = codebooks_f64(self.cbk if kind == 0 else self.cbv, self.l, self.jc, h)
            idx = np.zeros((n_vq, wl.groups), np.int64)
            d1 = np.zeros((n_vq, wl.groups))
            d2 = np.zeros((n_vq, wl.groups))
            for g in range(wl.groups):
                if n_vq:
                    idx[:, g], d1[:, g], d2[:, g] = O.encode(x[:, g], C[g])
            out[kind, b, h] = (idx, d1, d2, x)
        return out

    def oracle_pool(self, idx_of) -> np.ndarray:
        """Pool bytes of this (layer, loop group): [Hkv][num_pages][page_bytes]."""
        wl = self.wl
        lay = O.page_layout(wl.page_tokens, wl.groups, wl.index_bits)
        pool = np.zeros((wl.kv_heads, self.paging.num_pages, lay["page_bytes"]), np.uint8)
        for b in range(wl.batch):
            n_vq = int(self.n_vq[b])
            if n_vq == 0:
                continue
            for h in range(wl.kv_heads):
                pages = O.pack_sequence(idx_of(0, b, h), idx_of(1, b, h), wl.page_tokens, wl.index_bits)
                for p in range(pages.shape[0]):
                    pool[h, self.paging.table[b, p]] = pages[p]
        return pool

    def oracle_decode(self, idx_of, scale=None):
        wl = self.wl
        scale = 1.0 / np.sqrt(wl.head_dim) if scale is None else scale
        grp = wl.q_heads // wl.kv_heads
        o = np.zeros((wl.batch, wl.q_heads, wl.head_dim))
        lse = np.zeros((wl.batch, wl.q_heads))
        for b in range(wl.batch):
            n_pre, n_vq, n_rec = self.split[b]
            for hq in range(wl.q_heads):
                h = hq // grp
                o[b, hq], lse[b, hq] = O.decode_query(
                    f64(self.q[b, hq]), f64(self.kp[b, h, :n_pre]), f64(self.vp[b, h, :n_pre]),
                    idx_of(0, b, h), idx_of(1, b, h),
                    codebooks_f64(self.cbk, self.l, self.jc, h), codebooks_f64(self.cbv, self.l, self.jc, h),
                    f64(self.kr[b, h, :n_rec]), f64(self.vr[b, h, :n_rec]), self.tau, wl.chans, scale,
                    self.rot)
        return o, lse

    # ---------------- GPU side ----------------
    def gpu_setup(self):
        wl = self.wl
        self.cfg = lvq.make_config(wl)
        lay = lvq.loopvq_layout_query(self.cfg, wl.batch, self.paging.num_pages)
        self.lay = lay
        self.d_cb = {0: dev_u16(self.cbk), 1: dev_u16(self.cbv)}
        self.d_prep, self.d_norm, self.d_grp = {}, {}, {}
        for kind in (0, 1):
            self.d_prep[kind] = torch.empty_like(self.d_cb[kind])
            self.d_grp[kind] = torch.empty_like(self.d_cb[kind])
            self.d_norm[kind] = torch.empty(lay.norms_elems, dtype=torch.float32, device=DEV)
            lvq.loopvq_codebook_prepare(self.cfg, self.d_cb[kind], self.d_prep[kind], self.d_norm[kind])
            lvq.loopvq_codebook_prepare_groups(self.cfg, self.d_cb[kind], self.d_grp[kind])
        self.d_bt = dev_i32(self.paging.table)
        self.d_lens = dev_i32(self.lens)
        self.d_q = dev_u16(self.q)
        self.d_win = [dev_u16(a) for a in (self.kp, self.vp, self.kr, self.vr)]
        self.d_rot = dev_f32(self.rot) if self.rot is not None else None
        # the pool holds only this (layer, loop group): hand the library a base shifted back by the
        # slice's offset in the whole pool (the oracle's statement of the pool order)
        self.slice_bytes = wl.kv_heads * lay.pool_head_stride_bytes
        self.d_pool = torch.zeros(self.slice_bytes, dtype=torch.uint8, device=DEV)
        self.pool_shift = O.pool_offset(self.l, self.j, 0, 0, wl.loop_groups, wl.kv_heads, self.paging.num_pages,
                                        lay.page_bytes)

    def pool_base(self) -> int:
        return self.d_pool.data_ptr() - self.pool_shift

    def gpu_encode(self, kind: int):
        """Encode every VQ token of the loop group; returns out_idx [rows][Hkv][NG] and the row map."""
        wl = self.wl
        G, H, d = wl.loop_group, wl.kv_heads, wl.head_dim
        rows = [(b, u) for b in range(wl.batch) for u in range(int(self.n_vq[b]))]
        n = len(rows)
        src = np.zeros((G, max(n, 1), H, d), np.uint16)
        for r, (b, u) in enumerate(rows):
            n_pre = self.split[b][0]
            for h in range(H):
                src[:, r, h] = self.kv[kind, b, h][n_pre + u]
        d_src = dev_u16(src)
        seq = dev_i32([b for b, _ in rows] or [0])
        pos = dev_i32([u for _, u in rows] or [0])
        out_idx = torch.full((max(n, 1), H, wl.groups), -1, dtype=torch.int32, device=DEV)
        cnt = torch.zeros(1, dtype=torch.int64, device=DEV)
        lvq.loopvq_encode(self.cfg, layer=self.l, loop_group=self.j, kind=kind, n_tokens=n, src=d_src,
                          stride_loop=max(n, 1) * H * d, stride_token=H * d, stride_head=d, seq_id=seq, vq_pos=pos,
                          block_table=self.d_bt, batch=wl.batch, max_pages_per_seq=self.paging.max_pages,
                          num_pages=self.paging.num_pages, cb=self.d_cb[kind], cb_norms=self.d_norm[kind],
                          pool=self.pool_base(), out_idx=out_idx, rerank_count=cnt)
        torch.cuda.synchronize()
        return out_idx[:n].cpu().numpy(), rows, int(cnt.item())

    def gpu_decode(self, num_splits=0, scale=0.0, want_lse=True):
        wl = self.wl
        out = torch.full((wl.batch, wl.q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((wl.batch, wl.q_heads), float("nan"), dtype=torch.float32, device=DEV) if want_lse else None
        max_len = int(self.lens.max())
        S = num_splits or 0
        ws_bytes = max(lvq.loopvq_decode_attn_workspace(self.cfg, wl.batch, max_len),
                       (S * wl.batch * wl.q_heads * (wl.head_dim + 4) * 4) if S > 1 else 0)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
        lvq.loopvq_decode_attn(self.cfg, layer=self.l, loop=self.t, batch=wl.batch, q=self.d_q,
                               seq_lens=self.d_lens, max_seq_len=max_len, out=out, block_table=self.d_bt,
                               pool=self.pool_base(), max_pages_per_seq=self.paging.max_pages,
                               num_pages=self.paging.num_pages, cb_k_prep=self.d_prep[0], cb_v_prep=self.d_prep[1],
                               k_prefix=self.d_win[0], v_prefix=self.d_win[1], k_recent=self.d_win[2],
                               v_recent=self.d_win[3], rot=self.d_rot, softmax_scale=scale, lse=lse,
                               num_splits=num_splits, workspace=ws, workspace_bytes=ws_bytes)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), (lse.cpu().numpy().astype(np.float64) if want_lse else None)


def check_indices(gpu_idx, exp_idx, d1, d2, x, C, rel=1e-6):
    """Bit-exact index parity; a different index is excused only if its exact distance ties the best within rel.

    Returns the number of excused entries.
    """
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    assert gpu_idx.min() >= 0 and gpu_idx.max() < C.shape[0], "index out of range"
    diff = np.nonzero(gpu_idx != exp_idx)[0]
    for i in diff:
        dk = O.sq_dists(x[i:i + 1], C[gpu_idx[i]:gpu_idx[i] + 1])[0, 0]
        assert dk - d1[i] <= rel * d2[i], (
            f"index mismatch at {i}: gpu {gpu_idx[i]} (dist {dk!r}) vs oracle {exp_idx[i]} "
            f"(d1 {d1[i]!r}, d2 {d2[i]!r})")
    return len(diff)


def check_attention(o_gpu, o_ref, lse_gpu=None, lse_ref=None):
    o_gpu = o_gpu.reshape(-1, o_gpu.shape[-1])
    o_ref = o_ref.reshape(-1, o_ref.shape[-1])
    assert np.isfinite(o_gpu).all(), "non-finite output"
    num = np.linalg.norm(o_gpu - o_ref, axis=1)
    den = np.maximum(np.linalg.norm(o_ref, axis=1), 1e-30)
    rel = num / den
    mx = np.abs(o_gpu - o_ref).max()
    assert rel.max() <= REL_L2, f"rel-L2 {rel.max():.3e} (query {int(rel.argmax())}) > {REL_L2}"
    assert mx <= MAX_ABS, f"max-abs {mx:.3e} > {MAX_ABS}"
    if lse_gpu is not None:
        err = np.abs(lse_gpu.ravel() - lse_ref.ravel())
        assert err.max() <= 1e-3 * max(1.0, np.abs(lse_ref).max()), f"lse error {err.max():.3e}"
    return float(rel.max()), float(mx)


class FullCase:
    """A decode launch at a workload's full shape, checked on sampled queries.

    The packed cache of the sampled (sequence, kv-head) pairs holds uniform
    random indices from the generator, packed by the oracle; every other
    sequence's pages stay zero (its outputs are computed but not checked).
    Windows, queries and codebooks come from the host generator.
    """

    def __init__(self, wl: Workload, layer: int, loop: int, samples, lens=None, seed: int = 0):
        self.wl, self.l, self.t = wl, layer, loop
        self.j, self.tau = loop // wl.loop_group, loop % wl.loop_group
        self.jc = self.j if wl.codebook_per_loop_group else 0
        B, H, d, P, R = wl.batch, wl.kv_heads, wl.head_dim, wl.prefix, wl.recent
        self.lens = np.full(B, wl.context, np.int32) if lens is None else np.asarray(lens, np.int32)
        self.samples = list(samples)          # (b, hq)
        self.sc = gen.scales(wl)
        self.cbk = gen.codebooks(wl, 0, self.sc, layers=[layer])
        self.cbv = gen.codebooks(wl, 1, self.sc, layers=[layer])
        self.q = gen.queries(wl, layer, loop)
        self.rot = gen.rotation_matrix_f32(wl) if wl.rotate_keys else None
        self.split = [O.split_context(int(n), P, R) for n in self.lens]
        self.n_vq = np.array([s[1] for s in self.split], dtype=np.int64)
        self.paging = Paging(self.n_vq, wl.page_tokens, seed, spare=1)
        self.kp = np.zeros((B, H, P, d), np.uint16)
        self.vp = np.zeros((B, H, P, d), np.uint16)
        self.kr = np.zeros((B, H, R, d), np.uint16)
        self.vr = np.zeros((B, H, R, d), np.uint16)
        for b in range(B):
            n_pre, _, n_rec = self.split[b]
            N = int(self.lens[b])
            for h in range(H):
                for kind, pre, rec in ((0, self.kp, self.kr), (1, self.vp, self.vr)):
                    if n_pre:
                        pre[b, h, :n_pre] = gen.kv_tokens(wl, kind, layer, b, h, 0, n_pre, loop, loop + 1,
                                                          self.sc)[:, 0]
                    if n_rec:
                        rec[b, h, :n_rec] = gen.kv_tokens(wl, kind, layer, b, h, N - n_rec, N, loop, loop + 1,
                                                          self.sc)[:, 0]
        grp = wl.q_heads // wl.kv_heads
        self.pairs = sorted({(b, hq // grp) for b, hq in self.samples})
        self.idx = {}
        for b, h in self.pairs:
            for kind in (0, 1):
                self.idx[kind, b, h] = gen.random_indices(wl, kind, layer, self.j, b, h, int(self.n_vq[b]))

    def idx_of(self, kind, b, h):
        return self.idx[kind, b, h]

    def upload(self):
        wl = self.wl
        self.cfg = lvq.make_config(wl)
        lay = lvq.loopvq_layout_query(self.cfg, wl.batch, self.paging.num_pages)
        self.d_prep = {}
        for kind, cb in ((0, self.cbk), (1, self.cbv)):
            d_cb = dev_u16(cb)
            self.d_prep[kind] = torch.empty_like(d_cb)
            lvq.loopvq_codebook_prepare(self.cfg, d_cb, self.d_prep[kind], None)
            del d_cb
        self.d_bt = dev_i32(self.paging.table)
        self.d_lens = dev_i32(self.lens)
        self.d_q = dev_u16(self.q)
        self.d_win = [dev_u16(a) for a in (self.kp, self.vp, self.kr, self.vr)]
        self.d_rot = dev_f32(self.rot) if self.rot is not None else None
        slice_bytes = wl.kv_heads * lay.pool_head_stride_bytes
        self.d_pool = torch.zeros(slice_bytes, dtype=torch.uint8, device=DEV)
        pb = lay.page_bytes
        at = lambda h, page: O.pool_offset(self.l, self.j, h, page, wl.loop_groups, wl.kv_heads,  # noqa: E731
                                           self.paging.num_pages, pb)
        self.pool_shift = at(0, 0)
        for b, h in self.pairs:
            pages = O.pack_sequence(self.idx[0, b, h], self.idx[1, b, h], wl.page_tokens, wl.index_bits)
            for p in range(pages.shape[0]):
                off = at(h, int(self.paging.table[b, p])) - self.pool_shift
                self.d_pool[off:off + pb] = torch.from_numpy(pages[p]).to(DEV)
        torch.cuda.synchronize()

    def gpu_decode(self, num_splits=0, scale=0.0):
        wl = self.wl
        out = torch.full((wl.batch, wl.q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((wl.batch, wl.q_heads), float("nan"), dtype=torch.float32, device=DEV)
        max_len = int(self.lens.max())
        ws_bytes = lvq.loopvq_decode_attn_workspace(self.cfg, wl.batch, max_len)
        if num_splits > 1:
            ws_bytes = max(ws_bytes, num_splits * wl.batch * wl.q_heads * (wl.head_dim + 4) * 4)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=DEV)
        lvq.loopvq_decode_attn(self.cfg, layer=self.l, loop=self.t, batch=wl.batch, q=self.d_q,
                               seq_lens=self.d_lens, max_seq_len=max_len, out=out, block_table=self.d_bt,
                               pool=self.d_pool.data_ptr() - self.pool_shift,
                               max_pages_per_seq=self.paging.max_pages, num_pages=self.paging.num_pages,
                               cb_k_prep=self.d_prep[0], cb_v_prep=self.d_prep[1], k_prefix=self.d_win[0],
                               v_prefix=self.d_win[1], k_recent=self.d_win[2], v_recent=self.d_win[3],
                               rot=self.d_rot, softmax_scale=scale, lse=lse, num_splits=num_splits, workspace=ws,
                               workspace_bytes=ws_bytes)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)

    def oracle(self, b, hq, scale=None):
        wl = self.wl
        h = hq // (wl.q_heads // wl.kv_heads)
        n_pre, _, n_rec = self.split[b]
        return O.decode_query(
            f64(self.q[b, hq]), f64(self.kp[b, h, :n_pre]), f64(self.vp[b, h, :n_pre]),
            self.idx[0, b, h], self.idx[1, b, h], codebooks_f64(self.cbk, self.l, self.jc, h),
            codebooks_f64(self.cbv, self.l, self.jc, h), f64(self.kr[b, h, :n_rec]), f64(self.vr[b, h, :n_rec]),
            self.tau, wl.chans, 1.0 / np.sqrt(wl.head_dim) if scale is None else scale, self.rot)
