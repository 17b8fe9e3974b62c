"""Benchmark: LoopVQ decode-attention throughput on one MI355X.

One step = one decode step of a looped transformer stack over a packed,
loop-axis vector-quantized KV cache: for every loop step t (outer) and layer l
(inner), one decode-attention launch over all B sequences x Hq heads; then one
eviction launch that encodes, for every layer, loop group and K/V, the B tokens
that leave the bf16 recent window (written to a fixed VQ position so the cache
stays the same size).

Default workload: 24 layers x 4 loop steps, 16 heads, head_dim 128, batch 64,
32768-token context, 0.5 bit/elem (c=4, G=4, 8-bit indices), 8 prefix + 64 recent
bf16 tokens.  The cache is built on the GPU (device generator -> GPU encode).

Prints one JSON line.  `value` is decode queries per second (one query = one
(layer, loop step, sequence, q-head) attention row over the whole context).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "VQ decode-attn queries/s + effective HBM GB/s (% peak), 32K ctx, 0.5 bit/elem"
BF16_METRIC = "bf16-cache decode-attn queries/s + effective HBM GB/s (% peak), same kernel, 32K ctx"
HBM_PEAK_GBPS = 8000.0
MIN_ROTATED_CACHE_BYTES = 4 * 256 * 2**20   # 4x the Infinity Cache
DEFAULT_WORKLOAD = "stack24x4_h16_d128_b64_n32k"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_stack32k_traffic.md")
DECODE_SRC = os.path.join(ROOT, "sub_bit_loop_loopvq_amd", "csrc", "decode_attn.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(wl) -> dict:
    """Bytes one decode launch must move: index streams, bf16 windows, codebook slices, q in / out."""
    B, H, Hq, d, c = wl.batch, wl.kv_heads, wl.q_heads, wl.head_dim, wl.chans
    idx = B * H * wl.n_vq * (d // c) * (wl.index_bits / 8) * 2
    window = B * H * min(wl.context, wl.prefix + wl.recent) * d * 2 * 2
    slices = H * (d // c) * wl.codewords * c * 2 * 2 if wl.n_vq > 0 else 0   # read only with VQ rows
    qo = B * Hq * d * (2 + 4)
    rot = d * d * 4 if wl.rotate_keys else 0
    return {"idx": idx, "window": window, "slices": slices, "q_out": qo, "rot": rot,
            "total": idx + window + slices + qo + rot}


def traffic_from_profile():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it was taken
    on the current decode kernel source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_val):
        return None
    sha = hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()
    return float(m_val.group(1)) if sha == m_sha.group(1) else None


class Bench:
    def __init__(self, wl, seed=0):
        import torch
        import sub_bit_loop_loopvq_amd as lvq
        from synth import gen
        from synth.device import DeviceGen
        self.torch, self.lvq, self.wl = torch, lvq, wl
        dev = "cuda"
        L, T, G, J = wl.layers, wl.loops, wl.loop_group, wl.loop_groups
        B, H, Hq, d, P, R = wl.batch, wl.kv_heads, wl.q_heads, wl.head_dim, wl.prefix, wl.recent
        self.cfg = lvq.make_config(wl)
        n_vq = wl.n_vq
        self.pages_per_seq = -(-n_vq // wl.page_tokens)
        self.num_pages = B * self.pages_per_seq
        self.lay = lvq.loopvq_layout_query(self.cfg, B, self.num_pages)
        perm = np.random.default_rng(seed).permutation(self.num_pages).astype(np.int32)
        self.bt = torch.from_numpy(perm.reshape(B, self.pages_per_seq)).to(dev)
        self.lens = torch.full((B,), wl.context, dtype=torch.int32, device=dev)
        t0 = time.time()
        sc = gen.scales(wl)
        self.prep, self.cb, self.norms = {}, {}, {}
        for kind in (0, 1):
            cbh = gen.codebooks(wl, kind, sc)
            self.cb[kind] = torch.from_numpy(cbh.view(np.int16)).to(dev)
            self.prep[kind] = torch.empty_like(self.cb[kind])
            self.norms[kind] = torch.empty(self.lay.norms_elems, dtype=torch.float32, device=dev)
            lvq.loopvq_codebook_prepare(self.cfg, self.cb[kind], self.prep[kind], self.norms[kind])
        log(f"codebooks ready ({time.time() - t0:.1f}s)")
        q = np.stack([np.stack([gen.queries(wl, l, t) for t in range(T)]) for l in range(L)])
        self.q = torch.from_numpy(q.view(np.int16)).to(dev)                  # [L][T][B][Hq][d]
        self.rot = (torch.from_numpy(gen.rotation_matrix_f32(wl)).to(dev) if wl.rotate_keys else None)
        log(f"queries ready ({time.time() - t0:.1f}s)")
        dg = DeviceGen(wl)
        # bf16 windows of every (layer, loop step): [2][L][T][B][Hkv][P or R][d]
        self.pre = torch.empty((2, L, T, B, H, P, d), dtype=torch.int16, device=dev)
        self.rec = torch.empty((2, L, T, B, H, R, d), dtype=torch.int16, device=dev)
        for kind in (0, 1):
            for l in range(L):
                dg.kv(self.pre[kind, l], kind=kind, layer=l, b0=0, nb=B, h0=0, nh=H, n0=0, nn=P, t0=0, nt=T,
                      s_loop=B * H * P * d, s_b=H * P * d, s_h=P * d, s_n=d)
                dg.kv(self.rec[kind, l], kind=kind, layer=l, b0=0, nb=B, h0=0, nh=H, n0=wl.context - R, nn=R,
                      t0=0, nt=T, s_loop=B * H * R * d, s_b=H * R * d, s_h=R * d, s_n=d)
        torch.cuda.synchronize()
        log(f"windows ready ({time.time() - t0:.1f}s)")
        # packed index pool: device-generated K/V of every VQ token, encoded on the GPU
        self.pool = torch.zeros(self.lay.pool_bytes, dtype=torch.uint8, device=dev)
        chunk = max(1, min(B, int(2.5e9 // (G * n_vq * H * d * 2))))
        src = torch.empty((G, chunk * n_vq, H, d), dtype=torch.int16, device=dev)
        rows = chunk * n_vq
        self.rerank = torch.zeros(1, dtype=torch.int64, device=dev)
        for l in range(L):
            for j in range(J):
                for kind in (0, 1):
                    for b0 in range(0, B, chunk):
                        nb = min(chunk, B - b0)
                        for bi in range(nb):
                            dg.kv(src[:, bi * n_vq:], kind=kind, layer=l, b0=b0 + bi, nb=1, h0=0, nh=H, n0=P,
                                  nn=n_vq, t0=j * G, nt=G, s_loop=rows * H * d, s_b=0, s_h=d, s_n=H * d)
                        r = torch.arange(nb * n_vq, dtype=torch.int32, device=dev)
                        lvq.loopvq_encode(self.cfg, layer=l, loop_group=j, kind=kind, n_tokens=nb * n_vq, src=src,
                                          stride_loop=rows * H * d, stride_token=H * d, stride_head=d,
                                          seq_id=r // n_vq + b0, vq_pos=r % n_vq, block_table=self.bt, batch=B,
                                          max_pages_per_seq=self.pages_per_seq, num_pages=self.num_pages,
                                          cb=self.cb[kind], cb_norms=self.norms[kind], pool=self.pool,
                                          rerank_count=self.rerank)
            torch.cuda.synchronize()
            log(f"layer {l} encoded ({time.time() - t0:.1f}s)")
        del src
        torch.cuda.empty_cache()
        self.ws_bytes = lvq.loopvq_decode_attn_workspace(self.cfg, B, wl.context)
        self.ws = torch.empty(max(16, self.ws_bytes), dtype=torch.uint8, device=dev)
        self.out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        self.evict_pos = torch.full((B,), n_vq - 1, dtype=torch.int32, device=dev)
        self.evict_slot = torch.zeros((B,), dtype=torch.int32, device=dev)
        # A cache smaller than 4x the 256 MB Infinity Cache would be served from it when launches
        # repeat: decode launches then rotate over copies of the pool and windows, so every
        # launch reads its bytes from HBM (the eviction keeps writing copy 0).
        cache_bytes = self.lay.pool_bytes + 2 * (self.pre[0].numel() + self.rec[0].numel()) * 2
        self.replicas = max(1, min(16, -(-MIN_ROTATED_CACHE_BYTES // cache_bytes)))
        self.reps = [(self.pool, self.pre, self.rec)]
        for _ in range(self.replicas - 1):
            self.reps.append((self.pool.clone(), self.pre.clone(), self.rec.clone()))
        self.rep_i = 0
        self.setup_s = time.time() - t0
        log(f"setup done in {self.setup_s:.1f}s; re-ranked sub-vectors during build: {int(self.rerank.item())}")

    def decode(self, l, t):
        wl = self.wl
        pool, pre, rec = self.reps[self.rep_i]
        self.rep_i = (self.rep_i + 1) % self.replicas
        self.lvq.loopvq_decode_attn(
            self.cfg, layer=l, loop=t, batch=wl.batch, q=self.q[l, t], seq_lens=self.lens, max_seq_len=wl.context,
            out=self.out, block_table=self.bt, pool=pool, max_pages_per_seq=self.pages_per_seq,
            num_pages=self.num_pages, cb_k_prep=self.prep[0], cb_v_prep=self.prep[1], k_prefix=pre[0, l, t],
            v_prefix=pre[1, l, t], k_recent=rec[0, l, t], v_recent=rec[1, l, t], rot=self.rot,
            workspace=self.ws, workspace_bytes=self.ws_bytes)

    def evict(self):
        """Encode the token leaving the recent window of every sequence (ring slot 0), for every layer,
        loop group and kind, in one launch."""
        wl = self.wl
        self.lvq.loopvq_evict(self.cfg, batch=wl.batch, max_pages_per_seq=self.pages_per_seq,
                              num_pages=self.num_pages, k_ring=self.rec[0], v_ring=self.rec[1],
                              ring_slot=self.evict_slot, vq_pos=self.evict_pos, block_table=self.bt,
                              cb_k=self.cb[0], cb_v=self.cb[1], norms_k=self.norms[0], norms_v=self.norms[1],
                              pool=self.pool)

    def step(self, events=None, evict_events=None):
        wl = self.wl
        E = self.torch.cuda.Event
        for t in range(wl.loops):
            for l in range(wl.layers):
                if events is not None:
                    e0, e1 = E(enable_timing=True), E(enable_timing=True)
                    e0.record()
                    self.decode(l, t)
                    e1.record()
                    events.append((e0, e1))
                else:
                    self.decode(l, t)
        if evict_events is not None:
            e0, e1 = E(enable_timing=True), E(enable_timing=True)
            e0.record()
            self.evict()
            e1.record()
            evict_events.append((e0, e1))
        else:
            self.evict()


def parse_plan(text: str, wl):
    """Per-(layer, loop range) choice of (c, G): layers separated by '/', each a comma list of
    'LOOPS:cxG' segments covering the layer's loop steps in order (LOOPS % G == 0), e.g.
    '8:4x4,24:8x4/32:8x2/32:4x8/32:8x4'.  A layer list of one entry applies to every layer.
    Returns [[(loops, c, G)]] per layer."""
    layers = []
    for lt in text.split("/"):
        segs = []
        for st in lt.split(","):
            n, cg = st.split(":")
            c, G = cg.lower().split("x")
            segs.append((int(n), int(c), int(G)))
        layers.append(segs)
    if len(layers) == 1:
        layers = layers * wl.layers
    if len(layers) != wl.layers:
        raise ValueError(f"plan has {len(layers)} layers, the workload {wl.layers}")
    for segs in layers:
        if sum(n for n, _, _ in segs) != wl.loops or any(n % G for n, _, G in segs):
            raise ValueError(f"plan segments {segs} must cover {wl.loops} loop steps in whole loop groups")
    return layers


def plan_bits_per_elem(plan, index_bits: int) -> float:
    """Index bits per cached element, averaged over every (layer, loop step)."""
    tot = sum(n for segs in plan for n, _, _ in segs)
    return sum(n * index_bits / (c * G) for segs in plan for n, c, G in segs) / tot


class MixedBench:
    """A stack whose (layer, loop range) segments each pick their own (c, G): one config, pool,
    codebook set and windows per segment; decode (l, t) runs on the segment holding loop step t,
    eviction runs once per segment."""

    def __init__(self, wl, plan):
        self.wl, self.plan = wl, plan
        self.segs = []      # per layer: [(start, Bench)]
        for l, segs in enumerate(plan):
            row, start = [], 0
            for n, c, G in segs:
                sub = wl.with_(name=f"{wl.name}_l{l}_t{start}_c{c}g{G}", layers=1, loops=n, chans=c, loop_group=G,
                               wid=wl.wid * 64 + l * 8 + len(row))
                log(f"segment layer {l} loops [{start}, {start + n}) c={c} G={G}")
                row.append((start, Bench(sub)))
                start += n
            self.segs.append(row)
        self.torch = self.segs[0][0][1].torch

    def decode(self, l, t):
        for start, b in reversed(self.segs[l]):
            if t >= start:
                b.decode(0, t - start)
                return

    def step(self, events=None, evict_events=None):
        E = self.torch.cuda.Event
        for t in range(self.wl.loops):
            for l in range(self.wl.layers):
                if events is not None:
                    e0, e1 = E(enable_timing=True), E(enable_timing=True)
                    e0.record()
                    self.decode(l, t)
                    e1.record()
                    events.append((e0, e1))
                else:
                    self.decode(l, t)
        if evict_events is not None:
            e0 = E(enable_timing=True)
            e0.record()
        for row in self.segs:
            for _, b in row:
                b.evict()
        if evict_events is not None:
            e1 = E(enable_timing=True)
            e1.record()
            evict_events.append((e0, e1))


class Bf16Bench:
    """The same decode kernel over an uncompressed bf16 cache: the recent window covers the whole
    context (recent = context - prefix), so no token is vector-quantized and every launch streams
    bf16 K and V rows.  The bf16 cache of the whole stack would not fit in HBM (1.65 TB at the 32K
    workload), so one (layer, loop step) window pair is generated and every launch of the step
    reads it; each launch still streams its full bytes from HBM (17.2 GB per launch, far beyond
    the 256 MB Infinity Cache)."""

    def __init__(self, wl):
        import torch
        import sub_bit_loop_loopvq_amd as lvq
        from synth import gen
        from synth.device import DeviceGen
        self.torch, self.lvq = torch, lvq
        wl = wl.with_(name=wl.name + "_bf16", recent=wl.context - wl.prefix)
        self.wl = wl
        dev = "cuda"
        L, T = wl.layers, wl.loops
        B, H, d, P, R = wl.batch, wl.kv_heads, wl.head_dim, wl.prefix, wl.recent
        self.cfg = lvq.make_config(wl)
        t0 = time.time()
        q = np.stack([np.stack([gen.queries(wl, l, t) for t in range(T)]) for l in range(L)])
        self.q = torch.from_numpy(q.view(np.int16)).to(dev)                  # [L][T][B][Hq][d]
        self.rot = (torch.from_numpy(gen.rotation_matrix_f32(wl)).to(dev) if wl.rotate_keys else None)
        self.lens = torch.full((B,), wl.context, dtype=torch.int32, device=dev)
        dg = DeviceGen(wl)
        self.pre = torch.empty((2, B, H, P, d), dtype=torch.int16, device=dev)
        self.rec = torch.empty((2, B, H, R, d), dtype=torch.int16, device=dev)
        for kind in (0, 1):
            dg.kv(self.pre[kind], kind=kind, layer=0, b0=0, nb=B, h0=0, nh=H, n0=0, nn=P, t0=0, nt=1,
                  s_loop=B * H * P * d, s_b=H * P * d, s_h=P * d, s_n=d)
            dg.kv(self.rec[kind], kind=kind, layer=0, b0=0, nb=B, h0=0, nh=H, n0=P, nn=R, t0=0, nt=1,
                  s_loop=B * H * R * d, s_b=H * R * d, s_h=R * d, s_n=d)
        torch.cuda.synchronize()
        self.ws_bytes = lvq.loopvq_decode_attn_workspace(self.cfg, B, wl.context)
        self.ws = torch.empty(max(16, self.ws_bytes), dtype=torch.uint8, device=dev)
        self.out = torch.empty((B, wl.q_heads, d), dtype=torch.float32, device=dev)
        self.setup_s = time.time() - t0
        log(f"bf16 windows ready ({self.setup_s:.1f}s): {self.rec.numel() * 2 / 1e9:.1f} GB")

    def decode(self, l, t):
        wl = self.wl
        self.lvq.loopvq_decode_attn(
            self.cfg, layer=l, loop=t, batch=wl.batch, q=self.q[l, t], seq_lens=self.lens, max_seq_len=wl.context,
            out=self.out, k_prefix=self.pre[0], v_prefix=self.pre[1], k_recent=self.rec[0], v_recent=self.rec[1],
            rot=self.rot, workspace=self.ws, workspace_bytes=self.ws_bytes)

    def step(self, events=None, evict_events=None):
        E = self.torch.cuda.Event
        for t in range(self.wl.loops):
            for l in range(self.wl.layers):
                if events is not None:
                    e0, e1 = E(enable_timing=True), E(enable_timing=True)
                    e0.record()
                    self.decode(l, t)
                    e1.record()
                    events.append((e0, e1))
                else:
                    self.decode(l, t)


def host_cores() -> dict:
    """What the host offers the CPU baseline: logical CPUs, the ones this process may run on, and the
    BLAS pool's default thread count (the baseline itself pins BLAS to one thread)."""
    from threadpoolctl import threadpool_info
    blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"host_cpus": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)),
            "blas_threads_default": max(blas) if blas else None}


def cpu_baseline(wl, seconds: float) -> dict:
    """The CPU oracle (fp64, single BLAS thread) on sampled decode queries of the same workload, with
    generator indices (the workloads whose GPU pool is not one Bench pool: --plan, --bf16-cache)."""
    from threadpoolctl import threadpool_limits
    from oracle import loopvq_oracle as O
    from synth import gen
    t_start = time.time()
    sc = gen.scales(wl)
    l, t = 0, 0
    j, tau = t // wl.loop_group, t % wl.loop_group
    cbk = gen.bf16_to_f64(gen.codebooks(wl, 0, sc, layers=[l])[l, 0])
    cbv = gen.bf16_to_f64(gen.codebooks(wl, 1, sc, layers=[l])[l, 0])
    q = gen.queries(wl, l, t)
    n_pre, n_vq, n_rec = O.split_context(wl.context, wl.prefix, wl.recent)
    grp = wl.q_heads // wl.kv_heads
    done, busy = 0, 0.0
    with threadpool_limits(limits=1):
        for qi in range(wl.batch * wl.q_heads):
            b, hq = divmod(qi, wl.q_heads)
            h = hq // grp
            win = {}
            for kind in (0, 1):
                pre = gen.bf16_to_f64(gen.kv_tokens(wl, kind, l, b, h, 0, n_pre, t, t + 1, sc)[:, 0])
                rec = gen.bf16_to_f64(gen.kv_tokens(wl, kind, l, b, h, wl.context - n_rec, wl.context, t, t + 1,
                                                    sc)[:, 0])
                win[kind] = (pre, rec)
            ik = gen.random_indices(wl, 0, l, j, b, h, n_vq)
            iv = gen.random_indices(wl, 1, l, j, b, h, n_vq)
            pages = O.pack_sequence(ik, iv, wl.page_tokens, wl.index_bits)
            c0 = time.perf_counter()
            ik2, iv2 = O.unpack_sequence(pages, n_vq, wl.groups, wl.page_tokens, wl.index_bits)
            O.decode_query(gen.bf16_to_f64(q[b, hq]), win[0][0], win[1][0], ik2, iv2, cbk[h], cbv[h], win[0][1],
                           win[1][1], tau, wl.chans, 1.0 / np.sqrt(wl.head_dim))
            busy += time.perf_counter() - c0
            done += 1
            if busy >= seconds:
                break
    return {"value": done / busy, "unit": "queries/s", "cores": 1, "kind": "oracle", **host_cores(),
            "sample": (f"{done} decode queries (layer 0, loop step 0, sequences 0..{(done - 1) // wl.q_heads}) at "
                       f"full context {wl.context}: unpack packed pages (generator indices) + dequantize + fp64 "
                       f"softmax attention; {busy:.1f}s of timed oracle work, 1 BLAS thread; input setup untimed "
                       f"(wall {time.time() - t_start:.1f}s)")}


def cpu_baseline_gpu_pages(bench, seconds: float) -> dict:
    """The CPU oracle (fp64, one BLAS thread) on sampled decode queries of (layer 0, loop step 0), fed
    with exactly what the GPU decodes: the packed pages the GPU encode wrote (copied back through the
    block table), the bf16 windows, queries and codebooks in HBM.  The GPU's own output for the same
    launch is compared with the oracle's on the sampled queries (rel-L2 and max-abs)."""
    import torch
    from threadpoolctl import threadpool_limits
    from oracle import loopvq_oracle as O
    from synth import gen
    t_start = time.time()
    wl, lvq = bench.wl, bench.lvq
    l, t = 0, 0
    j, tau = t // wl.loop_group, t % wl.loop_group
    jc = j if wl.codebook_per_loop_group else 0
    # the GPU's output of this launch, over the same pool the oracle reads
    out = torch.empty_like(bench.out)
    lvq.loopvq_decode_attn(bench.cfg, layer=l, loop=t, batch=wl.batch, q=bench.q[l, t], seq_lens=bench.lens,
                           max_seq_len=wl.context, out=out, block_table=bench.bt, pool=bench.pool,
                           max_pages_per_seq=bench.pages_per_seq, num_pages=bench.num_pages,
                           cb_k_prep=bench.prep[0], cb_v_prep=bench.prep[1], k_prefix=bench.pre[0, l, t],
                           v_prefix=bench.pre[1, l, t], k_recent=bench.rec[0, l, t], v_recent=bench.rec[1, l, t],
                           rot=bench.rot, workspace=bench.ws, workspace_bytes=bench.ws_bytes)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    u16 = lambda x: x.cpu().numpy().view(np.uint16)   # noqa: E731
    q = u16(bench.q[l, t])
    cb = {k: gen.bf16_to_f64(u16(bench.cb[k][l, jc])) for k in (0, 1)}          # [H][NG][K][E]
    bt = bench.bt.cpu().numpy()
    rot = bench.rot.cpu().numpy().astype(np.float64) if bench.rot is not None else None
    n_pre, n_vq, n_rec = O.split_context(wl.context, wl.prefix, wl.recent)
    grp = wl.q_heads // wl.kv_heads
    page_bytes = bench.lay.page_bytes
    n_pages = -(-n_vq // wl.page_tokens)
    done, busy, rel, mx = 0, 0.0, 0.0, 0.0
    with threadpool_limits(limits=1):
        for qi in range(wl.batch * wl.q_heads):
            b, hq = divmod(qi, wl.q_heads)
            h = hq // grp
            offs = [O.pool_offset(l, j, h, int(bt[b, pg]), wl.loop_groups, wl.kv_heads, bench.num_pages, page_bytes)
                    for pg in range(n_pages)]
            idx = torch.tensor(offs, dtype=torch.int64, device=bench.pool.device)[:, None] + \
                torch.arange(page_bytes, device=bench.pool.device)[None]
            pages = bench.pool[idx].cpu().numpy()                              # [n_pages][page_bytes]
            win = [gen.bf16_to_f64(u16(a[kind, l, t, b, h, :n])) for kind in (0, 1)
                   for a, n in ((bench.pre, n_pre), (bench.rec, n_rec))]       # kp, kr, vp, vr
            c0 = time.perf_counter()
            ik, iv = O.unpack_sequence(pages, n_vq, wl.groups, wl.page_tokens, wl.index_bits)
            o, _ = O.decode_query(gen.bf16_to_f64(q[b, hq]), win[0], win[2], ik, iv, cb[0][h], cb[1][h], win[1],
                                  win[3], tau, wl.chans, 1.0 / np.sqrt(wl.head_dim), rot)
            busy += time.perf_counter() - c0
            rel = max(rel, float(np.linalg.norm(out[b, hq] - o) / max(np.linalg.norm(o), 1e-30)))
            mx = max(mx, float(np.abs(out[b, hq] - o).max()))
            done += 1
            if busy >= seconds:
                break
    return {"value": done / busy, "unit": "queries/s", "cores": 1, "kind": "oracle", **host_cores(),
            "gpu_vs_oracle": {"queries": done, "rel_l2_max": rel, "max_abs": mx},
            "sample": (f"{done} decode queries (layer 0, loop step 0, sequences 0..{(done - 1) // wl.q_heads}) at "
                       f"full context {wl.context}, on the GPU's own inputs copied back (the packed pages its "
                       f"encode wrote, bf16 windows, queries, codebooks): unpack + dequantize + fp64 softmax "
                       f"attention; {busy:.1f}s of timed oracle work, 1 BLAS thread; copies untimed "
                       f"(wall {time.time() - t_start:.1f}s)")}


ENCODE_METRIC = "LoopVQ bulk encode sub-vectors/s (one layer, loop group and kind)"
# VALU lane-operations per second of one MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
VALU_PEAK_OPS = 256 * 4 * 16 * 2.4e9


class EncodeBench:
    """Bulk encode of one (layer, loop group, kind) slice: all rows, kv-heads and groups in one call."""

    def __init__(self, wl, layer=0, loop_group=0, kind=0, seed=0):
        import torch
        import sub_bit_loop_loopvq_amd as lvq
        from synth import gen
        from synth.device import DeviceGen
        self.torch, self.lvq, self.wl = torch, lvq, wl
        self.layer, self.j, self.kind = layer, loop_group, kind
        dev = "cuda"
        B, H, d, G, P = wl.batch, wl.kv_heads, wl.head_dim, wl.loop_group, wl.prefix
        self.rows = rows = wl.encode_tokens
        per_seq = rows // B
        self.cfg = lvq.make_config(wl)
        self.pps = -(-per_seq // wl.page_tokens)
        self.num_pages = B * self.pps
        self.lay = lvq.loopvq_layout_query(self.cfg, B, self.num_pages)
        perm = np.random.default_rng(seed).permutation(self.num_pages).astype(np.int32)
        self.bt = torch.from_numpy(perm.reshape(B, self.pps)).to(dev)
        sc = gen.scales(wl)
        cb = gen.codebooks(wl, kind, sc, layers=[layer])
        self.cb = torch.from_numpy(cb.view(np.int16)).to(dev)
        self.norms = torch.empty(self.lay.norms_elems, dtype=torch.float32, device=dev)
        lvq.loopvq_codebook_prepare(self.cfg, self.cb, torch.empty_like(self.cb), self.norms)
        self.src = torch.empty((G, rows, H, d), dtype=torch.int16, device=dev)
        dg = DeviceGen(wl)
        for b in range(B):
            dg.kv(self.src[:, b * per_seq:], kind=kind, layer=layer, b0=b, nb=1, h0=0, nh=H, n0=P, nn=per_seq,
                  t0=loop_group * G, nt=G, s_loop=rows * H * d, s_b=0, s_h=d, s_n=H * d)
        r = torch.arange(rows, dtype=torch.int32, device=dev)
        self.seq, self.pos = r // per_seq, r % per_seq
        # the pool slice of this (layer, loop group); the library addresses it from the pool base
        slice_bytes = H * self.lay.pool_head_stride_bytes
        self.pool = torch.zeros(slice_bytes, dtype=torch.uint8, device=dev)
        self.shift = (layer * wl.loop_groups + loop_group) * slice_bytes
        self.rerank = torch.zeros(1, dtype=torch.int64, device=dev)
        torch.cuda.synchronize()

    def run(self, count=None):
        wl = self.wl
        self.lvq.loopvq_encode(self.cfg, layer=self.layer, loop_group=self.j, kind=self.kind, n_tokens=self.rows,
                               src=self.src, stride_loop=self.rows * wl.kv_heads * wl.head_dim,
                               stride_token=wl.kv_heads * wl.head_dim, stride_head=wl.head_dim, seq_id=self.seq,
                               vq_pos=self.pos, block_table=self.bt, batch=wl.batch, max_pages_per_seq=self.pps,
                               num_pages=self.num_pages, cb=self.cb, cb_norms=self.norms,
                               pool=self.pool.data_ptr() - self.shift, rerank_count=count)


def encode_cpu_baseline(wl, seconds: float, layer=0, loop_group=0, kind=0) -> dict:
    """The CPU oracle's brute-force encode (fp64, single BLAS thread) on sampled sub-vectors of the slice."""
    from threadpoolctl import threadpool_limits
    from oracle import loopvq_oracle as O
    from synth import gen
    t_start = time.time()
    sc = gen.scales(wl)
    cb = gen.bf16_to_f64(gen.codebooks(wl, kind, sc, layers=[layer])[layer, 0])   # [H][NG][K][E]
    per_seq = wl.encode_tokens // wl.batch
    G = wl.loop_group
    done, busy, rows = 0, 0.0, 0
    with threadpool_limits(limits=1):
        for h in range(wl.kv_heads):
            planes = gen.kv_tokens(wl, kind, layer, 0, h, wl.prefix, wl.prefix + per_seq, loop_group * G,
                                   loop_group * G + G, sc)                                  # [n][G][d]
            x = O.subvectors(gen.bf16_to_f64(planes).transpose(1, 0, 2), wl.chans)            # [n][NG][E]
            for n0 in range(0, per_seq, 256):
                c0 = time.perf_counter()
                for g in range(wl.groups):
                    O.encode(x[n0:n0 + 256, g], cb[h, g])
                busy += time.perf_counter() - c0
                done += 256 * wl.groups
                rows += 256
                if busy >= seconds:
                    break
            if busy >= seconds:
                break
    return {"value": done / busy, "unit": "sub-vectors/s", "cores": 1, "kind": "oracle", **host_cores(),
            "sample": (f"{done} sub-vectors ({rows} (token, kv-head) rows of sequence 0 x {wl.groups} groups) of "
                       f"layer {layer}, loop group {loop_group}, kind {kind}: brute-force fp64 distances to all "
                       f"{wl.codewords} codewords + argmin; {busy:.1f}s of timed oracle work, 1 BLAS thread; input "
                       f"setup untimed (wall {time.time() - t_start:.1f}s)")}


def encode_main(args):
    import torch
    from synth import workloads as W
    wl = W.BY_NAME[args.workload]
    torch.cuda.set_device(0)
    eb = EncodeBench(wl)
    for _ in range(args.warmup):
        eb.run()
    eb.rerank.zero_()
    events = []
    E = torch.cuda.Event
    torch.cuda.synchronize()
    for _ in range(args.steps):
        e0, e1 = E(enable_timing=True), E(enable_timing=True)
        e0.record()
        eb.run(eb.rerank)
        e1.record()
        events.append((e0, e1))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in events])
    avg = float(us.mean())
    subvec = wl.encode_tokens * wl.kv_heads * wl.groups
    in_bytes = subvec * wl.sub_len * 2
    out_bytes = subvec * wl.index_bits // 8
    compares = subvec * wl.codewords
    rec = {
        "metric": ENCODE_METRIC, "value": subvec / (avg * 1e-6), "unit": "sub-vectors/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": avg * 1e-3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.encode_tokens, "kv_heads": wl.kv_heads, "groups": wl.groups,
                   "sub_len": wl.sub_len, "codewords": wl.codewords, "layer": 0, "loop_group": 0, "kind": "K"},
        "tokens_per_s": wl.encode_tokens / (avg * 1e-6),
        # the binding roofline is the vector ALU (the argmin's compares); HBM and MFMA beside it
        "roofline": {"bound": "alu", "achieved": compares / (avg * 1e-6) / 1e12,
                     "peak": VALU_PEAK_OPS / 1e12, "unit": "Tcompare/s at one VALU op per compare",
                     "frac": compares / (avg * 1e-6) / VALU_PEAK_OPS, "traffic": None},
        "hbm_roofline": {"bound": "hbm", "achieved": (in_bytes + out_bytes) / (avg * 1e-6) / 1e9,
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": (in_bytes + out_bytes) / (avg * 1e-6) / 1e9 / HBM_PEAK_GBPS},
        "mfma_roofline": {"bound": "mfma", "achieved": 2 * compares * wl.sub_len / (avg * 1e-6) / 1e12,
                          "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": 2 * compares * wl.sub_len / (avg * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "launch_us": {"mean": avg, "p10": float(np.percentile(us, 10)), "p50": float(np.percentile(us, 50)),
                      "p90": float(np.percentile(us, 90))},
        "reranked_fraction": int(eb.rerank.item()) / (subvec * args.steps),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = encode_cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


EXTEND_METRIC = "LoopVQ extend (chunked prefill) attention TFLOP/s over the packed cache"
MFMA_BF16_PEAK_TFLOPS = 2500.0


class ExtendBench:
    """Chunked prefill of M new tokens per sequence over a full packed cache of N tokens, one (layer, loop)."""

    def __init__(self, wl, chunk, seed=0):
        import torch
        import sub_bit_loop_loopvq_amd as lvq
        from synth import gen
        from synth.device import DeviceGen
        self.torch, self.lvq, self.wl, self.M = torch, lvq, wl, chunk
        dev = "cuda"
        B, H, Hq, d, P, R, T = wl.batch, wl.kv_heads, wl.q_heads, wl.head_dim, wl.prefix, wl.recent, wl.loops
        self.cfg = lvq.make_config(wl)
        self.pps = -(-wl.n_vq // wl.page_tokens)
        self.num_pages = B * self.pps
        lay = lvq.loopvq_layout_query(self.cfg, B, self.num_pages)
        perm = np.random.default_rng(seed).permutation(self.num_pages).astype(np.int32)
        self.bt = torch.from_numpy(perm.reshape(B, self.pps)).to(dev)
        self.lens = torch.full((B,), wl.context, dtype=torch.int32, device=dev)
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        # one (layer, loop group) slice of uniformly random 8-bit indices; the library addresses it from the pool base
        slice_bytes = H * lay.pool_head_stride_bytes
        self.pool = torch.randint(0, 256, (slice_bytes,), dtype=torch.uint8, device=dev, generator=g)
        sc = gen.scales(wl)
        self.grp = []   # the group-major codebook copies extend reads
        for kind in (0, 1):
            cb = torch.from_numpy(gen.codebooks(wl, kind, sc, layers=[0]).view(np.int16)).to(dev)
            grp = torch.empty_like(cb)
            lvq.loopvq_codebook_prepare_groups(self.cfg, cb, grp)
            self.grp.append(grp)
        dg = DeviceGen(wl)
        self.win = []
        for kind in (0, 1):
            pre = torch.empty((B, H, P, d), dtype=torch.int16, device=dev)
            rec = torch.empty((B, H, R, d), dtype=torch.int16, device=dev)
            dg.kv(pre, kind=kind, layer=0, b0=0, nb=B, h0=0, nh=H, n0=0, nn=P, t0=0, nt=1, s_loop=0, s_b=H * P * d,
                  s_h=P * d, s_n=d)
            dg.kv(rec, kind=kind, layer=0, b0=0, nb=B, h0=0, nh=H, n0=wl.context - R, nn=R, t0=0, nt=1, s_loop=0,
                  s_b=H * R * d, s_h=R * d, s_n=d)
            self.win += [pre, rec]
        # the chunk: the next M tokens of every sequence (generator positions past the cache)
        self.kn = torch.empty((B, H, chunk, d), dtype=torch.int16, device=dev)
        self.vn = torch.empty((B, H, chunk, d), dtype=torch.int16, device=dev)
        for kind, buf in ((0, self.kn), (1, self.vn)):
            dg.kv(buf, kind=kind, layer=0, b0=0, nb=B, h0=0, nh=H, n0=0, nn=chunk, t0=0, nt=1, s_loop=0,
                  s_b=H * chunk * d, s_h=chunk * d, s_n=d)
        self.q = (torch.randn((B, chunk, Hq, d), device=dev, generator=g)).to(torch.bfloat16).view(torch.int16)
        self.out = torch.empty((B, chunk, Hq, d), dtype=torch.float32, device=dev)
        self.rot = torch.from_numpy(gen.rotation_matrix_f32(wl)).to(dev) if wl.rotate_keys else None
        torch.cuda.synchronize()

    def run(self):
        wl = self.wl
        self.lvq.loopvq_extend_attn(self.cfg, layer=0, loop=0, batch=wl.batch, chunk=self.M, q=self.q, k_new=self.kn,
                                    v_new=self.vn, seq_lens=self.lens, max_seq_len=wl.context, out=self.out,
                                    block_table=self.bt, pool=self.pool, max_pages_per_seq=self.pps,
                                    num_pages=self.num_pages, cb_k_grp=self.grp[0], cb_v_grp=self.grp[1],
                                    k_prefix=self.win[0], v_prefix=self.win[2], k_recent=self.win[1],
                                    v_recent=self.win[3], rot=self.rot)

    def flops(self):
        """Algorithmic flops of one launch: 2 per multiply-add of q.k and of p.v over every visible key."""
        wl, M = self.wl, self.M
        visible = M * wl.context + M * (M + 1) // 2
        return 4.0 * wl.head_dim * wl.batch * wl.q_heads * visible


def extend_cpu_baseline(wl, chunk, seconds: float) -> dict:
    """The CPU oracle's extend attention (fp64, single BLAS thread) on sampled chunk rows of the workload."""
    from threadpoolctl import threadpool_limits
    from oracle import loopvq_oracle as O
    from synth import gen
    t_start = time.time()
    sc = gen.scales(wl)
    cbk = gen.bf16_to_f64(gen.codebooks(wl, 0, sc, layers=[0])[0, 0])
    cbv = gen.bf16_to_f64(gen.codebooks(wl, 1, sc, layers=[0])[0, 0])
    n_pre, n_vq, n_rec = O.split_context(wl.context, wl.prefix, wl.recent)
    rng = np.random.default_rng(0)
    rows, busy = 0, 0.0
    with threadpool_limits(limits=1):
        for b in range(wl.batch):
            h = b % wl.kv_heads
            win = [gen.bf16_to_f64(gen.kv_tokens(wl, kind, 0, b, h, n0, n1, 0, 1, sc)[:, 0])
                   for kind in (0, 1) for (n0, n1) in ((0, n_pre), (wl.context - n_rec, wl.context))]
            ik = gen.random_indices(wl, 0, 0, 0, b, h, n_vq)
            iv = gen.random_indices(wl, 1, 0, 0, b, h, n_vq)
            kc = gen.bf16_to_f64(gen.to_bf16_bits(rng.normal(size=(chunk, wl.head_dim))))
            vc = gen.bf16_to_f64(gen.to_bf16_bits(rng.normal(size=(chunk, wl.head_dim))))
            q = gen.bf16_to_f64(gen.to_bf16_bits(rng.normal(size=(8, wl.head_dim))))
            c0 = time.perf_counter()
            for i in range(8):     # rows chunk-8 .. chunk-1 of the chunk (the longest)
                O.decode_query(q[i], win[0], win[2], ik, iv, cbk[h], cbv[h], np.concatenate([win[1], kc[:chunk - 7 + i]]),
                               np.concatenate([win[3], vc[:chunk - 7 + i]]), 0, wl.chans, 1 / np.sqrt(wl.head_dim))
            busy += time.perf_counter() - c0
            rows += 8
            if busy >= seconds:
                break
    vis = wl.context + chunk
    return {"value": rows * 4.0 * wl.head_dim * vis / busy / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            **host_cores(),
            "sample": (f"{rows} chunk rows (the last 8 of a {chunk}-row chunk, sequences 0..{rows // 8 - 1}) over "
                       f"the full {wl.context}-token cache: unpack + dequantize + fp64 softmax attention, "
                       f"{busy:.1f}s of timed oracle work, 1 BLAS thread; input setup untimed "
                       f"(wall {time.time() - t_start:.1f}s)")}


def extend_main(args):
    import torch
    from synth import workloads as W
    wl = W.BY_NAME[args.workload]
    torch.cuda.set_device(0)
    eb = ExtendBench(wl, args.chunk)
    for _ in range(args.warmup):
        eb.run()
    events = []
    E = torch.cuda.Event
    torch.cuda.synchronize()
    for _ in range(args.steps):
        e0, e1 = E(enable_timing=True), E(enable_timing=True)
        e0.record()
        eb.run()
        e1.record()
        events.append((e0, e1))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in events])
    avg = float(us.mean())
    tflops = eb.flops() / (avg * 1e-6) / 1e12
    rec = {
        "metric": EXTEND_METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": avg * 1e-3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "layers_timed": 1, "batch": wl.batch, "q_heads": wl.q_heads,
                   "kv_heads": wl.kv_heads, "head_dim": wl.head_dim, "cached_tokens": wl.context,
                   "chunk": args.chunk, "bits_per_elem": wl.index_bits / (wl.chans * wl.loop_group)},
        "chunk_tokens_per_s": wl.batch * args.chunk / (avg * 1e-6),
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None},
        "launch_us": {"mean": avg, "p10": float(np.percentile(us, 10)), "p50": float(np.percentile(us, 50)),
                      "p90": float(np.percentile(us, 90))},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = extend_cpu_baseline(wl, args.chunk, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


LLOYD_METRIC = "LoopVQ weighted Lloyd iteration sub-vectors/s (one codebook set: assignment + weighted update)"


class LloydBench:
    """One weighted k-means iteration of one (layer, loop group, kind) codebook set over the encode
    workload's tokens as samples: the assignment (the encode kernels without a pool), then the
    weighted update (sums, weights, new codewords and norms)."""

    def __init__(self, wl, layer=0, loop_group=0, kind=0):
        import torch
        import sub_bit_loop_loopvq_amd as lvq
        from synth import gen
        from synth.device import DeviceGen
        self.torch, self.lvq, self.wl = torch, lvq, wl
        self.layer, self.j = layer, loop_group
        dev = "cuda"
        B, H, d, G, P = wl.batch, wl.kv_heads, wl.head_dim, wl.loop_group, wl.prefix
        self.n = n = wl.encode_tokens
        per_seq = n // B
        self.cfg = lvq.make_config(wl)
        lay = lvq.loopvq_layout_query(self.cfg, 1, 1)
        sc = gen.scales(wl)
        self.cb = torch.from_numpy(gen.codebooks(wl, kind, sc, layers=[layer]).view(np.int16)).to(dev)
        self.norms = torch.empty(lay.norms_elems, dtype=torch.float32, device=dev)
        lvq.loopvq_codebook_prepare(self.cfg, self.cb, torch.empty_like(self.cb), self.norms)
        self.src = torch.empty((G, n, H, d), dtype=torch.int16, device=dev)
        dg = DeviceGen(wl)
        for b in range(B):
            dg.kv(self.src[:, b * per_seq:], kind=kind, layer=layer, b0=b, nb=1, h0=0, nh=H, n0=P, nn=per_seq,
                  t0=loop_group * G, nt=G, s_loop=n * H * d, s_b=0, s_h=d, s_n=H * d)
        self.w = torch.from_numpy(gen.sample_weights(wl, n)).to(dev)
        self.assign = torch.empty((n, H, wl.groups), dtype=torch.int32, device=dev)
        self.ws = torch.empty(lvq.loopvq_lloyd_workspace(self.cfg, n), dtype=torch.uint8, device=dev)
        self.dist = torch.empty((H, wl.groups), dtype=torch.float64, device=dev)
        self.strides = dict(stride_loop=n * H * d, stride_token=H * d, stride_head=d)
        self.jc = loop_group if wl.codebook_per_loop_group else 0
        torch.cuda.synchronize()

    def step(self, e0=None, e1=None, e2=None):
        wl, lvq = self.wl, self.lvq
        if e0 is not None:
            e0.record()
        lvq.loopvq_encode(self.cfg, layer=self.layer, loop_group=self.j, kind=0, n_tokens=self.n, src=self.src,
                          seq_id=None, vq_pos=None, block_table=None, batch=1, max_pages_per_seq=1, num_pages=1,
                          cb=self.cb, cb_norms=self.norms, pool=None, out_idx=self.assign, **self.strides)
        if e1 is not None:
            e1.record()
        lvq.loopvq_lloyd_update(self.cfg, layer=self.layer, cb_set=self.jc, n_samples=self.n, src=self.src,
                                weight=self.w, cb=self.cb, cb_norms=self.norms, assign=self.assign,
                                workspace=self.ws, distortion=self.dist, **self.strides)
        if e2 is not None:
            e2.record()


def lloyd_cpu_baseline(wl, seconds: float, layer=0, loop_group=0, kind=0) -> dict:
    """The oracle's Lloyd iteration (fp64 brute-force assignment + plain weighted accumulation, one BLAS
    thread) on whole (kv-head, group) sample sets of the same workload."""
    from threadpoolctl import threadpool_limits
    from oracle import loopvq_oracle as O
    from synth import gen
    t_start = time.time()
    sc = gen.scales(wl)
    cb = gen.bf16_to_f64(gen.codebooks(wl, kind, sc, layers=[layer])[layer, 0])   # [H][NG][K][E]
    per_seq = wl.encode_tokens // wl.batch
    G, n = wl.loop_group, wl.encode_tokens
    w = gen.sample_weights(wl, n)
    planes = np.concatenate([gen.kv_tokens(wl, kind, layer, b, 0, wl.prefix, wl.prefix + per_seq, loop_group * G,
                                           loop_group * G + G, sc) for b in range(wl.batch)])     # [n][G][d], head 0
    x = O.subvectors(gen.bf16_to_f64(planes).transpose(1, 0, 2), wl.chans)                       # [n][NG][E]
    done, busy, groups = 0, 0.0, 0
    with threadpool_limits(limits=1):
        for g in range(wl.groups):
            c0 = time.perf_counter()
            O.lloyd_step(x[:, g], w[:, 0, g].astype(np.float64), cb[0, g])
            busy += time.perf_counter() - c0
            done += n
            groups += 1
            if busy >= seconds:
                break
    return {"value": done / busy, "unit": "sub-vectors/s", "cores": 1, "kind": "oracle", **host_cores(),
            "sample": (f"{groups} whole (kv-head 0, group) sample sets of {n} sub-vectors each of layer {layer}, "
                       f"loop group {loop_group}, kind {kind}: one weighted Lloyd iteration each (fp64 brute-force "
                       f"assignment over {wl.codewords} codewords, weighted means, bf16 rounding); {busy:.1f}s of "
                       f"timed oracle work, 1 BLAS thread; input setup untimed (wall {time.time() - t_start:.1f}s)")}


def lloyd_main(args):
    import torch
    from synth import workloads as W
    wl = W.BY_NAME[args.workload]
    torch.cuda.set_device(0)
    lb = LloydBench(wl)
    for _ in range(args.warmup):
        lb.step()
    E = torch.cuda.Event
    ev = [(E(enable_timing=True), E(enable_timing=True), E(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e in ev:
        lb.step(*e)
    torch.cuda.synchronize()
    t_as = np.array([a.elapsed_time(b) * 1e3 for a, b, _ in ev])
    t_up = np.array([b.elapsed_time(c) * 1e3 for _, b, c in ev])
    t_st = np.array([a.elapsed_time(c) * 1e3 for a, _, c in ev])
    subvec = wl.encode_tokens * wl.kv_heads * wl.groups
    compares = subvec * wl.codewords
    # update: every sample element read once, its index and weight once, the set's codebook read and written
    up_bytes = subvec * (wl.sub_len * 2 + 4 + 4) + 2 * wl.kv_heads * wl.groups * wl.codewords * wl.sub_len * 2
    a_us, u_us, s_us = float(t_as.mean()), float(t_up.mean()), float(t_st.mean())
    rec = {
        "metric": LLOYD_METRIC, "value": subvec / (s_us * 1e-6), "unit": "sub-vectors/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": s_us * 1e-3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "samples": wl.encode_tokens, "kv_heads": wl.kv_heads, "groups": wl.groups,
                   "sub_len": wl.sub_len, "codewords": wl.codewords, "layer": 0, "loop_group": 0, "kind": "K",
                   "weights": "seeded stand-ins for Fisher information, one per sample, 1 in 16 zero"},
        "roofline": {"bound": "alu", "achieved": compares / (a_us * 1e-6) / 1e12, "peak": VALU_PEAK_OPS / 1e12,
                     "unit": "Tcompare/s at one VALU op per compare", "frac": compares / (a_us * 1e-6) / VALU_PEAK_OPS,
                     "traffic": None, "kernel": "assignment (encode kernels without a pool)"},
        "update_roofline": {"bound": "hbm", "achieved": up_bytes / (u_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": up_bytes / (u_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                            "traffic": None, "bytes": up_bytes},
        "assign_us": a_us, "update_us": u_us,
        "step_us": {"mean": s_us, "p10": float(np.percentile(t_st, 10)), "p50": float(np.percentile(t_st, 50)),
                    "p90": float(np.percentile(t_st, 90))},
        "distortion_sum_last": float(lb.dist.sum().item()),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = lloyd_cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def copy_calibration(nbytes: int, reps: int) -> None:
    """A plain device copy of known size, for scaling HBM counters (rocprofv3 --pmc)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=None,
                    help="workload name (default: the 32K decode stack; --encode and --extend have their own)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, help="bytes; run only a plain copy (counter scaling)")
    ap.add_argument("--encode", action="store_true",
                    help="time the bulk encode of one (layer, loop group, kind) slice instead of the decode step "
                         "(default workload for this mode: deep4x32_h32_d128_b16_n8k)")
    ap.add_argument("--extend", action="store_true",
                    help="time extend (chunked prefill) attention over a packed cache instead of the decode step "
                         "(default workload for this mode: layer16h_d128_b32_n4k)")
    ap.add_argument("--chunk", type=int, default=512, help="chunk rows per sequence for --extend")
    ap.add_argument("--cb-per-loop-group", action="store_true",
                    help="decode mode: one codebook set per loop group instead of one shared by all loop groups")
    ap.add_argument("--plan", default=None,
                    help="decode mode: per-(layer, loop range) choice of (c, G), e.g. '8:4x4,24:8x4' "
                         "(layers separated by '/'; one entry applies to every layer)")
    ap.add_argument("--bf16-cache", action="store_true",
                    help="decode mode: the same kernel over an uncompressed bf16 cache (recent window = whole "
                         "context, no vector-quantized tokens), for the comparison with the packed cache")
    ap.add_argument("--eager", action="store_true",
                    help="decode mode: the headline times the step's launches issued one by one; by default it "
                         "times replays of the step captured in a HIP graph (the per-launch kernel times always "
                         "come from the eager steps)")
    ap.add_argument("--lloyd", action="store_true",
                    help="time one weighted Lloyd iteration of one codebook set instead of the decode step "
                         "(default workload for this mode: deep4x32_h32_d128_b16_n8k)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return
    if args.extend:
        args.workload = args.workload or "layer16h_d128_b32_n4k"
        extend_main(args)
        return
    if args.encode:
        args.workload = args.workload or "deep4x32_h32_d128_b16_n8k"
        encode_main(args)
        return
    if args.lloyd:
        args.workload = args.workload or "deep4x32_h32_d128_b16_n8k"
        lloyd_main(args)
        return
    args.workload = args.workload or DEFAULT_WORKLOAD
    import torch
    from synth import workloads as W
    wl = W.BY_NAME[args.workload]
    if args.cb_per_loop_group:
        wl = wl.with_(name=wl.name + "_cbj", codebook_per_loop_group=True)
    torch.cuda.set_device(0)
    plan = parse_plan(args.plan, wl) if args.plan else None
    if args.bf16_cache and plan:
        print(json.dumps({"error": "--bf16-cache takes no --plan"}))
        sys.exit(2)
    if args.bf16_cache:
        bench = Bf16Bench(wl)
        wl = bench.wl
    else:
        bench = MixedBench(wl, plan) if plan else Bench(wl)
    for _ in range(args.warmup):
        bench.step()
    torch.cuda.synchronize()
    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    evict_events = []
    for _ in range(args.steps):
        bench.step(events, evict_events)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = ev0.elapsed_time(ev1) / args.steps
    launch_us = np.array([a.elapsed_time(b) * 1e3 for a, b in events])
    graph = None
    if not args.eager:
        # the same step captured once and replayed: a serving loop replays its decode step the same
        # way; the difference to the eager step is the host launch overhead
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            bench.step()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            bench.step()
        g.replay()
        torch.cuda.synchronize()
        gv0, gv1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gv0.record()
        for _ in range(args.steps):
            g.replay()
        gv1.record()
        torch.cuda.synchronize()
        g_ms = gv0.elapsed_time(gv1) / args.steps
        graph = {"ms_per_step": g_ms, "queries_per_s": wl.layers * wl.loops * wl.queries_per_launch / (g_ms * 1e-3),
                 "eager_minus_graph_ms": step_ms - g_ms}
        log(f"graph replay: {g_ms:.3f} ms per step (eager {step_ms:.3f} ms)")
    eager_ms = step_ms
    if graph is not None:
        step_ms = graph["ms_per_step"]
    if plan:   # bytes of a launch averaged over the segments' launches
        ab_l = [algorithmic_bytes(wl.with_(chans=c, loop_group=G)) for segs in plan for n, c, G in segs
                for _ in range(n)]
        ab = {k: sum(a[k] for a in ab_l) / len(ab_l) for k in ab_l[0]}
    else:
        ab = algorithmic_bytes(wl)
    q_per_step = wl.layers * wl.loops * wl.queries_per_launch
    value = q_per_step / (step_ms * 1e-3)
    avg_us = float(launch_us.mean())
    achieved = ab["total"] / (avg_us * 1e-6) / 1e9
    # the committed counter summary covers the default workload's launches only
    traffic = traffic_from_profile() if (wl.name == DEFAULT_WORKLOAD and not plan) else None
    log(f"wall {wall:.2f}s for {args.steps} steps; launch avg {avg_us:.1f} us (p10 {np.percentile(launch_us, 10):.1f}, "
        f"p90 {np.percentile(launch_us, 90):.1f}); {achieved:.0f} GB/s")
    rec = {
        "metric": BF16_METRIC if args.bf16_cache else METRIC, "value": value, "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "loop_steps": wl.loops, "loop_group": wl.loop_group,
                   "q_heads": wl.q_heads, "kv_heads": wl.kv_heads, "head_dim": wl.head_dim, "batch": wl.batch,
                   "context": wl.context, "prefix_tokens": wl.prefix, "recent_tokens": wl.recent,
                   "chans_per_group": wl.chans, "index_bits": wl.index_bits,
                   "bits_per_elem": (16.0 if args.bf16_cache else
                                     plan_bits_per_elem(plan, wl.index_bits) if plan
                                     else wl.index_bits / (wl.chans * wl.loop_group)),
                   "cache": ("bf16: recent window = context - prefix, no vector-quantized tokens; one (layer, "
                             "loop step) K / V window pair (17.2 GB at 32K) is read by every launch of the step"
                             if args.bf16_cache else "packed indices + bf16 prefix / recent windows"),
                   "page_tokens": wl.page_tokens,
                   "codebook_per_loop_group": bool(wl.codebook_per_loop_group),
                   "plan": args.plan,
                   "launches_per_step": wl.layers * wl.loops,
                   "cache_replicas": (1 if args.bf16_cache else
                                      min(b.replicas for row in bench.segs for _, b in row) if plan
                                      else bench.replicas),
                   "eviction_launches_per_step": 0 if args.bf16_cache else (sum(len(s) for s in plan) if plan else 1),
                   "evicted_sub_vectors_per_step": (
                       0 if args.bf16_cache else
                       sum((n // G) * 2 * wl.batch * wl.kv_heads * (wl.head_dim // c)
                           for segs in plan for n, c, G in segs) if plan
                       else wl.layers * wl.loop_groups * 2 * wl.batch * wl.kv_heads * wl.groups)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic},
        "decode_launch_us": {"mean": avg_us, "p10": float(np.percentile(launch_us, 10)),
                             "p50": float(np.percentile(launch_us, 50)), "p90": float(np.percentile(launch_us, 90))},
        "algorithmic_bytes_per_launch": ab,
        "evict_launch_us": (float(np.mean([a.elapsed_time(b) * 1e3 for a, b in evict_events]))
                            if evict_events else None),
        "step_gbps": ab["total"] * wl.layers * wl.loops / (step_ms * 1e-3) / 1e9,
        "step_timing": "eager" if graph is None else "hip_graph_replay",
        "eager_ms_per_step": eager_ms,
        "eager_queries_per_s": q_per_step / (eager_ms * 1e-3),
    }
    if not args.no_cpu_baseline:
        # with a plan: the oracle on the workload of layer 0's first segment
        if plan or args.bf16_cache:
            base = wl.with_(chans=plan[0][0][1], loop_group=plan[0][0][2]) if plan else wl
            rec["cpu_baseline"] = cpu_baseline(base, args.cpu_seconds)
        else:
            rec["cpu_baseline"] = cpu_baseline_gpu_pages(bench, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
