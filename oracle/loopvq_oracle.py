"""Plain fp64 CPU oracle for LoopVQ decode attention and encode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module:
only the tests, the smoke check and the CPU-baseline leg of the benchmark use it.
It shares no code with the HIP library (no headers, kernels, tables or helpers);
the only thing both sides consume is the seeded input generator in ``synth/``.

Sources (pages as titled; sections named, never line numbers)
-------------------------------------------------------------
[ABS]  "LoopVQ: Sub 1-bit KV Cache Quantization for Looped Transformers",
       shd-paper.top listing of arXiv 2611.05304, English abstract: every loop step
       keeps its own K and V; LoopVQ vector-quantizes the KV cache by coding the
       channels of several loop steps jointly; 0.5 and 0.25 bits per element.
[AIR]  airadar.tv summary of LoopVQ, opening summary: the channels of several
       *consecutive* loop steps form one sub-vector that shares a single codebook
       index; section "Raisons": the serving branch stores packed indices and
       uses fused decode kernels; section "Utilisation": 8 prefix and 64 recent
       tokens stay bf16.
[KC]   kongchang.com entry "LoopVQ": channels across several recurrent steps are
       encoded jointly instead of step by step.

Readings where the pages are silent (each one is listed in the design notes)
--------------------------------------------------------------------------
* sub-vector element order is loop-major: element tau*c + i is channel g*c + i
  of loop step j*G + tau;
* loop groups are [j*G, j*G + G) and T must be a multiple of G;
* encode distance is the plain squared Euclidean distance, ties go to the
  lowest index; K and V are quantized with separate codebooks;
* bits per element = b / (c * G) counts index bits only;
* context split: tokens [0, P) prefix, [P, N - R) vector-quantized, the rest
  recent; N includes the token being decoded; no mask inside the cache;
* softmax scale 1/sqrt(d) unless given; a key rotation R is undone by q' = R^T q;
* packed layout: see ``page_layout`` below;
* codebook learning ([AIR] opening summary, Fisher-weighted k-means): one scalar
  weight per sample (sub-vector) stands in for the Fisher weight, the assignment is
  the encode rule, a codeword that receives no weight keeps its value, and the new
  codeword is the weighted mean rounded to bf16 (the codebook's storage type).

Pins that tie this file to something other than itself live in
``tests/test_oracle_pins.py`` (brute force, scipy, closed forms, hand-worked
examples under ``tests/golden/``, exact-codebook and special-case identities).
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# Configuration
# ---------------------------------------------------------------------------
def check_config(T: int, G: int, Hq: int, Hkv: int, d: int, c: int, b: int,
                 PT: int = 64) -> None:
    """Raise ValueError unless the shape is one the method defines.

    [AIR] opening summary: one index covers c channels of G consecutive loop
    steps, so G must divide T and c must divide d.  K = 2**b codewords.
    """
    if min(T, G, Hq, Hkv, d, c, b, PT) <= 0:
        raise ValueError("all sizes must be positive")
    if T % G:
        raise ValueError("loop count T must be a multiple of the loop group G")
    if d % c:
        raise ValueError("head_dim must be a multiple of c")
    if Hq % Hkv:
        raise ValueError("q heads must be a multiple of kv heads")
    if not 1 <= b <= 16:
        raise ValueError("index bits must be in [1, 16]")
    if (d // c) % 4 or PT % 4:
        raise ValueError("packed micro-tiles need d/c and page_tokens divisible by 4")


def bits_per_elem(b: int, c: int, G: int) -> float:
    """One b-bit index per c*G cache elements ([ABS]: 0.5 and 0.25 bit/elem)."""
    return b / (c * G)


# ---------------------------------------------------------------------------
# Sub-vectors and encode
# ---------------------------------------------------------------------------
def subvectors(planes: np.ndarray, c: int) -> np.ndarray:
    """[G][n][d] values of one loop group -> [n][d/c][c*G] sub-vectors.

    [AIR] opening summary / [ABS]: channels of several consecutive loop steps are
    grouped into one sub-vector.  Element tau*c + i of group g is channel
    g*c + i of loop step tau of the group.
    """
    G, n, d = planes.shape
    NG = d // c
    x = np.empty((n, NG, c * G), dtype=np.float64)
    for tau in range(G):
        for g in range(NG):
            x[:, g, tau * c:(tau + 1) * c] = planes[tau, :, g * c:(g + 1) * c]
    return x


def sq_dists(x: np.ndarray, C: np.ndarray) -> np.ndarray:
    """Squared Euclidean distance of every row of x [n][E] to every codeword C [K][E], fp64."""
    D = np.zeros((x.shape[0], C.shape[0]), dtype=np.float64)
    for e in range(x.shape[1]):
        diff = x[:, e][:, None] - C[:, e][None, :]
        D += diff * diff
    return D


def encode(x: np.ndarray, C: np.ndarray, chunk: int = 2048):
    """Nearest codeword by brute force over all K codewords.

    Returns (idx, d1, d2): the lowest index attaining the minimum squared
    distance, the minimum, and the second-smallest distance over the other
    codewords (d2 = d1 when the minimum is shared).
    """
    n = x.shape[0]
    idx = np.empty(n, dtype=np.int64)
    d1 = np.empty(n, dtype=np.float64)
    d2 = np.empty(n, dtype=np.float64)
    for s in range(0, n, chunk):
        D = sq_dists(x[s:s + chunk], C)
        k = np.argmin(D, axis=1)               # first occurrence = lowest index
        rows = np.arange(D.shape[0])
        best = D[rows, k]
        D[rows, k] = np.inf
        idx[s:s + chunk] = k
        d1[s:s + chunk] = best
        d2[s:s + chunk] = D.min(axis=1) if C.shape[0] > 1 else np.inf
    return idx, d1, d2


# ---------------------------------------------------------------------------
# Packed index layout
# ---------------------------------------------------------------------------
def page_layout(PT: int, NG: int, b: int) -> dict:
    """Byte layout of one page ([AIR] "Raisons": indices are stored packed).

    A page holds PT consecutive vector-quantized positions of one
    (layer, loop group, kv-head): [kind K then V][PT/4 token quads][NG/4 group
    quads][one micro-tile of 2*b bytes].  A micro-tile packs 16 indices,
    element e = 4*i + r being token 4*Q + i, group 4*u + r; bit beta of element
    e sits at bit e*b + beta of the tile read as a little-endian integer.
    """
    tile = 2 * b
    kind_bytes = (PT // 4) * (NG // 4) * tile
    return {"tile_bytes": tile, "kind_bytes": kind_bytes, "page_bytes": 2 * kind_bytes}


def pack_tile(vals, b: int) -> bytes:
    """16 b-bit integers -> 2*b bytes, bit by bit."""
    out = bytearray(2 * b)
    for e, v in enumerate(vals):
        v = int(v)
        if not 0 <= v < (1 << b):
            raise ValueError("index out of range")
        for beta in range(b):
            if (v >> beta) & 1:
                pos = e * b + beta
                out[pos // 8] |= 1 << (pos % 8)
    return bytes(out)


def unpack_tile(data: bytes, b: int) -> list:
    vals = []
    for e in range(16):
        v = 0
        for beta in range(b):
            pos = e * b + beta
            v |= ((data[pos // 8] >> (pos % 8)) & 1) << beta
        vals.append(v)
    return vals


def pack_tiles(vals: np.ndarray, b: int) -> np.ndarray:
    """Array form of pack_tile: [..., 16] ints -> [..., 2*b] uint8, one bit field at a time."""
    vals = np.asarray(vals, dtype=np.int64)
    if vals.size and (vals.min() < 0 or vals.max() >= (1 << b)):
        raise ValueError("index out of range")
    out = np.zeros(vals.shape[:-1] + (2 * b,), dtype=np.int64)
    for e in range(16):
        for beta in range(b):
            pos = e * b + beta
            out[..., pos // 8] |= ((vals[..., e] >> beta) & 1) << (pos % 8)
    return out.astype(np.uint8)


def unpack_tiles(data: np.ndarray, b: int) -> np.ndarray:
    data = np.asarray(data, dtype=np.int64)
    vals = np.zeros(data.shape[:-1] + (16,), dtype=np.int64)
    for e in range(16):
        for beta in range(b):
            pos = e * b + beta
            vals[..., e] |= ((data[..., pos // 8] >> (pos % 8)) & 1) << beta
    return vals


def _to_tiles(idx: np.ndarray, n_pages: int, PT: int) -> np.ndarray:
    """[n][NG] -> [n_pages][PT/4][NG/4][16] with element 4*i + r = (token 4Q+i, group 4u+r); pad with 0."""
    n, NG = idx.shape
    full = np.zeros((n_pages * PT, NG), dtype=np.int64)
    full[:n] = idx
    t = full.reshape(n_pages, PT // 4, 4, NG // 4, 4)          # [p][Q][i][u][r]
    return t.transpose(0, 1, 3, 2, 4).reshape(n_pages, PT // 4, NG // 4, 16)


def _from_tiles(vals: np.ndarray, n: int, NG: int) -> np.ndarray:
    n_pages, Qn, Un, _ = vals.shape
    t = vals.reshape(n_pages, Qn, Un, 4, 4).transpose(0, 1, 3, 2, 4)   # [p][Q][i][u][r]
    return t.reshape(n_pages * Qn * 4, Un * 4)[:n]


def pack_sequence(idx_k: np.ndarray, idx_v: np.ndarray, PT: int, b: int) -> np.ndarray:
    """Indices of one (layer, loop group, kv-head, sequence) -> its pages, uint8 [n_pages][page_bytes]."""
    n, NG = idx_k.shape
    lay = page_layout(PT, NG, b)
    n_pages = max(1, -(-n // PT))
    pages = np.empty((n_pages, 2, lay["kind_bytes"]), dtype=np.uint8)
    for kind, idx in enumerate((idx_k, idx_v)):
        tiles = pack_tiles(_to_tiles(idx, n_pages, PT), b)
        pages[:, kind, :] = tiles.reshape(n_pages, -1)
    return pages.reshape(n_pages, lay["page_bytes"])


def unpack_sequence(pages: np.ndarray, n: int, NG: int, PT: int, b: int):
    """Inverse of pack_sequence: pages [n_pages][page_bytes] -> (idx_k, idx_v) [n][NG]."""
    lay = page_layout(PT, NG, b)
    n_pages = pages.shape[0]
    p = pages.reshape(n_pages, 2, PT // 4, NG // 4, lay["tile_bytes"])
    return tuple(_from_tiles(unpack_tiles(p[:, kind], b), n, NG) for kind in range(2))


def pool_offset(l: int, j: int, h: int, page: int, J: int, Hkv: int, num_pages: int,
                page_bytes: int) -> int:
    """Byte offset of a page in the pool [L][J][Hkv][num_pages][page_bytes].

    [AIR] "Raisons" says only that the indices are stored packed; this pool order (layer,
    loop group, kv-head, page, row-major) is the reading that the library shares.
    """
    return (((l * J + j) * Hkv + h) * num_pages + page) * page_bytes


# ---------------------------------------------------------------------------
# Dequantize and attend
# ---------------------------------------------------------------------------
def dequantize(idx: np.ndarray, C: np.ndarray, tau: int, c: int) -> np.ndarray:
    """Rebuild loop step tau of the cache: row n, channels [g*c, g*c+c) = C[g][idx[n][g]][tau*c : tau*c+c]."""
    n, NG = idx.shape
    out = np.empty((n, NG * c), dtype=np.float64)
    for g in range(NG):
        out[:, g * c:(g + 1) * c] = C[g][idx[:, g], tau * c:(tau + 1) * c]
    return out


def attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
              rot: np.ndarray | None = None):
    """Softmax attention of one query over all cached rows, fp64.

    Scores s_n = scale * (q' . k_n) with q' = R^T q when keys are stored rotated
    (k' = R^T k, so q' . k' = q . k for orthogonal R).  Returns (o, lse) with
    lse the natural log of sum_n exp(s_n).
    """
    qq = np.asarray(q, dtype=np.float64)
    if rot is not None:
        qq = np.asarray(rot, dtype=np.float64).T @ qq
    if keys.shape[0] == 0:
        # an empty context (N = 0): the softmax sum is empty, so lse = ln 0 = -inf, and the
        # output is the empty sum of weighted values, 0 (reading: the pages never decode
        # with nothing cached; this is the limit a caller can rely on)
        return np.zeros(values.shape[1], dtype=np.float64), -np.inf
    s = scale * (keys @ qq)
    m = s.max()
    p = np.exp(s - m)
    z = p.sum()
    o = (p[:, None] * values).sum(axis=0) / z
    return o, m + np.log(z)


def split_context(N: int, P: int, R: int):
    """(n_prefix, n_vq, n_recent) for a sequence of N >= 0 cached tokens ([AIR] "Utilisation")."""
    if N < 0:
        raise ValueError("a sequence holds N >= 0 tokens")
    n_prefix = min(P, N)
    n_vq = max(0, N - P - R)
    return n_prefix, n_vq, N - n_prefix - n_vq


def decode_query(q, k_prefix, v_prefix, idx_k, idx_v, cb_k, cb_v, k_recent, v_recent,
                 tau: int, c: int, scale: float, rot=None):
    """Attention output of one decode query over [prefix | vector-quantized | recent] rows.

    Window rows are exact bf16; VQ rows are dequantized from the loop-step-tau
    slice of the key and value codebooks of the query's (layer, head).
    """
    keys = np.concatenate([k_prefix, dequantize(idx_k, cb_k, tau, c), k_recent], axis=0)
    vals = np.concatenate([v_prefix, dequantize(idx_v, cb_v, tau, c), v_recent], axis=0)
    return attention(q, keys, vals, scale, rot)


def extend_attention(q_rows, k_prefix, v_prefix, idx_k, idx_v, cb_k, cb_v, k_recent, v_recent,
                     k_chunk, v_chunk, tau: int, c: int, scale: float, rot=None):
    """Chunked prefill ("extend") of M new tokens over one sequence's cache, fp64.

    The serving command in [AIR] "Utilisation" names a separate prefill backend; the
    pages say nothing more.  Reading: row i of the chunk attends over the whole cached
    context exactly as a decode query does ([prefix | vector-quantized | recent]) plus
    the chunk's own bf16 rows 0..i (causal inside the chunk).  Window order does not
    matter, so the chunk rows join the recent window.  Returns (o [M][d], lse [M]).
    """
    M = q_rows.shape[0]
    d = k_chunk.shape[1]
    o = np.empty((M, d), dtype=np.float64)
    lse = np.empty(M, dtype=np.float64)
    for i in range(M):
        kr = np.concatenate([k_recent, k_chunk[:i + 1]], axis=0)
        vr = np.concatenate([v_recent, v_chunk[:i + 1]], axis=0)
        o[i], lse[i] = decode_query(q_rows[i], k_prefix, v_prefix, idx_k, idx_v, cb_k, cb_v, kr, vr, tau, c,
                                    scale, rot)
    return o, lse


# ---------------------------------------------------------------------------
# Codebook learning: weighted Lloyd iterations
# ---------------------------------------------------------------------------
def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 value (round half to even), returned as fp64.

    Written out from the format: bf16 keeps 8 significant bits and the fp32 exponent
    range.  With v = m * 2**e, 0.5 <= |m| < 1, a normal bf16 near v is spaced 2**(e - 8)
    apart; below the smallest normal 2**-126 (e < -125) the spacing stays 2**-133
    (subnormals).  So the result is round_half_even(v / q) * q with q = 2**(max(e, -125) - 8).
    A magnitude that rounds above the largest finite bf16, (2 - 2**-7) * 2**127, becomes
    an infinity of the same sign (the tie at the overflow threshold rounds up, to the
    even significand), as IEEE round-to-nearest-even prescribes.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    qe = np.maximum(e, -125) - 8
    r = np.ldexp(np.round(np.ldexp(v, -qe)), qe)
    big = np.abs(r) > BF16_MAX
    return np.where(big, np.copysign(np.inf, v), r)


BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def lloyd_step(x: np.ndarray, w: np.ndarray, C: np.ndarray, to_bf16: bool = True):
    """One Fisher-weighted Lloyd iteration for one codebook ([AIR] opening summary: the codebook
    comes from k-means weighted by Fisher information, before the output-matching fine-tune,
    which is not part of this path).

    x [n][E] sub-vectors, w [n] non-negative weights (the Fisher weights; synthetic here),
    C [K][E] current codebook.  Assignment: the encode rule (nearest, lowest index on ties).
    Update: each codeword that received weight becomes the weighted mean of its sub-vectors,
    sum_n w_n x_n / sum_n w_n; a codeword with no weight keeps its value (reading: the pages
    are silent on empty clusters).  Codebooks are stored in bf16, so the new codeword is the
    mean rounded to bf16 (to_bf16=False keeps fp64, for the pins).
    Returns (assign [n], C_new [K][E], distortion), distortion = sum_n w_n ||x_n - C[a_n]||^2
    against the codebook the assignment used.
    """
    K, E = C.shape
    a, d1, _ = encode(x, C)
    distortion = float(np.sum(w * d1))
    wsum = np.zeros(K)
    sums = np.zeros((K, E))
    for n in range(x.shape[0]):            # plain accumulation, row order
        wsum[a[n]] += w[n]
        sums[a[n]] += w[n] * x[n]
    C_new = C.astype(np.float64).copy()
    hit = wsum > 0
    mean = sums[hit] / wsum[hit][:, None]
    C_new[hit] = round_to_bf16(mean) if to_bf16 else mean
    return a, C_new, distortion


def near_tie(d1: np.ndarray, d2: np.ndarray, rel: float = 1e-6) -> np.ndarray:
    """Sub-vectors whose two best distances are within rel of each other (several correct indices)."""
    return (d2 - d1) <= rel * d2
