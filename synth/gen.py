"""Seeded, counter-based synthetic inputs (host side, NumPy).

Both the CPU oracle and the GPU path consume these values; the GPU side either
uploads them or regenerates the same bits on the device with the twin kernel in
``synth/synth_device.hip``.  Nothing here computes any part of LoopVQ itself
(no distances, no argmin, no packing, no attention): it only draws the K/V
cache, the codebooks and the queries, and rounds them to bf16.

Generator (identical on host and device, bit for bit)
-----------------------------------------------------
* Uniform bits: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014) evaluated at a position: the i-th output of
  the stream keyed by ``key`` is ``mix64(key + (i + 1) * GAMMA)``.  Being a pure
  function of (key, i), it is a counter-based generator.
* Standard normals: each 64-bit output is cut into four 16-bit fields r, and a
  field maps to the normal quantile ``ndtri((r + 0.5) / 65536)`` looked up in a
  65536-entry fp64 table (inverse-CDF sampling on a 2**16-point grid).
* Loop-axis correlation: AR(1) along loop steps, ``x_0 = e_0`` and
  ``x_t = 0.9 * x_{t-1} + sqrt(1 - 0.81) * e_t`` (stationary, unit variance),
  evaluated in fp64 as two rounded products and one rounded sum.
* Per-channel scale ``s = exp(0.5 z)``, z ~ N(0, 1) (lognormal(0, 0.5)), one per
  (layer, kv-head, K/V, channel); ``outlier_channels`` key channels per
  (layer, kv-head) are multiplied by ``outlier_scale``.  Scales come from NumPy's
  PCG64 and are handed to the device as a table.
* Optional key rotation (the 0.25-bit workload): keys are multiplied by R^T
  where R = diag(sigma) H / sqrt(d), H the Sylvester-Hadamard matrix and sigma a
  seeded +-1 vector.  R^T k is evaluated as sign flips, an in-place fast
  Walsh-Hadamard transform with stages h = 1, 2, 4, ... (a + b, a - b), then one
  rounded product by 1/sqrt(d).
* Rounding: fp64 -> fp32 (round to nearest even) -> bf16 (round to nearest even).
"""
from __future__ import annotations

import numpy as np
from scipy.special import ndtri

from .workloads import Workload

BASE_SEED = 20261103
GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
AR_RHO = 0.9
AR_INNOV = float(np.sqrt(1.0 - AR_RHO * AR_RHO))

# stream ids
S_DATA, S_CODEBOOK, S_QUERY, S_SCALES, S_ROT, S_INDEX, S_WEIGHT = 1, 2, 3, 4, 5, 6, 7

_TABLE = None


def normal_table() -> np.ndarray:
    """fp64[65536]: standard-normal quantiles at (r + 0.5) / 65536."""
    global _TABLE
    if _TABLE is None:
        r = np.arange(65536, dtype=np.float64)
        _TABLE = ndtri((r + 0.5) / 65536.0)
        _TABLE.setflags(write=False)
    return _TABLE


def mix64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    z = (z ^ (z >> np.uint64(30))) * M1
    z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def stream_key(wl: Workload, stream: int) -> np.uint64:
    v = (np.uint64(BASE_SEED) << np.uint64(16)) + (np.uint64(wl.wid) << np.uint64(8)) + np.uint64(stream)
    return mix64(np.array([v], dtype=np.uint64))[0]


def uniform_u64(key: np.uint64, i: np.ndarray) -> np.ndarray:
    i = np.asarray(i, dtype=np.uint64)
    return mix64(np.uint64(key) + (i + np.uint64(1)) * GAMMA)


def normals(key: np.uint64, j: np.ndarray) -> np.ndarray:
    """Standard normal number j of the stream (j: uint64 array)."""
    j = np.asarray(j, dtype=np.uint64)
    u = uniform_u64(key, j >> np.uint64(2))
    r = (u >> ((j & np.uint64(3)) * np.uint64(16))) & np.uint64(0xFFFF)
    return normal_table()[r.astype(np.int64)]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE); returns uint16 bit patterns."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def sample_weights(wl: Workload, n: int, salt: int = 0) -> np.ndarray:
    """fp32 [n][Hkv][NG] per-sample weights standing in for Fisher information in codebook
    learning: (1 + m) * 2**-23 with m the top 24 bits of the stream (so in (0, 2], exact in
    fp32), and 0 for one sample in 16 (the low 4 bits zero)."""
    cnt = n * wl.kv_heads * wl.groups
    with np.errstate(over="ignore"):
        key = stream_key(wl, S_WEIGHT) + np.uint64(salt) * GAMMA
    u = uniform_u64(key, np.arange(cnt, dtype=np.uint64))
    w = ((u >> np.uint64(40)).astype(np.float64) + 1.0) * 2.0 ** -23
    w[(u & np.uint64(15)) == 0] = 0.0
    return w.astype(np.float32).reshape(n, wl.kv_heads, wl.groups)


def loops_padded(T: int) -> int:
    return 4 * ((T + 3) // 4)


# ---------------------------------------------------------------------------
# Host-only tables (scales, outliers, rotation signs)
# ---------------------------------------------------------------------------
def scales(wl: Workload) -> np.ndarray:
    """fp64 [L][Hkv][2 (K, V)][d] per-channel scales, outliers folded in."""
    out = np.empty((wl.layers, wl.kv_heads, 2, wl.head_dim), dtype=np.float64)
    for l in range(wl.layers):
        for h in range(wl.kv_heads):
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
                [BASE_SEED, wl.wid, S_SCALES, l, h])))
            z = rng.standard_normal((2, wl.head_dim))
            s = np.exp(0.5 * z)
            if wl.outlier_channels:
                ch = rng.choice(wl.head_dim, wl.outlier_channels, replace=False)
                s[0, ch] *= wl.outlier_scale
            out[l, h] = s
    return out


def rotation_signs(wl: Workload) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, wl.wid, S_ROT])))
    return (rng.integers(0, 2, wl.head_dim) * 2 - 1).astype(np.float64)


def inv_sqrt_d(wl: Workload) -> float:
    return float(1.0 / np.sqrt(np.float64(wl.head_dim)))


def rotation_matrix_f32(wl: Workload) -> np.ndarray:
    """R (fp32 [d][d], row-major) with keys stored as R^T k; None-equivalent identity if unrotated.

    R = diag(sigma) H / sqrt(d): R[i][j] = sigma_i * H[i][j] / sqrt(d), H[i][j] = (-1)^popcount(i & j).
    """
    d = wl.head_dim
    i = np.arange(d)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    H = np.where(pc % 2 == 0, 1.0, -1.0)
    R = rotation_signs(wl)[:, None] * H * inv_sqrt_d(wl)
    return R.astype(np.float32)


def _fwht_rows(v: np.ndarray) -> np.ndarray:
    """In-place-order fast Walsh-Hadamard transform along the last axis (fp64)."""
    v = v.copy()
    d = v.shape[-1]
    h = 1
    while h < d:
        w = v.reshape(v.shape[:-1] + (d // (2 * h), 2, h))
        a = w[..., 0, :].copy()
        b = w[..., 1, :].copy()
        w[..., 0, :] = a + b
        w[..., 1, :] = a - b
        v = w.reshape(v.shape)
        h *= 2
    return v


# ---------------------------------------------------------------------------
# K/V process
# ---------------------------------------------------------------------------
def _kv_raw(wl: Workload, key: np.uint64, elem_base: np.ndarray, sc: np.ndarray, t1: int,
            kind: int) -> np.ndarray:
    """fp64 [..., t1, d] values s * x_t for loops [0, t1) of the elements elem_base[..., ch]."""
    T4 = loops_padded(wl.loops)
    x = None
    outs = []
    for t in range(t1):
        e = normals(key, elem_base * np.uint64(T4) + np.uint64(t))
        x = e if x is None else AR_RHO * x + AR_INNOV * e
        outs.append(sc * x)
    v = np.stack(outs, axis=-2)
    if kind == 0 and wl.rotate_keys:
        v = _fwht_rows(v * rotation_signs(wl)) * inv_sqrt_d(wl)
    return v


def kv_tokens(wl: Workload, kind: int, l: int, b: int, h: int, n0: int, n1: int,
              t0: int, t1: int, sc: np.ndarray | None = None) -> np.ndarray:
    """bf16 bits [n1-n0][t1-t0][d]: cache values of tokens [n0, n1), loops [t0, t1).

    kind 0 = keys, 1 = values.  Token n of sequence b is the same value wherever
    it sits (prefix window, VQ region or recent window).
    """
    d = wl.head_dim
    if sc is None:
        sc = scales(wl)
    n = np.arange(n0, n1, dtype=np.uint64)
    ch = np.arange(d, dtype=np.uint64)
    row = np.uint64((((kind * wl.layers + l) * wl.batch + b) * wl.kv_heads + h) * wl.context)
    elem = (row + n[:, None]) * np.uint64(d) + ch[None, :]
    v = _kv_raw(wl, stream_key(wl, S_DATA), elem, sc[l, h, kind][None, :], t1, kind)
    return to_bf16_bits(v[:, t0:t1, :])


def codebook_tokens(wl: Workload, kind: int, l: int, h: int,
                    sc: np.ndarray | None = None) -> np.ndarray:
    """bf16 bits [K][T][d]: the K fresh tokens (independent stream) whose sub-vectors form the codebooks."""
    d, K = wl.head_dim, wl.codewords
    if sc is None:
        sc = scales(wl)
    n = np.arange(K, dtype=np.uint64)
    ch = np.arange(d, dtype=np.uint64)
    row = np.uint64(((kind * wl.layers + l) * wl.kv_heads + h) * K)
    elem = (row + n[:, None]) * np.uint64(d) + ch[None, :]
    v = _kv_raw(wl, stream_key(wl, S_CODEBOOK), elem, sc[l, h, kind][None, :], wl.loops, kind)
    return to_bf16_bits(v)


def codebooks(wl: Workload, kind: int, sc: np.ndarray | None = None, layers=None) -> np.ndarray:
    """bf16 bits [L][Jcb][Hkv][d/c][K][c*G]: codebook rows in the library's input format.

    Row k of (layer l, codebook loop group jc, head h, group g) is fresh token k's
    channels [g*c, g*c + c) over loop steps jc*G .. jc*G + G - 1, loop-major
    (element tau*c + i).  With ``layers`` given, only those layers are filled (the rest stay zero).
    """
    if sc is None:
        sc = scales(wl)
    L, Jc, H, NG, K, c, G = (wl.layers, wl.cb_loop_groups, wl.kv_heads, wl.groups,
                             wl.codewords, wl.chans, wl.loop_group)
    out = np.zeros((L, Jc, H, NG, K, c * G), dtype=np.uint16)
    for l in (range(L) if layers is None else layers):
        for h in range(H):
            tok = codebook_tokens(wl, kind, l, h, sc)          # [K][T][d]
            for jc in range(Jc):
                blk = tok[:, jc * G:(jc + 1) * G, :]            # [K][G][d]
                blk = blk.reshape(K, G, NG, c).transpose(2, 0, 1, 3)   # [NG][K][G][c]
                out[l, jc, h] = blk.reshape(NG, K, G * c)
    return out


def queries(wl: Workload, l: int, t: int) -> np.ndarray:
    """bf16 bits [B][Hq][d]: decode queries of layer l, loop step t (N(0, 1))."""
    B, Hq, d = wl.batch, wl.q_heads, wl.head_dim
    j = ((np.uint64((l * wl.loops + t) * B) + np.arange(B, dtype=np.uint64)[:, None, None])
         * np.uint64(Hq) + np.arange(Hq, dtype=np.uint64)[None, :, None]) * np.uint64(d) \
        + np.arange(d, dtype=np.uint64)[None, None, :]
    return to_bf16_bits(normals(stream_key(wl, S_QUERY), j))


def random_indices(wl: Workload, kind: int, l: int, j: int, b: int, h: int, n_tok: int) -> np.ndarray:
    """int64 [n_tok][d/c]: uniform codebook indices (top b bits of one 64-bit draw each).

    Used where a test needs a packed cache at full size without encoding it.
    """
    NG = wl.groups
    row = np.uint64(((((kind * wl.layers + l) * wl.loop_groups + j) * wl.batch + b)
                     * wl.kv_heads + h) * wl.context)
    i = (row + np.arange(n_tok, dtype=np.uint64)[:, None]) * np.uint64(NG) \
        + np.arange(NG, dtype=np.uint64)[None, :]
    u = uniform_u64(stream_key(wl, S_INDEX), i)
    return (u >> np.uint64(64 - wl.index_bits)).astype(np.int64)


def context_lengths(wl: Workload, ragged: bool = False, seed: int = 0) -> np.ndarray:
    """int32 [B] cached-token counts (includes the token being decoded)."""
    if not ragged:
        return np.full(wl.batch, wl.context, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, wl.wid, 99, seed])))
    n = rng.integers(1, wl.context + 1, wl.batch)
    n[0] = wl.context
    return n.astype(np.int32)
