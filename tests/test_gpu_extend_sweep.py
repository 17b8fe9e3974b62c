"""Seeded random extend shapes against the oracle (needs an MI355X).

Each case draws head_dim / channels per group / rotation, the GQA ratio, the page size, the
cached lengths (empty, prefix-only and vector-quantized caches alike), the chunk size and the
per-sequence chunk lengths from a fixed seed, so the sweep is the same on every run.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

pytest.importorskip("torch")
pytest.importorskip("lvq_harness")

from synth import workloads as W  # noqa: E402
from test_gpu_extend import _run_extend_case  # noqa: E402


def _draw(seed):
    rng = np.random.default_rng(1000 + seed)
    kind = seed % 4
    if kind == 0:      # d=64, c=4
        base = W.TINY
    elif kind == 1:    # d=128, c=4
        base = W.LAYER_4K
    elif kind == 2:    # d=128, c=8, rotated keys
        base = W.QUARTER_16K.with_(layers=1)
    else:              # d=128, c=8 without a rotation
        base = W.QUARTER_16K.with_(layers=1, rotate_keys=False)
    kv = int(rng.choice([1, 2]))
    grp = int(rng.choice([1, 2, 4]))
    batch = int(rng.integers(1, 4))
    lens = [int(x) for x in rng.choice([0, 5, 72, 73, 137, 300, 641, 1000], size=batch)]
    M = int(rng.choice([1, 17, 64, 100, 200]))
    clens = [int(x) for x in rng.integers(0, M + 1, size=batch)] if rng.random() < 0.5 else None
    page = int(rng.choice([64, 128, 256]))
    wl = base.with_(batch=batch, q_heads=kv * grp, kv_heads=kv, context=max(lens + [1]), page_tokens=page)
    loop = int(rng.integers(0, wl.loops))
    return wl, 0, loop, lens, M, clens


@pytest.mark.parametrize("seed", range(8))
def test_extend_random_shapes(seed):
    wl, layer, loop, lens, M, clens = _draw(seed)
    name = (f"sweep{seed}: d={wl.head_dim} c={wl.chans} rot={wl.rotate_keys} Hq/Hkv={wl.q_heads}/{wl.kv_heads} "
            f"page={wl.page_tokens} loop={loop} chunk_lens={clens}")
    _run_extend_case(name, wl, layer, loop, lens, M, clens, seed=seed)
