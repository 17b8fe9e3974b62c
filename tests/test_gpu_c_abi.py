"""Decode driven from plain C through loopvq.h alone (needs an MI355X).

tests/c_abi/decode_c.c (linked by build()) owns every device buffer, sizes them
with loopvq_layout_query and loopvq_decode_attn_workspace, prepares the
codebooks and runs one decode launch; its output must equal the Python
binding's output on the same inputs bit for bit (the decode kernel's fixed-point
histograms make it reproducible) and the oracle's within the attention
tolerance.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("lvq_harness")

from synth import workloads as W  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi", "decode_c")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _write_inputs(path, case, pool_slice, num_splits, scale):
    wl, cfg = case.wl, case.cfg
    args = {name: getattr(cfg, name) for name, _ in cfg._fields_}
    args.update(layer=case.l, loop=case.t, batch=wl.batch, max_pages_per_seq=case.paging.max_pages,
                max_seq_len=int(case.lens.max()), num_splits=num_splits, num_pages=case.paging.num_pages,
                pool_offset=case.pool_shift, pool_slice_bytes=pool_slice.size, softmax_scale=scale,
                has_rot=int(case.rot is not None))
    with open(os.path.join(path, "args.txt"), "w") as f:
        for k, v in args.items():
            f.write(f"{k} {v}\n")
    files = {"q.bin": case.q, "lens.bin": case.lens.astype(np.int32), "bt.bin": case.paging.table.astype(np.int32),
             "pool.bin": pool_slice, "cbk.bin": case.cbk, "cbv.bin": case.cbv, "kp.bin": case.kp,
             "vp.bin": case.vp, "kr.bin": case.kr, "vr.bin": case.vr}
    if case.rot is not None:
        files["rot.bin"] = np.asarray(case.rot, np.float32)
    for name, arr in files.items():
        np.ascontiguousarray(arr).tofile(os.path.join(path, name))


CASES = [
    ("tiny_ragged", W.TINY.with_(batch=3, q_heads=2, kv_heads=2, context=900), 0, 2, [900, 73, 300], 0),
    ("quarter_rot_layer1", W.QUARTER_16K.with_(layers=2, batch=2, q_heads=4, kv_heads=2, context=1300),
     1, 3, [1300, 650], 3),
]


@pytest.mark.parametrize("name,wl,layer,loop,lens,splits", CASES, ids=[c[0] for c in CASES])
def test_c_caller_matches_binding_and_oracle(tmp_path, name, wl, layer, loop, lens, splits):
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build() first"
    case = H.Case(wl, layer, loop, lens, seed=12)
    exp = case.oracle_encode()
    idx_of = lambda k, b, h: exp[k, b, h][0]  # noqa: E731
    pool_ref = case.oracle_pool(idx_of)
    case.gpu_setup()
    scale = 0.0
    _write_inputs(str(tmp_path), case, pool_ref.reshape(-1), splits, scale)

    _say(f"c caller {name}: layer={layer} loop={loop} lens={lens} splits={splits}")
    r = subprocess.run([BIN, str(tmp_path)], capture_output=True, text=True, timeout=120)
    _say(r.stdout.strip())
    assert r.returncode == 0, r.stderr
    shape = (wl.batch, wl.q_heads, wl.head_dim)
    o_c = np.fromfile(os.path.join(tmp_path, "out.bin"), np.float32).reshape(shape)
    lse_c = np.fromfile(os.path.join(tmp_path, "lse.bin"), np.float32).reshape(shape[:2])

    _say(f"  binding decode {name}")
    case.d_pool.copy_(torch.from_numpy(pool_ref.reshape(-1)).to(H.DEV))
    o_py, lse_py = case.gpu_decode(num_splits=splits, scale=scale)
    assert np.array_equal(o_c.astype(np.float64), o_py), "C caller and binding outputs differ"
    assert np.array_equal(lse_c.astype(np.float64), lse_py), "C caller and binding lse differ"

    o_ref, lse_ref = case.oracle_decode(idx_of)
    rel, mx = H.check_attention(o_c.astype(np.float64), o_ref, lse_c.astype(np.float64), lse_ref)
    _say(f"  ok: rel-L2 {rel:.2e}, max-abs {mx:.2e}")


ENC_CASES = [
    ("tiny_encode", W.TINY.with_(batch=3, q_heads=2, kv_heads=2, context=700), 0, 1, [700, 73, 301], 0),
    ("quarter_rot_encode_layer1", W.QUARTER_16K.with_(layers=2, batch=2, q_heads=2, kv_heads=2, context=600), 1, 2,
     [600, 200], 2),
]


@pytest.mark.parametrize("name,wl,layer,loop,lens,splits", ENC_CASES, ids=[c[0] for c in ENC_CASES])
def test_c_caller_encodes_then_decodes(tmp_path, name, wl, layer, loop, lens, splits):
    """The C caller encodes the loop group's K and V rows into a zeroed pool (loopvq_encode with the
    norms of loopvq_codebook_prepare), then decodes: its pages equal the oracle's packing of the
    oracle's indices and the binding's encode byte for byte, and its output equals the binding's
    decode over the binding's pages bit for bit and the oracle's within the attention tolerance."""
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build() first"
    case = H.Case(wl, layer, loop, lens, seed=17)
    exp = case.oracle_encode()
    idx_of = lambda k, b, h: exp[k, b, h][0]  # noqa: E731
    pool_ref = case.oracle_pool(idx_of).reshape(-1)
    case.gpu_setup()
    G, Hkv, d = wl.loop_group, wl.kv_heads, wl.head_dim
    rows = [(b, u) for b in range(wl.batch) for u in range(int(case.n_vq[b]))]
    n = len(rows)
    _write_inputs(str(tmp_path), case, pool_ref, splits, 0.0)
    for kind, fname in ((0, "src_k.bin"), (1, "src_v.bin")):
        src = np.zeros((G, n, Hkv, d), np.uint16)
        for r, (b, u) in enumerate(rows):
            for h in range(Hkv):
                src[:, r, h] = case.kv[kind, b, h][case.split[b][0] + u]
        src.tofile(os.path.join(tmp_path, fname))
    np.array([b for b, _ in rows], np.int32).tofile(os.path.join(tmp_path, "seq_id.bin"))
    np.array([u for _, u in rows], np.int32).tofile(os.path.join(tmp_path, "vq_pos.bin"))
    with open(os.path.join(tmp_path, "args.txt"), "a") as f:
        f.write(f"encode 1\nn_rows {n}\n")

    _say(f"c caller {name}: encode {n} rows x {Hkv} kv-heads, then decode (splits {splits})")
    r = subprocess.run([BIN, str(tmp_path)], capture_output=True, text=True, timeout=120)
    _say(r.stdout.strip())
    assert r.returncode == 0, r.stderr
    pool_c = np.fromfile(os.path.join(tmp_path, "pool_out.bin"), np.uint8)
    assert np.array_equal(pool_c, pool_ref), "C caller's pages differ from the oracle's"
    shape = (wl.batch, wl.q_heads, wl.head_dim)
    o_c = np.fromfile(os.path.join(tmp_path, "out.bin"), np.float32).reshape(shape).astype(np.float64)
    lse_c = np.fromfile(os.path.join(tmp_path, "lse.bin"), np.float32).reshape(shape[:2]).astype(np.float64)

    _say(f"  binding encode and decode {name}")
    for kind in (0, 1):
        case.gpu_encode(kind)
    assert np.array_equal(case.d_pool.cpu().numpy(), pool_c), "binding and C caller pages differ"
    o_py, lse_py = case.gpu_decode(num_splits=splits)
    assert np.array_equal(o_c, o_py) and np.array_equal(lse_c, lse_py), "C caller and binding outputs differ"
    o_ref, lse_ref = case.oracle_decode(idx_of)
    rel, mx = H.check_attention(o_c, o_ref, lse_c, lse_ref)
    _say(f"  ok: rel-L2 {rel:.2e}, max-abs {mx:.2e}")
