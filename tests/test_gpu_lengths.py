"""Decode's length contract on the GPU (needs an MI355X).

seq_lens[b] = 0 is an empty context: the oracle's empty softmax gives an output row of 0 and
lse = -inf.  A length outside [0, max_seq_len] is a caller error that only the device sees: its
output row and lse are NaN, while every other query of the launch is unaffected.  Both the
single-split write and the split merge are covered, at c = 4 and c = 8.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
H = pytest.importorskip("lvq_harness")

from synth import workloads as W  # noqa: E402


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


WLS = {
    "c4": W.LAYER_4K.with_(batch=4, q_heads=4, kv_heads=2, context=700),
    "c8": W.QUARTER_16K.with_(layers=1, batch=4, q_heads=2, kv_heads=2, context=700),
}


def _encode_all(case):
    exp = case.oracle_encode()
    case.gpu_setup()
    pool_ref = case.oracle_pool(lambda k, b, h: exp[k, b, h][0])
    case.d_pool.copy_(torch.from_numpy(pool_ref.reshape(-1)).to(H.DEV))
    return case.oracle_decode(lambda k, b, h: exp[k, b, h][0])


@pytest.mark.parametrize("name", sorted(WLS))
@pytest.mark.parametrize("splits", [1, 3])
def test_empty_and_out_of_range_lengths(name, splits):
    wl = WLS[name]
    lens = [700, 0, 300, 73]                       # max_seq_len = 700
    _say(f"lengths {name} splits={splits} lens={lens}")
    case = H.Case(wl, 0, 1, lens)
    o_ref, lse_ref = _encode_all(case)
    assert np.all(o_ref[1] == 0.0) and np.all(lse_ref[1] == -np.inf)   # the oracle's empty context

    o, lse = case.gpu_decode(num_splits=splits)
    live = [0, 2, 3]
    H.check_attention(o[live], o_ref[live], lse[live], lse_ref[live])
    assert np.all(o[1] == 0.0), "empty context: output must be 0"
    assert np.all(lse[1] == -np.inf), "empty context: lse must be -inf"

    # lengths the host cannot see as wrong: -3 and max_seq_len + 1; the other rows are unchanged
    bad = np.array([-3, 0, 300, 701], np.int32)
    case.d_lens.copy_(torch.from_numpy(bad).to(H.DEV))
    o2, lse2 = case.gpu_decode(num_splits=splits)
    assert np.all(np.isnan(o2[0])) and np.all(np.isnan(lse2[0])), "negative length must give NaN"
    assert np.all(np.isnan(o2[3])) and np.all(np.isnan(lse2[3])), "length above max_seq_len must give NaN"
    assert np.all(o2[1] == 0.0) and np.all(lse2[1] == -np.inf)
    assert np.array_equal(o2[2], o[2]) and np.array_equal(lse2[2], lse[2]), "a valid row changed"
    _say("  ok")
