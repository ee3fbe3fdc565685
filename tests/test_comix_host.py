"""Host-side checks of the CoMixKV controller entry points (no GPU).

comix_allocate_bits is host code: it must reproduce the oracle's greedy
allocation exactly (same double arithmetic, same tie rule) on random
instances with real pool byte costs, and reject what the header says it
rejects.  pkv_lloyd_max_distortion must equal the oracle's closed form over
the same fp32 table.  comix_sensitivity's argument validation runs on the host
before anything is enqueued, so its error paths are checked here too.
"""
import ctypes

import numpy as np
import pytest

from oracle import comixkv
from quantized_shared_kv_amd import polykv as pk


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_distortion_equals_oracle(bits):
    assert pk.lloyd_max_distortion(bits) == pytest.approx(comixkv.distortion(bits), rel=1e-12)


def test_distortion_rejects_other_bits():
    assert pk.lib().pkv_lloyd_max_distortion(1) < 0 and pk.lib().pkv_lloyd_max_distortion(5) < 0


@pytest.mark.parametrize("seed", range(12))
def test_allocation_equals_oracle(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 200))
    sens = rng.lognormal(0.0, 1.0, n).astype(np.float32)
    sens[rng.random(n) < 0.1] = 0.0
    if seed % 3 == 0:
        sens[:] = 1.0  # all ties
    hkv = int(rng.choice([1, 4, 8]))
    cost = np.stack([comixkv.block_cost(int(t), hkv, int(rng.choice([64, 128]))) for t in rng.integers(1, 600, n)])
    err = comixkv.error_factors()
    lo, hi = int(cost[:, 0].sum()), int(cost[:, 2].sum())
    for budget in [lo, hi, hi + 1000] + [int(x) for x in rng.integers(lo, hi, 6)]:
        want = comixkv.allocate(sens, cost, err, budget)
        got = pk.comix_allocate_bits(sens, cost, err, budget)
        assert got == list(want), (seed, budget)
        assert int(cost[np.arange(n), np.array(got) - 2].sum()) <= budget


def test_allocation_budget_and_input_errors():
    err = comixkv.error_factors()
    cost = [[200, 300, 400]] * 3
    with pytest.raises(pk.PolyKVError) as e:
        pk.comix_allocate_bits([1, 1, 1], cost, err, 599)
    assert e.value.code == -4
    assert pk.comix_allocate_bits([1, 1, 1], cost, err, 600) == [2, 2, 2]
    assert pk.comix_allocate_bits([], [], err, 0) == []
    for bad_sens, bad_cost, bad_err in (([-1, 1, 1], cost, err), ([float("nan"), 1, 1], cost, err),
                                        ([1, 1, 1], [[200, 200, 400]] + cost[1:], err),
                                        ([1, 1, 1], cost, [0.1, 0.2, 0.05])):
        with pytest.raises(pk.PolyKVError) as e:
            pk.comix_allocate_bits(bad_sens, bad_cost, bad_err, 10_000)
        assert e.value.code == -1


def test_sensitivity_validation_runs_on_host():
    f = pk.lib().comix_sensitivity
    lens = (ctypes.c_int32 * 2)(4, 4)
    ok = dict(n_agents=2, layer_count=3, n_q_heads=8, n_kv_heads=2, head_dim=128, softmax_scale=0.0, n_recent=2,
              q=0x1000, q_dtype=pk.PKV_BF16, win_k=0x2000, win_v=0x3000, win_dtype=pk.PKV_BF16, win_cap=4,
              win_len=lens, out=0x4000)

    def call(**kw):
        d = dict(ok, **kw)
        a = pk.ComixArgs(*[d[n] for n, _ in pk.ComixArgs._fields_])
        return f(ctypes.byref(a), None)

    assert f(None, None) == -1
    assert call(n_agents=0) == 0 and call(layer_count=0) == 0        # no-ops: nothing enqueued
    assert call(head_dim=96) == -2
    assert call(q_dtype=7) == -2 and call(win_dtype=7) == -2
    assert call(n_q_heads=7) == -1 and call(n_recent=0) == -1 and call(n_kv_heads=0) == -1
    assert call(softmax_scale=-1.0) == -1
    assert call(win_cap=3) == -1                                       # a length above the capacity
    assert call(win_k=0x2008) == -1                                    # window rows read in 16-byte pieces
    assert call(q=None) == -1 and call(out=None) == -1
    assert call(win_k=None) == -1
