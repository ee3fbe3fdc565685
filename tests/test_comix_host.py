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


def test_refresh_cycle_equals_oracle_at_qwen3_32b_shape():
    """A refresh cycle on the Qwen3-32B controller shape (8 agents x 64 layers = 512 items,
    8 kv heads, d 128, 1024 tokens of capacity per agent, 256-token blocks).

    The caller's side keeps its own books (stored blocks, remaining capacity) and calls
    comix_allocate_bits with item costs for each agent's remaining tokens and the budget left
    by the stored blocks; at every refresh the widths equal the oracle's.  After an exit the
    remaining agents' next blocks get the freed bytes (no item narrower than without the exit,
    more bytes in total); stored blocks keep their widths.  Also times the allocation at 512
    items."""
    import time

    A, L, Hkv, d, cap, n = 8, 64, 8, 128, 1024, 256

    def row(tokens):  # bytes of one layer of `tokens` tokens at 2, 3, 4 bits (header layout)
        return [tokens * (Hkv * (d + d * b // 8 + 4) + 4) for b in (2, 3, 4)]

    err = [pk.lloyd_max_distortion(b) ** 0.5 for b in (2, 3, 4)]
    budget = A * L * row(cap)[1]  # 3 bits on average over every agent's capacity
    ref = comixkv.RefreshCycle(budget, L, Hkv, d)
    stored = {}  # agent -> list of per-layer widths of its 256-token blocks
    rng = np.random.default_rng(7)
    for a in range(A):
        ref.start(a, cap)
        stored[a] = []
    times = []

    def refresh(sens):
        agents = [a for a in sorted(stored) if len(stored[a]) * n < cap]
        held = sum(row(n)[b - 2] for a in stored for blk in stored[a] for b in blk)
        s = np.concatenate([sens[a] for a in agents]).astype(np.float32)
        cost = [row(cap - len(stored[a]) * n) for a in agents for _ in range(L)]
        t0 = time.perf_counter()
        bits = pk.comix_allocate_bits(s, cost, err, budget - held)
        times.append(time.perf_counter() - t0)
        got = {a: bits[i * L:(i + 1) * L] for i, a in enumerate(agents)}
        want = ref.refresh({a: sens[a] for a in agents})
        assert {a: [int(x) for x in v] for a, v in want.items()} == got
        return got

    for _ in range(2):
        sens = {a: rng.lognormal(0.0, 1.0, L).astype(np.float32) for a in stored}
        w = refresh(sens)
        ref.commit(w, n)
        for a, b in w.items():
            stored[a].append(list(b))
    snapshot = {a: [list(b) for b in bl] for a, bl in stored.items()}
    sens = {a: rng.lognormal(0.0, 1.0, L).astype(np.float32) for a in stored}
    without_exit = refresh(sens)
    # agent 5 exits: its two blocks' bytes and its remaining capacity are released
    freed = ref.exit(5)
    assert freed == sum(row(n)[b - 2] for blk in stored.pop(5) for b in blk)
    with_exit = refresh(sens)
    assert sorted(with_exit) == [a for a in range(A) if a != 5]
    assert all(x >= y for a in with_exit for x, y in zip(with_exit[a], without_exit[a]))
    assert sum(with_exit[a].count(4) for a in with_exit) > sum(without_exit[a].count(4) for a in with_exit)
    assert all(stored[a] == snapshot[a] for a in stored)
    # a refresh at 512 items is host work of well under a millisecond; bound it loosely
    print(f"comix_allocate_bits at {A * L} items: median {1e6 * np.median(times):.0f} us")
    assert np.median(times) < 0.05
