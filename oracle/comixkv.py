"""CoMixKV controller: local attention-error sensitivity and joint V bit allocation.

Test infrastructure, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

CoMixKV news article, abstract and method paragraphs: a controller estimates
each (agent, layer)'s quantisation sensitivity online from the recently seen
queries, keys and values, as a local attention-error bound (no calibration
set, no trial quantisation, no extra forward pass), and allocates 2, 3 or 4
bits jointly over every resident agent and layer under one shared memory
budget, using the real byte costs.  New widths apply only to blocks quantised
afterwards ("incremental quantization strategy").

The article gives no formula.  The readings taken here:

* Local attention.  For agent a, layer l and one recent query row q (one of
  the agent's last R decode steps, one of its Hq query heads; kv head
  g = h // G), over the agent's native window (its most recent tokens, kept in
  bf16): p_t = softmax_t(sigma * q . k_t), sigma = 1 / sqrt(d) unless given.
* V error at b bits.  The codec writes v as ||v|| times the rotated, normalised
  coordinates y (E y_i^2 = 1) replaced by centroids, so
  ||v - v_hat||^2 = (||v||^2 / d) * sum_i (y_i - c(y_i))^2, whose expectation
  is D_b ||v||^2 with D_b the Lloyd-Max distortion of N(0, 1).
* Bound.  ||sum_t p_t (v_t - v_hat_t)|| <= sum_t p_t ||v_t - v_hat_t||, and by
  Jensen E[.] <= sqrt(D_b) * sum_t p_t ||v_t||.  The sensitivity is that sum
  averaged over the rows: s_{a,l} = mean_rows sum_t p_t ||v_t||, and the
  predicted error at b bits is s_{a,l} * sqrt(D_b).  An empty window gives 0.
* Allocation.  Minimise sum_i s_i * e[b_i] subject to sum_i cost_i[b_i] <=
  budget, b_i in {2, 3, 4}: every item starts at 2 bits; repeatedly the
  single-width upgrade b -> b + 1 with the largest error decrease per added
  byte, s_i (e[b] - e[b + 1]) / (cost_i[b + 1] - cost_i[b]), is taken if it
  fits the remaining budget (ties to the lower item index); an item whose
  best upgrade does not fit is not upgraded further; stop when nothing fits.
  (The article says the allocation is incremental and not globally optimal.)
"""
from __future__ import annotations

import math

import numpy as np

from . import lloyd_max


def distortion(bits: int) -> float:
    """D_b = E[(X - Q(X))^2], X ~ N(0, 1), for the fp32 table the codec uses."""
    c, t = lloyd_max.table_f32(bits)
    return lloyd_max.mse_closed_form(c.astype(np.float64), t.astype(np.float64))


def error_factors() -> np.ndarray:
    """[sqrt(D_2), sqrt(D_3), sqrt(D_4)]: predicted error per unit of sensitivity."""
    return np.array([math.sqrt(distortion(b)) for b in (2, 3, 4)], dtype=np.float64)


def sensitivity(q: np.ndarray, win_k: np.ndarray, win_v: np.ndarray, win_len, n_kv_heads: int,
                softmax_scale: float = 0.0) -> np.ndarray:
    """s[a, l] in fp64.

    q: [R][A][L][Hq][d] recent query rows; win_k, win_v: [A][L][Hkv][cap][d] the
    agents' native windows, of which the first win_len[a] tokens are used.
    """
    q = np.asarray(q, dtype=np.float64)
    R, A, L, Hq, d = q.shape
    G = Hq // n_kv_heads
    sigma = softmax_scale if softmax_scale > 0 else 1.0 / math.sqrt(d)
    out = np.zeros((A, L), dtype=np.float64)
    for a in range(A):
        n = int(win_len[a])
        if n == 0:
            continue
        for l in range(L):
            total = 0.0
            for g in range(n_kv_heads):
                k = np.asarray(win_k[a, l, g, :n], dtype=np.float64)
                v = np.asarray(win_v[a, l, g, :n], dtype=np.float64)
                vnorm = np.sqrt(np.sum(v * v, axis=1))
                for r in range(R):
                    for h in range(g * G, (g + 1) * G):
                        s = sigma * (k @ q[r, a, l, h])
                        p = np.exp(s - np.max(s))
                        p /= np.sum(p)
                        total += float(p @ vnorm)
            out[a, l] = total / (R * Hq)
    return out


def allocate(sens, cost, err, budget: int) -> np.ndarray | None:
    """Bits (2..4) per item by the greedy rule above; None if 2 bits everywhere exceed the budget.

    sens: [n] sensitivities (the float32 values the library receives);
    cost: [n][3] integer bytes at 2, 3, 4 bits; err: [3] error per unit of sensitivity.
    """
    s = np.asarray(sens, dtype=np.float32).astype(np.float64)
    cost = np.asarray(cost, dtype=np.uint64)
    err = np.asarray(err, dtype=np.float64)
    n = s.shape[0]
    bits = np.full(n, 2, dtype=np.int64)
    used = int(np.sum(cost[:, 0], dtype=np.uint64)) if n else 0
    if used > budget:
        return None
    frozen = np.zeros(n, dtype=bool)
    while True:
        best, best_ratio = -1, -1.0
        for i in range(n):
            if frozen[i] or bits[i] == 4:
                continue
            b = bits[i] - 2
            dc = int(cost[i, b + 1]) - int(cost[i, b])
            ratio = s[i] * (err[b] - err[b + 1]) / float(dc) if dc > 0 else math.inf
            if ratio > best_ratio:
                best, best_ratio = i, ratio
        if best < 0:
            break
        b = bits[best] - 2
        dc = int(cost[best, b + 1]) - int(cost[best, b])
        if used + dc <= budget:
            used += dc
            bits[best] += 1
        else:
            frozen[best] = True
    return bits


def objective(sens, err, bits) -> float:
    s = np.asarray(sens, dtype=np.float32).astype(np.float64)
    return float(np.sum(s * np.asarray(err, dtype=np.float64)[np.asarray(bits) - 2]))


def block_cost(n_tokens: int, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """Bytes one layer of a pool block of n_tokens takes at 2, 3, 4 V bits.

    Per token and kv head: d bytes of K codes, d * b / 8 of V codes, 4 of the
    V norm; per token: 4 bytes of K scale (the pool image's layout).
    """
    return np.array([n_tokens * (n_kv_heads * (head_dim + head_dim * b // 8 + 4) + 4) for b in (2, 3, 4)],
                    dtype=np.uint64)


class RefreshCycle:
    """The controller's budget bookkeeping over agent starts, exits and refreshes.

    CoMixKV news article, "online sensitivity estimation" paragraphs: the
    controller weighs the sensitivities, the capacity each agent still has to
    quantise and the real byte costs, chooses widths within the total budget,
    recomputes the choice when an agent starts or ends and when new
    observations arrive, and the budget an exiting agent held becomes
    available to the others; "incremental quantization strategy": a block,
    once quantised, keeps its encoding.  The readings taken here:

    * one byte budget covers every resident agent's quantised blocks;
    * each agent declares at start how many tokens it may quantise in all
      (its capacity); what it has not yet quantised is its remaining capacity;
    * a refresh has one item per (agent with remaining capacity, layer),
      ordered by agent id then layer; an item at b bits costs what the
      agent's remaining tokens take in that layer at b bits
      (``block_cost(remaining, ...)``); the budget for the items is the total
      minus the bytes the resident agents' stored blocks hold;
    * the chosen widths apply to the agent's next block (a commit of up to
      its remaining tokens); a stored block keeps its widths and bytes until
      its agent exits;
    * an exit releases that agent's blocks and its remaining capacity;
    * an agent with no sensitivity given (it has seen nothing yet) counts 0.
    """

    def __init__(self, budget: int, n_layers: int, n_kv_heads: int, head_dim: int):
        self.budget = int(budget)
        self.n_layers, self.n_kv_heads, self.head_dim = n_layers, n_kv_heads, head_dim
        self.capacity: dict[int, int] = {}
        self.blocks: dict[int, list[tuple[int, np.ndarray]]] = {}  # agent -> [(tokens, bits [L])]

    def start(self, agent: int, capacity_tokens: int) -> None:
        if agent in self.blocks or capacity_tokens < 1:
            raise ValueError("agent already resident, or no capacity")
        self.capacity[agent] = int(capacity_tokens)
        self.blocks[agent] = []

    def exit(self, agent: int) -> int:
        """Release the agent, its blocks and its remaining capacity; returns the stored bytes freed."""
        freed = sum(self.block_bytes(n, b) for n, b in self.blocks.pop(agent))
        del self.capacity[agent]
        return int(freed)

    def block_bytes(self, n_tokens: int, bits) -> int:
        c = block_cost(n_tokens, self.n_kv_heads, self.head_dim)
        return int(sum(int(c[b - 2]) for b in bits))

    def stored_bytes(self) -> int:
        return int(sum(self.block_bytes(n, b) for blocks in self.blocks.values() for n, b in blocks))

    def remaining(self, agent: int) -> int:
        return self.capacity[agent] - sum(n for n, _ in self.blocks[agent])

    def refresh(self, sens: dict) -> dict | None:
        """Widths of the next block of every resident agent with remaining capacity
        ({agent: [L] bits}), or None when 2 bits everywhere does not fit."""
        agents = [a for a in sorted(self.blocks) if self.remaining(a) > 0]
        L = self.n_layers
        if not agents:
            return {}
        s = np.concatenate([np.asarray(sens.get(a, np.zeros(L)), dtype=np.float32).reshape(L) for a in agents])
        cost = np.concatenate([np.tile(block_cost(self.remaining(a), self.n_kv_heads, self.head_dim), (L, 1))
                               for a in agents])
        free = self.budget - self.stored_bytes()
        if free < 0:
            return None
        bits = allocate(s, cost, error_factors(), free)
        if bits is None:
            return None
        return {a: bits[i * L:(i + 1) * L] for i, a in enumerate(agents)}

    def commit(self, widths: dict, n_tokens: int) -> None:
        """Store the next block of n_tokens of each agent in widths, at those widths."""
        for a, bits in widths.items():
            if a not in self.blocks or not 0 < n_tokens <= self.remaining(a):
                raise ValueError("agent not resident, or block beyond its remaining capacity")
            self.blocks[a].append((int(n_tokens), np.asarray(bits, dtype=np.int64).copy()))
        if self.stored_bytes() > self.budget:
            raise ValueError("blocks exceed the budget")
