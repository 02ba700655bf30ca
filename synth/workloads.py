"""Synthetic workloads shaped like the pages' model (input generation only).

Shapes: GLM-5.2 as the pages report it -- hidden 6144, 256 routed experts per
MoE layer, top-8 (tech.takumi3488.com "Trying colibri", section on the real
744B model), and an expert intermediate of 2048, the width at which three
int4 matrices make the pages' "about 19 MB" expert (agentlenshq.com "Colibri
...", section "Memory split"). The tiny shape is the pages' self-test fixture:
hidden 128, 8 experts per layer, top-2 (takumi3488, self-test and CLI
sections), with intermediate 64.

Distributions: expert and router weights N(0, 0.02^2), router bias
N(0, 0.1^2), hidden states N(0, 1), all fp32 from the counter-based
generator. Zipf routing: logits ln p_rank(e) + Gumbel with p_r proportional
to r^-1.1 and bias 0, so top-k samples experts without replacement with Zipf
popularity.
"""
from __future__ import annotations

import queue
import threading
from dataclasses import dataclass

import numpy as np

from . import (K_TRACE, expert_weights, gumbel, hidden, router_bias, router_weights, stream_id, uniform, zipf_logits,
               zipf_rank)


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    I: int
    E: int
    k: int
    T: int
    seed: int
    routing: str = "hidden"   # "hidden": router on hidden states; "zipf": given Zipf logits
    bits: int = 4
    has_shared: bool = True
    std: float = 0.02
    bias_std: float = 0.1


TINY = Workload("tiny", H=128, I=64, E=8, k=2, T=32, seed=0)
DECODE1 = Workload("glm_decode_t1", H=6144, I=2048, E=256, k=8, T=1, seed=1)
DECODE64 = Workload("glm_decode_t64_zipf", H=6144, I=2048, E=256, k=8, T=64, seed=2, routing="zipf")
PREFILL2048 = Workload("glm_prefill_t2048", H=6144, I=2048, E=256, k=8, T=2048, seed=3)
PREFILL2048_ZIPF = Workload("glm_prefill_t2048_zipf", H=6144, I=2048, E=256, k=8, T=2048, seed=4, routing="zipf")
MTP96 = Workload("glm_mtp_verify_t96", H=6144, I=2048, E=256, k=8, T=96, seed=5)

ALL = {w.name: w for w in (TINY, DECODE1, DECODE64, PREFILL2048, PREFILL2048_ZIPF, MTP96)}


def expert_fp32(w: Workload, e: int, layer: int = 0):
    return expert_weights(w.seed, layer, e, w.H, w.I, w.std)


def shared_fp32(w: Workload, layer: int = 0):
    return expert_weights(w.seed, layer, 0, w.H, w.I, w.std, shared=True)


def router_fp32(w: Workload, layer: int = 0):
    """(w_router [E][H], bias [E] or None). Zipf workloads route on logits: bias 0."""
    wr = router_weights(w.seed, layer, w.E, w.H, w.std)
    b = None if w.routing == "zipf" else router_bias(w.seed, layer, w.E, w.bias_std)
    return wr, b


def hidden_fp32(w: Workload, T: int | None = None, batch: int = 0):
    return hidden(w.seed, w.T if T is None else T, w.H, batch)


def logits_fp32(w: Workload, T: int | None = None, batch: int = 0):
    return zipf_logits(w.seed, 0, w.T if T is None else T, w.E, 1.1, batch)


def iter_experts(w: Workload, experts, layer: int = 0, prefetch: int = 2):
    """Yield (e, gate, up, down) fp32 arrays, generating the next experts on a
    background thread while the caller consumes the current one."""
    q: queue.Queue = queue.Queue(maxsize=prefetch)
    experts = list(experts)

    def work():
        for e in experts:
            q.put((e, *expert_fp32(w, e, layer)))
        q.put(None)

    th = threading.Thread(target=work, daemon=True)
    th.start()
    while True:
        item = q.get()
        if item is None:
            break
        yield item
    th.join()


def correlated_trace(seed: int, layer: int, T: int, E: int, k: int, reuse: float = 0.6, s: float = 1.1):
    """Routing trace int32 [T][k] of one layer of a decoding stack: each slot
    keeps the previous token's expert in that slot with probability `reuse`
    (when this token has not taken it already); the other slots draw from the
    layer's Zipf(s) popularity without replacement (Gumbel-top-k over
    ln p_rank + Gumbel noise, one noise vector per token)."""
    rank_of = zipf_rank(seed, layer, E)
    logp = -s * np.log(rank_of.astype(np.float64))
    g = gumbel(seed, stream_id(K_TRACE, layer, 0), T * E).reshape(T, E)
    u = uniform(seed, stream_id(K_TRACE, layer, 1), T * k).reshape(T, k)
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        taken = np.zeros(E, dtype=bool)
        row = np.full(k, -1, dtype=np.int64)
        if t > 0:
            for j in range(k):
                e = out[t - 1, j]
                if u[t, j] < reuse and not taken[e]:
                    row[j] = e
                    taken[e] = True
        order = np.argsort(-(logp + g[t]), kind="stable")
        pos = 0
        for j in range(k):
            if row[j] < 0:
                while taken[order[pos]]:
                    pos += 1
                row[j] = order[pos]
                taken[row[j]] = True
        out[t] = row
    return out
