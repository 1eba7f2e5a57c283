"""Seeded synthetic inputs for the CompKV decode step.

This module only draws random inputs; it holds none of the method's arithmetic.
Both the GPU path (tests, bench) and the fp64 oracle are fed from it.

The recipe stands in for the real model activations and long-context datasets
that the CompKV page (onedev.kr/papers/157, section "Assumptions and limits")
evaluates on, which are not available here. It keeps that page's settings:
16-token blocks, r variance groups, token budgets, 32K-128K contexts, GQA groups
of the Llama-3.1-8B / Qwen3-8B / Qwen3-32B layer shapes.

Per (sequence s, KV head h) one ``numpy.random.default_rng([cfg_id, s, h])``
draws, in this order:
  q0    [G][d]      N(0, 1)                         step-0 queries
  mu    [NBcap][d]  N(0, 1)                         block mean key
  logsb [NBcap]     U(ln 0.05, ln 2)                block noise scale s_b = exp(logsb)
  aniso [d]         U(ln 0.1, ln 3)   (if aniso)    per-coordinate key scale exp(.)
  eps   [cap][d]    N(0, 1)                         token key noise
  nu    [cap]       U(0, 1)                         needle lottery (needle if < 0.01)
  v     [cap][d]    N(0, 1)                         values
  xi    [steps][G][d] N(0, 1)                       per-step query noise
key_j = (mu_b + s_b * eps_j) * aniso;  needles add DELTA*sqrt(d)*qbar/|qbar|^2
(qbar = mean of the G step-0 queries), which raises qbar's logit by DELTA.
The step-t query is q0 for t = 0 and q0 + 0.5*xi_t after that.
K and V are rounded to bfloat16 (round to nearest even); queries stay fp32.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK = 16
NEEDLE_P = 0.01
NEEDLE_DELTA = 8.0
QUERY_STEP_NOISE = 0.5


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> fp32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    S: int
    H: int
    G: int
    d: int
    r: int
    budget: int
    prefill: tuple          # tokens in the cache per sequence before step 0
    steps: int              # decode steps; each appends one token
    aniso: bool = False
    needles: bool = True
    block: int = BLOCK
    extra_cap: int = 0      # spare capacity (tokens) beyond prefill + steps

    @property
    def cap_tokens(self) -> int:
        need = max(self.prefill) + self.steps + self.extra_cap
        return int(math.ceil(need / self.block) * self.block)

    @property
    def cap_blocks(self) -> int:
        return self.cap_tokens // self.block

    @property
    def Kb(self) -> int:
        return self.budget // self.block

    def max_blocks_after(self, step: int) -> int:
        """Largest block count over sequences after ``step + 1`` appends."""
        return max(int(math.ceil((p + step + 1) / self.block)) for p in self.prefill)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _ragged_lengths(n: int, lo: int, hi: int, seed: int) -> tuple:
    rng = np.random.default_rng([5, 999, seed])
    return tuple(int(t) for t in rng.integers(lo, hi + 1, size=n))


# The five workloads. Prefill lengths are set so that the first decode step
# (which appends one token) lands on the context length the workload names.
WORKLOADS = {
    "tiny": Workload("tiny single-layer decode, 1K ctx, d=64", 1, S=1, H=1, G=4, d=64, r=4,
                     budget=128, prefill=(1023,), steps=1, needles=False),
    "llama8b_32k": Workload("Llama-3.1-8B layer, 32K ctx, budget 512, r=4", 2, S=1, H=8, G=4,
                            d=128, r=4, budget=512, prefill=(32767,), steps=1),
    "qwen8b_128k": Workload("Qwen3-8B layer, 128K ctx, budget 2048, r=4, 64-step stream", 3,
                            S=1, H=8, G=4, d=128, r=4, budget=2048,
                            prefill=(131072 - 64,), steps=64),
    "qwen32b_64k": Workload("Qwen3-32B layer, 64K ctx, budget 1024, r=128, anisotropic keys", 4,
                            S=1, H=8, G=8, d=128, r=128, budget=1024, prefill=(65535,),
                            steps=1, aniso=True),
    "ragged16": Workload("16-seq ragged 8K-128K, Llama-3.1-8B layer, r=4", 5, S=16, H=8, G=4,
                         d=128, r=4, budget=1024,
                         prefill=_ragged_lengths(16, 8192, 131072, 0), steps=256),
}


def gen_unit(w: Workload, s: int, h: int, ntok: int | None = None) -> dict:
    """Draw one (sequence, KV head) unit: all tokens it will ever hold.

    Returns dict with k, v: uint16 bf16 bits [ntok][d] (ntok defaults to the
    sequence's prefill + steps), q: fp32 [steps][G][d].
    """
    if ntok is None:
        ntok = w.prefill[s] + w.steps
    d, G, B = w.d, w.G, w.block
    nbk = int(math.ceil(ntok / B))
    rng = np.random.default_rng([w.cfg_id, s, h])
    q0 = rng.standard_normal((G, d), dtype=np.float32)
    mu = rng.standard_normal((nbk, d), dtype=np.float32)
    lo, hi = math.log(0.05), math.log(2.0)
    sb = np.exp(lo + (hi - lo) * rng.random(nbk, dtype=np.float32)).astype(np.float32)
    if w.aniso:
        alo, ahi = math.log(0.1), math.log(3.0)
        scale = np.exp(alo + (ahi - alo) * rng.random(d, dtype=np.float32)).astype(np.float32)
    eps = rng.standard_normal((ntok, d), dtype=np.float32)
    nu = rng.random(ntok, dtype=np.float32)
    v = rng.standard_normal((ntok, d), dtype=np.float32)
    xi = rng.standard_normal((max(w.steps, 1), G, d), dtype=np.float32)

    blk = np.arange(ntok) // B
    k = mu[blk] + sb[blk, None] * eps
    if w.aniso:
        k *= scale[None, :]
    if w.needles:
        qbar = q0.astype(np.float64).mean(axis=0)
        shift = (NEEDLE_DELTA * math.sqrt(d) * qbar / float(qbar @ qbar)).astype(np.float32)
        k[nu < NEEDLE_P] += shift[None, :]
    q = np.empty((max(w.steps, 1), G, d), dtype=np.float32)
    q[0] = q0
    if w.steps > 1:
        q[1:] = q0[None] + np.float32(QUERY_STEP_NOISE) * xi[1:]
    return {"k": bf16_bits(k), "v": bf16_bits(v), "q": q}


def gen_layer(w: Workload, units=None, threads: int = 1) -> dict:
    """Draw every unit of a layer into cache-shaped arrays.

    Returns k, v: uint16 [S][H][cap_tokens][d] (tokens beyond each sequence's
    prefill + steps are zero), q: fp32 [steps][S][H*G][d],
    prefill: int32 [S]. `threads` > 1 draws units concurrently (each unit has
    its own generator, so the result does not depend on it).
    """
    S, H, G, d, cap = w.S, w.H, w.G, w.d, w.cap_tokens
    k = np.zeros((S, H, cap, d), dtype=np.uint16)
    v = np.zeros((S, H, cap, d), dtype=np.uint16)
    q = np.zeros((max(w.steps, 1), S, H * G, d), dtype=np.float32)
    todo = [(s, h) for s in range(S) for h in range(H) if units is None or (s, h) in units]

    def one(sh):
        s, h = sh
        u = gen_unit(w, s, h)
        n = u["k"].shape[0]
        k[s, h, :n] = u["k"]
        v[s, h, :n] = u["v"]
        q[:, s, h * G:(h + 1) * G] = u["q"]

    if threads > 1 and len(todo) > 1:
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, todo))
    else:
        for sh in todo:
            one(sh)
    return {"k": k, "v": v, "q": q, "prefill": np.asarray(w.prefill, dtype=np.int32)}
