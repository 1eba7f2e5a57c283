"""Exact quantities of CompKV's selection analysis -- TEST INFRASTRUCTURE ONLY.

CompKV page (onedev.kr/papers/157), section "How it works": under Mean
compensation the selection loss of a GQA group is the sum over its G query
heads of the KL divergence between the compensated and the original attention
distribution, minimised under a budget of K blocks. Expanding it, a skipped
block b costs p_{g,b}(1 - |b| e^{z̄}/Z) = p_{g,b}(σ²/2 + O(σ³)) with Z the
block's partition sum Z_{g,b}; so keeping the blocks with the largest
sum_g p_{g,b} σ²_{g,b} minimises the second-order objective. Without Mean
compensation and with one query head, the same objective selects by attention
mass (Top-K). These functions compute the exact quantities directly from the
token logits, independently of ``compkv``'s block summaries, so that the
oracle can be checked against the page's statements.

Derivation used (reading of "exact log-partition identity"): with Q the
compensated distribution (token i of a skipped block gets logit z̄_b, the
block-mean logit), Z' = sum_kept Z_b + sum_skipped |b| e^{z̄_b} and
KL(Q||P) = sum_i Q_i (z'_i - z_i) + ln(Z / Z'). The sum vanishes because Q is
constant on each skipped block and the logits there average to z̄_b, so
KL(Q||P) = ln Z - ln Z' = -ln(1 - sum_skipped δ_b) with
δ_b = p_b (1 - |b| e^{z̄_b} / Z_b).
"""
from __future__ import annotations

import itertools
import math

import numpy as np

BLOCK = 16


def token_logits(q, k, T: int) -> np.ndarray:
    """z_{g,i} = q_g . k_i / sqrt(d), [G][T]."""
    q = np.asarray(q, dtype=np.float64)
    return q @ np.asarray(k, dtype=np.float64)[:T].T / math.sqrt(q.shape[1])


def _logsumexp(x, axis):
    m = np.max(x, axis=axis, keepdims=True)
    return np.squeeze(m, axis) + np.log(np.exp(x - m).sum(axis=axis))


def exact_block_quantities(q, k, T: int, block: int = BLOCK) -> dict:
    """Per (g, b), from the token logits:
    logZ  = ln sum_{i in b} e^{z_i}        (block partition sum, log)
    p     = Z_b / sum_c Z_c                (block attention mass)
    zmean = mean_{i in b} z_i              (block-mean logit)
    sigma2 = population variance of z over b
    delta = p (1 - |b| e^{zmean} / Z_b)    (mass a skipped block loses)
    size  = |b|
    """
    z = token_logits(q, k, T)
    G = z.shape[0]
    NB = (T + block - 1) // block
    logZ = np.empty((G, NB))
    zmean = np.empty((G, NB))
    sigma2 = np.empty((G, NB))
    size = np.empty(NB)
    for b in range(NB):
        zb = z[:, b * block:min(b * block + block, T)]
        size[b] = zb.shape[1]
        logZ[:, b] = _logsumexp(zb, axis=1)
        zmean[:, b] = zb.mean(axis=1)
        sigma2[:, b] = zb.var(axis=1)
    logp = logZ - _logsumexp(logZ, axis=1)[:, None]
    p = np.exp(logp)
    # 1 - |b| e^{zmean}/Z_b, through expm1 to keep precision when it is small
    delta = p * (-np.expm1(np.log(size)[None, :] + zmean - logZ))
    return {"z": z, "logZ": logZ, "p": p, "zmean": zmean, "sigma2": sigma2,
            "delta": delta, "size": size}


def exact_loss(delta, kept) -> float:
    """sum_g KL(Q_g || P_g) = sum_g -ln(1 - sum_{b skipped} δ_{g,b})."""
    delta = np.asarray(delta)
    skip = np.ones(delta.shape[1], dtype=bool)
    skip[list(kept)] = False
    return float(-np.log1p(-delta[:, skip].sum(axis=1)).sum())


def second_order_loss(p, sigma2, kept) -> float:
    """(1/2) sum_g sum_{b skipped} p_{g,b} σ²_{g,b}."""
    skip = np.ones(np.asarray(p).shape[1], dtype=bool)
    skip[list(kept)] = False
    return float(0.5 * (np.asarray(p) * np.asarray(sigma2))[:, skip].sum())


def estimated_loss(S, kept) -> float:
    """(1/2) sum_{b skipped} S_b."""
    skip = np.ones(len(S), dtype=bool)
    skip[list(kept)] = False
    return float(0.5 * np.asarray(S)[skip].sum())


def no_compensation_loss(p, kept) -> float:
    """sum_g KL(P restricted to kept blocks || P) = sum_g -ln sum_{b kept} p_{g,b}."""
    p = np.asarray(p)
    return float(-np.log(p[:, list(kept)].sum(axis=1)).sum())


def compensated_token_distribution(q, k, T: int, kept, block: int = BLOCK):
    """Token-level compensated distribution: logits z_i on kept blocks, the
    block-mean logit on skipped blocks. Returns (log Q [G][T], log P [G][T])."""
    z = token_logits(q, k, T)
    zc = z.copy()
    keep = set(int(b) for b in kept)
    NB = (T + block - 1) // block
    for b in range(NB):
        if b not in keep:
            s, e = b * block, min(b * block + block, T)
            zc[:, s:e] = z[:, s:e].mean(axis=1, keepdims=True)
    logQ = zc - _logsumexp(zc, axis=1)[:, None]
    logP = z - _logsumexp(z, axis=1)[:, None]
    return logQ, logP


def feasible_selections(NB: int, Kb: int):
    """Every kept set that holds the forced set {0, NB-2, NB-1} and Kb blocks."""
    F = sorted({0, NB - 2, NB - 1})
    rest = [b for b in range(NB) if b not in F]
    for extra in itertools.combinations(rest, Kb - len(F)):
        yield tuple(sorted(F + list(extra)))


def brute_force_best(loss, NB: int, Kb: int):
    """(best kept set, its loss, the runner-up's loss) over feasible_selections."""
    scored = sorted((loss(s), s) for s in feasible_selections(NB, Kb))
    best_loss, best = scored[0]
    second = scored[1][0] if len(scored) > 1 else math.inf
    return np.array(best), best_loss, second
