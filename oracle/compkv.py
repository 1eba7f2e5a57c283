"""CompKV decode step in plain fp64 NumPy -- TEST INFRASTRUCTURE ONLY.

Written from the CompKV page (onedev.kr/papers/157). Section names used in the
citations below:
  "How it works"  (어떻게 동작하나): Mean compensation, GQA group of G query
                   heads sharing one KV head, budget of K blocks.
  "What differs"  (무엇과 다른가): the estimators z̄, σ̂², p̂, S_b, the block
                   summary {|b|, k̄_b, D̄_b, v̄_b}, the forced set and Top-K,
                   joint normalisation of exact and compensated terms.
  "How to use it" (어떻게 쓰나): per-step update of the current block's
                   statistics, BF16 KV cache with FP32 summaries.
  "Assumptions and limits" (전제와 한계): block size 16, default r = 4.

Everything is per (sequence, KV head) unit: q is [G][d] (the G query heads of
that KV head), k and v are the unit's tokens [T][d].

Readings of points the page leaves open (each is the plainest one the rest of
the page supports):
  * variances are population variances (divide by |b|); this is the variance
    for which the page's second-order expansion of the block partition sum
    holds exactly (ln(Z_b/|b|) = z̄_b + σ²_b/2 + O(σ³));
  * the r groups are contiguous: G_t = [t*d/r, (t+1)*d/r), r must divide d;
  * p̂ is normalised over all blocks of the unit (forced ones included);
  * logits are q.k/sqrt(d) throughout, so the 1/d of σ̂² is (1/sqrt(d))**2;
  * the two most recent blocks are the last two blocks (the last one may be
    partial); every kept block costs one budget slot; Kb = budget // 16;
  * if the unit has no more blocks than the budget, every block is kept;
  * ties in S_b go to the lower block index;
  * compensation uses e^{z̄_b} (Mean compensation); the ½σ̂² term enters
    only the mass estimate used for scoring.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 16
N_FORCED = 3


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def num_blocks(T: int, block: int = BLOCK) -> int:
    return (T + block - 1) // block


def _summaries_equal_blocks(kb: np.ndarray, vb: np.ndarray, r: int):
    """Summaries of n blocks that all hold m tokens: kb, vb are [n][m][d]."""
    n, m, d = kb.shape
    if d % r:
        raise ValueError("r must divide d")
    cnt = np.full(n, float(m))
    kbar = kb.mean(axis=1)                                  # mean key
    vbar = vb.mean(axis=1)                                  # mean value
    c = ((kb - kbar[:, None, :]) ** 2).mean(axis=1)         # per-coordinate population variance
    dbar = c.reshape(n, r, d // r).mean(axis=2)             # group mean of coordinate variances
    return cnt, kbar, dbar, vbar


def block_summaries(k: np.ndarray, v: np.ndarray, T: int, r: int, block: int = BLOCK):
    """The block summary {|b|, k̄_b, D̄_b, v̄_b} of every block of the first T tokens.

    CompKV page, "What differs": the key coordinates are split into r groups
    and D̄_b holds, per group, the mean of the coordinate variances of block
    b's keys; with the mean key and mean value and the token count the summary
    is 2d + r + 1 scalars per block.

    k, v: float64 [>=T][d]. Returns cnt [NB], kbar [NB][d], dbar [NB][r], vbar [NB][d].
    """
    k = np.asarray(k, dtype=np.float64)[:T]
    v = np.asarray(v, dtype=np.float64)[:T]
    d = k.shape[1]
    nfull, rem = divmod(T, block)
    parts = []
    if nfull:
        parts.append(_summaries_equal_blocks(k[:nfull * block].reshape(nfull, block, d),
                                             v[:nfull * block].reshape(nfull, block, d), r))
    if rem:
        parts.append(_summaries_equal_blocks(k[nfull * block:T][None], v[nfull * block:T][None], r))
    if not parts:
        return (np.zeros(0), np.zeros((0, d)), np.zeros((0, r)), np.zeros((0, d)))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(4))


def group_query_energy(q: np.ndarray, r: int) -> np.ndarray:
    """Q_{g,t} = sum over i in G_t of q_{g,i}^2, for contiguous groups. q: [G][d] -> [G][r]."""
    G, d = q.shape
    return (q ** 2).reshape(G, r, d // r).sum(axis=2)


def block_scores(q: np.ndarray, cnt, kbar, dbar, *, mass_order: int = 2,
                 variance_factor: bool = True) -> dict:
    """Estimated compensation-error scores of every block of one KV head.

    CompKV page, "What differs":
      z̄_{g,b}  = q_g . k̄_b / sqrt(d)
      σ̂²_{g,b} = (1/d) sum_t (sum_{i in G_t} q_{g,i}^2) (D̄_b)_t
      p̂_{g,b}  = |b| exp(z̄_{g,b} + σ̂²_{g,b}/2) / sum_c |c| exp(z̄_{g,c} + σ̂²_{g,c}/2)
      S_b      = sum_g p̂_{g,b} σ̂²_{g,b}
    with the G query heads of the GQA group ("How it works") summed.

    mass_order=1 drops the σ̂²/2 term of the mass estimate and
    variance_factor=False scores by sum_g p̂ alone; these are the two ablations
    the page reports ("Assumptions and limits"); the method itself is
    mass_order=2, variance_factor=True.

    q: [G][d] float. Returns dict with zbar, sig2, a (log of the unnormalised
    mass estimate), phat ([G][NB] each) and S ([NB]).
    """
    q = np.asarray(q, dtype=np.float64)
    cnt = np.asarray(cnt, dtype=np.float64)
    kbar = np.asarray(kbar, dtype=np.float64)
    dbar = np.asarray(dbar, dtype=np.float64)
    G, d = q.shape
    r = dbar.shape[1]
    zbar = q @ kbar.T / math.sqrt(d)
    sig2 = group_query_energy(q, r) @ dbar.T / d
    a = np.log(cnt)[None, :] + zbar
    if mass_order == 2:
        a = a + 0.5 * sig2
    if a.shape[1] == 0:
        return {"zbar": zbar, "sig2": sig2, "a": a, "phat": a.copy(), "S": np.zeros(0)}
    amax = a.max(axis=1, keepdims=True)
    lse = amax + np.log(np.exp(a - amax).sum(axis=1, keepdims=True))
    phat = np.exp(a - lse)
    S = (phat * sig2).sum(axis=0) if variance_factor else phat.sum(axis=0)
    return {"zbar": zbar, "sig2": sig2, "a": a, "phat": phat, "S": S}


def forced_blocks(NB: int) -> list:
    """The forced set F: the first (sink) block and the two most recent blocks."""
    return sorted({0, NB - 2, NB - 1} & set(range(NB)))


def select_blocks(S: np.ndarray, Kb: int) -> np.ndarray:
    """Kept blocks under a budget of Kb blocks, ascending.

    CompKV page, "What differs": the sink block and the two most recent
    blocks are always kept and count against the budget; the remaining slots
    go to the blocks with the largest S_b. Ties go to the lower block index.
    If there are no more blocks than slots, every block is kept.
    """
    S = np.asarray(S, dtype=np.float64)
    NB = S.shape[0]
    if Kb < N_FORCED:
        raise ValueError("budget must hold the forced set (3 blocks)")
    if NB <= Kb:
        return np.arange(NB)
    F = forced_blocks(NB)
    cand = np.setdiff1d(np.arange(NB), F)
    order = cand[np.lexsort((cand, -S[cand]))]          # S descending, index ascending
    return np.sort(np.concatenate([F, order[:Kb - len(F)]]))


def compensated_attention(q, k, v, T: int, sel, cnt, kbar, vbar, block: int = BLOCK,
                          compensate: bool = True):
    """Output of the G query heads: exact terms for kept blocks, Mean compensation for the rest.

    CompKV page, "How it works" and "What differs": every logit of an
    unselected block is replaced by the block-mean logit z̄_b = q.k̄_b/sqrt(d),
    so the block contributes |b| e^{z̄_b} to the partition sum and
    |b| e^{z̄_b} v̄_b to the weighted value sum; kept blocks contribute their
    tokens' exact terms; both share one normaliser.
    compensate=False drops the unselected blocks (the page's ablation).

    Returns o [G][d] and lse [G] = log of the shared normaliser.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    G, d = q.shape
    NB = num_blocks(T, block)
    sel = np.asarray(sel, dtype=np.int64)
    kept = np.zeros(NB, dtype=bool)
    kept[sel] = True
    tok = np.concatenate([np.arange(b * block, min(b * block + block, T)) for b in sel]) \
        if len(sel) else np.zeros(0, dtype=np.int64)
    z = q @ k[tok].T / math.sqrt(d)                        # exact logits of kept tokens [G][n]
    un = np.nonzero(~kept)[0] if compensate else np.zeros(0, dtype=np.int64)
    zbar_u = q @ np.asarray(kbar, dtype=np.float64)[un].T / math.sqrt(d)     # [G][nu]
    logw_u = zbar_u + np.log(np.asarray(cnt, dtype=np.float64)[un])[None, :]
    allw = np.concatenate([z, logw_u], axis=1)
    if allw.shape[1] == 0:
        return np.zeros((G, d)), np.full(G, -np.inf)
    m = allw.max(axis=1, keepdims=True)
    e_tok = np.exp(z - m)
    e_un = np.exp(logw_u - m)
    num = e_tok @ v[tok] + e_un @ np.asarray(vbar, dtype=np.float64)[un]
    den = e_tok.sum(axis=1) + e_un.sum(axis=1)
    return num / den[:, None], m[:, 0] + np.log(den)


def dense_attention(q, k, v, T: int):
    """Full softmax attention of the G query heads over all T tokens: o [G][d], lse [G]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)[:T]
    v = np.asarray(v, dtype=np.float64)[:T]
    z = q @ k.T / math.sqrt(q.shape[1])
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    den = e.sum(axis=1)
    return e @ v / den[:, None], m[:, 0] + np.log(den)


def decode_step(q, k_bits, v_bits, T: int, r: int, budget: int, block: int = BLOCK,
                sel=None, compensate: bool = True, mass_order: int = 2,
                variance_factor: bool = True) -> dict:
    """One CompKV decode step of one unit, from the cache contents (summaries rebuilt).

    q: fp32/fp64 [G][d]; k_bits, v_bits: bf16 bit patterns [>=T][d].
    ``sel`` overrides the selection (used to evaluate the output on another,
    equally valid, selection). ``compensate``, ``mass_order`` and
    ``variance_factor`` select the page's ablation variants ("Assumptions and
    limits": Mean compensation removed, first-order mass estimate, score
    without the outer variance factor); the defaults are CompKV itself.
    Returns summaries, scores, sel, o, lse.
    """
    k = decode_bf16(np.asarray(k_bits)[:T])
    v = decode_bf16(np.asarray(v_bits)[:T])
    cnt, kbar, dbar, vbar = block_summaries(k, v, T, r, block)
    sc = block_scores(q, cnt, kbar, dbar, mass_order=mass_order, variance_factor=variance_factor)
    chosen = select_blocks(sc["S"], budget // block)
    use = chosen if sel is None else np.asarray(sel)
    o, lse = compensated_attention(q, k, v, T, use, cnt, kbar, vbar, block, compensate=compensate)
    return {"cnt": cnt, "kbar": kbar, "dbar": dbar, "vbar": vbar, **sc,
            "sel": chosen, "o": o, "lse": lse}


class StreamingUnit:
    """The per-step oracle of one unit: summaries kept alongside the cache.

    CompKV page, "How to use it": each step first updates the statistics of
    the current (open) block with the new token, then scores, selects and
    attends. The open block's summary is recomputed from its tokens, which
    equals the from-scratch summary (tested).
    """

    def __init__(self, k_bits, v_bits, T: int, r: int, cap_tokens: int, block: int = BLOCK):
        d = np.asarray(k_bits).shape[1]
        self.block, self.r, self.T = block, r, T
        self.k = np.zeros((cap_tokens, d))
        self.v = np.zeros((cap_tokens, d))
        self.k[:T] = decode_bf16(np.asarray(k_bits)[:T])
        self.v[:T] = decode_bf16(np.asarray(v_bits)[:T])
        nb_cap = num_blocks(cap_tokens, block)
        self.cnt = np.zeros(nb_cap)
        self.kbar = np.zeros((nb_cap, d))
        self.dbar = np.zeros((nb_cap, r))
        self.vbar = np.zeros((nb_cap, d))
        NB = num_blocks(T, block)
        if NB:
            c, kb, db, vb = block_summaries(self.k, self.v, T, r, block)
            self.cnt[:NB], self.kbar[:NB], self.dbar[:NB], self.vbar[:NB] = c, kb, db, vb

    def append(self, k_bits_tok, v_bits_tok):
        T, B = self.T, self.block
        self.k[T] = decode_bf16(np.asarray(k_bits_tok))
        self.v[T] = decode_bf16(np.asarray(v_bits_tok))
        self.T = T + 1
        b = T // B
        s = b * B
        c, kb, db, vb = _summaries_equal_blocks(self.k[s:self.T][None], self.v[s:self.T][None], self.r)
        self.cnt[b], self.kbar[b], self.dbar[b], self.vbar[b] = c[0], kb[0], db[0], vb[0]

    def summaries(self):
        NB = num_blocks(self.T, self.block)
        return self.cnt[:NB], self.kbar[:NB], self.dbar[:NB], self.vbar[:NB]

    def step(self, q, budget: int) -> dict:
        cnt, kbar, dbar, vbar = self.summaries()
        sc = block_scores(q, cnt, kbar, dbar)
        sel = select_blocks(sc["S"], budget // self.block)
        o, lse = compensated_attention(q, self.k, self.v, self.T, sel, cnt, kbar, vbar, self.block)
        return {**sc, "sel": sel, "o": o, "lse": lse}
