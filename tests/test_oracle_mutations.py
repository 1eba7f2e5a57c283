"""The pins catch plausible mistakes in the oracle.

Each case replaces one oracle function with a copy carrying one planted
mistake (on the CPU, inside this process only) and checks that at least one
of the named pins then fails.
"""
import math

import numpy as np
import pytest

from oracle import compkv as ok
from tests import test_bf16_pins as bf16
from tests import test_oracle_pins as pins


def _summ_sample_variance(kb, vb, r):
    n, m, d = kb.shape
    cnt = np.full(n, float(m))
    kbar = kb.mean(axis=1)
    vbar = vb.mean(axis=1)
    c = ((kb - kbar[:, None, :]) ** 2).sum(axis=1) / max(m - 1, 1)
    return cnt, kbar, c.reshape(n, r, d // r).mean(axis=2), vbar


def _summ_group_sum(kb, vb, r):
    n, m, d = kb.shape
    cnt = np.full(n, float(m))
    kbar = kb.mean(axis=1)
    vbar = vb.mean(axis=1)
    c = ((kb - kbar[:, None, :]) ** 2).mean(axis=1)
    return cnt, kbar, c.reshape(n, r, d // r).sum(axis=2), vbar


def _summ_strided_groups(kb, vb, r):
    n, m, d = kb.shape
    cnt = np.full(n, float(m))
    kbar = kb.mean(axis=1)
    vbar = vb.mean(axis=1)
    c = ((kb - kbar[:, None, :]) ** 2).mean(axis=1)
    return cnt, kbar, c.reshape(n, d // r, r).mean(axis=1), vbar


def _energy_strided(q, r):
    G, d = q.shape
    return (q ** 2).reshape(G, d // r, r).sum(axis=1)


def _scores_variant(kind):
    real = ok.block_scores

    def f(q, cnt, kbar, dbar, *, mass_order=2, variance_factor=True):
        q = np.asarray(q, dtype=np.float64)
        G, d = q.shape
        r = np.asarray(dbar).shape[1]
        zbar = q @ np.asarray(kbar).T / math.sqrt(d)
        sig2 = ok.group_query_energy(q, r) @ np.asarray(dbar).T / d
        if kind == "sqrt_d":
            sig2 = sig2 * math.sqrt(d)
        if kind == "zbar_unscaled":
            zbar = zbar * math.sqrt(d)
        half = {"no_half": 0.0, "minus_half": -0.5}.get(kind, 0.5)
        a = np.log(np.asarray(cnt))[None, :] + zbar + half * sig2
        if kind == "norm_without_forced":
            NB = a.shape[1]
            keep = np.ones(NB, dtype=bool)
            keep[[0, NB - 2, NB - 1]] = False
            lse = np.log(np.exp(a[:, keep]).sum(axis=1, keepdims=True))
        else:
            lse = np.log(np.exp(a).sum(axis=1, keepdims=True))
        phat = np.exp(a - lse)
        S = (phat * sig2).max(axis=0) if kind == "max_over_g" else (phat * sig2).sum(axis=0)
        return {"zbar": zbar, "sig2": sig2, "a": a, "phat": phat, "S": S}
    return f


def _select_no_forced(S, Kb):
    S = np.asarray(S)
    NB = len(S)
    if NB <= Kb:
        return np.arange(NB)
    idx = np.arange(NB)
    return np.sort(idx[np.lexsort((idx, -S))][:Kb])


def _select_ties_high(S, Kb):
    S = np.asarray(S)
    NB = len(S)
    if NB <= Kb:
        return np.arange(NB)
    F = [0, NB - 2, NB - 1]
    cand = np.setdiff1d(np.arange(NB), F)
    order = cand[np.lexsort((-cand, -S[cand]))]
    return np.sort(np.concatenate([F, order[:Kb - 3]]))


def _attention_no_count(q, k, v, T, sel, cnt, kbar, vbar, block=16, compensate=True):
    return _real_attention(q, k, v, T, sel, np.ones_like(np.asarray(cnt)), kbar, vbar, block,
                           compensate)


_real_attention = ok.compensated_attention


def _attention_always_compensates(q, k, v, T, sel, cnt, kbar, vbar, block=16, compensate=True):
    return _real_attention(q, k, v, T, sel, cnt, kbar, vbar, block, True)

P9 = lambda: pins.test_p9_second_order_mass_estimate_converges_at_fourth_order()


def _decode_as_fp16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _decode_truncated(bits):
    b = np.asarray(bits, dtype=np.uint16) & np.uint16(0xFFF0)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


MUTATIONS = {
    "sample variance": (("_summaries_equal_blocks", _summ_sample_variance),
                        [lambda: pins.test_p3_single_coordinate_keys_give_exact_logit_variance(192)]),
    "group sum instead of mean": (("_summaries_equal_blocks", _summ_group_sum),
                                  [lambda: pins.test_p4_isotropic_blocks_closed_form_any_r(4)]),
    "strided groups": (("_summaries_equal_blocks", _summ_strided_groups),
                       [pins.test_p11_group_permutation_invariance]),
    "strided query energy": (("group_query_energy", _energy_strided),
                             [pins.test_p11_group_permutation_invariance]),
    "variance scaled by 1/sqrt(d)": (("block_scores", _scores_variant("sqrt_d")),
                                     [lambda: pins.test_p3_single_coordinate_keys_give_exact_logit_variance(192)]),
    "mean logit without 1/sqrt(d)": (("block_scores", _scores_variant("zbar_unscaled")),
                                     [lambda: pins.test_p3_single_coordinate_keys_give_exact_logit_variance(192)]),
    "mass estimate without half variance": (("block_scores", _scores_variant("no_half")), [P9]),
    "mass estimate with minus half variance": (("block_scores", _scores_variant("minus_half")), [P9]),
    "mass normalised without forced blocks": (("block_scores", _scores_variant("norm_without_forced")), [P9]),
    "max over query heads": (("block_scores", _scores_variant("max_over_g")),
                             [pins.test_p8_small_spread_selection_minimises_exact_kl]),
    "no forced set": (("select_blocks", _select_no_forced),
                      [lambda: pins.test_p8_forced_set_and_budget_by_brute_force(0),
                       pins.test_p2_constant_blocks_compensate_exactly]),
    "ties to higher index": (("select_blocks", _select_ties_high),
                             [pins.test_p2_constant_blocks_compensate_exactly]),
    "variance factor kept in the mass-only ablation": (("block_scores", _scores_variant("plain")),
        [lambda: pins.test_p7_ablation_mass_score_without_compensation_is_optimal(0)]),
    "compensation kept in the no-compensation ablation": (
        ("compensated_attention", _attention_always_compensates),
        [lambda: pins.test_p7_no_compensation_single_head_is_topk_mass(0),
         lambda: pins.test_p7_ablation_mass_score_without_compensation_is_optimal(0)]),
    "compensation without block size": (("compensated_attention", _attention_no_count),
                                        [lambda: pins.test_p5_log_partition_identity_and_token_level_output(0)]),
    "bf16 read as fp16": (("decode_bf16", _decode_as_fp16), [bf16.test_decode_every_bit_pattern]),
    "bf16 low mantissa bits dropped": (("decode_bf16", _decode_truncated),
                                       [bf16.test_decode_every_bit_pattern]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    (attr, fake), checks = MUTATIONS[name]
    monkeypatch.setattr(ok, attr, fake)
    failed = 0
    for check in checks:
        try:
            check()
        except (AssertionError, ValueError):
            failed += 1
    assert failed >= 1, f"no pin caught the planted mistake: {name}"
