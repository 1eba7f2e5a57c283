"""The oracle against the constants the CompKV page states (tests/golden)."""
import json
import os

import numpy as np
import pytest

from oracle import compkv as ok
from block_sparse_kv_stats_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_block_size_and_default_r():
    assert ok.BLOCK == GOLD["block_size"]["value"]
    assert synth.BLOCK == GOLD["block_size"]["value"]
    assert synth.WORKLOADS["llama8b_32k"].r == GOLD["default_r"]["value"]


@pytest.mark.parametrize("d,r", [(128, 4), (128, 128), (64, 4)])
def test_summary_is_2d_plus_r_plus_1_scalars(d, r):
    rng = np.random.default_rng(0)
    T = 16 * 3
    cnt, kbar, dbar, vbar = ok.block_summaries(rng.standard_normal((T, d)),
                                               rng.standard_normal((T, d)), T, r)
    per_block = 1 + kbar.shape[1] + dbar.shape[1] + vbar.shape[1]
    assert GOLD["summary_scalars_per_block"]["value"] == "2d + r + 1"
    assert per_block == 2 * d + r + 1


def test_r4_metadata_is_one_32nd_of_r128():
    num, den = GOLD["r4_metadata_fraction_of_r128"]["value"]
    rng = np.random.default_rng(1)
    k = rng.standard_normal((32, 128))
    d4 = ok.block_summaries(k, k, 32, 4)[2]
    d128 = ok.block_summaries(k, k, 32, 128)[2]
    assert d4.size * den == d128.size * num


@pytest.mark.parametrize("ctx,budget", [(c, b) for c in GOLD["efficiency_contexts_tokens"]["value"]
                                        for b in GOLD["efficiency_budgets_tokens"]["value"]])
def test_forced_set_counts_against_budget(ctx, budget):
    NB = ctx // GOLD["block_size"]["value"]
    Kb = budget // GOLD["block_size"]["value"]
    S = np.random.default_rng(ctx + budget).exponential(size=NB)
    sel = ok.select_blocks(S, Kb)
    assert len(sel) == Kb
    assert {0, NB - 2, NB - 1} <= set(sel.tolist())
    assert GOLD["forced_blocks"]["counts_against_budget"] is True
