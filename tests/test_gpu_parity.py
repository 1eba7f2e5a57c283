"""GPU parity: the C-ABI decode path against the fp64 oracle.

Tolerances (fp32 GPU arithmetic vs fp64 oracle on identical BF16 bytes):
identical kept sets except swaps inside a 1e-5 relative band around the cut
score; S_b within 1e-4 relative (floor 1e-7 max S); outputs within 2e-3
relative L2 per query head, evaluated on the GPU's kept set; lse within 1e-3.
"""
import sys

import numpy as np
import pytest

from block_sparse_kv_stats_amd import cknv, synth
from oracle import compkv as ok
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def run_single_step(w, units=None, check_summaries=True, flags=0):
    say(f"workload {w.name}: S={w.S} H={w.H} G={w.G} d={w.d} r={w.r} budget={w.budget} "
        f"prefill={w.prefill[:4]} flags={flags}")
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(0)
    cache = gu.upload(w, data, max_blocks=mb, flags=flags)
    dec = cknv.DecodeStep(cache, mb, w.budget, want_scores=True)
    return gu.step_and_check(w, data, cache, dec, 0, units, check_summaries)


def test_tiny_step():
    run_single_step(synth.WORKLOADS["tiny"])


def test_llama8b_32k_step():
    run_single_step(synth.WORKLOADS["llama8b_32k"])


def test_one_head_150k_step():
    """9376 blocks: the selection kernel's runs of 12 blocks nearly full."""
    run_single_step(synth.WORKLOADS["qwen8b_128k"].replace(name="one head 150K", H=1,
                                                           prefill=(150000,), steps=1))


def test_llama8b_32k_partial_open_block():
    w = synth.WORKLOADS["llama8b_32k"].replace(prefill=(32768 + 6,), extra_cap=16)
    run_single_step(w)


def test_qwen32b_64k_r128_step():
    run_single_step(synth.WORKLOADS["qwen32b_64k"])


@pytest.mark.parametrize("flags", range(1, 8))
def test_ablation_variants(flags):
    """The page's ablations through append + score_select + attend, against
    the oracle's same variant; a partial open block and a short sequence."""
    w = synth.WORKLOADS["llama8b_32k"].replace(S=2, prefill=(16 * 900 + 3, 33), budget=1024)
    run_single_step(w, flags=flags)


def test_streaming_with_block_closes_shortened():
    """Qwen3-8B layer shape, 40 appends from a partial block across 3 block
    closes; every step checked; the streamed store equals a rebuild."""
    w = synth.WORKLOADS["qwen8b_128k"].replace(prefill=(16 * 300 - 5,), steps=40)
    say(f"streaming {w.prefill} x {w.steps}")
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(w.steps - 1)
    cache = gu.upload(w, data, max_blocks=mb)
    dec = cknv.DecodeStep(cache, mb, w.budget, want_scores=True)
    for step in range(w.steps):
        gu.step_and_check(w, data, cache, dec, step, check_summaries=(step % 13 == 0))
    T = w.prefill[0] + w.steps
    for h in range(w.H):
        gu.summaries_equal(cache, data, w, 0, h, T)
    streamed = [t.clone() for t in (cache.kbar, cache.dbar, cache.cnt, cache.vbar)]
    cknv.build_summaries(cache, mb)
    torch.cuda.synchronize()
    NB = ok.num_blocks(T)
    for a, b in zip(streamed, (cache.kbar, cache.dbar, cache.cnt, cache.vbar)):
        assert torch.equal(a[:, :, :NB], b[:, :, :NB])


def test_streaming_qwen8b_128k_full():
    """The 128K, budget-2048 workload as timed: 64 steps, 4 block closes;
    sampled steps checked on every KV head."""
    w = synth.WORKLOADS["qwen8b_128k"]
    say(f"streaming {w.name}")
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(w.steps - 1)
    cache = gu.upload(w, data, max_blocks=mb)
    dec = cknv.DecodeStep(cache, mb, w.budget, want_scores=True)
    for step in range(w.steps):
        if step in (0, 15, 16, 47, 63):
            say(f"  step {step} checked")
            gu.step_and_check(w, data, cache, dec, step, check_summaries=(step == 63))
        else:
            t_idx = [p + step for p in data["prefill"]]
            nk, nv = gu.new_token(data, t_idx)
            dec(torch.from_numpy(data["q"][step]).cuda(), nk, nv)


def test_ragged_batch_shortened():
    """16 sequences of different lengths (some shorter than the budget, some
    with fewer than 3 blocks), 12 steps."""
    rng = np.random.default_rng(5)
    pre = tuple(int(x) for x in rng.integers(20, 5000, 16))
    pre = (1, 17, 40) + pre[3:]
    w = synth.WORKLOADS["ragged16"].replace(prefill=pre, steps=12, budget=512)
    say(f"ragged {pre}")
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(w.steps - 1)
    cache = gu.upload(w, data, max_blocks=mb)
    dec = cknv.DecodeStep(cache, mb, w.budget, want_scores=True)
    for step in range(w.steps):
        gu.step_and_check(w, data, cache, dec, step, check_summaries=(step == w.steps - 1))


@pytest.mark.parametrize("budget", [48, 128])
def test_short_contexts_keep_everything(budget):
    pre = (0, 1, 14, 15, 16, 31, 46, 47, 48, 63, 100, 200)
    w = synth.Workload("short", 77, S=len(pre), H=2, G=4, d=64, r=4, budget=budget, prefill=pre,
                       steps=2, extra_cap=16)
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(w.steps - 1)
    cache = gu.upload(w, data, max_blocks=mb)
    dec = cknv.DecodeStep(cache, mb, w.budget, want_scores=True)
    for step in range(w.steps):
        gu.step_and_check(w, data, cache, dec, step, check_summaries=True)


def test_empty_sequence_outputs_zero():
    w = synth.Workload("empty", 78, S=2, H=2, G=2, d=64, r=4, budget=64, prefill=(0, 100),
                       steps=1, extra_cap=16)
    data = synth.gen_layer(w)
    cache = gu.upload(w, data, max_blocks=w.cap_blocks)
    dec = cknv.DecodeStep(cache, w.cap_blocks, w.budget, want_scores=True)
    q = torch.from_numpy(data["q"][0]).cuda()
    dec(q)  # no append: sequence 0 holds no token
    torch.cuda.synchronize()
    assert dec.n_sel[:2].cpu().tolist() == [0, 0]
    assert torch.all(dec.out[0] == 0)
    assert torch.all(torch.isneginf(dec.lse[0]))
    o = dec.out.cpu().numpy()
    lse = dec.lse.cpu().numpy()
    for h in range(2):
        gu.check_unit(w, data, 1, h, 100, 0, data["q"][0], dec.sel.cpu().numpy(),
                      dec.n_sel.cpu().numpy(), o, lse, dec.scores.cpu().numpy(), w.budget)


def test_constant_blocks_tie_to_lower_index():
    """Identical keys inside every block: every S_b is 0, so the kept set is
    the forced set plus the lowest indices; compensation is then exact."""
    w = synth.Workload("const", 79, S=1, H=2, G=4, d=128, r=4, budget=160, prefill=(16 * 50 - 1,),
                       steps=1, needles=False)
    data = synth.gen_layer(w)
    k = data["k"]
    for b in range(50):
        k[:, :, 16 * b:16 * b + 16] = k[:, :, 16 * b:16 * b + 1]
    cache = gu.upload(w, data, max_blocks=50)
    dec = cknv.DecodeStep(cache, 50, w.budget, want_scores=True)
    gu.step_and_check(w, data, cache, dec, 0, check_summaries=True)
    sel = dec.sel.cpu().numpy()
    for u in range(2):
        assert sel[u].tolist() == list(range(8)) + [48, 49]
    assert torch.all(dec.scores[:, :, :50] == 0)


def test_long_ties_take_lowest_indices():
    """600 blocks of identical keys: every S_b is 0, far more tied candidates
    than the exact-ranking list holds, so the selection pins the threshold
    with extra radix passes and takes the tied blocks in index order."""
    NBk = 600
    w = synth.Workload("const-long", 82, S=1, H=2, G=4, d=64, r=4, budget=160,
                       prefill=(16 * NBk - 1,), steps=1, needles=False)
    data = synth.gen_layer(w)
    k = data["k"]
    for b in range(NBk):
        k[:, :, 16 * b:16 * b + 16] = k[:, :, 16 * b:16 * b + 1]
    cache = gu.upload(w, data, max_blocks=NBk)
    dec = cknv.DecodeStep(cache, NBk, w.budget, want_scores=True)
    gu.step_and_check(w, data, cache, dec, 0, check_summaries=False)
    sel = dec.sel.cpu().numpy()
    for u in range(2):
        assert sel[u].tolist() == list(range(8)) + [NBk - 2, NBk - 1]


def test_mixed_ties_at_the_cut():
    """Half the blocks constant (score 0), the rest noisy, with the budget
    reaching into the zero-score run: the cut falls inside a long tie."""
    NBk = 700
    w = synth.Workload("mixed-ties", 83, S=1, H=2, G=4, d=64, r=4, budget=16 * 400,
                       prefill=(16 * NBk - 1,), steps=1, needles=False)
    data = synth.gen_layer(w)
    k = data["k"]
    for b in range(0, NBk, 2):
        k[:, :, 16 * b:16 * b + 16] = k[:, :, 16 * b:16 * b + 1]
    cache = gu.upload(w, data, max_blocks=NBk)
    dec = cknv.DecodeStep(cache, NBk, w.budget, want_scores=True)
    gu.step_and_check(w, data, cache, dec, 0, check_summaries=False)


@pytest.mark.parametrize("d,G,r", [(64, 1, 1), (64, 2, 16), (64, 8, 64), (128, 1, 8),
                                   (128, 2, 32), (128, 8, 4), (128, 4, 64), (64, 4, 2)])
def test_shape_variants(d, G, r):
    w = synth.Workload(f"shape{d}-{G}-{r}", 80, S=2, H=3, G=G, d=d, r=r, budget=256,
                       prefill=(1500, 2333), steps=2, aniso=True)
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(w.steps - 1)
    cache = gu.upload(w, data, max_blocks=mb)
    dec = cknv.DecodeStep(cache, mb, w.budget, want_scores=True)
    for step in range(w.steps):
        gu.step_and_check(w, data, cache, dec, step, check_summaries=True)


def test_determinism_bitwise():
    w = synth.WORKLOADS["llama8b_32k"]
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(0)
    res = []
    for rep in range(2):
        cache = gu.upload(w, data, max_blocks=mb)
        dec = cknv.DecodeStep(cache, mb, w.budget, want_scores=True)
        nk, nv = gu.new_token(data, list(data["prefill"]))
        dec(torch.from_numpy(data["q"][0]).cuda(), nk, nv)
        torch.cuda.synchronize()
        res.append([t.clone() for t in (dec.scores, dec.sel, dec.n_sel, dec.out, dec.lse,
                                         cache.kbar, cache.dbar)])
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_attend_other_valid_selection():
    """cknv_attend with a caller-chosen kept list (random, unsorted) matches
    the oracle's output for that list."""
    w = synth.WORKLOADS["llama8b_32k"].replace(prefill=(9000,))
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(0)
    cache = gu.upload(w, data, max_blocks=mb)
    dec = cknv.DecodeStep(cache, mb, w.budget, want_scores=False)
    nk, nv = gu.new_token(data, list(data["prefill"]))
    q = torch.from_numpy(data["q"][0]).cuda()
    dec(q, nk, nv)
    T = w.prefill[0] + 1
    NB = ok.num_blocks(T)
    rng = np.random.default_rng(0)
    Kb = w.Kb
    sel = np.stack([rng.permutation(NB)[:Kb - 3] for _ in range(w.H)]).astype(np.int32)
    sel = np.concatenate([sel, np.full((w.H, 3), -1, np.int32)], axis=1)  # padding ignored
    n_sel = np.full(w.H, Kb, np.int32)
    dec.sel.copy_(torch.from_numpy(sel))
    dec.n_sel.copy_(torch.from_numpy(n_sel))
    cknv.attend(cache, q, dec.sel, dec.n_sel, w.budget, mb, dec.out, dec.ws, dec.lse)
    torch.cuda.synchronize()
    out = dec.out.cpu().numpy()
    for h in range(w.H):
        qh = data["q"][0][0, h * w.G:(h + 1) * w.G]
        ref = ok.decode_step(qh, data["k"][0, h], data["v"][0, h], T, w.r, w.budget,
                             sel=np.sort(sel[h, :Kb - 3]))
        assert np.all(gu.rel_l2(out[0, h * w.G:(h + 1) * w.G], ref["o"]) <= gu.OUT_RTOL_L2)


@pytest.mark.parametrize("name", ["tiny", "llama8b_32k"])
def test_dense_attend(name):
    w = synth.WORKLOADS[name]
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(0)
    cache = gu.upload(w, data, max_blocks=mb)
    ws = cknv.allocate_workspace(cache.shape, mb, w.budget)
    out = torch.zeros((w.S, w.H * w.G, w.d), dtype=torch.float32, device="cuda")
    lse = torch.zeros((w.S, w.H * w.G), dtype=torch.float32, device="cuda")
    q = torch.from_numpy(data["q"][0]).cuda()
    cknv.dense_attend(cache, q, w.budget, mb, out, ws, lse)
    torch.cuda.synchronize()
    T = w.prefill[0]
    for h in range(w.H):
        qh = data["q"][0][0, h * w.G:(h + 1) * w.G]
        o, l = ok.dense_attention(qh, ok.decode_bf16(data["k"][0, h]), ok.decode_bf16(data["v"][0, h]), T)
        assert np.all(gu.rel_l2(out[0, h * w.G:(h + 1) * w.G].cpu().numpy(), o) <= gu.OUT_RTOL_L2)
        np.testing.assert_allclose(lse[0, h * w.G:(h + 1) * w.G].cpu().numpy(), l, rtol=1e-4)


def test_append_at_capacity_is_a_no_op():
    w = synth.Workload("full", 81, S=1, H=2, G=2, d=64, r=4, budget=64, prefill=(64,), steps=1)
    data = synth.gen_layer(w)
    cache = gu.upload(w, data, cap_blocks=4, max_blocks=4)
    before = [t.clone() for t in (cache.k, cache.v, cache.kbar, cache.cnt, cache.seq_len)]
    nk = torch.ones((1, 2, 64), dtype=torch.bfloat16, device="cuda")
    cknv.append(cache, nk, nk)
    torch.cuda.synchronize()
    for a, b in zip(before, (cache.k, cache.v, cache.kbar, cache.cnt, cache.seq_len)):
        assert torch.equal(a, b)
