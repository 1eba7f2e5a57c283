"""GPU parity of the fused decode step (cknv_decode_step) against the fp64
oracle, to the same tolerances as the three-call path (see
test_gpu_parity.py), plus its agreement with that path and its handling of
a full cache."""
import sys

import numpy as np
import pytest

from block_sparse_kv_stats_amd import cknv, synth
from oracle import compkv as ok
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(f"[gpu fused] {msg}", flush=True)
    sys.stdout.flush()


def fused_dec(cache, mb, budget, want_scores=True):
    return cknv.DecodeStep(cache, mb, budget, want_scores=want_scores, fused=True)


def run_steps(w, steps=None, check_every=1, summaries_every=0, flags=0):
    say(f"{w.name}: S={w.S} H={w.H} G={w.G} d={w.d} r={w.r} budget={w.budget} "
        f"prefill={w.prefill[:4]} steps={w.steps} flags={flags}")
    data = synth.gen_layer(w)
    n = w.steps if steps is None else steps
    mb = w.max_blocks_after(n - 1)
    cache = gu.upload(w, data, max_blocks=mb, flags=flags)
    dec = fused_dec(cache, mb, w.budget)
    for step in range(n):
        if step % check_every == 0 or step == n - 1:
            say(f"  step {step} checked")
            summ = summaries_every and (step % summaries_every == 0 or step == n - 1)
            gu.step_and_check(w, data, cache, dec, step, check_summaries=bool(summ))
        else:
            t_idx = [p + step for p in data["prefill"]]
            nk, nv = gu.new_token(data, t_idx)
            dec(torch.from_numpy(data["q"][step]).cuda(), nk, nv)
    return data, cache, mb


@pytest.mark.parametrize("name", ["tiny", "llama8b_32k", "qwen32b_64k"])
def test_fused_single_step(name):
    w = synth.WORKLOADS[name]
    run_steps(w.replace(steps=1), summaries_every=1)


def test_fused_longest_bucket_150k():
    """One KV head at 150K tokens (9376 blocks): the step kernel's largest
    bucket (24 blocks per thread) and 32 parts per unit, against the oracle."""
    w = synth.WORKLOADS["qwen8b_128k"].replace(name="one head 150K", H=1, prefill=(150000,),
                                              steps=2)
    run_steps(w, summaries_every=1)


def test_fused_partial_open_block():
    w = synth.WORKLOADS["llama8b_32k"].replace(prefill=(32768 + 6,), extra_cap=16, steps=1)
    run_steps(w, summaries_every=1)


def test_fused_streaming_with_block_closes_equals_rebuild():
    """40 fused steps from a partial block across 3 block closes, every step
    checked; the streamed summary store is bit-identical to a rebuild."""
    w = synth.WORKLOADS["qwen8b_128k"].replace(prefill=(16 * 300 - 5,), steps=40)
    data, cache, mb = run_steps(w, summaries_every=13)
    T = w.prefill[0] + w.steps
    streamed = [t.clone() for t in (cache.kbar, cache.dbar, cache.cnt, cache.vbar)]
    cknv.build_summaries(cache, mb)
    torch.cuda.synchronize()
    NB = ok.num_blocks(T)
    for a, b in zip(streamed, (cache.kbar, cache.dbar, cache.cnt, cache.vbar)):
        assert torch.equal(a[:, :, :NB], b[:, :, :NB])


def test_fused_streaming_qwen8b_128k_full():
    """The 128K, budget-2048 stream as timed: 64 fused steps, sampled steps
    checked on every KV head."""
    run_steps(synth.WORKLOADS["qwen8b_128k"], check_every=16, summaries_every=63)


def test_fused_ragged_batch_shortened():
    rng = np.random.default_rng(5)
    pre = tuple(int(x) for x in rng.integers(20, 5000, 16))
    pre = (1, 17, 40) + pre[3:]
    w = synth.WORKLOADS["ragged16"].replace(prefill=pre, steps=12, budget=512)
    run_steps(w, summaries_every=11)


@pytest.mark.parametrize("budget", [48, 128, 1024])
def test_fused_short_contexts(budget):
    """Empty sequences (the first token), fewer than 3 blocks, NB <= Kb."""
    pre = (0, 1, 14, 15, 16, 31, 46, 47, 48, 63, 100, 200)
    w = synth.Workload("short", 77, S=len(pre), H=2, G=4, d=64, r=4, budget=budget, prefill=pre,
                       steps=3, extra_cap=16)
    run_steps(w, summaries_every=1)


@pytest.mark.parametrize("d,G,r", [(64, 1, 1), (64, 2, 16), (64, 8, 64), (128, 1, 8),
                                   (128, 2, 32), (128, 8, 4), (128, 4, 64), (64, 4, 2),
                                   (128, 8, 128), (128, 4, 128)])
def test_fused_shape_variants(d, G, r):
    w = synth.Workload(f"shape{d}-{G}-{r}", 80, S=2, H=3, G=G, d=d, r=r, budget=256,
                       prefill=(1500, 2333), steps=2, aniso=True)
    run_steps(w, summaries_every=1)


def test_fused_many_parts_and_records():
    """A budget of 2048 tokens at 20K context: many workgroups per unit,
    each folding several chunk records."""
    w = synth.WORKLOADS["llama8b_32k"].replace(prefill=(20000,), budget=2048, steps=2)
    run_steps(w, summaries_every=1)


def test_fused_more_than_64_parts():
    """One KV head, 40K context, a budget of 8192 tokens: 128 parts per unit,
    past the 64 whose records the last part merges lane-parallel, so the
    merge takes its batched path, against the oracle."""
    w = synth.WORKLOADS["llama8b_32k"].replace(name="one head, 128 parts", H=1, prefill=(40000,),
                                              budget=8192, steps=2)
    run_steps(w, summaries_every=1)


def test_fused_part_groups_with_a_partial_last_group():
    """Two KV heads, 12K context, a budget of 1296 tokens (81 blocks): 21
    parts per unit, past the 16 that count in on one counter, so they count
    in by groups of 8, 8 and 5, and the last part merges 21 records, against
    the oracle over three steps."""
    w = synth.WORKLOADS["llama8b_32k"].replace(name="two heads, 21 parts", H=2, prefill=(12000,),
                                              budget=1296, steps=3)
    run_steps(w, summaries_every=1)


def test_fused_constant_blocks_tie_to_lower_index():
    w = synth.Workload("const", 79, S=1, H=2, G=4, d=128, r=4, budget=160, prefill=(16 * 50 - 1,),
                       steps=1, needles=False)
    data = synth.gen_layer(w)
    k = data["k"]
    for b in range(50):
        k[:, :, 16 * b:16 * b + 16] = k[:, :, 16 * b:16 * b + 1]
    cache = gu.upload(w, data, max_blocks=50)
    dec = fused_dec(cache, 50, w.budget)
    gu.step_and_check(w, data, cache, dec, 0, check_summaries=True)
    sel = dec.sel.cpu().numpy()
    for u in range(2):
        assert sel[u].tolist() == list(range(8)) + [48, 49]
    assert torch.all(dec.scores[:, :, :50] == 0)


def test_fused_long_ties_take_lowest_indices():
    NBk = 600
    w = synth.Workload("const-long", 82, S=1, H=2, G=4, d=64, r=4, budget=160,
                       prefill=(16 * NBk - 1,), steps=1, needles=False)
    data = synth.gen_layer(w)
    k = data["k"]
    for b in range(NBk):
        k[:, :, 16 * b:16 * b + 16] = k[:, :, 16 * b:16 * b + 1]
    cache = gu.upload(w, data, max_blocks=NBk)
    dec = fused_dec(cache, NBk, w.budget)
    gu.step_and_check(w, data, cache, dec, 0, check_summaries=False)
    sel = dec.sel.cpu().numpy()
    for u in range(2):
        assert sel[u].tolist() == list(range(8)) + [NBk - 2, NBk - 1]


def test_fused_mixed_ties_at_the_cut():
    NBk = 700
    w = synth.Workload("mixed-ties", 83, S=1, H=2, G=4, d=64, r=4, budget=16 * 400,
                       prefill=(16 * NBk - 1,), steps=1, needles=False)
    data = synth.gen_layer(w)
    k = data["k"]
    for b in range(0, NBk, 2):
        k[:, :, 16 * b:16 * b + 16] = k[:, :, 16 * b:16 * b + 1]
    cache = gu.upload(w, data, max_blocks=NBk)
    dec = fused_dec(cache, NBk, w.budget)
    gu.step_and_check(w, data, cache, dec, 0, check_summaries=False)


@pytest.mark.parametrize("flags", range(1, 8))
def test_fused_ablation_variants(flags):
    """The page's ablations (no compensation, mass-only score, first-order
    mass, and their combinations) against the oracle's same variant, across
    a block close, with a partial open block and a short sequence."""
    w = synth.WORKLOADS["llama8b_32k"].replace(S=2, prefill=(16 * 700 - 2, 40), steps=3,
                                                budget=512)
    run_steps(w, summaries_every=2, flags=flags)


@pytest.mark.parametrize("flags", [1, 2, 4, 7])
def test_fused_ablation_variants_many_parts(flags):
    w = synth.WORKLOADS["qwen8b_128k"].replace(prefill=(16 * 3000 + 5,), steps=1)
    run_steps(w, flags=flags)


@pytest.mark.parametrize("G,budget", [(4, 2048), (8, 512), (4, 320)])
def test_fused_many_units_several_blocks_per_wave(G, budget):
    """More units than the step kernel's resident workgroups: fewer parts per
    unit, each attending wave taking several kept blocks in turn (16, 2 and
    3 of them here; the last part's slots run past the kept list), every
    unit checked against the oracle at two steps."""
    rng = np.random.default_rng(11)
    pre = tuple(int(x) for x in rng.integers(300, 6000, 16))
    w = synth.Workload(f"many units G={G}", 84, S=16, H=8 if G == 4 else 4, G=G, d=128, r=4,
                       budget=budget, prefill=pre, steps=2)
    run_steps(w, check_every=1)


@pytest.mark.parametrize("flags", [0, 1, 6])
def test_fused_equals_three_calls(flags):
    """Same inputs through cknv_decode_step and through append + score_select
    + attend: identical kept lists and summaries, outputs and scores equal to
    fp32 rounding."""
    w = synth.WORKLOADS["llama8b_32k"].replace(prefill=(12345,))
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(0)
    res = []
    for fused in (False, True):
        cache = gu.upload(w, data, max_blocks=mb, flags=flags)
        dec = cknv.DecodeStep(cache, mb, w.budget, want_scores=True, fused=fused)
        nk, nv = gu.new_token(data, list(data["prefill"]))
        dec(torch.from_numpy(data["q"][0]).cuda(), nk, nv)
        torch.cuda.synchronize()
        res.append(dict(sel=dec.sel.clone(), n=dec.n_sel.clone(), out=dec.out.clone(),
                        lse=dec.lse.clone(), scores=dec.scores.clone(), seq=cache.seq_len.clone(),
                        k=cache.k.clone(), v=cache.v.clone(), kbar=cache.kbar.clone(),
                        dbar=cache.dbar.clone(), vbar=cache.vbar.clone(), cnt=cache.cnt.clone()))
    a, b = res
    for key in ("sel", "n", "seq", "k", "v", "kbar", "dbar", "vbar", "cnt"):
        assert torch.equal(a[key], b[key]), key
    NB = ok.num_blocks(w.prefill[0] + 1)
    torch.testing.assert_close(a["scores"][:, :, :NB], b["scores"][:, :, :NB], rtol=2e-5, atol=1e-30)
    torch.testing.assert_close(a["out"], b["out"], rtol=1e-4, atol=1e-5)
    torch.testing.assert_close(a["lse"], b["lse"], rtol=1e-5, atol=1e-5)


def test_fused_determinism_bitwise():
    w = synth.WORKLOADS["llama8b_32k"]
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(0)
    res = []
    for rep in range(2):
        cache = gu.upload(w, data, max_blocks=mb)
        dec = fused_dec(cache, mb, w.budget)
        nk, nv = gu.new_token(data, list(data["prefill"]))
        dec(torch.from_numpy(data["q"][0]).cuda(), nk, nv)
        torch.cuda.synchronize()
        res.append([t.clone() for t in (dec.scores, dec.sel, dec.n_sel, dec.out, dec.lse,
                                         cache.kbar, cache.dbar)])
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_fused_full_cache_attends_existing_tokens():
    """A sequence whose cache is full keeps its tokens and seq_len; the step
    scores, selects and attends those tokens. The other sequence appends."""
    w = synth.Workload("full", 81, S=2, H=2, G=4, d=64, r=4, budget=64, prefill=(160, 100),
                       steps=1)
    data = synth.gen_layer(w)
    cap = 10  # 160 tokens: sequence 0 is full
    cache = gu.upload(w, data, cap_blocks=cap, max_blocks=cap)
    before_k = cache.k[0].clone()
    dec = fused_dec(cache, cap, w.budget)
    nk, nv = gu.new_token(data, [159, 100])  # sequence 0's token is ignored
    q = torch.from_numpy(data["q"][0]).cuda()
    dec(q, nk, nv)
    torch.cuda.synchronize()
    assert cache.seq_len.cpu().tolist() == [160, 101]
    assert torch.equal(cache.k[0], before_k)
    sel, nsel = dec.sel.cpu().numpy(), dec.n_sel.cpu().numpy()
    out, lse, scores = dec.out.cpu().numpy(), dec.lse.cpu().numpy(), dec.scores.cpu().numpy()
    for s, T in ((0, 160), (1, 101)):
        for h in range(w.H):
            gu.check_unit(w, data, s, h, T, 0, data["q"][0], sel, nsel, out, lse, scores, w.budget)


def test_fused_halves_equal_one_call():
    """cknv_decode_score then cknv_decode_finish give the same bits as
    cknv_decode_step."""
    w = synth.WORKLOADS["llama8b_32k"].replace(prefill=(7777,))
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(0)
    q = torch.from_numpy(data["q"][0]).cuda()
    nk, nv = gu.new_token(data, list(data["prefill"]))
    res = []
    for halves in (False, True):
        cache = gu.upload(w, data, max_blocks=mb)
        dec = fused_dec(cache, mb, w.budget)
        b = cknv.BoundStep(cache, mb, w.budget, dec.ws, dec.sel, dec.n_sel, dec.out, dec.lse, q,
                           nk, nv, torch.cuda.current_stream(), scores=dec.scores)
        if halves:
            b.decode_score()
            b.decode_finish()
        else:
            b.fused_step()
        torch.cuda.synchronize()
        res.append([t.clone() for t in (dec.scores, dec.sel, dec.n_sel, dec.out, dec.lse,
                                         cache.kbar, cache.seq_len)])
    for a, b in zip(*res):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name,prefill", [("llama8b_32k", 9999), ("qwen8b_128k", 16 * 3000 + 5)])
def test_fused_finish_repeats_bitwise(name, prefill):
    """With several parts per unit, the part that completes a unit's count
    merges the parts and resets the count: cknv_decode_finish run three times
    after one cknv_decode_score gives the same bits each time, and the same
    bits as cknv_decode_step."""
    w = synth.WORKLOADS[name].replace(prefill=(prefill,))
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(0)
    q = torch.from_numpy(data["q"][0]).cuda()
    nk, nv = gu.new_token(data, list(data["prefill"]))
    cache = gu.upload(w, data, max_blocks=mb)
    dec = fused_dec(cache, mb, w.budget)
    b = cknv.BoundStep(cache, mb, w.budget, dec.ws, dec.sel, dec.n_sel, dec.out, dec.lse, q, nk, nv,
                       torch.cuda.current_stream(), scores=dec.scores)
    say(f"{name}: P = {-(-w.Kb // 4)} parts per unit")
    b.decode_score()
    res = []
    for rep in range(3):
        b.decode_finish()
        torch.cuda.synchronize()
        res.append([t.clone() for t in (dec.out, dec.lse, dec.sel, dec.n_sel, cache.seq_len)])
    for r in res[1:]:
        for x, y in zip(res[0], r):
            assert torch.equal(x, y)
    cache2 = gu.upload(w, data, max_blocks=mb)
    dec2 = fused_dec(cache2, mb, w.budget)
    dec2(q, nk, nv)
    torch.cuda.synchronize()
    for x, y in zip(res[0], (dec2.out, dec2.lse, dec2.sel, dec2.n_sel, cache2.seq_len)):
        assert torch.equal(x, y)


@pytest.mark.parametrize("method", ["fused_step", "step"])
def test_graph_replay_of_layer_sweep_matches_eager(method):
    """A HIP graph of one decode step per layer (three layers, several parts
    per unit), replayed three times with new tokens and queries written into
    the bound buffers between replays, gives the same bits as the same calls
    issued eagerly on a twin set of layers, at every replay (eager work and
    synchronisations run between the replays); the last replay also matches
    the oracle."""
    stream = torch.cuda.Stream()
    reps, L = 3, 3
    ws_ = [synth.WORKLOADS["llama8b_32k"].replace(cfg_id=90 + li, prefill=(3000 + 53 * li,),
                                                   steps=reps) for li in range(L)]
    datas = [synth.gen_layer(w) for w in ws_]

    def make_twin():
        layers = []
        for w, data in zip(ws_, datas):
            mb = w.max_blocks_after(reps - 1)
            cache = gu.upload(w, data, max_blocks=mb)
            dec = fused_dec(cache, mb, w.budget, want_scores=False)
            q = torch.from_numpy(data["q"][0]).cuda()
            nk, nv = gu.new_token(data, list(data["prefill"]))
            b = cknv.BoundStep(cache, mb, w.budget, dec.ws, dec.sel, dec.n_sel, dec.out, dec.lse,
                               q, nk, nv, stream)
            layers.append((cache, dec, q, nk, nv, b))
        return layers

    def feed(layers, rep):
        for (cache, dec, q, nk, nv, b), data in zip(layers, datas):
            q.copy_(torch.from_numpy(data["q"][rep]))
            k1, v1 = gu.new_token(data, [p + rep for p in data["prefill"]])
            nk.copy_(k1)
            nv.copy_(v1)
        torch.cuda.synchronize()

    def state(layers):
        return [[t.clone() for t in (dec.out, dec.lse, dec.sel, dec.n_sel, cache.seq_len,
                                     cache.kbar, cache.dbar, cache.cnt, cache.vbar, cache.k)]
                for (cache, dec, q, nk, nv, b) in layers]

    eager, graphed = make_twin(), make_twin()
    g = cknv.DecodeGraph([x[5] for x in graphed], stream, method=method)
    say(f"graph of {L} layers ({method}) captured")
    for rep in range(reps):
        feed(eager, rep)
        with torch.cuda.stream(stream):
            for x in eager:
                getattr(x[5], method)()
        torch.cuda.synchronize()
        feed(graphed, rep)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for la, lb in zip(state(eager), state(graphed)):
            for a, b in zip(la, lb):
                assert torch.equal(a, b), f"replay {rep}"
        say(f"  replay {rep} equals eager")
    w, data = ws_[-1], datas[-1]
    cache, dec = graphed[-1][0], graphed[-1][1]
    T = data["prefill"][0] + reps
    assert int(cache.seq_len[0]) == T
    sel, nsel = dec.sel.cpu().numpy(), dec.n_sel.cpu().numpy()
    out, lse = dec.out.cpu().numpy(), dec.lse.cpu().numpy()
    for h in (0, w.H - 1):
        gu.check_unit(w, data, 0, h, T, reps - 1, data["q"][reps - 1], sel, nsel, out, lse, None,
                      w.budget)
