"""GPU parity at the 16-sequence ragged batch's full size: 16 sequences of the
Llama-3.1-8B layer shape (8 KV heads, 4 query heads each, d = 128, r = 4),
contexts drawn uniformly from 8K-128K, budgets of 512, 1024 and 2048 tokens,
256 fused decode steps (cknv_decode_step) per budget, each appending one
token to every sequence. Checked against the oracle at steps 0, 15, 16 and
255 on both KV heads 0 and 7 of the shortest and of the longest sequence,
and at step 255 on every KV head of one more sequence: kept sets (up to the
tie band), scores and outputs to the parity tolerances.

The oracle side keeps each checked unit as an oracle StreamingUnit (its
summaries updated per appended token, pinned against a rebuild on the CPU),
so a check at 128K costs one scoring pass rather than a rebuild."""
import sys

import numpy as np
import pytest

from block_sparse_kv_stats_amd import cknv, synth
from oracle import compkv as ok
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CHECK_STEPS = (0, 15, 16, 255)
_DATA = {}


def say(msg):
    print(f"[gpu ragged16] {msg}", flush=True)
    sys.stdout.flush()


def layer():
    if "d" not in _DATA:
        w = synth.WORKLOADS["ragged16"]
        say(f"generating {w.S} x {w.H} units, contexts {min(w.prefill)}..{max(w.prefill)}")
        _DATA["w"], _DATA["d"] = w, synth.gen_layer(w, threads=16)
    return _DATA["w"], _DATA["d"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("budget", [512, 1024, 2048])
def test_ragged16_full_size(budget):
    w0, data = layer()
    w = w0.replace(budget=budget)
    pre = np.asarray(w.prefill)
    s_short, s_long = int(np.argmin(pre)), int(np.argmax(pre))
    s_all = next(s for s in range(w.S) if s not in (s_short, s_long))
    units = {(s, h): CHECK_STEPS for s in (s_short, s_long) for h in (0, w.H - 1)}
    units.update({(s_all, h): (w.steps - 1,) for h in range(w.H)})
    say(f"budget {budget}: shortest seq {s_short} ({pre[s_short]}), longest {s_long} "
        f"({pre[s_long]}), all heads of seq {s_all}")
    mb = w.max_blocks_after(w.steps - 1)
    cache = gu.upload(w, data, max_blocks=mb)
    dec = cknv.DecodeStep(cache, mb, w.budget, want_scores=True, fused=True)
    say(f"  {dec.n_sel.numel()} units, {w.steps} steps")
    cap = int(pre.max()) + w.steps + 16
    su = {u: ok.StreamingUnit(data["k"][u[0], u[1]], data["v"][u[0], u[1]], int(pre[u[0]]), w.r,
                              cap_tokens=cap) for u in units}
    G = w.G
    for step in range(w.steps):
        t_idx = [int(p) + step for p in pre]
        nk, nv = gu.new_token(data, t_idx)
        dec(torch.from_numpy(data["q"][step]).cuda(), nk, nv)
        for (s, h), x in su.items():
            x.append(data["k"][s, h, t_idx[s]], data["v"][s, h, t_idx[s]])
        todo = [u for u, steps in units.items() if step in steps]
        if not todo:
            continue
        torch.cuda.synchronize()
        sel, nsel = dec.sel.cpu().numpy(), dec.n_sel.cpu().numpy()
        out, lse = dec.out.cpu().numpy(), dec.lse.cpu().numpy()
        scores = dec.scores.cpu().numpy()
        worst = 0.0
        for (s, h) in todo:
            x = su[(s, h)]
            u = s * w.H + h
            q = data["q"][step][s, h * G:(h + 1) * G]
            ref = x.step(q, budget)
            n = int(nsel[u])
            gu.check_selection(ref["S"], sel[u], n, w.Kb)
            NB = ok.num_blocks(x.T)
            gu.check_scores(scores[s, h, :NB], ref["S"])
            cnt, kbar, dbar, vbar = x.summaries()
            o_ref, lse_ref = ok.compensated_attention(q, x.k, x.v, x.T, np.sort(sel[u][:n]), cnt,
                                                      kbar, vbar)
            err = gu.rel_l2(out[s, h * G:(h + 1) * G], o_ref)
            assert np.all(err <= gu.OUT_RTOL_L2), f"step {step} unit {(s, h)}: rel L2 {err}"
            lerr = np.abs(lse[s, h * G:(h + 1) * G] - lse_ref)
            assert np.all(lerr <= 1e-3 * np.maximum(1.0, np.abs(lse_ref))), lerr
            worst = max(worst, float(err.max()))
        say(f"  step {step}: {len(todo)} units match (worst output rel L2 {worst:.2e})")
    assert cache.seq_len.cpu().tolist() == [int(p) + w.steps for p in pre]
