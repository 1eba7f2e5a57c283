"""Helpers for the GPU parity tests: upload seeded inputs, run the C-ABI
path, compare with the fp64 oracle to the stated tolerances."""
import math

import numpy as np

from block_sparse_kv_stats_amd import cknv, synth
from oracle import compkv as ok

SCORE_RTOL = 1e-4      # S_b relative tolerance
SCORE_FLOOR = 1e-7     # ... with an absolute floor of this times max_b S_b
TIE_BAND = 1e-5        # kept sets may differ only between blocks this close to the cut score
OUT_RTOL_L2 = 2e-3     # relative L2 error of each query head's output


def to_dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def oracle_variant(flags: int) -> dict:
    """The oracle's keyword arguments for the ablation flags of a shape."""
    return dict(compensate=not flags & cknv.FLAG_NO_COMPENSATION,
                variance_factor=not flags & cknv.FLAG_MASS_ONLY_SCORE,
                mass_order=1 if flags & cknv.FLAG_FIRST_ORDER_MASS else 2)


def upload(w: synth.Workload, data: dict, cap_blocks=None, max_blocks=None, flags=0,
           kv_on_host=False, summaries_on_host=False):
    """LayerCache holding each sequence's prefill tokens (later slots zero),
    seq_len = prefill, summaries built on the GPU. kv_on_host /
    summaries_on_host: the host-offload placement (pinned host memory)."""
    import torch
    cb = cap_blocks or w.cap_blocks
    shape = cknv.make_shape(w.S, w.H, w.G, w.d, w.r, cb, flags)
    cache = cknv.LayerCache.allocate(shape, kv_on_host=kv_on_host,
                                     summaries_on_host=summaries_on_host)
    k = np.zeros((w.S, w.H, cb * 16, w.d), dtype=np.uint16)
    v = np.zeros_like(k)
    n = min(cb * 16, data["k"].shape[2])
    for s, T in enumerate(data["prefill"]):
        T = int(min(T, n))
        k[s, :, :T] = data["k"][s, :, :T]
        v[s, :, :T] = data["v"][s, :, :T]
    cache.k.copy_(to_dev_bf16(k))
    cache.v.copy_(to_dev_bf16(v))
    cache.seq_len.copy_(torch.tensor(np.asarray(data["prefill"], dtype=np.int32)))
    cknv.build_summaries(cache, max_blocks or cb)
    return cache


def new_token(data: dict, t_index):
    """bf16 [S][H][d] of token position t_index[s] of every sequence."""
    S = data["k"].shape[0]
    kt = np.stack([data["k"][s, :, t_index[s]] for s in range(S)])
    vt = np.stack([data["v"][s, :, t_index[s]] for s in range(S)])
    return to_dev_bf16(kt), to_dev_bf16(vt)


def check_selection(S_ref, sel_gpu, n_gpu, Kb):
    """The GPU kept set equals the oracle's, up to swaps between blocks whose
    fp64 scores lie within TIE_BAND (relative) of the cut score."""
    NB = len(S_ref)
    sel_gpu = np.asarray(sel_gpu[:n_gpu])
    if NB <= Kb:
        assert n_gpu == NB
        np.testing.assert_array_equal(sel_gpu, np.arange(NB))
        return
    assert n_gpu == Kb
    assert np.all(np.diff(sel_gpu) > 0), "kept list must be ascending and distinct"
    assert {0, NB - 2, NB - 1} <= set(sel_gpu.tolist())
    ref = ok.select_blocks(S_ref, Kb)
    diff = set(ref.tolist()) ^ set(sel_gpu.tolist())
    if not diff:
        return
    cand = np.setdiff1d(np.arange(NB), [0, NB - 2, NB - 1])
    order = cand[np.lexsort((cand, -S_ref[cand]))]
    cut = S_ref[order[Kb - 4]]
    band = TIE_BAND * max(cut, 1e-300)
    bad = [b for b in diff if abs(S_ref[b] - cut) > band]
    assert not bad, f"kept sets differ beyond the tie band: {sorted(diff)} cut={cut} " \
                    f"scores={[S_ref[b] for b in sorted(diff)]}"


def check_scores(S_gpu, S_ref):
    S_gpu = np.asarray(S_gpu, dtype=np.float64)
    floor = SCORE_FLOOR * max(S_ref.max(initial=0.0), 1e-300)
    err = np.abs(S_gpu - S_ref)
    ok_ = err <= SCORE_RTOL * np.abs(S_ref) + floor
    assert ok_.all(), f"score mismatch at {np.nonzero(~ok_)[0][:10]}: " \
                      f"gpu={S_gpu[~ok_][:5]} ref={S_ref[~ok_][:5]}"


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-30)


def check_unit(w, data, s, h, T, step, q_all, sel_all, nsel_all, out_all, lse_all, scores_all,
               budget, flags=0):
    """Compare one unit's GPU results with the oracle's from-scratch step."""
    G = w.G
    u = s * w.H + h
    q = q_all[s, h * G:(h + 1) * G]
    var = oracle_variant(flags)
    ref = ok.decode_step(q, data["k"][s, h], data["v"][s, h], T, w.r, budget, **var)
    Kb = budget // 16
    n = int(nsel_all[u])
    check_selection(ref["S"], sel_all[u], n, Kb)
    if scores_all is not None:
        NB = ok.num_blocks(T)
        check_scores(scores_all[s, h, :NB], ref["S"])
    # output against the oracle evaluated on the GPU's (valid) kept set
    o_ref = ok.decode_step(q, data["k"][s, h], data["v"][s, h], T, w.r, budget,
                           sel=np.asarray(sel_all[u][:n]), **var)
    err = rel_l2(out_all[s, h * G:(h + 1) * G], o_ref["o"])
    assert np.all(err <= OUT_RTOL_L2), f"unit {u}: output rel L2 {err}"
    lse_err = np.abs(lse_all[s, h * G:(h + 1) * G] - o_ref["lse"])
    assert np.all(lse_err <= 1e-3 * np.maximum(1.0, np.abs(o_ref["lse"]))), lse_err
    return err.max()


def summaries_equal(cache, data, w, s, h, T, rtol=1e-4, atol=2e-6):
    """GPU summary store of one unit vs the oracle's from-scratch summaries."""
    NB = ok.num_blocks(T)
    ref = ok.block_summaries(ok.decode_bf16(data["k"][s, h][:T]), ok.decode_bf16(data["v"][s, h][:T]),
                             T, w.r)
    got = (cache.cnt[s, h, :NB].cpu().numpy(), cache.kbar[s, h, :NB].cpu().numpy(),
           cache.dbar[s, h, :NB].cpu().numpy(), cache.vbar[s, h, :NB].cpu().numpy())
    for name, g, r in zip(("cnt", "kbar", "dbar", "vbar"), got, ref):
        np.testing.assert_allclose(g, r, rtol=rtol, atol=atol, err_msg=name)


def step_and_check(w, data, cache, dec, step, units=None, check_summaries=False):
    """Append token prefill+step, score/select, attend; compare the listed units."""
    t_idx = [p + step for p in data["prefill"]]
    nk, nv = new_token(data, t_idx)
    import torch
    q = torch.from_numpy(data["q"][step]).cuda()
    flags = int(cache.shape.flags)
    dec(q, nk, nv)
    torch.cuda.synchronize()
    sel, nsel = dec.sel.cpu().numpy(), dec.n_sel.cpu().numpy()
    out, lse = dec.out.cpu().numpy(), dec.lse.cpu().numpy()
    scores = dec.scores.cpu().numpy() if dec.scores is not None else None
    assert np.all(cache.seq_len.cpu().numpy() == np.asarray(t_idx) + 1)
    worst = 0.0
    for s in range(w.S):
        for h in range(w.H):
            if units is not None and (s, h) not in units:
                continue
            T = t_idx[s] + 1
            worst = max(worst, check_unit(w, data, s, h, T, step, data["q"][step], sel, nsel,
                                             out, lse, scores, w.budget, flags))
            if check_summaries:
                summaries_equal(cache, data, w, s, h, T)
    return worst
