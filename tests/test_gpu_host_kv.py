"""The host-offload placement on the GPU: the KV cache (and optionally the
summary store) in pinned host memory, read and written by the same kernels
through the host link (cknv_kv_placement). The page keeps both in pinned CPU
memory and moves what a step needs over the link ("How to use it").

Checked: the placement the library reports, that pageable host memory is
refused before any kernel can touch it, and that every entry point gives
bit-for-bit the results of the all-HBM placement on the same inputs (same
kernels, same arithmetic), plus the oracle's parity at the last step."""
import ctypes
import sys

import numpy as np
import pytest

from block_sparse_kv_stats_amd import cknv, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(f"[gpu host kv] {msg}", flush=True)
    sys.stdout.flush()


def test_placement_reported_and_pageable_refused():
    w = synth.WORKLOADS["tiny"]
    shape = cknv.make_shape(w.S, w.H, w.G, w.d, w.r, w.cap_blocks)
    assert cknv.LayerCache.allocate(shape).placement() == 0
    h = cknv.LayerCache.allocate(shape, kv_on_host=True)
    assert h.placement() == cknv.KV_ON_HOST
    assert h.k.is_pinned() and h.v.is_pinned() and h.kbar.is_cuda and h.seq_len.is_cuda
    hs = cknv.LayerCache.allocate(shape, kv_on_host=True, summaries_on_host=True)
    assert hs.placement() == cknv.KV_ON_HOST | cknv.SUMMARIES_ON_HOST
    # pageable host memory: the binding refuses it ...
    pageable = cknv.LayerCache(shape, torch.zeros(h.k.shape, dtype=h.k.dtype), h.v,
                               h.kbar, h.dbar, h.cnt, h.vbar, h.seq_len)
    assert not pageable.k.is_pinned()
    with pytest.raises(ValueError):
        pageable.c_struct()
    # ... and so does the library (no kernel is launched by either check)
    raw = h._raw_struct()
    buf = np.zeros(h.k.numel(), dtype=np.uint16)
    raw.k = ctypes.c_void_p(buf.ctypes.data)
    raw.v = ctypes.c_void_p(buf.ctypes.data)
    out = ctypes.c_int32(-7)
    assert cknv.lib().cknv_kv_placement(ctypes.byref(shape), ctypes.byref(raw),
                                        ctypes.byref(out)) == cknv.EINVAL
    # mixed placements of k and v are refused
    raw = h._raw_struct()
    raw.v = ctypes.c_void_p(cknv.LayerCache.allocate(shape).v.data_ptr())
    assert cknv.lib().cknv_kv_placement(ctypes.byref(shape), ctypes.byref(raw),
                                        ctypes.byref(out)) == cknv.EINVAL
    assert out.value == -7


def _state(cache, dec):
    return [t.cpu().clone() for t in (dec.sel, dec.n_sel, dec.out, dec.lse, dec.scores,
                                      cache.seq_len, cache.k, cache.v, cache.kbar, cache.dbar,
                                      cache.cnt, cache.vbar)]


@pytest.mark.parametrize("summaries_on_host", [False, True])
def test_fused_steps_match_hbm_placement(summaries_on_host):
    """Fused steps on the Llama-3.1-8B 32K layer with the KV cache (and the
    summaries) in pinned host memory equal the all-HBM steps bit for bit;
    the last step also matches the oracle on two KV heads."""
    w = synth.WORKLOADS["llama8b_32k"].replace(steps=6)
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(w.steps - 1)
    say(f"uploading ({'KV + summaries' if summaries_on_host else 'KV'} on the host)")
    dev = gu.upload(w, data, max_blocks=mb)
    host = gu.upload(w, data, max_blocks=mb, kv_on_host=True, summaries_on_host=summaries_on_host)
    for a, b in zip(dev.tensors()[2:6], host.tensors()[2:6]):
        assert torch.equal(a.cpu(), b.cpu()), "summaries built through the host link differ"
    d_dev = cknv.DecodeStep(dev, mb, w.budget, want_scores=True, fused=True)
    d_host = cknv.DecodeStep(host, mb, w.budget, want_scores=True, fused=True)
    for step in range(w.steps):
        t_idx = [p + step for p in data["prefill"]]
        nk, nv = gu.new_token(data, t_idx)
        q = torch.from_numpy(data["q"][step]).cuda()
        d_dev(q, nk, nv)
        if step < w.steps - 1:
            d_host(q, nk, nv)
        else:
            gu.step_and_check(w, data, host, d_host, step, units={(0, 0), (0, w.H - 1)})
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_state(dev, d_dev), _state(host, d_host))):
            assert torch.equal(a, b), f"step {step}: state item {i} differs"
        say(f"  step {step}: identical")


def test_three_call_and_dense_match_hbm_placement():
    """cknv_append + cknv_score_select + cknv_attend and cknv_dense_attend
    over a host-resident KV cache equal their all-HBM results bit for bit."""
    w = synth.WORKLOADS["llama8b_32k"].replace(steps=2)
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(w.steps - 1)
    dev = gu.upload(w, data, max_blocks=mb)
    host = gu.upload(w, data, max_blocks=mb, kv_on_host=True)
    res = []
    for cache in (dev, host):
        dec = cknv.DecodeStep(cache, mb, w.budget, want_scores=True, fused=False)
        got = []
        for step in range(w.steps):
            t_idx = [p + step for p in data["prefill"]]
            nk, nv = gu.new_token(data, t_idx)
            dec(torch.from_numpy(data["q"][step]).cuda(), nk, nv)
            torch.cuda.synchronize()
            got += _state(cache, dec)
        out = torch.zeros_like(dec.out)
        lse = torch.zeros_like(dec.lse)
        cknv.dense_attend(cache, torch.from_numpy(data["q"][0]).cuda(), w.budget, mb, out, dec.ws,
                          lse)
        torch.cuda.synchronize()
        res.append(got + [out.cpu(), lse.cpu()])
    for i, (a, b) in enumerate(zip(*res)):
        assert torch.equal(a, b), f"item {i} differs"
