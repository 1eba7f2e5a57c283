"""cknv_decode_step_noalloc (no workspace argument: the library's per-GPU
scratch array) against cknv_decode_step with a caller workspace, on two calls
in a row, the second with a smaller input of another shape (so the scratch
layout changes between them). Same kernels, so the results must agree bit
for bit; the kept sets, scores and outputs are also checked against the
oracle at the parity tolerances."""
import sys

import numpy as np
import pytest

from block_sparse_kv_stats_amd import cknv, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def outputs(w, budget):
    U = w.S * w.H
    return dict(sel=torch.full((U, budget // 16), -7, dtype=torch.int32, device="cuda"),
                n_sel=torch.full((U,), -7, dtype=torch.int32, device="cuda"),
                out=torch.full((w.S, w.H * w.G, w.d), 7.0, device="cuda"),
                lse=torch.full((w.S, w.H * w.G), 7.0, device="cuda"),
                scores=torch.full((w.S, w.H, w.cap_blocks), 7.0, device="cuda"))


def one_call(w, oracle_units):
    say(f"no-alloc step: {w.name} S={w.S} H={w.H} G={w.G} d={w.d} prefill={w.prefill[:2]}")
    data = synth.gen_layer(w)
    mb = w.max_blocks_after(0)
    assert cknv.workspace_size(cknv.make_shape(w.S, w.H, w.G, w.d, w.r, w.cap_blocks), mb,
                               w.budget) <= cknv.NOALLOC_SCRATCH_BYTES
    ref_cache = gu.upload(w, data, max_blocks=mb)
    na_cache = gu.upload(w, data, max_blocks=mb)
    nk, nv = gu.new_token(data, list(data["prefill"]))
    q = torch.from_numpy(data["q"][0]).cuda()
    ws = cknv.allocate_workspace(ref_cache.shape, mb, w.budget)
    ref, got = outputs(w, w.budget), outputs(w, w.budget)
    cknv.decode_step(ref_cache, nk, nv, q, w.budget, mb, ref["sel"], ref["n_sel"], ref["out"], ws,
                     ref["lse"], ref["scores"])
    cknv.decode_step_noalloc(na_cache, nk, nv, q, w.budget, mb, got["sel"], got["n_sel"],
                             got["out"], got["lse"], got["scores"])
    torch.cuda.synchronize()
    for name in ("n_sel", "out", "lse"):
        assert torch.equal(ref[name], got[name]), name
    for u in range(w.S * w.H):
        n = int(ref["n_sel"][u])
        assert torch.equal(ref["sel"][u, :n], got["sel"][u, :n])
    for s, T0 in enumerate(w.prefill):
        NB = -(-(T0 + 1) // 16)
        assert torch.equal(ref["scores"][s, :, :NB], got["scores"][s, :, :NB])
    for a, b in zip((ref_cache.k, ref_cache.v, ref_cache.kbar, ref_cache.dbar, ref_cache.cnt,
                     ref_cache.vbar, ref_cache.seq_len),
                    (na_cache.k, na_cache.v, na_cache.kbar, na_cache.dbar, na_cache.cnt,
                     na_cache.vbar, na_cache.seq_len)):
        assert torch.equal(a, b)
    sel, nsel = got["sel"].cpu().numpy(), got["n_sel"].cpu().numpy()
    out, lse, scores = got["out"].cpu().numpy(), got["lse"].cpu().numpy(), got["scores"].cpu().numpy()
    for s, h in oracle_units:
        gu.check_unit(w, data, s, h, w.prefill[s] + 1, 0, data["q"][0], sel, nsel, out, lse,
                      scores, w.budget)


def test_noalloc_step_equals_workspace_step_twice_second_smaller():
    one_call(synth.WORKLOADS["llama8b_32k"], [(0, 0), (0, 5)])
    one_call(synth.WORKLOADS["tiny"].replace(prefill=(700,)), [(0, 0)])
