"""Host-side checks of libcknv: it loads, exports every entry point that
include/cknv.h declares, and rejects bad arguments before any HIP call.
No kernel is launched (these run without a GPU)."""
import ctypes
import os
import re

import pytest

from block_sparse_kv_stats_amd import cknv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cknv.h")
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cknv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = cknv.lib()
    names = declared_functions()
    assert len(names) == 13
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in (0, -1, -2, -3, -4):
        assert cknv.status_str(code).startswith("CKNV_")


def shape(**kw):
    base = dict(S=1, H=8, G=4, d=128, r=4, cap_blocks=2100)
    base.update(kw)
    return cknv.make_shape(**base)


def wsize(sh, max_blocks=2048, budget=512):
    n = ctypes.c_size_t(0)
    st = cknv.lib().cknv_workspace_size(ctypes.byref(sh), max_blocks, budget, ctypes.byref(n))
    return st, n.value


def test_workspace_size_valid_and_monotone():
    st, n1 = wsize(shape())
    assert st == cknv.OK and n1 > 0 and n1 % 256 == 0
    st, n2 = wsize(shape(), max_blocks=2100)
    assert st == cknv.OK and n2 >= n1


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), cknv.EUNSUPPORTED), (dict(G=3), cknv.EUNSUPPORTED), (dict(r=3), cknv.EUNSUPPORTED),
    (dict(r=256), cknv.EUNSUPPORTED), (dict(S=0), cknv.EINVAL), (dict(H=-1), cknv.EINVAL),
    (dict(flags=8), cknv.EUNSUPPORTED), (dict(flags=0x80000001), cknv.EUNSUPPORTED)])
def test_bad_shapes(kw, code):
    assert wsize(shape(**kw))[0] == code


@pytest.mark.parametrize("flags", range(8))
def test_ablation_flags_accepted(flags):
    """Every combination of the three ablation bits is a valid shape."""
    assert wsize(shape(flags=flags))[0] == cknv.OK


def test_flag_bits_match_header():
    text = open(os.path.join(ROOT, "include", "cknv.h")).read()
    for name in ("NO_COMPENSATION", "MASS_ONLY_SCORE", "FIRST_ORDER_MASS"):
        m = re.search(rf"#define CKNV_FLAG_{name} (0x[0-9a-f]+)u", text)
        assert m and int(m.group(1), 16) == getattr(cknv, f"FLAG_{name}")


def test_block_size_must_be_16():
    sh = shape()
    sh.block = 32
    assert wsize(sh)[0] == cknv.EUNSUPPORTED


@pytest.mark.parametrize("mb,budget,code", [(0, 512, cknv.EINVAL), (2101, 512, cknv.ENOSPACE),
                                            (2048, 47, cknv.EINVAL)])
def test_bad_sizes(mb, budget, code):
    assert wsize(shape(), mb, budget)[0] == code


def test_too_many_blocks_for_lds_is_unsupported():
    assert wsize(shape(cap_blocks=1 << 16), 12289, 512)[0] == cknv.EUNSUPPORTED
    assert wsize(shape(cap_blocks=1 << 16), 12288, 512)[0] == cknv.OK


def cache_struct(null=None):
    c = cknv.Cache(*([FAKE] * 7))
    if null:
        setattr(c, null, None)
    return c


@pytest.mark.parametrize("null", ["k", "v", "kbar", "dbar", "cnt", "vbar", "seq_len"])
def test_null_cache_pointer_rejected(null):
    sh = shape()
    c = cache_struct(null)
    L = cknv.lib()
    st = L.cknv_score_select(ctypes.byref(sh), ctypes.byref(c), FAKE, 512, 2048, None, FAKE, FAKE,
                             FAKE, 1 << 30, None)
    assert st == cknv.EINVAL
    assert L.cknv_build_summaries(ctypes.byref(sh), ctypes.byref(c), 2048, None) == cknv.EINVAL


def test_entry_points_reject_before_launch():
    sh = shape()
    c = cache_struct()
    L = cknv.lib()
    _, need = wsize(sh)
    # null outputs / query / workspace
    assert L.cknv_score_select(ctypes.byref(sh), ctypes.byref(c), None, 512, 2048, None, FAKE,
                               FAKE, FAKE, need, None) == cknv.EINVAL
    assert L.cknv_score_select(ctypes.byref(sh), ctypes.byref(c), FAKE, 512, 2048, None, None,
                               FAKE, FAKE, need, None) == cknv.EINVAL
    # workspace too small
    assert L.cknv_score_select(ctypes.byref(sh), ctypes.byref(c), FAKE, 512, 2048, None, FAKE,
                               FAKE, FAKE, need - 1, None) == cknv.ENOSPACE
    assert L.cknv_attend(ctypes.byref(sh), ctypes.byref(c), FAKE, FAKE, FAKE, 512, 2048, FAKE,
                         None, FAKE, need - 1, None) == cknv.ENOSPACE
    assert L.cknv_attend(ctypes.byref(sh), ctypes.byref(c), FAKE, None, FAKE, 512, 2048, FAKE,
                         None, FAKE, need, None) == cknv.EINVAL
    assert L.cknv_dense_attend(ctypes.byref(sh), ctypes.byref(c), FAKE, 512, 2048, None, None,
                               FAKE, need, None) == cknv.EINVAL
    # (budget_tokens, max_blocks) in that order, as in every other call: a
    # budget below the forced set is rejected, a max_blocks beyond capacity too
    assert L.cknv_dense_attend(ctypes.byref(sh), ctypes.byref(c), FAKE, 32, 2048, FAKE, None,
                               FAKE, need, None) == cknv.EINVAL
    assert L.cknv_dense_attend(ctypes.byref(sh), ctypes.byref(c), FAKE, 512, 5000, FAKE, None,
                               FAKE, need, None) == cknv.ENOSPACE
    assert L.cknv_append(ctypes.byref(sh), ctypes.byref(c), None, FAKE, None) == cknv.EINVAL
    assert L.cknv_append(ctypes.byref(sh), None, FAKE, FAKE, None) == cknv.EINVAL
    assert L.cknv_workspace_init(ctypes.byref(sh), 2048, 512, None, need, None) == cknv.EINVAL
    # budget below the forced set, max_blocks beyond capacity
    assert L.cknv_score_select(ctypes.byref(sh), ctypes.byref(c), FAKE, 32, 2048, None, FAKE, FAKE,
                               FAKE, need, None) == cknv.EINVAL
    assert L.cknv_build_summaries(ctypes.byref(sh), ctypes.byref(c), 5000, None) == cknv.ENOSPACE
    assert L.cknv_score_select(None, ctypes.byref(c), FAKE, 512, 2048, None, FAKE, FAKE, FAKE,
                               need, None) == cknv.EINVAL


def test_decode_step_rejects_before_launch():
    sh = shape()
    c = cache_struct()
    L = cknv.lib()
    _, need = wsize(sh)

    def call(new_k=FAKE, new_v=FAKE, q=FAKE, budget=512, mb=2048, sel=FAKE, n_sel=FAKE, out=FAKE,
             ws=FAKE, ws_bytes=need, cache=c, shp=sh):
        return L.cknv_decode_step(ctypes.byref(shp) if shp is not None else None,
                                  ctypes.byref(cache) if cache is not None else None, new_k, new_v,
                                  q, budget, mb, None, sel, n_sel, out, None, ws, ws_bytes, None)

    for kw in (dict(new_k=None), dict(new_v=None), dict(q=None), dict(sel=None),
               dict(n_sel=None), dict(out=None), dict(ws=None), dict(cache=None), dict(shp=None),
               dict(budget=47), dict(mb=0)):
        assert call(**kw) == cknv.EINVAL, kw
    assert call(ws_bytes=need - 1) == cknv.ENOSPACE
    assert call(mb=2101) == cknv.ENOSPACE
    assert call(cache=cache_struct("seq_len")) == cknv.EINVAL


def test_decode_halves_reject_before_launch():
    sh = shape()
    c = cache_struct()
    L = cknv.lib()
    _, need = wsize(sh)

    def score(nk=FAKE, nv=FAKE, q=FAKE, mb=2048, ws_bytes=need):
        return L.cknv_decode_score(ctypes.byref(sh), ctypes.byref(c), nk, nv, q, 512, mb, FAKE,
                                   ws_bytes, None)

    def finish(q=FAKE, sel=FAKE, n_sel=FAKE, out=FAKE, mb=2048, ws_bytes=need):
        return L.cknv_decode_finish(ctypes.byref(sh), ctypes.byref(c), q, 512, mb, None, sel, n_sel,
                                    out, None, FAKE, ws_bytes, None)

    for kw in (dict(nk=None), dict(nv=None), dict(q=None)):
        assert score(**kw) == cknv.EINVAL, kw
    assert score(ws_bytes=need - 1) == cknv.ENOSPACE
    assert score(mb=2101) == cknv.ENOSPACE
    for kw in (dict(q=None), dict(sel=None), dict(n_sel=None), dict(out=None)):
        assert finish(**kw) == cknv.EINVAL, kw
    assert finish(ws_bytes=need - 1) == cknv.ENOSPACE
    assert finish(mb=2101) == cknv.ENOSPACE


def test_noalloc_step_rejects_before_any_hip_call():
    """The no-allocation step validates like cknv_decode_step, and a
    workspace beyond its per-GPU array is refused (all before any HIP call)."""
    L = cknv.lib()
    c = cknv.Cache(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    sh = shape()
    args = lambda sh_, mb, budget: (ctypes.byref(sh_), ctypes.byref(c), FAKE, FAKE, FAKE, budget,
                                    mb, None, FAKE, FAKE, FAKE, None, None)
    assert L.cknv_decode_step_noalloc(None, *args(sh, 2048, 512)[1:]) == cknv.EINVAL
    assert L.cknv_decode_step_noalloc(*args(sh, 2048, 32)) == cknv.EINVAL
    assert L.cknv_decode_step_noalloc(*args(sh, 5000, 512)) == cknv.ENOSPACE
    a = list(args(sh, 2048, 512))
    a[2] = None  # new_k
    assert L.cknv_decode_step_noalloc(*a) == cknv.EINVAL
    big = shape(S=16, cap_blocks=8300)
    assert wsize(big, 8300, 2048)[1] > cknv.NOALLOC_SCRATCH_BYTES
    assert L.cknv_decode_step_noalloc(*args(big, 8300, 2048)) == cknv.ENOSPACE


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define CKNV_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == cknv.NOALLOC_SCRATCH_BYTES


def test_kv_placement_rejects_before_any_hip_call():
    """cknv_kv_placement validates its arguments before querying the runtime."""
    L = cknv.lib()
    sh = shape()
    out = ctypes.c_int32(-7)
    assert L.cknv_kv_placement(ctypes.byref(sh), ctypes.byref(cache_struct()), None) == cknv.EINVAL
    assert L.cknv_kv_placement(ctypes.byref(sh), ctypes.byref(cache_struct("vbar")),
                               ctypes.byref(out)) == cknv.EINVAL
    assert L.cknv_kv_placement(None, ctypes.byref(cache_struct()), ctypes.byref(out)) == cknv.EINVAL
    assert L.cknv_kv_placement(ctypes.byref(shape(d=96)), ctypes.byref(cache_struct()),
                               ctypes.byref(out)) == cknv.EUNSUPPORTED
    assert out.value == -7


def test_placement_bits_match_header():
    text = open(HEADER).read()
    for name in ("KV_ON_HOST", "SUMMARIES_ON_HOST"):
        m = re.search(rf"#define CKNV_{name} (0x[0-9a-f]+)", text)
        assert m and int(m.group(1), 16) == getattr(cknv, name)
