"""Thin Python binding of libcknv (the C ABI in include/cknv.h).

Argument marshalling only: torch tensors provide device memory and the HIP
stream; every step of the decode path runs in the library's kernels. The
library is loaded on first use; if it is missing this raises (there is no
fallback).
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcknv.so")

OK, EINVAL, EUNSUPPORTED, ENOSPACE, EHIP = 0, -1, -2, -3, -4
BLOCK = 16


class CknvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})")


class Shape(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int32), ("H", ctypes.c_int32), ("G", ctypes.c_int32),
                ("d", ctypes.c_int32), ("r", ctypes.c_int32), ("block", ctypes.c_int32),
                ("cap_blocks", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("kbar", ctypes.c_void_p),
                ("dbar", ctypes.c_void_p), ("cnt", ctypes.c_void_p), ("vbar", ctypes.c_void_p),
                ("seq_len", ctypes.c_void_p)]


_lib = None
P = ctypes.c_void_p
I32 = ctypes.c_int32
SZ = ctypes.c_size_t
SIGNATURES = {
    "cknv_workspace_size": [ctypes.POINTER(Shape), I32, I32, ctypes.POINTER(SZ)],
    "cknv_workspace_init": [ctypes.POINTER(Shape), I32, I32, P, SZ, P],
    "cknv_append": [ctypes.POINTER(Shape), ctypes.POINTER(Cache), P, P, P],
    "cknv_build_summaries": [ctypes.POINTER(Shape), ctypes.POINTER(Cache), I32, P],
    "cknv_score_select": [ctypes.POINTER(Shape), ctypes.POINTER(Cache), P, I32, I32, P, P, P, P,
                          SZ, P],
    "cknv_attend": [ctypes.POINTER(Shape), ctypes.POINTER(Cache), P, P, P, I32, I32, P, P, P, SZ,
                    P],
    "cknv_dense_attend": [ctypes.POINTER(Shape), ctypes.POINTER(Cache), P, I32, I32, P, P, P, SZ,
                          P],
    "cknv_decode_step": [ctypes.POINTER(Shape), ctypes.POINTER(Cache), P, P, P, I32, I32, P, P, P,
                         P, P, P, SZ, P],
    "cknv_decode_score": [ctypes.POINTER(Shape), ctypes.POINTER(Cache), P, P, P, I32, I32, P, SZ,
                          P],
    "cknv_decode_finish": [ctypes.POINTER(Shape), ctypes.POINTER(Cache), P, I32, I32, P, P, P, P,
                           P, P, SZ, P],
    "cknv_decode_step_noalloc": [ctypes.POINTER(Shape), ctypes.POINTER(Cache), P, P, P, I32, I32,
                                 P, P, P, P, P, P],
    "cknv_kv_placement": [ctypes.POINTER(Shape), ctypes.POINTER(Cache), ctypes.POINTER(I32)],
}
KV_ON_HOST = 0x1          # CKNV_KV_ON_HOST
SUMMARIES_ON_HOST = 0x2   # CKNV_SUMMARIES_ON_HOST
NOALLOC_SCRATCH_BYTES = 32 << 20  # CKNV_NOALLOC_SCRATCH_BYTES


def lib():
    """The loaded libcknv (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_kv_stats_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.cknv_status_str.argtypes = [ctypes.c_int]
        L.cknv_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().cknv_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != OK:
        raise CknvError(status, what)


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t, dtype=None, numel=None, what="", host_ok=False):
    """The address of tensor t, after checking its dtype, size and layout.
    host_ok: pinned host memory is accepted too (a cache's arrays in the
    host-offload placement); pageable host memory never is."""
    if t is None:
        return None
    if not t.is_cuda and not (host_ok and t.is_pinned()):
        raise ValueError(f"{what}: expected a device tensor" + (" or pinned host memory" if host_ok else ""))
    if not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous tensor")
    if dtype is not None and t.dtype not in dtype:
        raise ValueError(f"{what}: dtype {t.dtype} not in {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{what}: {t.numel()} elements, need {numel}")
    return ctypes.c_void_p(t.data_ptr())


# cknv_shape.flags bits: the page's ablation variants (cknv.h)
FLAG_NO_COMPENSATION = 0x1
FLAG_MASS_ONLY_SCORE = 0x2
FLAG_FIRST_ORDER_MASS = 0x4


def make_shape(S, H, G, d, r, cap_blocks, flags=0) -> Shape:
    return Shape(S, H, G, d, r, BLOCK, cap_blocks, flags)


@dataclasses.dataclass
class LayerCache:
    """Tensors of one layer's KV cache and summary store (see cknv.h): device
    tensors, or for k/v (and the summaries) pinned host tensors in the
    host-offload placement (cknv_kv_placement)."""
    shape: Shape
    k: object        # bf16 [S][H][cap_blocks*16][d]
    v: object
    kbar: object     # fp32 [S][H][cap_blocks][d]
    dbar: object     # fp32 [S][H][cap_blocks][r]
    cnt: object      # fp32 [S][H][cap_blocks]
    vbar: object     # fp32 [S][H][cap_blocks][d]
    seq_len: object  # int32 [S]
    _placement: object = dataclasses.field(default=None, repr=False, compare=False)

    @staticmethod
    def allocate(shape: Shape, device="cuda", kv_on_host=False, summaries_on_host=False):
        """Zeroed arrays; kv_on_host / summaries_on_host put k and v / the
        four summary arrays in pinned host memory (torch's pin_memory, which
        allocates with hipHostMalloc), seq_len always on the device."""
        import torch
        S, H, d, r, cb = shape.S, shape.H, shape.d, shape.r, shape.cap_blocks

        def zeros(size, dtype, host):
            if host:
                return torch.zeros(size, dtype=dtype, pin_memory=True)
            return torch.zeros(size, dtype=dtype, device=device)

        kv = lambda: zeros((S, H, cb * BLOCK, d), torch.bfloat16, kv_on_host)
        sm = lambda last: zeros((S, H, cb) + last, torch.float32, summaries_on_host)
        c = LayerCache(shape, kv(), kv(), sm((d,)), sm((r,)), sm(()), sm((d,)),
                       torch.zeros((S,), dtype=torch.int32, device=device))
        want = (KV_ON_HOST if kv_on_host else 0) | (SUMMARIES_ON_HOST if summaries_on_host else 0)
        if c.placement() != want:
            raise RuntimeError(f"cache placement {c.placement()} is not the requested {want}")
        return c

    def like(self):
        """A zeroed cache of the same shape and placement."""
        p = self.placement()
        return LayerCache.allocate(self.shape, self.seq_len.device, bool(p & KV_ON_HOST),
                                   bool(p & SUMMARIES_ON_HOST))

    def replicate(self):
        """A copy of this cache (same shape and placement, distinct memory)."""
        c = self.like()
        for a, b in zip(c.tensors(), self.tensors()):
            a.copy_(b)
        return c

    def tensors(self):
        return (self.k, self.v, self.kbar, self.dbar, self.cnt, self.vbar, self.seq_len)

    def placement(self) -> int:
        """cknv_kv_placement of this cache (checked once; host arrays are
        verified before any kernel can touch them)."""
        if self._placement is None:
            pl = I32(0)
            _check(lib().cknv_kv_placement(ctypes.byref(self.shape), ctypes.byref(self._raw_struct()),
                                           ctypes.byref(pl)), "cknv_kv_placement")
            self._placement = int(pl.value)
        return self._placement

    def _raw_struct(self) -> Cache:
        import torch
        s = self.shape
        n_tok = s.S * s.H * s.cap_blocks * BLOCK * s.d
        n_row = s.S * s.H * s.cap_blocks
        bf = (torch.bfloat16, torch.int16, torch.uint16)
        f32 = (torch.float32,)
        return Cache(_ptr(self.k, bf, n_tok, "k", True), _ptr(self.v, bf, n_tok, "v", True),
                     _ptr(self.kbar, f32, n_row * s.d, "kbar", True),
                     _ptr(self.dbar, f32, n_row * s.r, "dbar", True),
                     _ptr(self.cnt, f32, n_row, "cnt", True),
                     _ptr(self.vbar, f32, n_row * s.d, "vbar", True),
                     _ptr(self.seq_len, (torch.int32,), s.S, "seq_len"))

    def c_struct(self) -> Cache:
        if any(not t.is_cuda for t in self.tensors()):
            self.placement()  # host arrays: the device must map them at the same address
        return self._raw_struct()


def workspace_size(shape: Shape, max_blocks: int, budget: int) -> int:
    n = SZ(0)
    _check(lib().cknv_workspace_size(ctypes.byref(shape), max_blocks, budget, ctypes.byref(n)),
           "cknv_workspace_size")
    return int(n.value)


def allocate_workspace(shape: Shape, max_blocks: int, budget: int, device="cuda", stream=None):
    """A zeroed-counter workspace (uint8 tensor) for these sizes."""
    import torch
    ws = torch.empty(workspace_size(shape, max_blocks, budget), dtype=torch.uint8, device=device)
    _check(lib().cknv_workspace_init(ctypes.byref(shape), max_blocks, budget, _ptr(ws, what="ws"),
                                     ws.numel(), _stream(stream)), "cknv_workspace_init")
    return ws


def append(cache: LayerCache, new_k, new_v, stream=None):
    import torch
    s = cache.shape
    n = s.S * s.H * s.d
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    c = cache.c_struct()
    _check(lib().cknv_append(ctypes.byref(s), ctypes.byref(c), _ptr(new_k, bf, n, "new_k"),
                             _ptr(new_v, bf, n, "new_v"), _stream(stream)), "cknv_append")


def build_summaries(cache: LayerCache, max_blocks: int, stream=None):
    c = cache.c_struct()
    _check(lib().cknv_build_summaries(ctypes.byref(cache.shape), ctypes.byref(c), max_blocks,
                                      _stream(stream)), "cknv_build_summaries")


def score_select(cache: LayerCache, q, budget: int, max_blocks: int, sel, n_sel, ws,
                 scores=None, stream=None):
    import torch
    s = cache.shape
    Kb = budget // BLOCK
    c = cache.c_struct()
    _check(lib().cknv_score_select(
        ctypes.byref(s), ctypes.byref(c), _ptr(q, (torch.float32,), s.S * s.H * s.G * s.d, "q"),
        budget, max_blocks,
        _ptr(scores, (torch.float32,), s.S * s.H * s.cap_blocks, "scores"),
        _ptr(sel, (torch.int32,), s.S * s.H * Kb, "sel"),
        _ptr(n_sel, (torch.int32,), s.S * s.H, "n_sel"),
        _ptr(ws, what="ws"), ws.numel(), _stream(stream)), "cknv_score_select")


def attend(cache: LayerCache, q, sel, n_sel, budget: int, max_blocks: int, out, ws, lse=None,
           stream=None):
    import torch
    s = cache.shape
    Kb = budget // BLOCK
    nq = s.S * s.H * s.G
    c = cache.c_struct()
    _check(lib().cknv_attend(
        ctypes.byref(s), ctypes.byref(c), _ptr(q, (torch.float32,), nq * s.d, "q"),
        _ptr(sel, (torch.int32,), s.S * s.H * Kb, "sel"),
        _ptr(n_sel, (torch.int32,), s.S * s.H, "n_sel"), budget, max_blocks,
        _ptr(out, (torch.float32,), nq * s.d, "out"), _ptr(lse, (torch.float32,), nq, "lse"),
        _ptr(ws, what="ws"), ws.numel(), _stream(stream)), "cknv_attend")


def dense_attend(cache: LayerCache, q, budget: int, max_blocks: int, out, ws, lse=None,
                 stream=None):
    import torch
    s = cache.shape
    nq = s.S * s.H * s.G
    c = cache.c_struct()
    _check(lib().cknv_dense_attend(
        ctypes.byref(s), ctypes.byref(c), _ptr(q, (torch.float32,), nq * s.d, "q"), budget,
        max_blocks, _ptr(out, (torch.float32,), nq * s.d, "out"),
        _ptr(lse, (torch.float32,), nq, "lse"), _ptr(ws, what="ws"), ws.numel(),
        _stream(stream)), "cknv_dense_attend")


def decode_step(cache: LayerCache, new_k, new_v, q, budget: int, max_blocks: int, sel, n_sel,
                out, ws, lse=None, scores=None, stream=None):
    """cknv_decode_step: append + score/select + attend in one call."""
    import torch
    s = cache.shape
    Kb = budget // BLOCK
    nq = s.S * s.H * s.G
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    c = cache.c_struct()
    _check(lib().cknv_decode_step(
        ctypes.byref(s), ctypes.byref(c), _ptr(new_k, bf, s.S * s.H * s.d, "new_k"),
        _ptr(new_v, bf, s.S * s.H * s.d, "new_v"), _ptr(q, (torch.float32,), nq * s.d, "q"),
        budget, max_blocks, _ptr(scores, (torch.float32,), s.S * s.H * s.cap_blocks, "scores"),
        _ptr(sel, (torch.int32,), s.S * s.H * Kb, "sel"),
        _ptr(n_sel, (torch.int32,), s.S * s.H, "n_sel"),
        _ptr(out, (torch.float32,), nq * s.d, "out"), _ptr(lse, (torch.float32,), nq, "lse"),
        _ptr(ws, what="ws"), ws.numel(), _stream(stream)), "cknv_decode_step")


def decode_step_noalloc(cache: LayerCache, new_k, new_v, q, budget: int, max_blocks: int, sel,
                        n_sel, out, lse=None, scores=None, stream=None):
    """cknv_decode_step_noalloc: cknv_decode_step in the library's own per-GPU
    scratch array (no workspace argument; nothing is allocated)."""
    import torch
    s = cache.shape
    Kb = budget // BLOCK
    nq = s.S * s.H * s.G
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    c = cache.c_struct()
    _check(lib().cknv_decode_step_noalloc(
        ctypes.byref(s), ctypes.byref(c), _ptr(new_k, bf, s.S * s.H * s.d, "new_k"),
        _ptr(new_v, bf, s.S * s.H * s.d, "new_v"), _ptr(q, (torch.float32,), nq * s.d, "q"),
        budget, max_blocks, _ptr(scores, (torch.float32,), s.S * s.H * s.cap_blocks, "scores"),
        _ptr(sel, (torch.int32,), s.S * s.H * Kb, "sel"),
        _ptr(n_sel, (torch.int32,), s.S * s.H, "n_sel"),
        _ptr(out, (torch.float32,), nq * s.d, "out"), _ptr(lse, (torch.float32,), nq, "lse"),
        _stream(stream)), "cknv_decode_step_noalloc")


class DecodeStep:
    """Buffers for one CompKV decode step of a layer: append, score/select, attend.

    Holds the workspace and the sel/n_sel/out/lse tensors sized for
    (max_blocks, budget)."""

    def __init__(self, cache: LayerCache, max_blocks: int, budget: int, want_scores=False,
                 stream=None, fused=False):
        import torch
        self.fused = fused
        s = cache.shape
        dev = cache.seq_len.device  # k and v may be host-resident (host-offload placement)
        self.cache, self.max_blocks, self.budget = cache, max_blocks, budget
        self.Kb = budget // BLOCK
        self.ws = allocate_workspace(s, max_blocks, budget, device=dev, stream=stream)
        self.sel = torch.zeros((s.S * s.H, self.Kb), dtype=torch.int32, device=dev)
        self.n_sel = torch.zeros((s.S * s.H,), dtype=torch.int32, device=dev)
        self.out = torch.zeros((s.S, s.H * s.G, s.d), dtype=torch.float32, device=dev)
        self.lse = torch.zeros((s.S, s.H * s.G), dtype=torch.float32, device=dev)
        self.scores = (torch.zeros((s.S, s.H, s.cap_blocks), dtype=torch.float32, device=dev)
                       if want_scores else None)

    def __call__(self, q, new_k=None, new_v=None, stream=None):
        if self.fused and new_k is not None:
            decode_step(self.cache, new_k, new_v, q, self.budget, self.max_blocks, self.sel,
                        self.n_sel, self.out, self.ws, self.lse, self.scores, stream)
            return self.out
        if new_k is not None:
            append(self.cache, new_k, new_v, stream)
        score_select(self.cache, q, self.budget, self.max_blocks, self.sel, self.n_sel, self.ws,
                     self.scores, stream)
        attend(self.cache, q, self.sel, self.n_sel, self.budget, self.max_blocks, self.out,
               self.ws, self.lse, stream)
        return self.out


def blocks_for(tokens: int) -> int:
    return int(math.ceil(tokens / BLOCK))


class BoundStep:
    """Pre-marshalled arguments of one layer's decode step (append, score/select,
    attend) on a fixed stream, so that issuing a step is three foreign calls.
    The tensors passed in must stay alive while this object is used."""

    def __init__(self, cache: LayerCache, max_blocks: int, budget: int, ws, sel, n_sel, out,
                 lse, q, new_k, new_v, stream, scores=None):
        import torch
        s = cache.shape
        L = lib()
        self._keep = (cache, ws, sel, n_sel, out, lse, q, new_k, new_v, scores)
        self.shape = ctypes.byref(s)
        self.cache_c = cache.c_struct()
        cp = ctypes.byref(self.cache_c)
        st = _stream(stream)
        w, wn = _ptr(ws, what="ws"), ws.numel()
        qp = _ptr(q, (torch.float32,), s.S * s.H * s.G * s.d, "q")
        bf = (torch.bfloat16, torch.int16, torch.uint16)
        self.append_args = (self.shape, cp, _ptr(new_k, bf, s.S * s.H * s.d, "new_k"),
                            _ptr(new_v, bf, s.S * s.H * s.d, "new_v"), st)
        self.score_args = (self.shape, cp, qp, budget, max_blocks,
                           _ptr(scores, (torch.float32,), s.S * s.H * s.cap_blocks, "scores"),
                           _ptr(sel, (torch.int32,), s.S * s.H * (budget // BLOCK), "sel"),
                           _ptr(n_sel, (torch.int32,), s.S * s.H, "n_sel"), w, wn, st)
        self.attend_args = (self.shape, cp, qp, self.score_args[6], self.score_args[7], budget,
                            max_blocks, _ptr(out, (torch.float32,), s.S * s.H * s.G * s.d, "out"),
                            _ptr(lse, (torch.float32,), s.S * s.H * s.G, "lse"), w, wn, st)
        self.dense_args = (self.shape, cp, qp, budget, max_blocks, self.attend_args[7],
                           self.attend_args[8], w, wn, st)
        self.fused_args = (self.shape, cp, self.append_args[2], self.append_args[3], qp, budget,
                           max_blocks, self.score_args[5], self.score_args[6], self.score_args[7],
                           self.attend_args[7], self.attend_args[8], w, wn, st)
        self._append, self._score = L.cknv_append, L.cknv_score_select
        self._attend, self._dense = L.cknv_attend, L.cknv_dense_attend
        self.dscore_args = self.fused_args[:7] + (w, wn, st)
        self.dfinish_args = (self.shape, cp) + self.fused_args[4:]
        self._fused = L.cknv_decode_step
        self._dscore, self._dfinish = L.cknv_decode_score, L.cknv_decode_finish

    def append(self):
        st = self._append(*self.append_args)
        if st:
            raise CknvError(st, "cknv_append")

    def score_select(self):
        st = self._score(*self.score_args)
        if st:
            raise CknvError(st, "cknv_score_select")

    def attend(self):
        st = self._attend(*self.attend_args)
        if st:
            raise CknvError(st, "cknv_attend")

    def dense(self):
        st = self._dense(*self.dense_args)
        if st:
            raise CknvError(st, "cknv_dense_attend")

    def step(self):
        """One decode step as three calls (append, score_select, attend)."""
        self.append()
        self.score_select()
        self.attend()

    def fused_step(self):
        """One decode step as one call (cknv_decode_step)."""
        st = self._fused(*self.fused_args)
        if st:
            raise CknvError(st, "cknv_decode_step")

    def decode_score(self):
        """First half of cknv_decode_step (the append and the streaming scoring pass)."""
        st = self._dscore(*self.dscore_args)
        if st:
            raise CknvError(st, "cknv_decode_score")

    def decode_finish(self):
        """Second half of cknv_decode_step."""
        st = self._dfinish(*self.dfinish_args)
        if st:
            raise CknvError(st, "cknv_decode_finish")


class DecodeGraph:
    """Decode steps of several layers captured as one HIP graph.

    `steps` are BoundStep objects created on `stream`; each one's `method`
    ("fused_step" for cknv_decode_step, "step" for the three calls) is
    recorded once, in order, and replay() re-issues the whole sweep with one
    launch. The kernels read the context length from the device-resident
    seq_len, so every replay is the next decode step of every layer, with
    whatever the bound q, new_k and new_v tensors hold at replay time; the
    captured max_blocks bounds how many replays still append. Capture records
    kernels only (no memset: the step's counters are reset by its kernels).
    """

    def __init__(self, steps, stream, method="fused_step"):
        import torch
        if method not in ("fused_step", "step"):
            raise ValueError(f"method {method!r}: expected 'fused_step' or 'step'")
        self.steps = list(steps)
        self.graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(self.graph, stream=stream):
            for b in self.steps:
                getattr(b, method)()
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()
