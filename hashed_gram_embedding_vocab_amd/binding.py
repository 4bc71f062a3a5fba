"""Thin Python binding of libengram.so (argument marshalling only).

Every entry point mirrors a C function of ``include/engram.h`` /
``include/engram_synth.h`` with the same name.  Tensors are torch tensors on
the GPU; only their device pointers cross the boundary, together with the
current HIP stream.  All computation happens in the HIP kernels of the
library.  If the library is not built this module raises: there is no CPU
fallback.
"""

from __future__ import annotations

import atexit
import ctypes as C
import os
import threading
import weakref
from typing import Dict, Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libengram.so")

OK, E_INVALID_ARG, E_UNSUPPORTED, E_DEVICE, E_NOMEM = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
CONV_LINEAR, CONV_SILU_SKIP = 0, 1
OUT_DELTA = 1
RETRIEVE_IN_PROJECTION = 2  # engram_forward: retrieval inside the projection launches
WEIGHTS_PACKED = 4  # engram_forward / engram_gate_fuse: W_k and W_v as engram_pack_weight wrote them
MAX_TABLES, MAX_BRANCHES = 32, 4
NOALLOC_SCRATCH_BYTES = 64 << 20  # ENGRAM_NOALLOC_SCRATCH_BYTES
KERNEL_NAMES = ("hash", "gather", "gemm", "fuse", "aux", "gemm_v", "gate", "seam", "bwd_gemm", "bwd_fuse",
                "bwd_table")


class EngramError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))
        self.status = status


class Config(C.Structure):
    _fields_ = [
        ("vocab", C.c_int32), ("vocab_comp", C.c_int32), ("n_orders", C.c_int32),
        ("orders", C.c_int32 * 4), ("heads", C.c_int32), ("head_dim", C.c_int32),
        ("table_rows", C.c_uint32 * MAX_TABLES), ("hash_seed", C.c_uint64),
        ("d_model", C.c_int32), ("n_branches", C.c_int32), ("conv_kernel", C.c_int32),
        ("conv_mode", C.c_int32), ("rms_eps", C.c_float), ("dtype", C.c_int32),
        ("state_dtype", C.c_int32),
    ]


class WeightsC(C.Structure):
    _fields_ = [
        ("w_k", C.c_void_p * MAX_BRANCHES), ("w_v", C.c_void_p),
        ("gamma_h", C.c_void_p * MAX_BRANCHES), ("gamma_k", C.c_void_p * MAX_BRANCHES),
        ("conv_w", C.c_void_p),
    ]


class ProfileC(C.Structure):
    _fields_ = [("total_ms", C.c_double * len(KERNEL_NAMES)), ("launches", C.c_int64 * len(KERNEL_NAMES)),
                ("dropped", C.c_int64)]


class GradsC(C.Structure):
    _fields_ = [
        ("dw", C.c_void_p), ("dgamma_h", C.c_void_p), ("dgamma_k", C.c_void_p), ("dconv_w", C.c_void_p),
        ("row_ids", C.c_void_p), ("row_grads", C.c_void_p), ("row_counts", C.c_void_p),
    ]


class RowCacheC(C.Structure):
    _fields_ = [("keys", C.c_void_p), ("rows", C.c_void_p), ("capacity", C.c_uint32)]


_lib = None
_lock = threading.Lock()


def lib() -> C.CDLL:
    """Load libengram.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError("libengram.so not built at %s: run "
                              "`python -m hashed_gram_embedding_vocab_amd.build`" % LIB_PATH)
        L = C.CDLL(LIB_PATH)
        P, i32, i64, u32, u64 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_uint64
        L.engram_status_string.restype = C.c_char_p
        L.engram_status_string.argtypes = [C.c_int]
        L.engram_plan_create.restype = C.c_int
        L.engram_plan_create.argtypes = [C.POINTER(Config), C.POINTER(C.c_void_p)]
        L.engram_plan_destroy.restype = C.c_int
        L.engram_plan_destroy.argtypes = [P]
        L.engram_workspace_size.restype = C.c_size_t
        L.engram_workspace_size.argtypes = [P, i32, i32]
        L.engram_pack_weight.restype = C.c_int
        L.engram_pack_weight.argtypes = [P, P, P, P]
        L.engram_hash.restype = C.c_int
        L.engram_hash.argtypes = [P, P, i32, i32, P, P, P, P, P]
        L.engram_gather.restype = C.c_int
        L.engram_gather.argtypes = [P, P, i64, P, P, P]
        L.engram_gate_fuse.restype = C.c_int
        L.engram_gate_fuse.argtypes = [P, P, P, i32, i32, C.POINTER(WeightsC), P, P, P, u32, P,
                                       C.c_size_t, P]
        L.engram_forward.restype = C.c_int
        L.engram_forward.argtypes = [P, P, i32, i32, P, P, P, P, C.POINTER(WeightsC), P, P, P, u32,
                                     P, C.c_size_t, P, P]
        L.engram_retrieve.restype = C.c_int
        L.engram_retrieve.argtypes = [P, P, i32, i32, P, P, P, P, P, P]
        L.engram_forward_noalloc.restype = C.c_int
        L.engram_forward_noalloc.argtypes = [P, P, i32, i32, P, P, P, P, C.POINTER(WeightsC), P, P, P, u32,
                                             P, P]
        L.engram_backward_workspace_size.restype = C.c_size_t
        L.engram_backward_workspace_size.argtypes = [P, i32, i32]
        L.engram_backward.restype = C.c_int
        L.engram_backward.argtypes = [P, P, P, P, C.POINTER(WeightsC), P, i32, i32, u32, P, C.POINTER(GradsC),
                                      P, C.c_size_t, P]
        L.engram_profile_begin.restype = C.c_int
        L.engram_profile_begin.argtypes = [P, i32, u32]
        L.engram_profile_end.restype = C.c_int
        L.engram_profile_end.argtypes = [P, C.POINTER(ProfileC)]
        L.engram_profile_every.restype = C.c_int
        L.engram_profile_every.argtypes = [P, i32]
        L.engram_host_alloc.restype = C.c_int
        L.engram_host_alloc.argtypes = [C.c_size_t, C.POINTER(C.c_void_p)]
        L.engram_host_free.restype = C.c_int
        L.engram_host_free.argtypes = [P]
        L.engram_prefetcher_create.restype = C.c_int
        L.engram_prefetcher_create.argtypes = [P, P, C.POINTER(RowCacheC), i64, i32, C.POINTER(C.c_void_p)]
        L.engram_prefetcher_destroy.restype = C.c_int
        L.engram_prefetcher_destroy.argtypes = [P]
        L.engram_prefetch_begin.restype = C.c_int
        L.engram_prefetch_begin.argtypes = [P, P, i64, P]
        L.engram_prefetch_finish.restype = C.c_int
        L.engram_prefetch_finish.argtypes = [P, P, C.POINTER(C.c_uint32), P]
        L.engram_cache_build.restype = C.c_int
        L.engram_cache_build.argtypes = [P, P, i32, P, C.POINTER(RowCacheC), P]
        L.engram_gather_cached.restype = C.c_int
        L.engram_gather_cached.argtypes = [P, P, i64, P, C.POINTER(RowCacheC), P, i32, P]
        L.engram_synth_fill_table.restype = C.c_int
        L.engram_synth_fill_table.argtypes = [i32, u64, i32, i64, i32, P, P]
        L.engram_probe_stream.restype = C.c_int
        L.engram_probe_stream.argtypes = [i32, u32, i32, i32, P, P, i64, P]
        _lib = L
        return L


def _check(fn: str, status: int):
    if status != OK:
        raise EngramError(fn, status, lib().engram_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    return C.c_void_p(t.data_ptr())


_live_host_buffers = weakref.WeakSet()


class HostBuffer:
    """Pinned host memory from engram_host_alloc that the GPU reads directly
    (tables kept in host DRAM).  `tensor` is a CPU view of it; the memory is
    released by free(), when the object is collected, or at interpreter exit
    (before the HIP runtime shuts down); no kernel may still read it then."""

    def __init__(self, nbytes: int):
        p = C.c_void_p()
        _check("engram_host_alloc", lib().engram_host_alloc(nbytes, C.byref(p)))
        self.ptr = p.value
        self.nbytes = nbytes
        self.tensor = torch.frombuffer((C.c_uint8 * nbytes).from_address(self.ptr), dtype=torch.uint8)
        _live_host_buffers.add(self)

    def view(self, dtype, shape):
        return self.tensor.view(dtype).view(shape)

    def free(self):
        if getattr(self, "ptr", None):
            self.tensor = None
            lib().engram_host_free(C.c_void_p(self.ptr))
            self.ptr = None

    def __del__(self):
        self.free()


@atexit.register
def _free_host_buffers():
    for hb in list(_live_host_buffers):
        hb.free()


def _table_ptr(t) -> int:
    """Device address of a table: a HIP tensor, or a HostBuffer's memory."""
    if isinstance(t, HostBuffer):
        return t.ptr
    return _ptr(t, "table").value


def _host_table_ptr(t) -> int:
    """Host address of a table the host threads read: a HostBuffer or a
    contiguous CPU tensor."""
    if isinstance(t, HostBuffer):
        return t.ptr
    if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_contiguous():
        raise TypeError("host tables must be HostBuffer objects or contiguous CPU tensors")
    return t.data_ptr()


class Prefetcher:
    """engram_prefetcher_*: host threads gather the rows that miss the HBM
    cache from host tables; a DMA engine copies them to the GPU."""

    def __init__(self, plan: "Plan", host_tables, cache: Optional["RowCache"], max_tokens: int, n_threads: int = 8):
        self._tables = list(host_tables)  # kept alive while the prefetcher may read them
        self._cache = cache
        ptrs = (C.c_void_p * len(self._tables))(*[_host_table_ptr(t) for t in self._tables])
        h = C.c_void_p()
        _check("engram_prefetcher_create", lib().engram_prefetcher_create(
            plan._h, ptrs, None if cache is None else C.byref(cache.c), max_tokens, n_threads, C.byref(h)))
        self._h = h

    def begin(self, idx, stream=None):
        _check("engram_prefetch_begin", lib().engram_prefetch_begin(
            self._h, _ptr(idx, "idx", (torch.int32, torch.uint32)), idx.shape[0], _stream(stream)))

    def finish(self, emb, stream=None) -> int:
        """Enqueue E's assembly; returns how many (token, table) pairs missed the cache."""
        n = C.c_uint32(0)
        _check("engram_prefetch_finish", lib().engram_prefetch_finish(
            self._h, _ptr(emb, "emb"), C.byref(n), _stream(stream)))
        return int(n.value)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().engram_prefetcher_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()


class RowCache:
    """Device buffers of a hot-row cache: keys [n_tables][capacity] uint32 and
    rows [n_tables][capacity][d_e]."""

    def __init__(self, n_tables: int, capacity: int, head_dim: int, dtype, device="cuda"):
        self.capacity = capacity
        self.keys = torch.zeros((n_tables, max(capacity, 1)), dtype=torch.int32, device=device)
        self.rows = torch.zeros((n_tables, max(capacity, 1), head_dim), dtype=dtype, device=device)
        self.c = RowCacheC(C.c_void_p(self.keys.data_ptr()), C.c_void_p(self.rows.data_ptr()), capacity)


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _torch_dtype(dt: int):
    return torch.bfloat16 if dt == BF16 else torch.float32


class Grads:
    """Device tensors receiving engram_backward's gradients (fp32), plus their C struct."""

    def __init__(self, n_branches: int, d: int, emb_dim: int, conv_k: int, n_tables: int, n_tok: int,
                 head_dim: int, device="cuda"):
        f = dict(dtype=torch.float32, device=device)
        self.dw = torch.zeros((n_branches + 1, d, emb_dim), **f)
        self.dgamma_h = torch.zeros((n_branches, d), **f)
        self.dgamma_k = torch.zeros((n_branches, d), **f)
        self.dconv_w = torch.zeros((d, conv_k), **f)
        self.row_ids = torch.zeros((n_tables, n_tok), dtype=torch.int32, device=device)
        self.row_grads = torch.zeros((n_tables, n_tok, head_dim), **f)
        self.row_counts = torch.zeros((n_tables,), dtype=torch.int32, device=device)
        self.c = GradsC(*[C.c_void_p(t.data_ptr()) for t in (self.dw, self.dgamma_h, self.dgamma_k, self.dconv_w,
                                                            self.row_ids, self.row_grads, self.row_counts)])


class Weights:
    """Device tensors of one layer's weights, plus their C struct."""

    def __init__(self, w_k: Sequence[torch.Tensor], w_v: torch.Tensor, gamma_h: Sequence[torch.Tensor],
                 gamma_k: Sequence[torch.Tensor], conv_w: torch.Tensor):
        self.w_k, self.w_v = list(w_k), w_v
        self.gamma_h, self.gamma_k, self.conv_w = list(gamma_h), list(gamma_k), conv_w
        s = WeightsC()
        for m, t in enumerate(self.w_k):
            s.w_k[m] = _ptr(t, "w_k[%d]" % m).value
        for m, t in enumerate(self.gamma_h):
            s.gamma_h[m] = _ptr(t, "gamma_h[%d]" % m, torch.float32).value
        for m, t in enumerate(self.gamma_k):
            s.gamma_k[m] = _ptr(t, "gamma_k[%d]" % m, torch.float32).value
        s.w_v = _ptr(w_v, "w_v").value
        s.conv_w = _ptr(conv_w, "conv_w", torch.float32).value
        self.c = s


class Plan:
    """An engram_plan: immutable hashing and shape constants of one Engram layer."""

    def __init__(self, vocab: int, vocab_comp: int, heads: int, head_dim: int,
                 table_rows: Sequence[int], hash_seed: int, d_model: int, n_branches: int = 1,
                 conv_kernel: int = 4, conv_mode: int = CONV_LINEAR, rms_eps: float = 1e-6,
                 dtype: int = BF16, orders: Sequence[int] = (2, 3), state_dtype: int = F32):
        cfg = Config()
        cfg.vocab, cfg.vocab_comp = vocab, vocab_comp
        cfg.n_orders = len(orders)
        for i, o in enumerate(orders):
            cfg.orders[i] = o
        cfg.heads, cfg.head_dim = heads, head_dim
        if len(table_rows) > MAX_TABLES:
            raise ValueError("too many tables")
        for i, r in enumerate(table_rows):
            cfg.table_rows[i] = r
        cfg.hash_seed = hash_seed & 0xFFFFFFFFFFFFFFFF
        cfg.d_model, cfg.n_branches = d_model, n_branches
        cfg.conv_kernel, cfg.conv_mode, cfg.rms_eps, cfg.dtype = conv_kernel, conv_mode, rms_eps, dtype
        cfg.state_dtype = state_dtype
        self.cfg = cfg
        self.state_torch_dtype = _torch_dtype(state_dtype)
        self.n_tables = len(orders) * heads
        self.emb_dim = self.n_tables * head_dim
        self.dtype = dtype
        self.torch_dtype = _torch_dtype(dtype)
        h = C.c_void_p()
        _check("engram_plan_create", lib().engram_plan_create(C.byref(cfg), C.byref(h)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.engram_plan_destroy(h)
            self._h = None

    # ------------------------------------------------------------------ ABI calls
    def engram_workspace_size(self, batch: int, seqlen: int) -> int:
        return int(lib().engram_workspace_size(self._h, batch, seqlen))

    def engram_pack_weight(self, w, packed, stream=None):
        """Pack one [d][D_e] weight matrix into packed (same shape and dtype)."""
        _check("engram_pack_weight", lib().engram_pack_weight(
            self._h, _ptr(w, "w", self.torch_dtype), _ptr(packed, "packed", self.torch_dtype), _stream(stream)))

    def packed_weights(self, w: "Weights", stream=None) -> "Weights":
        """The weights with every W_k and W_v packed by engram_pack_weight into
        new tensors (pass flags=WEIGHTS_PACKED with them)."""
        def pk(t):
            out = torch.empty_like(t)
            self.engram_pack_weight(t, out, stream)
            return out
        return Weights([pk(t) for t in w.w_k], pk(w.w_v), w.gamma_h, w.gamma_k, w.conv_w)

    def engram_hash(self, tokens, comp_map, idx, prev_ctx=None, bad_tokens=None, stream=None):
        batch, seqlen = tokens.shape
        _check("engram_hash", lib().engram_hash(
            self._h, _ptr(tokens, "tokens", torch.int32), batch, seqlen,
            _ptr(comp_map, "comp_map", torch.int32), _ptr(prev_ctx, "prev_ctx", torch.int32),
            _ptr(idx, "idx", (torch.int32, torch.uint32)), _ptr(bad_tokens, "bad_tokens", (torch.int32, torch.uint32)),
            _stream(stream)))

    def engram_gather(self, idx, tables: Sequence[torch.Tensor], emb, stream=None):
        n_tok = idx.shape[0]
        ptrs = (C.c_void_p * len(tables))(*[_table_ptr(t) for t in tables])
        _check("engram_gather", lib().engram_gather(
            self._h, _ptr(idx, "idx", (torch.int32, torch.uint32)), n_tok, ptrs,
            _ptr(emb, "emb", self.torch_dtype), _stream(stream)))

    def engram_retrieve(self, tokens, comp_map, tables: Sequence[torch.Tensor], emb, prev_ctx=None,
                        bad_tokens=None, stream=None):
        """Hash and gather into emb ([batch*seqlen][D_e]); then roll prev_ctx if given."""
        batch, seqlen = tokens.shape
        ptrs = (C.c_void_p * len(tables))(*[_table_ptr(t) for t in tables])
        _check("engram_retrieve", lib().engram_retrieve(
            self._h, _ptr(tokens, "tokens", torch.int32), batch, seqlen, _ptr(comp_map, "comp_map", torch.int32),
            _ptr(prev_ctx, "prev_ctx", torch.int32), ptrs, _ptr(emb, "emb", self.torch_dtype),
            _ptr(bad_tokens, "bad_tokens", (torch.int32, torch.uint32)), _stream(stream)))

    def engram_cache_build(self, hot, tables, cache: RowCache, stream=None):
        """hot: [n_tables][n_hot] int32 device tensor of row numbers."""
        ptrs = (C.c_void_p * len(tables))(*[_table_ptr(t) for t in tables])
        n_hot = 0 if hot is None else hot.shape[1]
        _check("engram_cache_build", lib().engram_cache_build(
            self._h, _ptr(hot, "hot", (torch.int32, torch.uint32)), n_hot, ptrs, C.byref(cache.c),
            _stream(stream)))

    def engram_gather_cached(self, idx, tables, cache: Optional[RowCache], emb, max_workgroups: int = 0,
                             stream=None):
        n_tok = idx.shape[0]
        ptrs = (C.c_void_p * len(tables))(*[_table_ptr(t) for t in tables])
        _check("engram_gather_cached", lib().engram_gather_cached(
            self._h, _ptr(idx, "idx", (torch.int32, torch.uint32)), n_tok, ptrs,
            None if cache is None else C.byref(cache.c), _ptr(emb, "emb", self.torch_dtype), max_workgroups,
            _stream(stream)))

    def engram_gate_fuse(self, emb, h, weights: Weights, out, workspace, batch: int, seqlen: int,
                         conv_state=None, alpha=None, flags: int = 0, stream=None):
        _check("engram_gate_fuse", lib().engram_gate_fuse(
            self._h, _ptr(emb, "emb", self.torch_dtype), _ptr(h, "h", self.torch_dtype), batch, seqlen,
            C.byref(weights.c), _ptr(conv_state, "conv_state", self.state_torch_dtype),
            _ptr(out, "out", self.torch_dtype), _ptr(alpha, "alpha", torch.float32), flags,
            _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _stream(stream)))

    def engram_forward(self, tokens, comp_map, tables: Sequence[torch.Tensor], h, weights: Weights,
                       out, workspace, prev_ctx=None, conv_state=None, alpha=None, flags: int = 0,
                       bad_tokens=None, stream=None):
        batch, seqlen = tokens.shape
        ptrs = (C.c_void_p * len(tables))(*[_table_ptr(t) for t in tables])
        _check("engram_forward", lib().engram_forward(
            self._h, _ptr(tokens, "tokens", torch.int32), batch, seqlen,
            _ptr(comp_map, "comp_map", torch.int32), _ptr(prev_ctx, "prev_ctx", torch.int32), ptrs,
            _ptr(h, "h", self.torch_dtype), C.byref(weights.c),
            _ptr(conv_state, "conv_state", self.state_torch_dtype), _ptr(out, "out", self.torch_dtype),
            _ptr(alpha, "alpha", torch.float32), flags, _ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(),
            _ptr(bad_tokens, "bad_tokens", (torch.int32, torch.uint32)), _stream(stream)))

    def engram_forward_noalloc(self, tokens, comp_map, tables: Sequence[torch.Tensor], h, weights: Weights,
                               out, prev_ctx=None, conv_state=None, alpha=None, flags: int = 0,
                               bad_tokens=None, stream=None):
        """engram_forward on the library's per-GPU scratch array (no workspace argument)."""
        batch, seqlen = tokens.shape
        ptrs = (C.c_void_p * len(tables))(*[_table_ptr(t) for t in tables])
        _check("engram_forward_noalloc", lib().engram_forward_noalloc(
            self._h, _ptr(tokens, "tokens", torch.int32), batch, seqlen,
            _ptr(comp_map, "comp_map", torch.int32), _ptr(prev_ctx, "prev_ctx", torch.int32), ptrs,
            _ptr(h, "h", self.torch_dtype), C.byref(weights.c),
            _ptr(conv_state, "conv_state", self.state_torch_dtype), _ptr(out, "out", self.torch_dtype),
            _ptr(alpha, "alpha", torch.float32), flags,
            _ptr(bad_tokens, "bad_tokens", (torch.int32, torch.uint32)), _stream(stream)))

    def engram_backward_workspace_size(self, batch: int, seqlen: int) -> int:
        return int(lib().engram_backward_workspace_size(self._h, batch, seqlen))

    def engram_backward(self, idx, tables: Sequence[torch.Tensor], h, weights: "Weights", dout, dh,
                        grads: "Grads", workspace, batch: int, seqlen: int, flags: int = 0, stream=None):
        ptrs = (C.c_void_p * len(tables))(*[_table_ptr(t) for t in tables])
        _check("engram_backward", lib().engram_backward(
            self._h, _ptr(idx, "idx", (torch.int32, torch.uint32)), ptrs, _ptr(h, "h", self.torch_dtype),
            C.byref(weights.c), _ptr(dout, "dout", self.torch_dtype), batch, seqlen, flags,
            _ptr(dh, "dh", self.torch_dtype), C.byref(grads.c), _ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)))

    def backward_workspace(self, batch: int, seqlen: int, device="cuda") -> torch.Tensor:
        n = self.engram_backward_workspace_size(batch, seqlen)
        if n == 0:
            raise EngramError("engram_backward_workspace_size", E_UNSUPPORTED, "unsupported shape")
        return torch.empty(n, dtype=torch.uint8, device=device)

    def engram_profile_begin(self, max_launches: int = 4096, kinds: Optional[Sequence[str]] = None):
        """Time launches of the named kinds (KERNEL_NAMES; None: all)."""
        mask = 0 if kinds is None else sum(1 << KERNEL_NAMES.index(k) for k in kinds)
        _check("engram_profile_begin", lib().engram_profile_begin(self._h, max_launches, mask))

    def engram_profile_every(self, every: int):
        """Time one launch in `every` of each selected kind (1: all)."""
        _check("engram_profile_every", lib().engram_profile_every(self._h, every))

    def engram_profile_end(self) -> Dict[str, Dict[str, float]]:
        p = ProfileC()
        _check("engram_profile_end", lib().engram_profile_end(self._h, C.byref(p)))
        out = {n: {"total_ms": p.total_ms[i], "launches": int(p.launches[i])}
               for i, n in enumerate(KERNEL_NAMES)}
        out["dropped"] = int(p.dropped)
        return out

    # ------------------------------------------------------------------ helpers
    def workspace(self, batch: int, seqlen: int, device="cuda") -> torch.Tensor:
        """A caller-owned workspace tensor of the required size (256-byte aligned by torch)."""
        return torch.empty(self.engram_workspace_size(batch, seqlen), dtype=torch.uint8, device=device)


def engram_synth_fill_table(table: torch.Tensor, seed: int, tau: int, dtype: int, stream=None):
    rows, head_dim = table.shape
    _check("engram_synth_fill_table", lib().engram_synth_fill_table(
        dtype, seed & 0xFFFFFFFFFFFFFFFF, tau, rows, head_dim,
        _ptr(table, "table", _torch_dtype(dtype)), _stream(stream)))


PROBE_NONTEMPORAL = 1


def engram_probe_stream(mode: int, src: torch.Tensor, dst: torch.Tensor, nbytes: int, unroll: int = 8,
                        blocks: int = 2048, flags: int = 0, stream=None):
    """Streaming read (mode 0) or copy (mode 1) of nbytes of src: a
    measurement helper, not part of the method."""
    if nbytes > src.numel() * src.element_size() or (mode == 1 and nbytes > dst.numel() * dst.element_size()):
        raise ValueError("nbytes exceeds a buffer")
    if mode == 0 and dst.numel() * dst.element_size() < 16:
        raise ValueError("the read probe's sink needs 16 bytes")
    _check("engram_probe_stream", lib().engram_probe_stream(mode, flags, unroll, blocks, _ptr(src, "src"),
                                                            _ptr(dst, "dst"), nbytes, _stream(stream)))
