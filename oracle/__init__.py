"""CPU oracle for the Engram forward pass -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (the HIP library under
``hashed_gram_embedding_vocab_amd``) never imports it and shares no code with
it.  The arithmetic lives in ``engram_oracle.c`` (plain single-threaded C,
fp64 accumulation); this module only builds it with gcc and marshals NumPy
arrays through ctypes.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "engram_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F32, BF16 = 0, 1
CONV_LINEAR, CONV_SILU_SKIP = 0, 1
OUT_DELTA = 1


def build(force: bool = False) -> str:
    """Compile engram_oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = C.CDLL(_LIB)
            u64, i64, i32, u32 = C.c_uint64, C.c_int64, C.c_int32, C.c_uint32
            P = C.c_void_p
            L.orc_mix64.restype = u64
            L.orc_mix64.argtypes = [u64]
            L.orc_table_seed.restype = u64
            L.orc_table_seed.argtypes = [u64, i32]
            L.orc_ngram_key.restype = u64
            L.orc_ngram_key.argtypes = [P, i32, i32]
            L.orc_project.restype = None
            L.orc_project.argtypes = [P, P, i32, i32, i32, P]
            L.orc_ngram_slot.restype = u32
            L.orc_ngram_slot.argtypes = [P, i32, i32, u64, u32]
            L.orc_hash.restype = i64
            L.orc_hash.argtypes = [P, i64, i64, P, i32, i32, P, i32, P, i32, P, u64, P, P]
            L.orc_philox4x64_10.restype = None
            L.orc_philox4x64_10.argtypes = [P, P, P]
            L.orc_synth_value.restype = C.c_float
            L.orc_synth_value.argtypes = [u64, i32, u64, i32]
            L.orc_bf16_rne.restype = C.c_uint16
            L.orc_bf16_rne.argtypes = [C.c_float]
            L.orc_gather_synth.restype = None
            L.orc_gather_synth.argtypes = [P, i64, i32, i32, u64, i32, P]
            L.orc_gather_host.restype = None
            L.orc_gather_host.argtypes = [P, i64, i32, i32, P, i32, P]
            L.orc_gate_token.restype = C.c_double
            L.orc_gate_token.argtypes = [P, P, P, P, P, P, i32, i32, C.c_double, i32, P]
            L.orc_forward_range.restype = i32
            L.orc_forward_range.argtypes = [i64, i64, i64, i64, i64, i32, i32, i32, i32, i32,
                                            C.c_double, u32, i32, P, P, P, P, P, P, P, P, P, P, P]
            L.orc_conv_state_update.restype = None
            L.orc_conv_state_update.argtypes = [i64, i64, i32, i32, i32, P, P, P]
            L.orc_backward.restype = i32
            L.orc_backward.argtypes = [i64, i64, i32, i32, i32, i32, i32, C.c_double, u32, i32,
                                       P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
            L.orc_table_grad.restype = None
            L.orc_table_grad.argtypes = [P, i64, i32, i32, P, P, P, P]
            _lib = L
        return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- hashing

def mix64(z: int) -> int:
    return int(lib().orc_mix64(z & 0xFFFFFFFFFFFFFFFF))


def table_seed(hash_seed: int, tau: int) -> int:
    return int(lib().orc_table_seed(hash_seed, tau))


def ngram_key(g: Sequence[int], vocab_comp: int) -> int:
    ga = _c(list(g), np.int32)
    return int(lib().orc_ngram_key(_p(ga), len(g), vocab_comp))


def ngram_slot(g: Sequence[int], vocab_comp: int, seed_tau: int, prime: int) -> int:
    ga = _c(list(g), np.int32)
    return int(lib().orc_ngram_slot(_p(ga), len(g), vocab_comp, seed_tau, prime))


def hash_tokens(tokens: np.ndarray, comp_map: np.ndarray, vocab: int, vocab_comp: int,
                heads: int, primes: Sequence[int], hash_seed: int,
                prev_ctx: Optional[np.ndarray] = None, orders=(2, 3)):
    """idx [batch*seqlen][len(orders)*heads] uint32, bad-token count, new prev_ctx [batch][2]."""
    tokens = _c(tokens, np.int32)
    batch, seqlen = tokens.shape
    n_tables = len(orders) * heads
    idx = np.zeros((batch * seqlen, n_tables), np.uint32)
    new_ctx = np.zeros((batch, 2), np.int32)
    pc = None if prev_ctx is None else _c(prev_ctx, np.int32)
    bad = lib().orc_hash(_p(tokens), batch, seqlen, _p(_c(comp_map, np.int32)), vocab, vocab_comp,
                         _p(pc), len(orders), _p(_c(list(orders), np.int32)), heads,
                         _p(_c(list(primes), np.uint32)), hash_seed, _p(idx), _p(new_ctx))
    return idx, int(bad), new_ctx


# ---------------------------------------------------------------- synthetic tables

def philox4x64_10(ctr: Sequence[int], key: Sequence[int]) -> np.ndarray:
    c = _c(list(ctr), np.uint64)
    k = _c(list(key), np.uint64)
    out = np.zeros(4, np.uint64)
    lib().orc_philox4x64_10(_p(c), _p(k), _p(out))
    return out


def synth_value(seed: int, tau: int, row: int, col: int) -> float:
    return float(lib().orc_synth_value(seed, tau, row, col))


def bf16_rne(x: float) -> int:
    return int(lib().orc_bf16_rne(x))


def gather_synth(idx: np.ndarray, head_dim: int, table_seed: int, dtype: int) -> np.ndarray:
    """E [n_tok][n_tables*head_dim]: fp32 values, or bf16 bit patterns (uint16)."""
    idx = _c(idx, np.uint32)
    n_tok, n_tables = idx.shape
    emb = np.zeros((n_tok, n_tables * head_dim), np.uint16 if dtype == BF16 else np.float32)
    lib().orc_gather_synth(_p(idx), n_tok, n_tables, head_dim, table_seed, dtype, _p(emb))
    return emb


def gather_host(idx: np.ndarray, tables: Sequence[np.ndarray], dtype: int) -> np.ndarray:
    idx = _c(idx, np.uint32)
    n_tok, n_tables = idx.shape
    head_dim = tables[0].shape[1]
    tabs = [np.ascontiguousarray(t) for t in tables]
    ptrs = (C.c_void_p * n_tables)(*[t.ctypes.data for t in tabs])
    emb = np.zeros((n_tok, n_tables * head_dim), np.uint16 if dtype == BF16 else np.float32)
    lib().orc_gather_host(_p(idx), n_tok, n_tables, head_dim, ptrs, dtype, _p(emb))
    return emb


# ---------------------------------------------------------------- gate / fusion

def _stored(a: np.ndarray, dtype: int) -> np.ndarray:
    """Arrays in the workload dtype: fp32 as-is, bf16 as uint16 bit patterns."""
    if dtype == BF16:
        if a.dtype == np.uint16:
            return np.ascontiguousarray(a)
        a = np.ascontiguousarray(a, np.float32)
        return (a.view(np.uint32) >> 16).astype(np.uint16)
    return _c(a, np.float32)


def project(e, w, dtype: int) -> np.ndarray:
    d, De = w.shape
    y = np.zeros(d, np.float64)
    lib().orc_project(_p(_stored(e, dtype)), _p(_stored(w, dtype)), d, De, dtype, _p(y))
    return y


def gate_token(e, h, w_k, w_v, gamma_h, gamma_k, eps: float, dtype: int, want_u=True):
    d, De = w_k.shape
    u = np.zeros(d, np.float64) if want_u else None
    a = lib().orc_gate_token(_p(_stored(e, dtype)), _p(_stored(h, dtype)), _p(_stored(w_k, dtype)),
                             _p(_stored(w_v, dtype)), _p(_c(gamma_h, np.float32)),
                             _p(_c(gamma_k, np.float32)), d, De, eps, dtype, _p(u))
    return a, u


class Layer:
    """One Engram layer's dense inputs in stored form, ready for repeated oracle calls."""

    def __init__(self, emb, h, w_k, w_v, gamma_h, gamma_k, conv_w, batch, seqlen, dtype,
                 conv_state=None, conv_mode=CONV_LINEAR, eps=1e-6, flags=0):
        self.dtype = dtype
        self.emb = _stored(emb, dtype)
        self.h = _stored(h, dtype)
        self.w_k = _stored(w_k, dtype)
        self.w_v = _stored(w_v, dtype)
        self.gamma_h = _c(gamma_h, np.float32)
        self.gamma_k = _c(gamma_k, np.float32)
        self.conv_w = _c(conv_w, np.float32)
        self.conv_state = None if conv_state is None else _c(conv_state, np.float32)
        self.batch, self.seqlen = batch, seqlen
        self.n_branches, self.d, self.De = self.w_k.shape
        self.conv_k = self.conv_w.shape[1]
        self.conv_mode, self.eps, self.flags = conv_mode, eps, flags

    def forward_range(self, b: int, t0: int, t1: int, want_u=False):
        n = t1 - t0
        out = np.zeros((self.n_branches, n, self.d), np.float64)
        alpha = np.zeros((self.n_branches, n), np.float64)
        u = np.zeros((self.n_branches, n, self.d), np.float64) if want_u else None
        rc = lib().orc_forward_range(b, t0, t1, self.batch, self.seqlen, self.d, self.De,
                                     self.n_branches, self.conv_k, self.conv_mode, self.eps,
                                     self.flags, self.dtype, _p(self.emb), _p(self.h),
                                     _p(self.w_k), _p(self.w_v), _p(self.gamma_h),
                                     _p(self.gamma_k), _p(self.conv_w), _p(self.conv_state),
                                     _p(out), _p(alpha), _p(u))
        if rc != 0:
            raise ValueError("orc_forward_range: bad arguments")
        return out, alpha, u

    def forward_positions(self, rows: Sequence[int]):
        """out [B_r][len(rows)][d], alpha [B_r][len(rows)] at flat token rows b*seqlen+t."""
        outs, alphas = [], []
        for r in rows:
            b, t = divmod(int(r), self.seqlen)
            o, a, _ = self.forward_range(b, t, t + 1)
            outs.append(o[:, 0])
            alphas.append(a[:, 0])
        return np.stack(outs, 1), np.stack(alphas, 1)

    def forward_all(self, want_u=False):
        """Every position: out [B_r][n_tok][d], alpha [B_r][n_tok], u (optional)."""
        outs, alphas, us = [], [], []
        for b in range(self.batch):
            o, a, u = self.forward_range(b, 0, self.seqlen, want_u)
            outs.append(o)
            alphas.append(a)
            us.append(u)
        out = np.concatenate(outs, 1)
        alpha = np.concatenate(alphas, 1)
        u = np.concatenate(us, 1) if want_u else None
        return out, alpha, u

    def backward(self, dout) -> dict:
        """Gradients of <dout, out> over whole sequences (no carried conv state):
        dh [B_r][n_tok][d], demb [n_tok][De], dw_k [B_r][d][De], dw_v [d][De],
        dgamma_h, dgamma_k [B_r][d], dconv_w [d][K_c], all float64."""
        if self.conv_state is not None:
            raise ValueError("the backward oracle covers whole sequences (no carried state)")
        n_tok = self.batch * self.seqlen
        Br, d, De, kc = self.n_branches, self.d, self.De, self.conv_k
        g = {"dh": np.zeros((Br, n_tok, d)), "demb": np.zeros((n_tok, De)), "dw_k": np.zeros((Br, d, De)),
             "dw_v": np.zeros((d, De)), "dgamma_h": np.zeros((Br, d)), "dgamma_k": np.zeros((Br, d)),
             "dconv_w": np.zeros((d, kc))}
        rc = lib().orc_backward(self.batch, self.seqlen, d, De, Br, kc, self.conv_mode, self.eps, self.flags,
                                self.dtype, _p(self.emb), _p(self.h), _p(self.w_k), _p(self.w_v),
                                _p(self.gamma_h), _p(self.gamma_k), _p(self.conv_w),
                                _p(_stored(dout, self.dtype)), _p(g["dh"]), _p(g["demb"]), _p(g["dw_k"]),
                                _p(g["dw_v"]), _p(g["dgamma_h"]), _p(g["dgamma_k"]), _p(g["dconv_w"]))
        if rc != 0:
            raise ValueError("orc_backward: bad arguments")
        return g

    def new_conv_state(self, u_all: np.ndarray) -> np.ndarray:
        """State after this chunk, from the chunk's gated values u_all [B_r][n_tok][d]."""
        S = self.conv_k - 1
        tail = min(self.seqlen, S)
        u = u_all.reshape(self.n_branches, self.batch, self.seqlen, self.d)[:, :, self.seqlen - tail:]
        u = np.ascontiguousarray(u, np.float64)
        out = np.zeros((self.n_branches, self.batch, S, self.d), np.float32)
        lib().orc_conv_state_update(self.batch, self.seqlen, self.d, self.n_branches, self.conv_k,
                                    _p(u), _p(self.conv_state), _p(out))
        return out


def table_grad(idx: np.ndarray, demb: np.ndarray, head_dim: int):
    """Per table: distinct rows (ascending), their summed gradients and the
    count: rows [n_tables][n_tok] uint32, grads [n_tables][n_tok][head_dim]
    float64, counts [n_tables] (only the first counts[tau] entries are set)."""
    idx = _c(idx, np.uint32)
    n_tok, n_tables = idx.shape
    demb = _c(demb, np.float64)
    rows = np.zeros((n_tables, n_tok), np.uint32)
    grads = np.zeros((n_tables, n_tok, head_dim), np.float64)
    counts = np.zeros(n_tables, np.int64)
    lib().orc_table_grad(_p(idx), n_tok, n_tables, head_dim, _p(demb), _p(rows), _p(grads), _p(counts))
    return rows, grads, counts
