"""Shared helpers for the parity tests: oracle expectations and tolerances.

Expected values always come from the CPU oracle (``oracle/``) run on the
same seeded inputs; nothing here reads a result of the HIP path.
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

import oracle
from synthetic import workloads as W


def oracle_dtype(wl: W.Workload) -> int:
    return oracle.BF16 if wl.dtype == "bf16" else oracle.F32


def oracle_indices(wl: W.Workload, li: W.LayerInputs, tokens: np.ndarray, comp: np.ndarray,
                   prev_ctx: Optional[np.ndarray] = None):
    return oracle.hash_tokens(tokens, comp, wl.vocab, wl.vocab_comp, wl.heads, wl.primes(),
                              li.hash_seed, prev_ctx=prev_ctx, orders=wl.orders)


def rows_needed(positions: Iterable[int], seqlen: int, conv_k: int) -> np.ndarray:
    need = set()
    for r in positions:
        b, t = divmod(int(r), seqlen)
        for j in range(conv_k):
            if t - j >= 0:
                need.add(b * seqlen + t - j)
    return np.array(sorted(need), np.int64)


def oracle_layer(wl: W.Workload, li: W.LayerInputs, idx: np.ndarray, batch: int, seqlen: int,
                 rows: Optional[np.ndarray] = None, conv_state=None, conv_mode=oracle.CONV_LINEAR,
                 flags=0, eps=1e-6) -> oracle.Layer:
    """An oracle.Layer whose E holds the oracle's own gathered rows (all rows,
    or only ``rows``, the rest left zero and never read)."""
    dt = oracle_dtype(wl)
    n_tok = batch * seqlen
    if rows is None:
        emb = oracle.gather_synth(idx, wl.head_dim, li.table_seed, dt)
    else:
        emb = np.zeros((n_tok, wl.emb_dim), np.uint16 if dt == oracle.BF16 else np.float32)
        if len(rows):
            emb[rows] = oracle.gather_synth(idx[rows], wl.head_dim, li.table_seed, dt)
    return oracle.Layer(emb, li.h, li.w_k, li.w_v, li.gamma_h, li.gamma_k, li.conv_w, batch, seqlen,
                        dt, conv_state=conv_state, conv_mode=conv_mode, flags=flags, eps=eps)


def sample_positions(batch: int, seqlen: int, n: int, seed: int = 0) -> np.ndarray:
    """Edge positions (sequence starts, tile and block seams, ends) plus random ones.

    Seams are sequence-relative (positions around 32 and 128) and global:
    the tokens around multiples of 256, where one token tile of the
    projection kernels ends and the next begins."""
    rng = np.random.default_rng(seed)
    cand = set()
    for b in {0, batch - 1}:
        for t in (0, 1, 2, 3, 31, 32, 33, 127, 128, 129, seqlen - 2, seqlen - 1):
            if 0 <= t < seqlen:
                cand.add(b * seqlen + t)
    n_tok = batch * seqlen
    n_seams = (n_tok - 1) // 256
    for k in sorted({1, 2, (n_seams + 1) // 2, n_seams}):
        for dt in (-1, 0, 1, 2, 3):
            g = 256 * k + dt
            if 1 <= k <= n_seams and 0 <= g < n_tok:
                cand.add(g)
    while len(cand) < n:
        cand.add(int(rng.integers(0, batch * seqlen)))
    return np.array(sorted(cand), np.int64)


# ------------------------------------------------------------------ tolerances

def bf16_bound(ref: np.ndarray) -> np.ndarray:
    """bf16 storage with fp32 accumulation: |d| <= 1e-2 + 2e-2 |ref|."""
    return 1e-2 + 2e-2 * np.abs(ref)


def f32_bound(ref: np.ndarray) -> np.ndarray:
    """fp32 end to end: |d| <= 1e-5 * max(|ref|, rms of the row).

    On elements with |ref| >= the row's RMS this is the plain elementwise
    relative error 1e-5; below that the floor is 1e-5 x row RMS absolute, since
    the output of a sum of d_model products carries absolute (not relative)
    rounding error, and an element that cancels to near zero cannot keep 1e-5
    of its own size.  f32_split_errors reports the two parts apart."""
    rms = np.sqrt(np.mean(ref.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return 1e-5 * np.maximum(np.abs(ref), rms)


F32_REL_TOL = 1e-5

# worst errors of every fp32 check in this process, by part (printed at the
# end of a pytest session)
f32_stats = {"checks": 0, "n_large": 0, "max_rel_large": 0.0, "n_small": 0, "max_abs_over_rms_small": 0.0}


def f32_split_errors(got: np.ndarray, ref: np.ndarray):
    """(max elementwise relative error over elements with |ref| >= row RMS,
    their count, max |d| / row RMS over the rest, their count)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    rms_b = np.broadcast_to(rms, ref.shape)
    diff = np.abs(got - ref)
    large = (np.abs(ref) >= rms_b) & (rms_b > 0)
    small = ~large
    rel_large = float((diff[large] / np.abs(ref[large])).max()) if large.any() else 0.0
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(rms_b[small] > 0, diff[small] / rms_b[small], np.where(diff[small] > 0, np.inf, 0.0))
    abs_small = float(q.max()) if small.any() else 0.0
    return rel_large, int(large.sum()), abs_small, int(small.sum())


def assert_within(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bound = bf16_bound(ref) if dtype == "bf16" else f32_bound(ref)
    diff = np.abs(got - ref)
    ratio = diff / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite values"
    assert ratio.max() <= 1.0, "%s: max |d|/bound = %.3f at %s (got %r, ref %r)" % (
        what, ratio.max(), worst, got[worst], ref[worst])
    if dtype != "bf16" and ref.ndim >= 1 and ref.size:
        rel_large, n_large, abs_small, n_small = f32_split_errors(got, ref)
        f32_stats["checks"] += 1
        f32_stats["n_large"] += n_large
        f32_stats["n_small"] += n_small
        f32_stats["max_rel_large"] = max(f32_stats["max_rel_large"], rel_large)
        f32_stats["max_abs_over_rms_small"] = max(f32_stats["max_abs_over_rms_small"], abs_small)
        assert rel_large <= F32_REL_TOL, "%s: elementwise relative error %.3e on |ref| >= row RMS" % (
            what, rel_large)


def alpha_tol(dtype: str) -> float:
    # fp32 gate arithmetic on exact (bf16) or fp32 products; 2e-4 absolute
    # leaves a margin of several hundred fp32 ulps of the pre-sigmoid score.
    return 2e-4 if dtype == "bf16" else 1e-5
