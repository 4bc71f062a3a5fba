"""Workload shapes and seeded input generators (harness, not method).

Every workload below is a synthetic stand-in for the configurations the
Engram pages discuss ("Conditional Memory via Scalable Lookup", as
summarised on the five source pages): the pages name no dataset for the
throughput figures, only that n-gram access follows a Zipf law, so token
streams are finite-Zipf samples over the vocabulary and the embedding
tables hold procedurally generated values standing in for trained rows.

Nothing in this module computes any step of the Engram forward pass.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

# Default hash seed: the ASCII bytes "ENGRAM" followed by 0x00 0x01.  For a
# stack with Engram at several layers, the low byte holds the layer id.
HASH_SEED_BASE = 0x454E4752414D0000

# Procedural table recipe (shared definition, implemented independently by
# the oracle in C and by the HIP fill kernel; no code is shared):
#   words = Philox4x64-10(counter = (row, col // 4, tau, 0), key = (seed, 0))
#   w     = words[col % 4]                      (a uint64)
#   S     = sum of the four 16-bit fields of w  (0 .. 262140)
#   x     = fp32(S - 131070) * C, C = fp32 0x1.1bc77ap-21
#           (the fp32 nearest 0.02 / sqrt(4 * (2**32 - 1) / 12))
#   fp32 tables store x; bf16 tables store x rounded to nearest-even.
# S is an Irwin-Hall(4) sum of uniform 16-bit integers: mean 131070 and
# standard deviation sqrt((2**32 - 1) / 3), so x has mean 0 and sd 0.02.
TABLE_RECIPE = {
    "generator": "philox4x64_10",
    "counter": "(row, col // 4, tau, 0)",
    "key": "(seed, 0)",
    "offset": 131070,
    "scale_f32_bits": 0x350DE3BD,
    "sd": 0.02,
}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int               # stable id used to offset seeds
    vocab: int               # raw vocabulary V
    batch: int               # sequences per step
    seqlen: int              # tokens per sequence in this call
    zipf_s: Optional[float]  # None = uniform token ids
    heads: int               # K hash heads per n-gram order
    head_dim: int            # d_e, row width of every table
    table_target: int        # primes are the 2K largest primes <= this
    same_prime: bool         # every table uses the single largest prime
    dtype: str               # "f32" or "bf16" (tables, h, W, E, out)
    d_model: int             # hidden size d
    n_branches: int          # residual branches sharing tables and W_v
    conv_kernel: int = 4
    layers: tuple = (0,)     # Engram insertion layers (hash seed low byte)
    decode: bool = False     # carries prev_ctx / conv_state from a context
    orders: tuple = (2, 3)
    state_dtype: str = "f32"  # element type of the carried conv state ("f32" or "bf16")

    @property
    def vocab_comp(self) -> int:
        # The pages report a 23% smaller vocabulary after compression.
        return int(round(0.77 * self.vocab))

    @property
    def n_tables(self) -> int:
        return len(self.orders) * self.heads

    @property
    def emb_dim(self) -> int:
        return self.n_tables * self.head_dim

    @property
    def n_tokens(self) -> int:
        return self.batch * self.seqlen

    def primes(self) -> List[int]:
        if self.same_prime:
            p = largest_primes_at_most(self.table_target, 1)[0]
            return [p] * self.n_tables
        return largest_primes_at_most(self.table_target, self.n_tables)

    def table_bytes(self) -> int:
        eb = 4 if self.dtype == "f32" else 2
        return sum(self.primes()) * self.head_dim * eb

    def hash_seed(self, layer: int) -> int:
        return HASH_SEED_BASE | (layer & 0xFF) if self.layers != (0,) else HASH_SEED_BASE | 1

    def seed(self, base: int, layer_slot: int = 0) -> int:
        return base + 100 * self.index + 1000 * layer_slot

    def with_shape(self, batch: int, seqlen: int) -> "Workload":
        return dataclasses.replace(self, batch=batch, seqlen=seqlen)


def _w(**kw) -> Workload:
    return Workload(**kw)


# The five configurations the build is measured on (sizes and distributions
# as the workload statement gives them; table sizes follow from the stated
# parameter totals: 5.7B bf16 params over 16 tables of 80 dims is 4,453,125
# rows per table, 100B is 78,125,000 and 2 x 2.85B is 2,226,562).
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        _w(name="tiny", index=1, vocab=1000, batch=2, seqlen=128, zipf_s=1.1,
           heads=4, head_dim=32, table_target=10007, same_prime=True,
           dtype="f32", d_model=256, n_branches=1),
        _w(name="small", index=2, vocab=32000, batch=8, seqlen=4096, zipf_s=1.1,
           heads=8, head_dim=64, table_target=500009, same_prime=False,
           dtype="bf16", d_model=1024, n_branches=1),
        _w(name="layer27b", index=3, vocab=129280, batch=8, seqlen=4096, zipf_s=1.05,
           heads=8, head_dim=80, table_target=4453125, same_prime=False,
           dtype="bf16", d_model=2560, n_branches=1),
        _w(name="maxtable_zipf", index=4, vocab=129280, batch=8, seqlen=4096, zipf_s=1.05,
           heads=8, head_dim=80, table_target=78125000, same_prime=False,
           dtype="bf16", d_model=2560, n_branches=1),
        _w(name="maxtable_uniform", index=4, vocab=129280, batch=8, seqlen=4096, zipf_s=None,
           heads=8, head_dim=80, table_target=78125000, same_prime=False,
           dtype="bf16", d_model=2560, n_branches=1),
        _w(name="multibranch_prefill", index=5, vocab=129280, batch=1, seqlen=32768, zipf_s=1.05,
           heads=8, head_dim=80, table_target=2226562, same_prime=False,
           dtype="bf16", d_model=2560, n_branches=4, layers=(2, 6)),
        _w(name="multibranch_decode", index=5, vocab=129280, batch=256, seqlen=1, zipf_s=1.05,
           heads=8, head_dim=80, table_target=2226562, same_prime=False,
           dtype="bf16", d_model=2560, n_branches=4, layers=(2, 6), decode=True, state_dtype="bf16"),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


# ----------------------------------------------------------------------------
# primes
# ----------------------------------------------------------------------------

def _is_prime(n: int) -> bool:
    if n < 2:
        return False
    if n % 2 == 0:
        return n == 2
    r = math.isqrt(n)
    f = 3
    while f <= r:
        if n % f == 0:
            return False
        f += 2
    return True


def largest_primes_at_most(limit: int, count: int) -> List[int]:
    """The ``count`` largest distinct primes <= ``limit``, in descending order."""
    out = []
    n = limit
    while len(out) < count:
        if n < 2:
            raise ValueError("not enough primes below limit")
        if _is_prime(n):
            out.append(n)
        n -= 1
    return out


# ----------------------------------------------------------------------------
# compression map and tokens
# ----------------------------------------------------------------------------

def compression_map(vocab: int, vocab_comp: int, seed: int) -> np.ndarray:
    """A seeded surjective map [0, V) -> [0, V').

    Stand-in for the pages' tokenizer compression (surface variants of a
    token share one id, about 23% fewer ids); the real normalisation rules
    need the tokenizer, which is not available.  Every id in [0, V') appears
    at least once because the first V' entries before shuffling are 0..V'-1.
    """
    rng = np.random.default_rng(seed)
    p = np.concatenate([np.arange(vocab_comp, dtype=np.int64),
                        rng.integers(0, vocab_comp, vocab - vocab_comp)])
    rng.shuffle(p)
    return p.astype(np.int32)


def _zipf_ranks(n: int, vocab: int, s: float, rng: np.random.Generator) -> np.ndarray:
    """Finite Zipf over ranks 1..vocab, P(r) proportional to r**-s (0-based out)."""
    r = np.arange(1, vocab + 1, dtype=np.float64)
    p = r ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = rng.random(n)
    ranks = np.searchsorted(cdf, u, side="right")
    return np.minimum(ranks, vocab - 1)


def make_tokens(wl: Workload, seed: Optional[int] = None, batch: Optional[int] = None,
                seqlen: Optional[int] = None, zipf_s: Optional[float] = "default",
                perm_seed: Optional[int] = None) -> np.ndarray:
    """Raw token ids [batch][seqlen] int32: Zipf over a seeded rank->id
    permutation (seed + 1 unless perm_seed is given: batches that share a
    perm_seed share which tokens are frequent, as text of one language does)."""
    seed = wl.seed(2) if seed is None else seed
    batch = wl.batch if batch is None else batch
    seqlen = wl.seqlen if seqlen is None else seqlen
    s = wl.zipf_s if zipf_s == "default" else zipf_s
    rng = np.random.default_rng(seed)
    n = batch * seqlen
    if s is None:
        ids = rng.integers(0, wl.vocab, n)
    else:
        perm = np.random.default_rng(seed + 1 if perm_seed is None else perm_seed).permutation(wl.vocab)
        ids = perm[_zipf_ranks(n, wl.vocab, s, rng)]
    return ids.astype(np.int32).reshape(batch, seqlen)


# ----------------------------------------------------------------------------
# dense inputs
# ----------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of fp32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclasses.dataclass
class LayerInputs:
    """Dense inputs for one Engram layer; float arrays are fp32 holding values
    exactly representable in the workload dtype (bf16-rounded for bf16)."""
    h: np.ndarray            # [B_r][n_tok][d]
    w_k: np.ndarray          # [B_r][d][D_e]   (row n produces output channel n)
    w_v: np.ndarray          # [d][D_e]
    gamma_h: np.ndarray      # [B_r][d] fp32
    gamma_k: np.ndarray      # [B_r][d] fp32
    conv_w: np.ndarray       # [d][K_c] fp32, last tap = current token
    table_seed: int
    hash_seed: int
    prev_ctx: Optional[np.ndarray] = None    # [batch][2] int32 compressed ids
    conv_state: Optional[np.ndarray] = None  # [B_r][batch][K_c-1][d] fp32


def make_layer_inputs(wl: Workload, layer_slot: int = 0, batch: Optional[int] = None,
                      seqlen: Optional[int] = None, with_h: bool = True) -> LayerInputs:
    batch = wl.batch if batch is None else batch
    seqlen = wl.seqlen if seqlen is None else seqlen
    n_tok = batch * seqlen
    d, De, Br = wl.d_model, wl.emb_dim, wl.n_branches
    cast = round_to_bf16 if wl.dtype == "bf16" else (lambda a: np.ascontiguousarray(a, np.float32))

    rng_h = np.random.default_rng(wl.seed(4, layer_slot))
    h = cast(rng_h.standard_normal((Br, n_tok, d), dtype=np.float32)) if with_h else None

    rng_w = np.random.default_rng(wl.seed(5, layer_slot))
    w_k = cast(rng_w.standard_normal((Br, d, De), dtype=np.float32) * np.float32(1.0 / math.sqrt(De)))
    w_v = cast(rng_w.standard_normal((d, De), dtype=np.float32) *
               np.float32(1.0 / (0.02 * math.sqrt(De))))
    gamma_h = (1.0 + 0.1 * rng_w.standard_normal((Br, d))).astype(np.float32)
    gamma_k = (1.0 + 0.1 * rng_w.standard_normal((Br, d))).astype(np.float32)
    conv_w = (0.5 * rng_w.standard_normal((d, wl.conv_kernel))).astype(np.float32)

    layer = wl.layers[layer_slot]
    li = LayerInputs(h=h, w_k=w_k, w_v=w_v, gamma_h=gamma_h, gamma_k=gamma_k, conv_w=conv_w,
                     table_seed=wl.seed(3, layer_slot), hash_seed=wl.hash_seed(layer))
    if wl.decode:
        rng_s = np.random.default_rng(wl.seed(6, layer_slot))
        if wl.zipf_s is None:
            li.prev_ctx = rng_s.integers(0, wl.vocab_comp, (batch, 2)).astype(np.int32)
        else:
            li.prev_ctx = _zipf_ranks(batch * 2, wl.vocab_comp, wl.zipf_s, rng_s).astype(
                np.int32).reshape(batch, 2)
        li.conv_state = rng_s.standard_normal(
            (Br, batch, wl.conv_kernel - 1, d), dtype=np.float32)
        if wl.state_dtype == "bf16":  # a bf16 state holds bf16 values exactly
            li.conv_state = round_to_bf16(li.conv_state)
    return li
