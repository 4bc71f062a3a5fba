"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle step to a fact fixed outside the oracle: a
published generator's known-answer value, a library routine (NumPy's
Philox, NumPy fp64 matmul, torch's depthwise conv1d and bf16 rounding),
brute-force enumeration over tiny vocabularies, closed forms of the gate,
or invariants the pages state (token-only retrieval, determinism,
causality).  All of these run on the CPU.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synthetic import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# generators (harness)
# ----------------------------------------------------------------------------

def test_splitmix64_known_answer():
    # SplitMix64 seeded with 0 (Steele, Lea & Flood 2014; Vigna's reference
    # splitmix64.c): the state advances by 0x9E3779B97F4A7C15 and the first
    # output is 0xE220A8397B1DCDAF.
    assert oracle.mix64(0x9E3779B97F4A7C15) == 0xE220A8397B1DCDAF
    # the per-table seed of table 0 under hash seed 0 is that same first output
    assert oracle.table_seed(0, 0) == 0xE220A8397B1DCDAF


def test_mix64_is_a_bijection_sample():
    rng = np.random.default_rng(11)
    xs = set(int(x) for x in rng.integers(0, 2**63, 20000, dtype=np.int64))
    ys = set(oracle.mix64(x) for x in xs)
    assert len(ys) == len(xs)


def _numpy_philox(ctr, key):
    """Philox4x64-10 block at counter ``ctr`` from NumPy's bit generator.

    NumPy increments the 256-bit counter before producing a block, so start
    it one below ``ctr``.
    """
    c = sum(int(v) << (64 * i) for i, v in enumerate(ctr))
    c = (c - 1) % (1 << 256)
    cw = [(c >> (64 * i)) & (2**64 - 1) for i in range(4)]
    bg = np.random.Philox(counter=np.array(cw, np.uint64), key=np.array(key, np.uint64))
    return bg.random_raw(4)


@pytest.mark.parametrize("ctr,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 2, 3, 4), (5, 6)),
    ((2**64 - 1, 2**64 - 1, 2**64 - 1, 2**64 - 1), (2**64 - 1, 2**64 - 1)),
    ((123456789, 19, 31, 0), (0x454E4752414D0001, 0)),
    ((78124999, 0, 15, 0), (403, 0)),
])
def test_philox_matches_numpy(ctr, key):
    assert list(oracle.philox4x64_10(ctr, key)) == list(_numpy_philox(ctr, key))


def test_synth_scale_constant():
    c = np.float32(0.02 / math.sqrt(4 * (2**32 - 1) / 12))
    assert int(c.view(np.uint32)) == W.TABLE_RECIPE["scale_f32_bits"]


def test_synth_value_from_numpy_philox():
    rng = np.random.default_rng(5)
    scale = np.uint32(W.TABLE_RECIPE["scale_f32_bits"]).view(np.float32)
    for _ in range(200):
        seed = int(rng.integers(0, 2**63))
        tau = int(rng.integers(0, 32))
        row = int(rng.integers(0, 80_000_000))
        col = int(rng.integers(0, 80))
        words = _numpy_philox((row, col // 4, tau, 0), (seed, 0))
        w = int(words[col % 4])
        s = sum((w >> (16 * i)) & 0xFFFF for i in range(4))
        expect = np.float32(s - 131070) * scale
        assert oracle.synth_value(seed, tau, row, col) == float(expect)


def test_synth_distribution():
    rng = np.random.default_rng(6)
    vals = np.array([oracle.synth_value(3, int(t), int(r), int(c))
                     for t, r, c in zip(rng.integers(0, 16, 20000), rng.integers(0, 10**7, 20000),
                                        rng.integers(0, 80, 20000))])
    assert abs(vals.mean()) < 4 * 0.02 / math.sqrt(len(vals))
    assert abs(vals.std() / 0.02 - 1) < 0.03
    assert np.abs(vals).max() <= 131070 * 5.3e-7


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(5000).astype(np.float32) * 0.02,
        rng.standard_normal(5000).astype(np.float32) * 100,
        # exact ties between two bf16 values, both parities
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        ((np.arange(1, 2000, dtype=np.uint32) << 16) | 0x8001).view(np.float32),
        ((np.arange(1, 2000, dtype=np.uint32) << 16) | 0x7FFF).view(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_rne(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)
    # the synthetic module's rounding of dense inputs agrees with torch too
    assert np.array_equal(W.bf16_bits(W.round_to_bf16(x)), ref)


# ----------------------------------------------------------------------------
# page facts and workloads
# ----------------------------------------------------------------------------

def _facts():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        return json.load(f)


def test_workloads_follow_page_facts():
    f = _facts()
    keep = f["compression_keep_fraction"]
    for wl in W.WORKLOADS.values():
        assert abs(wl.vocab_comp / wl.vocab - keep["value"]) <= keep["tolerance"]
        assert tuple(wl.orders) == tuple(f["ngram_orders"]["value"])
    # a 3-gram space of about 2e15 for a ~128k vocabulary
    v = W.workload("layer27b").vocab
    assert 0.5 < v**3 / f["trigram_space_order_of_magnitude"]["value"] < 2
    assert abs(v / f["vocab_nominal"]["value"] - 1) < 0.05
    # the 27B-class memory and the 100B offloaded table, in bf16 parameters
    p27 = sum(W.workload("layer27b").primes()) * 80
    assert abs(p27 / f["engram_27b_memory_params"]["value"] - 1) < 1e-3
    pmax = sum(W.workload("maxtable_zipf").primes()) * 80
    assert abs(pmax / f["offloaded_table_params"]["value"] - 1) < 1e-3
    assert list(W.workload("multibranch_prefill").layers) == f["insertion_layers"]["value"]


def _is_prime_sieve(n):
    if n < 2:
        return False
    for p in range(2, int(n**0.5) + 1):
        if n % p == 0:
            return False
    return True


def test_primes():
    assert W.largest_primes_at_most(10007, 1) == [10007]
    ps = W.largest_primes_at_most(500009, 16)
    assert ps[0] == 500009 and len(set(ps)) == 16 and ps == sorted(ps, reverse=True)
    assert all(_is_prime_sieve(p) for p in ps)
    # no prime was skipped between consecutive picks
    for a, b in zip(ps, ps[1:]):
        assert not any(_is_prime_sieve(q) for q in range(b + 1, a))


def test_compression_map_surjective():
    for wl in W.WORKLOADS.values():
        p = W.compression_map(wl.vocab, wl.vocab_comp, wl.seed(1))
        assert p.shape == (wl.vocab,) and p.min() >= 0 and p.max() < wl.vocab_comp
        assert len(np.unique(p)) == wl.vocab_comp


# ----------------------------------------------------------------------------
# O1-O3: compression, suffix n-grams, hashing
# ----------------------------------------------------------------------------

TINY_V, TINY_VC = 7, 5


# Per-table primes of the tiny-vocabulary pins.  They all differ and are not
# sorted (the order-3 tables' primes exceed the order-2 tables'), and each is
# well below the number of distinct n-grams its table sees, so a hash that
# reduced every table by one table's prime, by a head's prime instead of the
# table's, or by the tables' primes in another order, leaves residues of p_tau
# unreached or reaches values >= p_tau, and these pins fail.
TINY_PRIMES = {2: [7, 5, 13, 11], 3: [5, 3, 2, 23, 19, 17]}


def _tiny_setup(heads=2, seed=0x1234):
    comp = W.compression_map(TINY_V, TINY_VC, 99)
    pre = {int(c): int(np.nonzero(comp == c)[0][0]) for c in range(TINY_VC)}  # one raw id per class
    primes = list(TINY_PRIMES[heads])
    assert len(set(primes)) == 2 * heads and all(_is_prime_sieve(q) for q in primes)
    return comp, pre, primes, seed


# SplitMix64 from its published definition (Steele, Lea & Flood 2014): the
# state advances by the golden-ratio increment and each output is the state
# passed through the finalizer.  Written here with Python integers, apart from
# the oracle, for direct evaluation of single n-grams.
_GOLDEN = 0x9E3779B97F4A7C15
_M64 = (1 << 64) - 1


def _py_mix64(z):
    z &= _M64
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & _M64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def _py_slot(g, vocab_comp, hash_seed, tau, prime):
    """Slot of n-gram g (oldest id first) in table tau: the base-(V'+1) key,
    mixed with the tau-th SplitMix64 output of the hash seed, reduced by that
    table's own prime."""
    key = 0
    for c in g:
        key = key * (vocab_comp + 1) + int(c)
    s_tau = _py_mix64(hash_seed + (tau + 1) * _GOLDEN)
    return _py_mix64(key ^ s_tau) % prime


def test_splitmix64_sequence_gives_table_seeds():
    # the first five outputs of SplitMix64 seeded with 0 (Vigna's reference
    # splitmix64.c); table tau's seed under hash seed 0 is output tau
    seq = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC,
           0x1B39896A51A8749B]
    assert [oracle.table_seed(0, t) for t in range(5)] == seq
    assert [_py_mix64((t + 1) * _GOLDEN) for t in range(5)] == seq


def _check_table_ranges(idx, primes):
    """Table tau's slots lie in [0, p_tau) and, over a stream that holds far
    more distinct n-grams than p_tau, reach every residue of p_tau."""
    for tau, p in enumerate(primes):
        col = idx[:, tau].astype(np.int64)
        assert col.min() >= 0 and col.max() < p, (tau, p, int(col.max()))
        assert len(np.unique(col)) == p, (tau, p, len(np.unique(col)))


def test_ngram_key_injective_exhaustive():
    vc = TINY_VC
    ids = range(vc + 1)  # PAD = vc included
    for n in (2, 3):
        keys = [oracle.ngram_key(g, vc) for g in itertools.product(ids, repeat=n)]
        assert len(set(keys)) == len(keys)
        assert max(keys) < (vc + 1) ** n
    # the largest configuration's 3-gram keys stay below 2^63
    assert (99546 + 1) ** 3 < 2**63


def test_hash_bruteforce_all_trigrams():
    """Every length-3 sequence over a 5-id compressed vocabulary: the streaming
    hash must equal direct evaluation of the suffix n-grams at each position."""
    heads = 2
    comp, pre, primes, seed = _tiny_setup(heads)
    seqs = list(itertools.product(range(TINY_VC), repeat=3))
    toks = np.array([[pre[a], pre[b], pre[c]] for a, b, c in seqs], np.int32)
    idx, bad, _ = oracle.hash_tokens(toks, comp, TINY_V, TINY_VC, heads, primes, seed)
    assert bad == 0
    P = TINY_VC
    for s, (a, b, c) in enumerate(seqs):
        grams = {0: [(P, a), (P, P, a)], 1: [(a, b), (P, a, b)], 2: [(b, c), (a, b, c)]}
        for t in range(3):
            row = idx[s * 3 + t]
            for o, g in enumerate(grams[t]):
                for k in range(heads):
                    tau = o * heads + k
                    assert row[tau] == oracle.ngram_slot(g, TINY_VC, oracle.table_seed(seed, tau),
                                                         primes[tau])
                    assert row[tau] == _py_slot(g, TINY_VC, seed, tau, primes[tau])
    _check_table_ranges(idx, primes)


def _de_bruijn(k, n):
    a = [0] * k * n
    seq = []

    def db(t, p):
        if t > n:
            if n % p == 0:
                seq.extend(a[1:p + 1])
        else:
            a[t] = a[t - p]
            db(t + 1, p)
            for j in range(a[t - p] + 1, k):
                a[t] = j
                db(t + 1, t)
    db(1, 1)
    return seq


def test_hash_de_bruijn_stream():
    heads = 3
    comp, pre, primes, seed = _tiny_setup(heads)
    s = _de_bruijn(TINY_VC, 3)
    s = s + s[:2]  # cyclic -> linear: every 3-gram appears exactly once
    assert len(set(zip(s, s[1:], s[2:]))) == TINY_VC**3 == len(s) - 2
    toks = np.array([[pre[c] for c in s]], np.int32)
    idx, _, _ = oracle.hash_tokens(toks, comp, TINY_V, TINY_VC, heads, primes, seed)
    for t in range(2, len(s)):
        for o, g in enumerate([(s[t - 1], s[t]), (s[t - 2], s[t - 1], s[t])]):
            for k in range(heads):
                tau = o * heads + k
                assert idx[t, tau] == oracle.ngram_slot(g, TINY_VC, oracle.table_seed(seed, tau),
                                                        primes[tau])
                assert idx[t, tau] == _py_slot(g, TINY_VC, seed, tau, primes[tau])
    # from position 2 on: 25 distinct 2-grams and 125 distinct 3-grams
    _check_table_ranges(idx[2:], primes)


def test_identical_ngrams_hit_identical_slots():
    """Determinism: the same suffix n-gram maps to the same slots wherever it
    occurs, and retrieval depends only on the token sequence."""
    wl = W.workload("tiny")
    comp = W.compression_map(wl.vocab, wl.vocab_comp, wl.seed(1))
    toks = W.make_tokens(wl)
    idx1, _, _ = oracle.hash_tokens(toks, comp, wl.vocab, wl.vocab_comp, wl.heads, wl.primes(), 77)
    idx2, _, _ = oracle.hash_tokens(toks.copy(), comp, wl.vocab, wl.vocab_comp, wl.heads,
                                    wl.primes(), 77)
    assert np.array_equal(idx1, idx2)
    c = comp[toks]
    seen = {}
    for b in range(c.shape[0]):
        for t in range(2, c.shape[1]):
            g = (int(c[b, t - 2]), int(c[b, t - 1]), int(c[b, t]))
            row = tuple(idx1[b * c.shape[1] + t, wl.heads:])
            assert seen.setdefault(g, row) == row


def test_hash_chunking_with_prev_ctx():
    wl = W.workload("tiny")
    comp = W.compression_map(wl.vocab, wl.vocab_comp, wl.seed(1))
    toks = W.make_tokens(wl, seqlen=50)
    args = (comp, wl.vocab, wl.vocab_comp, wl.heads, wl.primes(), 5)
    full, _, ctx_full = oracle.hash_tokens(toks, *args)
    full = full.reshape(toks.shape[0], toks.shape[1], -1)
    ctx = None
    parts = []
    for a, b in [(0, 1), (1, 2), (2, 17), (17, 50)]:
        p, _, ctx = oracle.hash_tokens(toks[:, a:b], *args, prev_ctx=ctx)
        parts.append(p.reshape(toks.shape[0], b - a, -1))
    assert np.array_equal(np.concatenate(parts, 1), full)
    assert np.array_equal(ctx, ctx_full)
    assert np.array_equal(ctx_full, comp[toks[:, -2:]])


def test_hash_out_of_range_tokens_are_pad():
    comp, pre, primes, seed = _tiny_setup(2)
    good = np.array([[pre[1], pre[2], pre[3], pre[4]]], np.int32)
    badt = good.copy()
    badt[0, 1] = -5
    badt[0, 3] = TINY_V
    idx_bad, nbad, _ = oracle.hash_tokens(badt, comp, TINY_V, TINY_VC, 2, primes, seed)
    assert nbad == 2
    # PAD id = vocab_comp occupies the bad positions
    P = TINY_VC
    c = [1, P, 3, P]
    ext = [P, P] + c
    for t in range(4):
        g2, g3 = ext[t + 1:t + 3], ext[t:t + 3]
        for tau in range(4):
            g = g2 if tau < 2 else g3
            assert idx_bad[t, tau] == oracle.ngram_slot(g, TINY_VC, oracle.table_seed(seed, tau), primes[tau])
            assert idx_bad[t, tau] == _py_slot(g, TINY_VC, seed, tau, primes[tau])


def test_hash_uniformity_chi2():
    rng = np.random.default_rng(3)
    p = 1009
    n = 200_000
    g = np.unique(rng.integers(0, 99546, (n, 3)), axis=0)
    toks_seed = oracle.table_seed(W.HASH_SEED_BASE | 1, 9)
    slots = np.array([oracle.ngram_slot(row, 99546, toks_seed, p) for row in g])
    counts = np.bincount(slots, minlength=p)
    exp = len(g) / p
    chi2 = ((counts - exp) ** 2 / exp).sum()
    df = p - 1
    assert abs(chi2 - df) < 5 * math.sqrt(2 * df)


def test_hash_collisions_and_head_independence():
    rng = np.random.default_rng(4)
    p = 10007
    g = np.unique(rng.integers(0, 770, (20000, 3)), axis=0)
    n = len(g)
    s0 = oracle.table_seed(1, 0)
    s1 = oracle.table_seed(1, 1)
    a = np.array([oracle.ngram_slot(r, 770, s0, p) for r in g])
    b = np.array([oracle.ngram_slot(r, 770, s1, p) for r in g])
    ca = np.bincount(a, minlength=p)
    pairs = int((ca * (ca - 1) // 2).sum())
    expect = n * (n - 1) / 2 / p
    assert abs(pairs - expect) < 5 * math.sqrt(expect)
    # pairs that collide in head 0 almost never collide in head 1 too
    both = 0
    order = np.argsort(a, kind="stable")
    sa, sb = a[order], b[order]
    for v in np.nonzero(ca > 1)[0]:
        grp = sb[sa == v]
        cb = np.bincount(grp)
        both += int((cb * (cb - 1) // 2).sum())
    assert both <= 5 + 10 * pairs / p


# ----------------------------------------------------------------------------
# O4: gather
# ----------------------------------------------------------------------------

def test_gather_host_matches_numpy_indexing():
    rng = np.random.default_rng(8)
    tabs = [rng.standard_normal((p, 8)).astype(np.float32) for p in (11, 13, 17, 19)]
    idx = np.stack([rng.integers(0, t.shape[0], 50) for t in tabs], 1).astype(np.uint32)
    emb = oracle.gather_host(idx, tabs, oracle.F32)
    ref = np.concatenate([tabs[i][idx[:, i]] for i in range(4)], 1)
    assert np.array_equal(emb, ref)


def test_gather_synth_matches_values():
    rng = np.random.default_rng(9)
    idx = rng.integers(0, 10007, (6, 8)).astype(np.uint32)
    e32 = oracle.gather_synth(idx, 32, 3, oracle.F32)
    e16 = oracle.gather_synth(idx, 32, 3, oracle.BF16)
    for t in range(6):
        for tau in range(8):
            for c in range(32):
                v = oracle.synth_value(3, tau, int(idx[t, tau]), c)
                assert e32[t, tau * 32 + c] == np.float32(v)
    ref16 = torch.from_numpy(e32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(e16, ref16)


# ----------------------------------------------------------------------------
# O5-O7: projections and gate
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
def test_project_matches_numpy_fp64(dtype):
    rng = np.random.default_rng(10)
    e = rng.standard_normal(96).astype(np.float32)
    w = rng.standard_normal((40, 96)).astype(np.float32)
    if dtype == oracle.BF16:
        e, w = W.round_to_bf16(e), W.round_to_bf16(w)
    y = oracle.project(e, w, dtype)
    ref = w.astype(np.float64) @ e.astype(np.float64)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def _gate_inputs(d, h, kvec, rng):
    """e = first basis vector, so W_k e is exactly W_k's first column."""
    e = np.zeros(d, np.float32)
    e[0] = 1.0
    w_k = rng.standard_normal((d, d)).astype(np.float32)
    w_k[:, 0] = kvec
    w_v = rng.standard_normal((d, d)).astype(np.float32)
    return e, h.astype(np.float32), w_k, w_v


def test_gate_closed_forms():
    d = 256
    rng = np.random.default_rng(12)
    ones = np.ones(d, np.float32)
    h = rng.standard_normal(d).astype(np.float32)
    sig = lambda x: 1 / (1 + math.exp(-x))
    # parallel, opposite, orthogonal key and query
    hp = h.copy()
    perp = rng.standard_normal(d).astype(np.float64)
    perp -= perp @ hp.astype(np.float64) / (hp.astype(np.float64) @ hp) * hp
    cases = [(h, sig(math.sqrt(d))), (-h, sig(-math.sqrt(d)))]
    for kvec, expect in cases:
        e, hh, wk, wv = _gate_inputs(d, h, kvec, rng)
        a, u = oracle.gate_token(e, hh, wk, wv, ones, ones, 0.0, oracle.F32)
        assert abs(a - expect) < 1e-12
        np.testing.assert_allclose(u, a * (wv.astype(np.float64) @ e), rtol=1e-12)
    # orthogonal: the dot is zero up to fp32 rounding of the key
    e, hh, wk, wv = _gate_inputs(d, h, perp.astype(np.float32), rng)
    a, _ = oracle.gate_token(e, hh, wk, wv, ones, ones, 0.0, oracle.F32)
    assert abs(a - 0.5) < 1e-6
    # RMSNorm weights: gamma_h * gamma_k = 1 everywhere gives the same gate
    e, hh, wk, wv = _gate_inputs(d, h, h, rng)
    a2, _ = oracle.gate_token(e, hh, wk, wv, 2 * ones, 0.5 * ones, 0.0, oracle.F32)
    assert abs(a2 - sig(math.sqrt(d))) < 1e-12


def test_gate_scale_invariance_and_zero_query():
    d = 64
    rng = np.random.default_rng(13)
    e = rng.standard_normal(d).astype(np.float32)
    h = rng.standard_normal(d).astype(np.float32)
    wk = rng.standard_normal((d, d)).astype(np.float32)
    wv = rng.standard_normal((d, d)).astype(np.float32)
    gh = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    gk = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    a, _ = oracle.gate_token(e, h, wk, wv, gh, gk, 0.0, oracle.F32, want_u=False)
    for c in (0.5, 4.0, 1024.0):  # powers of two keep the scaled inputs exact
        a1, _ = oracle.gate_token(e, c * h, wk, wv, gh, gk, 0.0, oracle.F32, want_u=False)
        a2, _ = oracle.gate_token(e, h, c * wk, wv, gh, gk, 0.0, oracle.F32, want_u=False)
        assert abs(a1 - a) < 1e-13 and abs(a2 - a) < 1e-13
    # a zero hidden state normalises to zero: the gate sits at sigmoid(0)
    a0, _ = oracle.gate_token(e, 0 * h, wk, wv, gh, gk, 1e-6, oracle.F32, want_u=False)
    assert a0 == 0.5


def test_gate_decreases_with_mismatch():
    """A larger disagreement between key and query gives a smaller gate."""
    d = 128
    rng = np.random.default_rng(14)
    ones = np.ones(d, np.float32)
    h = rng.standard_normal(d)
    hu = h / np.linalg.norm(h)
    q = rng.standard_normal(d)
    q -= (q @ hu) * hu
    q /= np.linalg.norm(q)
    prev = 2.0
    for theta in np.linspace(0, math.pi, 13):
        kvec = (math.cos(theta) * hu + math.sin(theta) * q).astype(np.float32)
        e, hh, wk, wv = _gate_inputs(d, h, kvec, rng)
        a, _ = oracle.gate_token(e, hh, wk, wv, ones, ones, 0.0, oracle.F32, want_u=False)
        assert 0 < a < 1
        assert abs(a - 1 / (1 + math.exp(-math.sqrt(d) * math.cos(theta)))) < 1e-6
        assert a < prev
        prev = a


# ----------------------------------------------------------------------------
# O8-O10: conv, residual, state
# ----------------------------------------------------------------------------

def _small_layer(dtype=oracle.F32, batch=2, seqlen=9, d=24, De=32, Br=2, conv_k=4,
                 conv_mode=oracle.CONV_LINEAR, flags=0, conv_state=None, seed=15):
    rng = np.random.default_rng(seed)
    cast = W.round_to_bf16 if dtype == oracle.BF16 else (lambda a: a.astype(np.float32))
    emb = cast(rng.standard_normal((batch * seqlen, De)).astype(np.float32) * 0.02)
    h = cast(rng.standard_normal((Br, batch * seqlen, d)).astype(np.float32))
    w_k = cast(rng.standard_normal((Br, d, De)).astype(np.float32) / math.sqrt(De))
    w_v = cast(rng.standard_normal((d, De)).astype(np.float32) / (0.02 * math.sqrt(De)))
    gh = (1 + 0.1 * rng.standard_normal((Br, d))).astype(np.float32)
    gk = (1 + 0.1 * rng.standard_normal((Br, d))).astype(np.float32)
    cw = (0.5 * rng.standard_normal((d, conv_k))).astype(np.float32)
    return oracle.Layer(emb, h, w_k, w_v, gh, gk, cw, batch, seqlen, dtype,
                        conv_state=conv_state, conv_mode=conv_mode, flags=flags)


def _h64(layer):
    h = layer.h
    if layer.dtype == oracle.BF16:
        h = (h.astype(np.uint32) << 16).view(np.float32)
    return h.astype(np.float64).reshape(layer.n_branches, layer.batch * layer.seqlen, layer.d)


@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
@pytest.mark.parametrize("mode", [oracle.CONV_LINEAR, oracle.CONV_SILU_SKIP])
def test_conv_matches_torch_depthwise(dtype, mode):
    L = _small_layer(dtype, conv_mode=mode)
    out, alpha, u = L.forward_all(want_u=True)
    assert np.all((alpha > 0) & (alpha < 1))
    y = out - _h64(L)
    ut = torch.from_numpy(u.reshape(L.n_branches, L.batch, L.seqlen, L.d))
    w = torch.from_numpy(L.conv_w.astype(np.float64))[:, None, :]  # [d][1][K]
    for m in range(L.n_branches):
        for b in range(L.batch):
            x = ut[m, b].T[None]  # [1][d][T]
            conv = F.conv1d(F.pad(x, (L.conv_k - 1, 0)), w, groups=L.d)[0].T
            ref = conv if mode == oracle.CONV_LINEAR else ut[m, b] + F.silu(conv)
            got = y[m, b * L.seqlen:(b + 1) * L.seqlen]
            np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_conv_special_taps():
    L = _small_layer()
    L.conv_w[:] = 0
    out, _, _ = L.forward_all()
    assert np.array_equal(out, _h64(L))  # zero taps: out = h exactly
    L.conv_w[:, -1] = 1  # identity on the current token
    out, _, u = L.forward_all(want_u=True)
    np.testing.assert_allclose(out - _h64(L), u, rtol=1e-12, atol=1e-14)
    # impulse: taps [1, 0, 0, 0] delay the gated value by conv_k - 1 positions
    L.conv_w[:] = 0
    L.conv_w[:, 0] = 1
    L.flags = oracle.OUT_DELTA
    y, _, u = L.forward_all(want_u=True)
    y = y.reshape(L.n_branches, L.batch, L.seqlen, L.d)
    u = u.reshape(L.n_branches, L.batch, L.seqlen, L.d)
    assert np.all(y[:, :, :3] == 0)
    np.testing.assert_allclose(y[:, :, 3:], u[:, :, :-3], rtol=1e-12)


def test_out_delta_flag():
    L = _small_layer()
    out, _, _ = L.forward_all()
    L.flags = oracle.OUT_DELTA
    y, _, _ = L.forward_all()
    np.testing.assert_allclose(out - _h64(L), y, rtol=1e-12, atol=1e-12)


def test_causality_and_batch_independence():
    L = _small_layer(seqlen=12)
    base, _, _ = L.forward_all()
    base = base.reshape(L.n_branches, L.batch, L.seqlen, L.d)
    t0 = 6
    rng = np.random.default_rng(1)
    # perturb future embeddings and hidden states of sequence 0
    rows = np.arange(t0 + 1, L.seqlen)
    L.emb[rows] = rng.standard_normal((len(rows), L.De)).astype(np.float32)
    L.h[:, rows] = rng.standard_normal((L.n_branches, len(rows), L.d)).astype(np.float32)
    pert, _, _ = L.forward_all()
    pert = pert.reshape(L.n_branches, L.batch, L.seqlen, L.d)
    assert np.array_equal(pert[:, 0, :t0 + 1], base[:, 0, :t0 + 1])
    assert not np.array_equal(pert[:, 0, t0 + 1:], base[:, 0, t0 + 1:])
    assert np.array_equal(pert[:, 1], base[:, 1])  # other sequence untouched


def test_chunked_forward_equals_full():
    """forward(x[0:T]) equals forward(x[0:T1]) then forward(x[T1:T]) with the
    carried conv state (decode is the case of chunks of length one)."""
    L = _small_layer(seqlen=10)
    full, alpha_full, u_full = L.forward_all(want_u=True)
    full = full.reshape(L.n_branches, L.batch, L.seqlen, L.d)
    u_full = u_full.reshape(L.n_branches, L.batch, L.seqlen, L.d)
    emb = L.emb.reshape(L.batch, L.seqlen, -1)
    h = L.h.reshape(L.n_branches, L.batch, L.seqlen, L.d)
    state = None
    got = []
    for a, b in [(0, 1), (1, 3), (3, 4), (4, 10)]:
        n = b - a
        C = oracle.Layer(emb[:, a:b].reshape(L.batch * n, -1), h[:, :, a:b].reshape(L.n_branches, -1, L.d),
                         L.w_k.view(np.float32), L.w_v.view(np.float32), L.gamma_h, L.gamma_k, L.conv_w,
                         L.batch, n, L.dtype, conv_state=state)
        o, _, u = C.forward_all(want_u=True)
        got.append(o.reshape(L.n_branches, L.batch, n, L.d))
        state = C.new_conv_state(u)
        # the carried state is exactly the last conv_k-1 gated values so far
        ref = np.zeros((L.n_branches, L.batch, 3, L.d))
        hist = u_full[:, :, :b]
        k = min(3, b)
        ref[:, :, 3 - k:] = hist[:, :, b - k:]
        np.testing.assert_allclose(state, ref.astype(np.float32), rtol=0, atol=0)
    got = np.concatenate(got, 2)
    # the carried state passes through fp32, so allow fp32 rounding of u
    np.testing.assert_allclose(got, full, rtol=1e-6, atol=1e-6)


def test_f32_split_errors_parts():
    """The fp32 parity report splits elements at the row RMS: plain relative
    error above it, |d| / row RMS below it."""
    from engram_harness import f32_split_errors
    ref = np.array([[4.0, -4.0, 0.0, 0.0]])  # row RMS = sqrt(8) ~ 2.83
    got = ref + np.array([[4e-6, 0.0, 2.83e-6, -1e-7]])
    rel_large, n_large, abs_small, n_small = f32_split_errors(got, ref)
    assert (n_large, n_small) == (2, 2)
    assert abs(rel_large - 1e-6) < 1e-12
    assert abs(abs_small - 2.83e-6 / np.sqrt(8.0)) < 1e-12
