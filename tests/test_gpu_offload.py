"""Tables in pinned host memory, read by the GPU over the host link, with a
hot-row cache in HBM (through the C ABI), against the CPU oracle.

Retrieval is a copy, so every gathered row must equal the oracle's row bit
for bit, whether it came from host memory, from device memory or from the
cache; the cache must hold exactly the valid distinct rows it was given.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from synthetic import workloads as W
from synthetic.device import make_device_layer, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B(gpu):
    from hashed_gram_embedding_vocab_amd import binding
    binding.lib()  # raises if the library is not built: no fallback
    return binding


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_i32(x):
    return to_device(np.asarray(x, np.int32), torch.int32, "cuda")


def tables_for(B, primes, head_dim, seed, dt, where):
    code = B.BF16 if dt == "bf16" else B.F32
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    out = []
    for tau, p in enumerate(primes):
        t = torch.empty((p, head_dim), dtype=tdt, device="cuda")
        B.engram_synth_fill_table(t, seed, tau, code)
        if where == "host":
            hb = B.HostBuffer(t.numel() * t.element_size())
            hb.view(tdt, t.shape).copy_(t.cpu())
            out.append(hb)
        else:
            out.append(t)
    torch.cuda.synchronize()
    return out


def emb_bytes(emb, dt):
    return (emb.view(torch.int16).cpu().numpy().view(np.uint16) if dt == "bf16" else emb.cpu().numpy()).view(np.uint8)


def plan_for(B, primes, head_dim, dt):
    code = B.BF16 if dt == "bf16" else B.F32
    n_tables = len(primes)
    return B.Plan(vocab=1000, vocab_comp=770, heads=n_tables // 2, head_dim=head_dim, table_rows=primes,
                  hash_seed=1, d_model=256, dtype=code)


def zipf_idx(primes, n_tok, seed):
    """Slots with a Zipf-like skew (a few rows take most accesses), plus the
    first and last row of every table."""
    rng = np.random.default_rng(seed)
    cols = []
    for p in primes:
        ranks = np.minimum(rng.zipf(1.3, n_tok) - 1, p - 1)
        perm = rng.permutation(p)
        cols.append(perm[ranks])
    idx = np.stack(cols, 1).astype(np.uint32)
    idx[0] = 0
    idx[-1] = np.array(primes) - 1
    return idx


CASES = [("f32", 32, [10007] * 8), ("bf16", 80, W.largest_primes_at_most(5000, 16)),
         ("bf16", 64, W.largest_primes_at_most(3001, 4)), ("bf16", 32, W.largest_primes_at_most(2003, 32))]


@pytest.mark.parametrize("dt,head_dim,primes", CASES)
@pytest.mark.parametrize("n_tok", [1, 1000, 4099])
def test_host_table_gather_bit_exact(B, dt, head_dim, primes, n_tok):
    say("host gather", dt, head_dim, len(primes), n_tok)
    seed = 17
    plan = plan_for(B, primes, head_dim, dt)
    tables = tables_for(B, primes, head_dim, seed, dt, "host")
    idx = zipf_idx(primes, n_tok, n_tok)
    ref = oracle.gather_synth(idx, head_dim, seed, oracle.BF16 if dt == "bf16" else oracle.F32).view(np.uint8)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    emb = torch.empty((n_tok, len(primes) * head_dim), dtype=tdt, device="cuda")
    plan.engram_gather(dev_i32(idx.view(np.int32)), tables, emb)
    torch.cuda.synchronize()
    assert np.array_equal(emb_bytes(emb, dt), ref)
    emb.fill_(0)
    plan.engram_gather_cached(dev_i32(idx.view(np.int32)), tables, None, emb)
    torch.cuda.synchronize()
    assert np.array_equal(emb_bytes(emb, dt), ref)


@pytest.mark.parametrize("dt,head_dim,primes", CASES)
@pytest.mark.parametrize("where", ["host", "device"])
@pytest.mark.parametrize("capacity,n_hot,max_wg", [(2, 1, 0), (64, 32, 7), (4096, 700, 0), (8, 0, 1),
                                                   (4096, 700, 64)])
def test_cached_gather_bit_exact_and_cache_contents(B, dt, head_dim, primes, where, capacity, n_hot, max_wg):
    say("cached gather", dt, head_dim, len(primes), where, capacity, n_hot, max_wg)
    seed = 23
    n_tok = 3001
    plan = plan_for(B, primes, head_dim, dt)
    tables = tables_for(B, primes, head_dim, seed, dt, where)
    idx = zipf_idx(primes, n_tok, 5)
    n_tables = len(primes)
    # hot rows: the most frequent slots of each table, with a repeated entry
    # and an entry past the table's end mixed in
    hot = np.zeros((n_tables, n_hot), np.uint32)
    for tau in range(n_tables):
        u, c = np.unique(idx[:, tau], return_counts=True)
        top = u[np.argsort(-c, kind="stable")]
        row = np.resize(top, n_hot) if n_hot else top[:0]
        if n_hot >= 4:
            row[1] = row[0]
            row[2] = primes[tau] + 5
        hot[tau] = row
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    cache = B.RowCache(n_tables, capacity, head_dim, tdt)
    plan.engram_cache_build(dev_i32(hot.view(np.int32)) if n_hot else None, tables, cache)
    emb = torch.empty((n_tok, n_tables * head_dim), dtype=tdt, device="cuda")
    plan.engram_gather_cached(dev_i32(idx.view(np.int32)), tables, cache, emb, max_workgroups=max_wg)
    torch.cuda.synchronize()
    odt = oracle.BF16 if dt == "bf16" else oracle.F32
    ref = oracle.gather_synth(idx, head_dim, seed, odt).view(np.uint8)
    assert np.array_equal(emb_bytes(emb, dt), ref)
    # the cache holds exactly the valid distinct hot rows, each a copy of its table row
    keys = cache.keys.cpu().numpy().view(np.uint32)
    rows = cache.rows.view(torch.int16).cpu().numpy() if dt == "bf16" else cache.rows.cpu().numpy()
    for tau in range(n_tables):
        want = np.unique(hot[tau][hot[tau] < primes[tau]]) if n_hot else np.zeros(0, np.uint32)
        held = keys[tau][keys[tau] != 0] - 1
        assert np.array_equal(np.sort(held), want), tau
        slots = np.nonzero(keys[tau])[0]
        if len(slots):
            one = np.zeros((len(slots), n_tables), np.uint32)
            one[:, tau] = keys[tau][slots] - 1
            exp = oracle.gather_synth(one, head_dim, seed, odt)[:, tau * head_dim:(tau + 1) * head_dim]
            assert np.array_equal(rows[tau][slots].view(np.uint8), np.ascontiguousarray(exp).view(np.uint8))


def test_every_row_cached(B):
    """A cache holding every row of small tables serves every access."""
    say("every row cached")
    primes = [97, 89, 83, 79]
    head_dim, dt, seed = 64, "bf16", 31
    plan = plan_for(B, primes, head_dim, dt)
    tables = tables_for(B, primes, head_dim, seed, dt, "host")
    hot = np.stack([np.arange(97) % p for p in primes]).astype(np.uint32)  # wraps: repeats, all rows
    cache = B.RowCache(len(primes), 256, head_dim, torch.bfloat16)
    plan.engram_cache_build(dev_i32(hot.view(np.int32)), tables, cache)
    idx = zipf_idx(primes, 2000, 9)
    emb = torch.empty((2000, len(primes) * head_dim), dtype=torch.bfloat16, device="cuda")
    plan.engram_gather_cached(dev_i32(idx.view(np.int32)), tables, cache, emb)
    torch.cuda.synchronize()
    ref = oracle.gather_synth(idx, head_dim, seed, oracle.BF16).view(np.uint8)
    assert np.array_equal(emb_bytes(emb, dt), ref)
    keys = cache.keys.cpu().numpy().view(np.uint32)
    for tau, p in enumerate(primes):
        assert np.array_equal(np.sort(keys[tau][keys[tau] != 0] - 1), np.arange(p))


def test_cache_arguments_rejected(B):
    primes = [97, 89]
    plan = plan_for(B, primes, 64, "bf16")
    tables = tables_for(B, primes, 64, 1, "bf16", "device")
    hot = dev_i32(np.zeros((2, 3), np.int32))
    for cap in (0, 4, 6):  # no cache, load factor above 1/2, not a power of two
        with pytest.raises(B.EngramError):
            plan.engram_cache_build(hot, tables, B.RowCache(2, cap, 64, torch.bfloat16))
    emb = torch.empty((4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.EngramError):
        plan.engram_gather_cached(dev_i32(np.zeros((4, 2), np.int32)), tables, B.RowCache(2, 6, 64, torch.bfloat16),
                                  emb)


@pytest.mark.parametrize("n_branches", [1, 4])
def test_forward_with_host_tables_equals_oracle_and_device(B, n_branches):
    """engram_forward reading its rows from host memory gives the bits it
    gives with device tables, and matches the oracle."""
    from engram_harness import assert_within, oracle_indices, oracle_layer
    say("forward host tables", n_branches)
    import dataclasses
    wl = dataclasses.replace(W.workload("small"), name="offload_custom", index=60 + n_branches, batch=2,
                             seqlen=130, d_model=256, heads=2, head_dim=32, table_target=10007, same_prime=False,
                             n_branches=n_branches)
    dl_h = make_device_layer(wl, host_tables=True)
    dl_d = make_device_layer(wl)
    tokens = W.make_tokens(wl)
    outs = []
    for dl in (dl_h, dl_d):
        out = torch.empty_like(dl.h)
        ws = dl.plan.workspace(wl.batch, wl.seqlen)
        dl.plan.engram_forward(dev_i32(tokens), dl.comp_map, dl.tables, dl.h, dl.weights, out, ws)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    idx, _, _ = oracle_indices(wl, dl_h.li, tokens, dl_h.comp_map_host)
    L = oracle_layer(wl, dl_h.li, idx, wl.batch, wl.seqlen)
    ref, _, _ = L.forward_all()
    got = torch.from_numpy(outs[0]).view(torch.bfloat16).float().numpy()
    assert_within(got.reshape(ref.shape), ref, "bf16", "forward, host tables")


def test_capped_gather_beside_busy_stream(B):
    """A host-table gather capped at a few workgroups, issued on its own
    stream while another stream runs matrix products, returns the oracle's
    rows (the prefetch arrangement of the offload path)."""
    say("capped gather beside a busy stream")
    primes = W.largest_primes_at_most(3001, 4)
    head_dim, dt, seed = 64, "bf16", 41
    plan = plan_for(B, primes, head_dim, dt)
    tables = tables_for(B, primes, head_dim, seed, dt, "host")
    idx = zipf_idx(primes, 5000, 3)
    cache = B.RowCache(len(primes), 64, head_dim, torch.bfloat16)
    hot = np.stack([np.unique(idx[:, t])[:32] for t in range(len(primes))]).astype(np.uint32)
    plan.engram_cache_build(dev_i32(hot.view(np.int32)), tables, cache)
    emb = torch.empty((5000, len(primes) * head_dim), dtype=torch.bfloat16, device="cuda")
    idx_d = dev_i32(idx.view(np.int32))
    x = torch.randn((2048, 2048), device="cuda").to(torch.bfloat16)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        for _ in range(4):
            x = torch.mm(x, x) * 0.01
    plan.engram_gather_cached(idx_d, tables, cache, emb, max_workgroups=3, stream=sb)
    torch.cuda.synchronize()
    ref = oracle.gather_synth(idx, head_dim, seed, oracle.BF16).view(np.uint8)
    assert np.array_equal(emb_bytes(emb, dt), ref)



@pytest.mark.parametrize("kind", ["pinned", "pageable"])
@pytest.mark.parametrize("cached", ["none", "some", "all"])
def test_prefetcher_bit_exact_over_jobs(B, kind, cached):
    """Host threads gather the missed rows, a DMA engine stages them, the GPU
    assembles E: bit-exact with the oracle over consecutive jobs of different
    sizes, and the reported miss count is the number of pairs not cached."""
    say("prefetcher", kind, cached)
    primes = W.largest_primes_at_most(2003, 6)
    head_dim, dt, seed = 80, "bf16", 53
    plan = plan_for(B, primes, head_dim, dt)
    dev_tables = tables_for(B, primes, head_dim, seed, dt, "device")
    if kind == "pinned":
        tables = []
        for t in dev_tables:
            hb = B.HostBuffer(t.numel() * t.element_size())
            hb.view(torch.bfloat16, t.shape).copy_(t.cpu())
            tables.append(hb)
    else:
        tables = [t.cpu().contiguous() for t in dev_tables]
    n_tables = len(primes)
    cache, hot_sets = None, [set() for _ in primes]
    if cached != "none":
        n_hot = 2003 if cached == "all" else 100
        hot = np.stack([(np.arange(n_hot) * 7 + tau) % p for tau, p in enumerate(primes)]).astype(np.uint32)
        cache = B.RowCache(n_tables, 4096, head_dim, torch.bfloat16)
        plan.engram_cache_build(dev_i32(hot.view(np.int32)), dev_tables, cache)
        hot_sets = [set(hot[tau].tolist()) for tau in range(n_tables)]
    pf = B.Prefetcher(plan, tables, cache, max_tokens=3000, n_threads=4)
    for job, n_tok in enumerate([3000, 1, 1777, 3000]):
        idx = zipf_idx(primes, n_tok, 100 + job)
        emb = torch.zeros((n_tok, n_tables * head_dim), dtype=torch.bfloat16, device="cuda")
        pf.begin(dev_i32(idx.view(np.int32)))
        if job == 0:
            with pytest.raises(B.EngramError):  # one job at a time
                pf.begin(dev_i32(idx.view(np.int32)))
        n_miss = pf.finish(emb)
        torch.cuda.synchronize()
        ref = oracle.gather_synth(idx, head_dim, seed, oracle.BF16).view(np.uint8)
        assert np.array_equal(emb_bytes(emb, dt), ref), (job, n_tok)
        want = sum(int(r) not in hot_sets[tau] for tau in range(n_tables) for r in idx[:, tau])
        assert n_miss == want, (job, n_miss, want)
    with pytest.raises(B.EngramError):  # nothing begun
        pf.finish(emb)
    pf.close()


def test_prefetcher_beside_busy_stream(B):
    """begin on one stream, matrix products on another, finish on a third:
    the assembled E still equals the oracle's rows."""
    say("prefetcher beside a busy stream")
    primes = W.largest_primes_at_most(3001, 4)
    head_dim, dt, seed = 64, "bf16", 61
    plan = plan_for(B, primes, head_dim, dt)
    tables = tables_for(B, primes, head_dim, seed, dt, "host")
    pf = B.Prefetcher(plan, tables, None, max_tokens=5000, n_threads=8)
    idx = zipf_idx(primes, 5000, 4)
    emb = torch.empty((5000, len(primes) * head_dim), dtype=torch.bfloat16, device="cuda")
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    x = torch.randn((2048, 2048), device="cuda").to(torch.bfloat16)
    idx_d = dev_i32(idx.view(np.int32))
    torch.cuda.synchronize()
    pf.begin(idx_d, stream=s1)
    with torch.cuda.stream(s2):
        for _ in range(4):
            x = torch.mm(x, x) * 0.01
    pf.finish(emb, stream=s3)
    torch.cuda.synchronize()
    ref = oracle.gather_synth(idx, head_dim, seed, oracle.BF16).view(np.uint8)
    assert np.array_equal(emb_bytes(emb, dt), ref)
    pf.close()
