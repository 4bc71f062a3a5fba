"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Indices and gathered rows must match bit for bit; floating-point outputs
within the tolerances of ``engram_harness`` (fp32: 1e-5 relative to the
larger of |ref| and the row's rms; bf16 storage with fp32 accumulation:
1e-2 absolute + 2e-2 relative).  Expected values come only from ``oracle/``
on the same seeded inputs.
"""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from engram_harness import (alpha_tol, assert_within, oracle_dtype, oracle_indices, oracle_layer,
                            rows_needed, sample_positions)
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


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def forward(dl, tokens, prev_ctx=None, conv_state=None, flags=0, h=None, out=None, stream=None):
    batch, seqlen = tokens.shape
    h = dl.h if h is None else h
    out = torch.empty_like(h) if out is None else out
    alpha = torch.full((dl.wl.n_branches, batch * seqlen), -1.0, dtype=torch.float32, device="cuda")
    ws = dl.plan.workspace(batch, seqlen)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    dl.plan.engram_forward(dev_i32(tokens), dl.comp_map, dl.tables, h, dl.weights, out, ws,
                           prev_ctx=prev_ctx, conv_state=conv_state, alpha=alpha, flags=flags,
                           bad_tokens=bad, stream=stream)
    torch.cuda.synchronize()
    return out, alpha, int(bad.item())


def small_wl(n_branches=1, batch=3, seqlen=77, d_model=256, heads=2, head_dim=32, conv_kernel=4,
             dtype="bf16", name="small_custom"):
    return dataclasses.replace(W.workload("small"), name=name, index=40 + n_branches, batch=batch,
                               seqlen=seqlen, d_model=d_model, heads=heads, head_dim=head_dim,
                               table_target=10007, same_prime=False, n_branches=n_branches,
                               conv_kernel=conv_kernel, dtype=dtype)


# ----------------------------------------------------------------------------
# synthetic tables: the device generator equals the oracle's generator
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dt,rows,hd", [("f32", 10007, 32), ("bf16", 4099, 80)])
def test_synth_fill_bit_exact(B, dt, rows, hd):
    say("synth fill", dt, rows, hd)
    code = B.BF16 if dt == "bf16" else B.F32
    t = torch.empty((rows, hd), dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device="cuda")
    B.engram_synth_fill_table(t, 3, 5, code)
    torch.cuda.synchronize()
    if dt == "bf16":
        got = t.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        got = t.cpu().numpy()
    rng = np.random.default_rng(1)
    sample = sorted({0, 1, rows - 1, *rng.integers(0, rows, 40).tolist()})
    for r in sample:
        for c in range(hd):
            v = oracle.synth_value(3, 5, r, c)
            if dt == "bf16":
                assert got[r, c] == oracle.bf16_rne(v), (r, c)
            else:
                assert got[r, c] == np.float32(v), (r, c)


# ----------------------------------------------------------------------------
# hashing: bit-exact slots
# ----------------------------------------------------------------------------

def _hash_gpu(B, plan, tokens, comp_dev, n_tables, prev_ctx=None):
    batch, seqlen = tokens.shape
    idx = torch.zeros((batch * seqlen, n_tables), dtype=torch.int32, device="cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    plan.engram_hash(dev_i32(tokens), comp_dev, idx,
                     prev_ctx=None if prev_ctx is None else dev_i32(prev_ctx), bad_tokens=bad)
    torch.cuda.synchronize()
    return idx.cpu().numpy().view(np.uint32), int(bad.item())


def test_hash_tiny_vocab_exhaustive(B):
    say("hash tiny vocab")
    V, Vc, heads = 7, 5, 2
    comp = W.compression_map(V, Vc, 99)
    pre = {int(c): int(np.nonzero(comp == c)[0][0]) for c in range(Vc)}
    seqs = [(a, b, c) for a in range(Vc) for b in range(Vc) for c in range(Vc)]
    toks = np.array([[pre[a], pre[b], pre[c]] for a, b, c in seqs], np.int32)
    primes = [13, 11, 7, 5]
    plan = B.Plan(vocab=V, vocab_comp=Vc, heads=heads, head_dim=32, table_rows=primes, hash_seed=0x1234,
                  d_model=256, dtype=B.F32)
    comp_dev = dev_i32(comp)
    got, bad = _hash_gpu(B, plan, toks, comp_dev, 4)
    ref, rbad, _ = oracle.hash_tokens(toks, comp, V, Vc, heads, primes, 0x1234)
    assert bad == rbad == 0
    assert np.array_equal(got, ref)
    ctx = np.random.default_rng(2).integers(0, Vc + 1, (len(seqs), 2)).astype(np.int32)
    got, _ = _hash_gpu(B, plan, toks, comp_dev, 4, prev_ctx=ctx)
    ref, _, _ = oracle.hash_tokens(toks, comp, V, Vc, heads, primes, 0x1234, prev_ctx=ctx)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("name,batch,seqlen", [
    ("tiny", 1, 1), ("tiny", 1, 2), ("tiny", 1, 3), ("tiny", 3, 63), ("tiny", 2, 64), ("tiny", 2, 65),
    ("tiny", 5, 200), ("layer27b", 2, 1000), ("maxtable_uniform", 1, 300), ("multibranch_prefill", 1, 129),
])
@pytest.mark.parametrize("with_ctx", [False, True])
def test_hash_shapes(B, name, batch, seqlen, with_ctx):
    say("hash", name, batch, seqlen, with_ctx)
    wl = W.workload(name)
    li = W.make_layer_inputs(wl, batch=1, seqlen=1)
    comp = W.compression_map(wl.vocab, wl.vocab_comp, wl.seed(1))
    toks = W.make_tokens(wl, batch=batch, seqlen=seqlen)
    ctx = None
    if with_ctx:
        ctx = np.random.default_rng(3).integers(0, wl.vocab_comp + 1, (batch, 2)).astype(np.int32)
    plan = B.Plan(vocab=wl.vocab, vocab_comp=wl.vocab_comp, heads=wl.heads, head_dim=wl.head_dim,
                  table_rows=wl.primes(), hash_seed=li.hash_seed, d_model=wl.d_model,
                  n_branches=wl.n_branches, dtype=B.BF16 if wl.dtype == "bf16" else B.F32)
    got, bad = _hash_gpu(B, plan, toks, dev_i32(comp), wl.n_tables, prev_ctx=ctx)
    ref, rbad, _ = oracle_indices(wl, li, toks, comp, prev_ctx=ctx)
    assert bad == rbad == 0
    assert np.array_equal(got, ref)


# More than 16 tables (a plan accepts up to 32): fewer tokens per retrieval
# block, 4-wide index stores across 24 or 32 slots, a single order of 32 heads.
MANY_TABLES = [(12, (2, 3)), (16, (2, 3)), (32, (3,))]


def many_tables_wl(heads, orders, batch, seqlen, dtype="bf16", name="many_tables"):
    return dataclasses.replace(W.workload("small"), name=name, index=60 + heads + len(orders), batch=batch,
                               seqlen=seqlen, d_model=256, heads=heads, head_dim=32, orders=orders,
                               table_target=2003, same_prime=False, n_branches=1, dtype=dtype)


@pytest.mark.parametrize("heads,orders", MANY_TABLES)
@pytest.mark.parametrize("batch,seqlen", [(1, 1), (3, 65), (2, 1000)])
@pytest.mark.parametrize("with_ctx", [False, True])
def test_hash_many_tables(B, heads, orders, batch, seqlen, with_ctx):
    say("hash many tables", heads, orders, batch, seqlen, with_ctx)
    wl = many_tables_wl(heads, orders, batch, seqlen)
    li = W.make_layer_inputs(wl, batch=1, seqlen=1)
    comp = W.compression_map(wl.vocab, wl.vocab_comp, wl.seed(1))
    toks = W.make_tokens(wl)
    ctx = None
    if with_ctx:
        ctx = np.random.default_rng(4).integers(0, wl.vocab_comp + 1, (batch, 2)).astype(np.int32)
    plan = B.Plan(vocab=wl.vocab, vocab_comp=wl.vocab_comp, heads=wl.heads, head_dim=wl.head_dim,
                  table_rows=wl.primes(), hash_seed=li.hash_seed, d_model=wl.d_model, dtype=B.BF16,
                  orders=wl.orders)
    got, bad = _hash_gpu(B, plan, toks, dev_i32(comp), wl.n_tables, prev_ctx=ctx)
    ref, rbad, _ = oracle_indices(wl, li, toks, comp, prev_ctx=ctx)
    assert wl.n_tables in (24, 32)
    assert bad == rbad == 0
    assert np.array_equal(got, ref)


def test_hash_out_of_range_tokens(B):
    say("hash bad tokens")
    wl = W.workload("tiny")
    li = W.make_layer_inputs(wl, batch=1, seqlen=1)
    comp = W.compression_map(wl.vocab, wl.vocab_comp, wl.seed(1))
    toks = W.make_tokens(wl, batch=2, seqlen=130)
    for b, t, v in [(0, 0, -1), (0, 1, wl.vocab), (0, 63, 2**31 - 1), (0, 64, -2**31), (1, 129, 5000),
                    (1, 65, -7)]:
        toks[b, t] = v
    plan = B.Plan(vocab=wl.vocab, vocab_comp=wl.vocab_comp, heads=wl.heads, head_dim=wl.head_dim,
                  table_rows=wl.primes(), hash_seed=li.hash_seed, d_model=wl.d_model, dtype=B.F32)
    got, bad = _hash_gpu(B, plan, toks, dev_i32(comp), wl.n_tables)
    ref, rbad, _ = oracle_indices(wl, li, toks, comp)
    assert bad == rbad == 6
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------------------
# gather: bit-exact rows
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dt,head_dim,primes", [
    ("f32", 32, [10007] * 8),
    ("bf16", 80, W.largest_primes_at_most(5000, 16)),
    ("bf16", 64, W.largest_primes_at_most(3001, 4)),
    ("bf16", 64, W.largest_primes_at_most(3001, 24)),
    ("bf16", 32, W.largest_primes_at_most(2003, 32)),
    ("f32", 32, W.largest_primes_at_most(1009, 32)),
])
@pytest.mark.parametrize("n_tok", [1, 1000, 4099])
def test_gather_bit_exact(B, dt, head_dim, primes, n_tok):
    say("gather", dt, head_dim, len(primes), n_tok)
    code = B.BF16 if dt == "bf16" else B.F32
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    n_tables = len(primes)
    plan = B.Plan(vocab=1000, vocab_comp=770, heads=n_tables // 2, head_dim=head_dim, table_rows=primes,
                  hash_seed=1, d_model=256, dtype=code)
    seed = 17
    tables = []
    for tau, p in enumerate(primes):
        t = torch.empty((p, head_dim), dtype=tdt, device="cuda")
        B.engram_synth_fill_table(t, seed, tau, code)
        tables.append(t)
    rng = np.random.default_rng(n_tok)
    idx = np.stack([rng.integers(0, p, n_tok) for p in primes], 1).astype(np.uint32)
    idx[0] = 0
    idx[-1] = np.array(primes) - 1
    emb = torch.empty((n_tok, n_tables * head_dim), dtype=tdt, device="cuda")
    plan.engram_gather(dev_i32(idx.view(np.int32)), tables, emb)
    torch.cuda.synchronize()
    got = emb.view(torch.int16).cpu().numpy().view(np.uint16) if dt == "bf16" else emb.cpu().numpy()
    ref = oracle.gather_synth(idx, head_dim, seed, oracle.BF16 if dt == "bf16" else oracle.F32)
    assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))


# ----------------------------------------------------------------------------
# whole forward pass
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("mode,flags", [(oracle.CONV_LINEAR, 0), (oracle.CONV_SILU_SKIP, 0),
                                        (oracle.CONV_LINEAR, oracle.OUT_DELTA)])
def test_forward_tiny_all_positions(B, mode, flags):
    say("forward tiny", mode, flags)
    wl = W.workload("tiny")
    dl = make_device_layer(wl, conv_mode=mode)
    toks = W.make_tokens(wl)
    out, alpha, bad = forward(dl, toks, flags=flags)
    idx, _, _ = oracle_indices(wl, dl.li, toks, dl.comp_map_host)
    L = oracle_layer(wl, dl.li, idx, wl.batch, wl.seqlen, conv_mode=mode, flags=flags)
    ref, ref_alpha, _ = L.forward_all()
    assert bad == 0
    assert_within(host(out), ref, "f32", "tiny out")
    assert np.abs(host(alpha) - ref_alpha).max() <= alpha_tol("f32")


@pytest.mark.parametrize("n_branches", [1, 2, 3, 4])
@pytest.mark.parametrize("batch,seqlen", [(3, 77), (1, 1), (2, 130), (3, 300), (3, 127)])
def test_forward_bf16_small_shapes_all_positions(B, n_branches, batch, seqlen):
    say("forward bf16 small", n_branches, batch, seqlen)
    wl = small_wl(n_branches=n_branches, batch=batch, seqlen=seqlen)
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    out, alpha, _ = forward(dl, toks)
    idx, _, _ = oracle_indices(wl, dl.li, toks, dl.comp_map_host)
    L = oracle_layer(wl, dl.li, idx, batch, seqlen)
    ref, ref_alpha, _ = L.forward_all()
    assert_within(host(out), ref, "bf16", "bf16 small out")
    assert np.abs(host(alpha) - ref_alpha).max() <= alpha_tol("bf16")
    # y alone, so an error in y cannot hide next to h
    dl2 = make_device_layer(wl, conv_mode=oracle.CONV_SILU_SKIP)
    y, _, _ = forward(dl2, toks, flags=oracle.OUT_DELTA)
    L2 = oracle_layer(wl, dl2.li, idx, batch, seqlen, conv_mode=oracle.CONV_SILU_SKIP,
                      flags=oracle.OUT_DELTA)
    ref_y, _, _ = L2.forward_all()
    assert_within(host(y), ref_y, "bf16", "bf16 small y (silu skip)")


@pytest.mark.parametrize("heads,orders", MANY_TABLES)
@pytest.mark.parametrize("dtype,batch,seqlen", [("bf16", 3, 77), ("bf16", 5, 1), ("bf16", 2, 300),
                                                ("f32", 2, 70)])
def test_forward_many_tables_all_positions(B, heads, orders, dtype, batch, seqlen):
    """engram_forward with 24 or 32 tables: fused retrieval and both fusion
    routes (prefill tiles, and the one-token route with its carried state),
    every position against the oracle; the retrieve-in-projection flag
    (which covers at most 16 tables, so with more the library keeps the
    separate retrieval) gives the same bits."""
    say("forward many tables", heads, orders, dtype, batch, seqlen)
    wl = many_tables_wl(heads, orders, batch, seqlen, dtype=dtype)
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    ctx = state = None
    if seqlen == 1:
        rng = np.random.default_rng(5)
        ctx = rng.integers(0, wl.vocab_comp + 1, (batch, 2)).astype(np.int32)
        state = rng.standard_normal((1, batch, 3, wl.d_model)).astype(np.float32)
    st_dev = None if state is None else to_device(state, torch.float32, "cuda")
    out, alpha, bad = forward(dl, toks, prev_ctx=None if ctx is None else dev_i32(ctx), conv_state=st_dev)
    assert bad == 0
    idx, _, _ = oracle_indices(wl, dl.li, toks, dl.comp_map_host, prev_ctx=ctx)
    L = oracle_layer(wl, dl.li, idx, batch, seqlen, conv_state=state)
    ref, ref_alpha, _ = L.forward_all()
    assert_within(host(out), ref, dtype, "many tables out")
    assert np.abs(host(alpha) - ref_alpha).max() <= alpha_tol(dtype)
    st2 = None if state is None else to_device(state, torch.float32, "cuda")
    out2, _, _ = forward(dl, toks, prev_ctx=None if ctx is None else dev_i32(ctx), conv_state=st2,
                         flags=B.RETRIEVE_IN_PROJECTION)
    assert torch.equal(out2.view(torch.int16) if dtype == "bf16" else out2,
                       out.view(torch.int16) if dtype == "bf16" else out)


def _sampled_check(wl, dl, toks, n_pos, what, prev_ctx=None, conv_state=None, seed=0, flags=0):
    batch, seqlen = toks.shape
    out, alpha, bad = forward(dl, toks, prev_ctx=None if prev_ctx is None else dev_i32(prev_ctx),
                              conv_state=None if conv_state is None else to_device(conv_state, torch.float32, "cuda"),
                              flags=flags)
    assert bad == 0
    pos = sample_positions(batch, seqlen, n_pos, seed)
    idx, _, _ = oracle_indices(wl, dl.li, toks, dl.comp_map_host, prev_ctx=prev_ctx)
    L = oracle_layer(wl, dl.li, idx, batch, seqlen, rows=rows_needed(pos, seqlen, wl.conv_kernel),
                     conv_state=conv_state)
    ref, ref_alpha = L.forward_positions(pos)
    got = host(out)[:, pos]
    assert_within(got, ref, wl.dtype, what)
    assert np.abs(host(alpha)[:, pos] - ref_alpha).max() <= alpha_tol(wl.dtype)
    return out, alpha


def _same_bits_in_projection(dl, toks, out, alpha, flag):
    """The forward with retrieval inside both projection launches gives the
    bits of the separate-retrieval forward."""
    out2, alpha2, bad2 = forward(dl, toks, flags=flag)
    assert bad2 == 0
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert torch.equal(alpha2, alpha)


def _same_bits_packed_weights(B, dl, toks, out, alpha):
    """The forward on W_k and W_v packed by engram_pack_weight gives the bits
    of the forward on the [d][D_e] matrices."""
    packed = dl.plan.packed_weights(dl.weights)
    saved, dl.weights = dl.weights, packed
    try:
        out2, alpha2, bad2 = forward(dl, toks, flags=B.WEIGHTS_PACKED)
    finally:
        dl.weights = saved
    assert bad2 == 0
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert torch.equal(alpha2, alpha)
    del packed


@pytest.mark.parametrize("name", ["small", "layer27b"])
def test_forward_full_size_sampled(B, name):
    """Sampled positions against the oracle; the same forward with retrieval
    inside the W_k and W_v launches (256 x 256 tiles at both sizes) gives
    the same bits, its sampled positions checked against the oracle too."""
    say("forward full size", name)
    wl = W.workload(name)
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    out, alpha = _sampled_check(wl, dl, toks, 48, name)
    say("forward full size, retrieval in projection", name)
    _same_bits_in_projection(dl, toks, out, alpha, B.RETRIEVE_IN_PROJECTION)
    _sampled_check(wl, dl, toks, 24, name + " (retrieval in projection)", seed=7, flags=B.RETRIEVE_IN_PROJECTION)
    say("forward full size, packed weights", name)
    _same_bits_packed_weights(B, dl, toks, out, alpha)
    del dl
    torch.cuda.empty_cache()


def test_forward_multibranch_prefill_two_layers_sampled(B):
    wl = W.workload("multibranch_prefill")
    toks = W.make_tokens(wl)
    for slot in range(len(wl.layers)):
        say("forward multibranch prefill layer", wl.layers[slot])
        dl = make_device_layer(wl, layer_slot=slot)
        out, alpha = _sampled_check(wl, dl, toks, 20, "multibranch layer %d" % wl.layers[slot], seed=slot)
        if slot == 0:  # four stacked W_k matrices and W_v, packed
            _same_bits_packed_weights(B, dl, toks, out, alpha)
        del dl
        torch.cuda.empty_cache()


def test_decode_step_batch_size_invariance(B):
    """A decode step of 3,328 sequences (260 narrow projection tiles, more
    than one round) and the same step of its first 128 sequences (10 tiles)
    give the same bits for those sequences: outputs, gates, conv state and
    context; sampled rows of the large step against the oracle."""
    say("decode step batch-size invariance")
    wl = dataclasses.replace(small_wl(n_branches=4, batch=3328, seqlen=1, head_dim=64), decode=True,
                             state_dtype="bf16")
    assert wl.emb_dim % 256 == 0
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    Br, d, nb = wl.n_branches, wl.d_model, 128
    ctx_a = dev_i32(dl.li.prev_ctx)
    st_a = to_device(dl.li.conv_state, dl.plan.state_torch_dtype, "cuda")
    out_a, alpha_a, bad = forward(dl, toks, prev_ctx=ctx_a, conv_state=st_a)
    assert bad == 0
    ctx_b = dev_i32(dl.li.prev_ctx[:nb])
    st_b = st_a.new_empty((Br, nb) + tuple(st_a.shape[2:]))
    st_b.copy_(to_device(dl.li.conv_state[:, :nb], dl.plan.state_torch_dtype, "cuda"))
    h_b = dl.h[:, :nb].contiguous()
    out_b, alpha_b, _ = forward(dl, np.ascontiguousarray(toks[:nb]), prev_ctx=ctx_b, conv_state=st_b, h=h_b)
    assert torch.equal(out_a[:, :nb], out_b)
    assert torch.equal(alpha_a[:, :nb], alpha_b)
    assert torch.equal(st_a[:, :nb], st_b)
    assert torch.equal(ctx_a[:nb], ctx_b)
    rows = np.arange(5, wl.batch, 211)
    idx, _, new_ctx = oracle_indices(wl, dl.li, toks, dl.comp_map_host, prev_ctx=dl.li.prev_ctx)
    L = oracle_layer(wl, dl.li, idx, wl.batch, 1, rows=rows, conv_state=dl.li.conv_state)
    ref, ref_alpha = L.forward_positions(rows)
    assert_within(host(out_a)[:, rows], ref, "bf16", "decode out, 3328 sequences")
    assert np.abs(host(alpha_a)[:, rows] - ref_alpha).max() <= alpha_tol("bf16")
    assert np.array_equal(ctx_a.cpu().numpy(), new_ctx)
    del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("state_dtype", ["bf16", "f32"])
def test_forward_multibranch_decode_with_state(B, state_dtype):
    wl = dataclasses.replace(W.workload("multibranch_decode"), state_dtype=state_dtype)
    toks = W.make_tokens(wl)
    for slot in range(len(wl.layers)):
        say("forward multibranch decode layer", wl.layers[slot], "state", state_dtype)
        dl = make_device_layer(wl, layer_slot=slot)
        ctx = dev_i32(dl.li.prev_ctx)
        state = to_device(dl.li.conv_state, dl.plan.state_torch_dtype, "cuda")
        out, alpha, bad = forward(dl, toks, prev_ctx=ctx, conv_state=state)
        assert bad == 0
        rows = np.arange(0, wl.batch, 7)
        idx, _, new_ctx = oracle_indices(wl, dl.li, toks, dl.comp_map_host, prev_ctx=dl.li.prev_ctx)
        L = oracle_layer(wl, dl.li, idx, wl.batch, 1, rows=rows, conv_state=dl.li.conv_state)
        ref, ref_alpha = L.forward_positions(rows)
        assert_within(host(out)[:, rows], ref, "bf16", "decode out")
        assert np.abs(host(alpha)[:, rows] - ref_alpha).max() <= alpha_tol("bf16")
        assert np.array_equal(ctx.cpu().numpy(), new_ctx)
        # new conv state = [old rows 1, 2, u_0]
        st = state.float().cpu().numpy()
        assert np.array_equal(st[:, :, :2], dl.li.conv_state[:, :, 1:])
        for r in rows[:8]:
            _, _, u = L.forward_range(int(r), 0, 1, want_u=True)
            np.testing.assert_allclose(st[:, r, 2], u[:, 0], rtol=2e-2, atol=1e-2)
        del dl
        torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def maxtable_layer(B):
    wl = W.workload("maxtable_zipf")
    say("allocating max-table layer (%.1f GB of tables)" % (wl.table_bytes() / 1e9))
    dl = make_device_layer(wl)
    yield dl
    dl.free_tables()
    del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["maxtable_zipf", "maxtable_uniform"])
def test_forward_maxtable_sampled(B, maxtable_layer, name):
    say("forward", name)
    wl = W.workload(name)
    toks = W.make_tokens(wl)
    out, alpha = _sampled_check(wl, maxtable_layer, toks, 24, name)
    say("forward, retrieval in projection", name)
    _same_bits_in_projection(maxtable_layer, toks, out, alpha, B.RETRIEVE_IN_PROJECTION)
    say("forward, packed weights", name)
    _same_bits_packed_weights(B, maxtable_layer, toks, out, alpha)


@pytest.mark.parametrize("dtype,d,heads,head_dim,orders,kc,br,batch,seqlen", [
    ("bf16", 256, 2, 32, (2, 3), 1, 2, 2, 300),   # no conv history
    ("bf16", 256, 2, 32, (2, 3), 2, 1, 3, 77),
    ("bf16", 512, 4, 32, (3,), 3, 3, 2, 130),     # trigrams only
    ("bf16", 256, 4, 32, (2,), 4, 1, 1, 257),     # bigrams only, one token past a tile
    ("bf16", 256, 2, 32, (2, 3), 2, 4, 4, 1),     # one-token chunks on the fused path (K_c - 1 = 1)
    ("bf16", 256, 2, 32, (2, 3), 3, 2, 5, 1),     # one-token chunks on the fusion kernel, K_c = 3
    ("f32", 200, 3, 4, (2, 3), 3, 2, 2, 45),      # d not a multiple of 64, D_e = 24
    ("f32", 72, 1, 12, (2, 3), 2, 3, 3, 33),      # a sequence over two fusion workgroups
])
def test_forward_other_shapes_all_positions(B, dtype, d, heads, head_dim, orders, kc, br, batch, seqlen):
    """Conv kernels shorter than 4, single-order n-grams and odd fp32 widths,
    with a carried context and conv state: every position against the oracle,
    and the new state and context."""
    say("other shapes", dtype, d, heads, head_dim, orders, kc, br, batch, seqlen)
    wl = dataclasses.replace(small_wl(n_branches=br, batch=batch, seqlen=seqlen, d_model=d, heads=heads,
                                      head_dim=head_dim, conv_kernel=kc, dtype=dtype), orders=orders)
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    rng = np.random.default_rng(d + kc)
    ctx0 = rng.integers(0, wl.vocab_comp + 1, (batch, 2)).astype(np.int32)
    st0 = (0.05 * rng.standard_normal((br, batch, max(kc - 1, 0), d))).astype(np.float32)
    ctx = dev_i32(ctx0)
    st = to_device(st0, torch.float32, "cuda") if kc > 1 else None
    out, alpha, bad = forward(dl, toks, prev_ctx=ctx, conv_state=st)
    assert bad == 0
    idx, _, new_ctx = oracle_indices(wl, dl.li, toks, dl.comp_map_host, prev_ctx=ctx0)
    L = oracle_layer(wl, dl.li, idx, batch, seqlen, conv_state=st0 if kc > 1 else None)
    ref, ref_alpha, u = L.forward_all(want_u=True)
    assert_within(host(out), ref, dtype, "out")
    assert np.abs(host(alpha) - ref_alpha).max() <= alpha_tol(dtype)
    assert np.array_equal(ctx.cpu().numpy(), new_ctx)
    if kc > 1:
        assert_within(st.cpu().numpy(), L.new_conv_state(u), dtype, "new conv state")
    del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("br,batch,seqlen", [
    (2, 3, 255),   # sequences start 1 and 2 tokens before tile seams: the seam rows read the state
    (1, 4, 254),
    (3, 2, 40),    # the fused W_v path reads the state at sequence starts, stages, converts
    (4, 5, 1),     # one-token chunks: the fusion kernel updates the bf16 state in place
    (2, 3, 2),
])
def test_forward_bf16_state_all_positions(B, br, batch, seqlen):
    """A bf16 conv state: the carried rows are read in bf16 on every route
    (fused W_v epilogue, seam rows, fusion kernel) and the new state is the
    last K_c-1 gated values rounded to bf16; every position against the
    oracle run on the same (bf16-exact) carried values."""
    say("bf16 state", br, batch, seqlen)
    wl = dataclasses.replace(small_wl(n_branches=br, batch=batch, seqlen=seqlen), state_dtype="bf16")
    dl = make_device_layer(wl)
    assert dl.plan.state_torch_dtype == torch.bfloat16
    toks = W.make_tokens(wl)
    rng = np.random.default_rng(31 + seqlen)
    ctx0 = rng.integers(0, wl.vocab_comp + 1, (batch, 2)).astype(np.int32)
    st0 = W.round_to_bf16((0.5 * rng.standard_normal((br, batch, 3, wl.d_model))).astype(np.float32))
    ctx = dev_i32(ctx0)
    st = to_device(st0, torch.bfloat16, "cuda")
    out, alpha, bad = forward(dl, toks, prev_ctx=ctx, conv_state=st)
    assert bad == 0
    idx, _, new_ctx = oracle_indices(wl, dl.li, toks, dl.comp_map_host, prev_ctx=ctx0)
    L = oracle_layer(wl, dl.li, idx, batch, seqlen, conv_state=st0)
    ref, ref_alpha, u = L.forward_all(want_u=True)
    assert_within(host(out), ref, "bf16", "out (bf16 state)")
    assert np.abs(host(alpha) - ref_alpha).max() <= alpha_tol("bf16")
    assert np.array_equal(ctx.cpu().numpy(), new_ctx)
    assert_within(st.float().cpu().numpy(), L.new_conv_state(u), "bf16", "new bf16 conv state")
    del dl
    torch.cuda.empty_cache()


def test_chunked_prefill_and_decode_with_bf16_state(B):
    """With a bf16 state the chunks carry rounded gated values: chunked calls
    agree with one whole call, and with the oracle's unchunked pass, within
    the bf16 tolerance (bit equality holds for the fp32 state)."""
    say("chunks, bf16 state")
    wl = dataclasses.replace(small_wl(n_branches=2, batch=3, seqlen=300), state_dtype="bf16")
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    Br, d = wl.n_branches, wl.d_model
    pad = np.full((wl.batch, 2), wl.vocab_comp, np.int32)
    full, alpha_full, _ = forward(dl, toks, prev_ctx=dev_i32(pad),
                                  conv_state=torch.zeros((Br, wl.batch, 3, d), dtype=torch.bfloat16, device="cuda"))
    ctx = dev_i32(pad)
    st = torch.zeros((Br, wl.batch, 3, d), dtype=torch.bfloat16, device="cuda")
    parts = []
    for a, b in [(0, 1), (1, 2), (2, 5), (5, 261), (261, 262), (262, 300)]:
        h = _split(dl.h, Br, wl.batch, wl.seqlen, a, b)
        o, _, _ = forward(dl, np.ascontiguousarray(toks[:, a:b]), prev_ctx=ctx, conv_state=st, h=h)
        parts.append(o.view(Br, wl.batch, b - a, d))
    chunked = host(torch.cat(parts, 2).view(Br, -1, d))
    idx, _, _ = oracle_indices(wl, dl.li, toks, dl.comp_map_host)
    ref, _, _ = oracle_layer(wl, dl.li, idx, wl.batch, wl.seqlen).forward_all()
    assert_within(chunked, ref, "bf16", "chunked (bf16 state) vs oracle")
    assert_within(host(full), ref, "bf16", "whole call vs oracle")
    assert np.array_equal(ctx.cpu().numpy(), dl.comp_map_host[toks[:, -2:]])


# ----------------------------------------------------------------------------
# the split calls: engram_hash -> engram_gather -> engram_gate_fuse
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["tiny", "bf16_1x2x300", "bf16_4x3x2", "bf16_2x2x77"])
def test_split_calls_equal_forward_and_oracle(B, case):
    """Retrieval and fusion as separate calls, with a carried context, a conv
    state and the caller's alpha buffer: indices and E bit-exact against the
    oracle; out, alpha and the new state within tolerance of the oracle and
    bit-identical to engram_forward on the same inputs."""
    say("split calls", case)
    if case == "tiny":
        wl = W.workload("tiny")
    else:
        br, batch, seqlen = (int(x) for x in case.split("_")[1].split("x"))
        wl = small_wl(n_branches=br, batch=batch, seqlen=seqlen)
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    batch, seqlen = toks.shape
    n_tok, Br, d, S = batch * seqlen, wl.n_branches, wl.d_model, wl.conv_kernel - 1
    rng = np.random.default_rng(23)
    ctx0 = rng.integers(0, wl.vocab_comp + 1, (batch, 2)).astype(np.int32)  # PAD = V' included
    ctx0[0] = wl.vocab_comp
    st0 = (0.05 * rng.standard_normal((Br, batch, S, d))).astype(np.float32)
    tdt = dl.h.dtype

    ctx_s = dev_i32(ctx0)
    idx = torch.zeros((n_tok, wl.n_tables), dtype=torch.int32, device="cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    dl.plan.engram_hash(dev_i32(toks), dl.comp_map, idx, prev_ctx=ctx_s, bad_tokens=bad)
    emb = torch.empty((n_tok, wl.emb_dim), dtype=tdt, device="cuda")
    dl.plan.engram_gather(idx, dl.tables, emb)
    st_s = to_device(st0, torch.float32, "cuda")
    out_s = torch.empty_like(dl.h)
    alpha_s = torch.full((Br, n_tok), -1.0, dtype=torch.float32, device="cuda")
    ws = dl.plan.workspace(batch, seqlen)
    dl.plan.engram_gate_fuse(emb, dl.h, dl.weights, out_s, ws, batch, seqlen, conv_state=st_s, alpha=alpha_s)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    assert np.array_equal(ctx_s.cpu().numpy(), ctx0)  # engram_hash leaves the context alone

    ctx_f = dev_i32(ctx0)
    st_f = to_device(st0, torch.float32, "cuda")
    out_f, alpha_f, _ = forward(dl, toks, prev_ctx=ctx_f, conv_state=st_f)
    assert torch.equal(out_s, out_f)
    assert torch.equal(alpha_s, alpha_f)
    assert torch.equal(st_s, st_f)

    idx_ref, _, new_ctx = oracle_indices(wl, dl.li, toks, dl.comp_map_host, prev_ctx=ctx0)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), idx_ref)
    assert np.array_equal(ctx_f.cpu().numpy(), new_ctx)
    dt = oracle_dtype(wl)
    emb_ref = oracle.gather_synth(idx_ref, wl.head_dim, dl.li.table_seed, dt)
    got_emb = emb.view(torch.int16).cpu().numpy().view(np.uint16) if wl.dtype == "bf16" else emb.cpu().numpy()
    assert np.array_equal(got_emb.view(np.uint8), emb_ref.view(np.uint8))
    L = oracle_layer(wl, dl.li, idx_ref, batch, seqlen, conv_state=st0)
    ref, ref_alpha, u = L.forward_all(want_u=True)
    assert_within(host(out_s), ref, wl.dtype, case + " out")
    assert np.abs(host(alpha_s) - ref_alpha).max() <= alpha_tol(wl.dtype)
    assert np.all((host(alpha_s) > 0) & (host(alpha_s) < 1))
    assert_within(st_s.cpu().numpy(), L.new_conv_state(u), wl.dtype, case + " new conv state")
    del dl
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# invariants on the GPU path
# ----------------------------------------------------------------------------

def _split(x, n_branches, batch, seqlen, a, b):
    d = x.shape[-1]
    return x.view(n_branches, batch, seqlen, d)[:, :, a:b].contiguous().view(n_branches, batch * (b - a), d)


@pytest.mark.parametrize("dt,br,kc,mode,flags", [
    ("bf16", 4, 4, oracle.CONV_LINEAR, 0),
    ("f32", 3, 4, oracle.CONV_SILU_SKIP, 0),
    ("bf16", 2, 2, oracle.CONV_SILU_SKIP, oracle.OUT_DELTA),
    ("bf16", 1, 3, oracle.CONV_LINEAR, 0),
])
def test_chunked_prefill_and_decode_equal_full_prefill_bitwise(B, dt, br, kc, mode, flags):
    """Chunks of 1, 1, 3, 32, 1 and 2 positions (one-token chunks take the
    decode-step kernel) against the whole sequence in one call."""
    say("chunk invariance", dt, br, kc, mode, flags)
    wl = small_wl(n_branches=br, batch=3, seqlen=40, dtype=dt, conv_kernel=kc)
    dl = make_device_layer(wl, conv_mode=mode)
    toks = W.make_tokens(wl)
    Br, d = wl.n_branches, wl.d_model
    pad = np.full((wl.batch, 2), wl.vocab_comp, np.int32)
    ctx_full = dev_i32(pad)
    st_full = torch.zeros((Br, wl.batch, kc - 1, d), dtype=torch.float32, device="cuda")
    full, alpha_full, _ = forward(dl, toks, prev_ctx=ctx_full, conv_state=st_full, flags=flags)
    ctx = dev_i32(pad)
    st = torch.zeros_like(st_full)
    parts, alphas = [], []
    for a, b in [(0, 1), (1, 2), (2, 5), (5, 37), (37, 38), (38, 40)]:
        h = _split(dl.h, Br, wl.batch, wl.seqlen, a, b)
        o, al, _ = forward(dl, np.ascontiguousarray(toks[:, a:b]), prev_ctx=ctx, conv_state=st, h=h, flags=flags)
        parts.append(o.view(Br, wl.batch, b - a, d))
        alphas.append(al.view(Br, wl.batch, b - a))
    chunked = torch.cat(parts, 2).view(Br, -1, d)
    assert torch.equal(chunked, full)
    assert torch.equal(torch.cat(alphas, 2).view(Br, -1), alpha_full)
    assert torch.equal(ctx, ctx_full)
    assert torch.equal(st, st_full)
    # and the carried context is the last two compressed ids
    assert np.array_equal(ctx.cpu().numpy(), dl.comp_map_host[toks[:, -2:]])


def test_determinism_streams_and_in_place(B):
    say("determinism")
    wl = W.workload("small")
    dl = make_device_layer(wl, batch=2, seqlen=1024)
    toks = W.make_tokens(wl, batch=2, seqlen=1024)
    o1, a1, _ = forward(dl, toks)
    o2, a2, _ = forward(dl, toks)
    assert torch.equal(o1, o2) and torch.equal(a1, a2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o3, a3, _ = forward(dl, toks, stream=s)
    assert torch.equal(o1, o3) and torch.equal(a1, a3)
    h_copy = dl.h.clone()
    o4, _, _ = forward(dl, toks, h=h_copy, out=h_copy)  # out aliases h
    assert torch.equal(o1, o4)


def test_causality_on_gpu(B):
    say("causality")
    wl = small_wl(n_branches=2, batch=2, seqlen=100)
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    base, _, _ = forward(dl, toks)
    t0 = 60
    toks2 = toks.copy()
    toks2[0, t0 + 1:] = np.random.default_rng(5).integers(0, wl.vocab, wl.seqlen - t0 - 1)
    h2 = dl.h.clone().view(2, 2, 100, -1)
    h2[:, 0, t0 + 1:] += 1.0
    pert, _, _ = forward(dl, toks2, h=h2.view(2, 200, -1))
    b4 = base.view(2, 2, 100, -1)
    p4 = pert.view(2, 2, 100, -1)
    assert torch.equal(p4[:, 0, :t0 + 1], b4[:, 0, :t0 + 1])
    assert not torch.equal(p4[:, 0, t0 + 1:], b4[:, 0, t0 + 1:])
    assert torch.equal(p4[:, 1], b4[:, 1])


def test_profiling_counts_launches(B):
    wl = W.workload("tiny")
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    dl.plan.engram_profile_begin(64)
    forward(dl, toks)
    forward(dl, toks)
    # engram_forward retrieves with one fused hash+gather kernel
    idx = torch.zeros((wl.n_tokens, wl.n_tables), dtype=torch.int32, device="cuda")
    dl.plan.engram_hash(dev_i32(toks), dl.comp_map, idx)
    torch.cuda.synchronize()
    prof = dl.plan.engram_profile_end()
    # the fusion-kernel path computes the gate inside the fusion kernel
    for k, n in (("hash", 1), ("gather", 2), ("gemm", 2), ("gate", 0), ("fuse", 2), ("gemm_v", 0)):
        assert prof[k]["launches"] == n, (k, prof)
        assert (prof[k]["total_ms"] > 0) == (n > 0)
    assert prof["dropped"] == 0
    # bf16 prefill: retrieval, the W_k launch, the gate, then the W_v launch
    # with the fusion step in its epilogue and, past one 256-token tile, the
    # seam rows; chunks shorter than K_c - 1 use the fusion kernel
    for seqlen, seams in ((50, 0), (300, 1)):
        wl = small_wl(n_branches=2, batch=2, seqlen=seqlen)
        dl = make_device_layer(wl)
        toks = W.make_tokens(wl)
        dl.plan.engram_profile_begin(64)
        forward(dl, toks)
        forward(dl, np.ascontiguousarray(toks[:, :2]), h=_split(dl.h, 2, 2, seqlen, 0, 2))
        torch.cuda.synchronize()
        prof = dl.plan.engram_profile_end()
        for k, n in (("hash", 0), ("gather", 2), ("gemm", 2), ("gate", 1), ("fuse", 1), ("gemm_v", 1),
                     ("seam", seams), ("aux", 0)):
            assert prof[k]["launches"] == n, (seqlen, k, prof)
    # sampled timing: one launch in three of each selected kind (the 1st, 4th, 7th)
    dl.plan.engram_profile_every(3)
    dl.plan.engram_profile_begin(64, ["gemm", "gemm_v"])
    for _ in range(7):
        forward(dl, toks)
    torch.cuda.synchronize()
    prof = dl.plan.engram_profile_end()
    dl.plan.engram_profile_every(1)
    assert prof["gemm"]["launches"] == 3 and prof["gemm_v"]["launches"] == 3, prof
    assert prof["gather"]["launches"] == 0 and prof["dropped"] == 0, prof


def test_unsupported_bf16_shape_is_rejected(B):
    wl = small_wl(d_model=200, batch=1, seqlen=8)
    with pytest.raises(B.EngramError) as e:
        dl = make_device_layer(wl)
        forward(dl, W.make_tokens(wl))
    assert e.value.status == B.E_UNSUPPORTED


# ----------------------------------------------------------------------------
# backward (training): engram_backward against the oracle's chain rule
# ----------------------------------------------------------------------------

def grad_within(got, ref, what, rel=2e-2, frac=1e-2):
    """fp32 gradients fed by bf16 operands (dk and dv enter the contractions
    rounded to bf16, as E and the weights do in the forward): |d| <= frac *
    rms(row of ref) + rel * |ref|, rows along the last axis."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite"
    bound = frac * (np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True)) + 1e-30) + rel * np.abs(ref)
    ratio = np.abs(got - ref) / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, "%s: max |d|/bound = %.3f at %s (got %r, ref %r)" % (
        what, ratio.max(), worst, got[worst], ref[worst])


def _backward(dl, idx, dout, flags=0):
    wl = dl.wl
    batch, seqlen = wl.batch, wl.seqlen
    n_tok = batch * seqlen
    from hashed_gram_embedding_vocab_amd import binding
    grads = binding.Grads(wl.n_branches, wl.d_model, wl.emb_dim, wl.conv_kernel, wl.n_tables, n_tok, wl.head_dim)
    dh = torch.empty_like(dl.h)
    ws = dl.plan.backward_workspace(batch, seqlen)
    dl.plan.engram_backward(idx, dl.tables, dl.h, dl.weights, dout, dh, grads, ws, batch, seqlen, flags=flags)
    torch.cuda.synchronize()
    return dh, grads


@pytest.mark.parametrize("br,batch,seqlen,kc,mode,flags,d", [
    (1, 2, 77, 4, oracle.CONV_LINEAR, 0, 256),
    (2, 2, 300, 4, oracle.CONV_SILU_SKIP, 0, 256),
    (4, 3, 33, 3, oracle.CONV_LINEAR, oracle.OUT_DELTA, 256),
    (1, 1, 1, 4, oracle.CONV_LINEAR, 0, 256),
    (3, 2, 40, 1, oracle.CONV_SILU_SKIP, 0, 256),
    (1, 1, 64, 2, oracle.CONV_LINEAR, 0, 1280),
])
def test_backward_matches_oracle(B, br, batch, seqlen, kc, mode, flags, d):
    say("backward", br, batch, seqlen, kc, mode, flags, d)
    wl = small_wl(n_branches=br, batch=batch, seqlen=seqlen, conv_kernel=kc, d_model=d)
    dl = make_device_layer(wl, conv_mode=mode)
    toks = W.make_tokens(wl)
    n_tok = batch * seqlen
    idx = torch.zeros((n_tok, wl.n_tables), dtype=torch.int32, device="cuda")
    dl.plan.engram_hash(dev_i32(toks), dl.comp_map, idx)
    rng = np.random.default_rng(br * 1000 + seqlen)
    dout_f = rng.standard_normal((br, n_tok, d)).astype(np.float32)
    dout = torch.from_numpy(dout_f).to(torch.bfloat16).cuda()
    dh, g = _backward(dl, idx, dout, flags)
    # the same call again: the same bits
    dh2, g2 = _backward(dl, idx, dout, flags)
    assert torch.equal(dh, dh2)
    for name in ("dw", "dgamma_h", "dgamma_k", "dconv_w", "row_ids", "row_grads", "row_counts"):
        assert torch.equal(getattr(g, name), getattr(g2, name)), name

    idx_ref, _, _ = oracle_indices(wl, dl.li, toks, dl.comp_map_host)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), idx_ref)
    L = oracle_layer(wl, dl.li, idx_ref, batch, seqlen, conv_mode=mode, flags=flags)
    ref = L.backward(dout.float().cpu().numpy())
    assert_within(host(dh), ref["dh"], "bf16", "dh")
    grad_within(g.dw[:br].cpu().numpy(), ref["dw_k"], "dW_k")
    grad_within(g.dw[br].cpu().numpy(), ref["dw_v"], "dW_v")
    grad_within(g.dgamma_h.cpu().numpy(), ref["dgamma_h"], "dgamma_h")
    grad_within(g.dgamma_k.cpu().numpy(), ref["dgamma_k"], "dgamma_k")
    grad_within(g.dconv_w.cpu().numpy(), ref["dconv_w"], "dconv_w")
    rows, grads, counts = oracle.table_grad(idx_ref, ref["demb"], wl.head_dim)
    got_counts = g.row_counts.cpu().numpy()
    assert np.array_equal(got_counts, counts)
    got_rows = g.row_ids.cpu().numpy().view(np.uint32)
    got_grads = g.row_grads.cpu().numpy()
    for tau in range(wl.n_tables):
        c = int(counts[tau])
        assert np.array_equal(got_rows[tau, :c], rows[tau, :c]), tau
        grad_within(got_grads[tau, :c], grads[tau, :c], "table %d rows" % tau)
    del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,br,batch,seqlen", [("small", 1, 1, 96), ("layer27b", 1, 1, 40),
                                                   ("multibranch_prefill", 4, 1, 12)])
def test_backward_full_width_against_oracle(B, name, br, batch, seqlen):
    """The configs' own widths (d, tables, d_e, branches), on few enough
    tokens for the oracle's chain rule to finish in seconds."""
    say("backward full width", name, batch, seqlen)
    wl = dataclasses.replace(W.workload(name), batch=batch, seqlen=seqlen)
    dl = make_device_layer(wl, batch=batch, seqlen=seqlen)
    toks = W.make_tokens(wl, batch=batch, seqlen=seqlen)
    n_tok = batch * seqlen
    idx = torch.zeros((n_tok, wl.n_tables), dtype=torch.int32, device="cuda")
    dl.plan.engram_hash(dev_i32(toks), dl.comp_map, idx)
    rng = np.random.default_rng(5)
    dout = torch.from_numpy(rng.standard_normal((br, n_tok, wl.d_model)).astype(np.float32)).to(torch.bfloat16).cuda()
    dh, g = _backward(dl, idx, dout)
    idx_ref, _, _ = oracle_indices(wl, dl.li, toks, dl.comp_map_host)
    L = oracle_layer(wl, dl.li, idx_ref, batch, seqlen)
    ref = L.backward(dout.float().cpu().numpy())
    assert_within(host(dh), ref["dh"], "bf16", "dh")
    grad_within(g.dw[:br].cpu().numpy(), ref["dw_k"], "dW_k")
    grad_within(g.dw[br].cpu().numpy(), ref["dw_v"], "dW_v")
    grad_within(g.dgamma_h.cpu().numpy(), ref["dgamma_h"], "dgamma_h")
    grad_within(g.dgamma_k.cpu().numpy(), ref["dgamma_k"], "dgamma_k")
    grad_within(g.dconv_w.cpu().numpy(), ref["dconv_w"], "dconv_w")
    rows, grads, counts = oracle.table_grad(idx_ref, ref["demb"], wl.head_dim)
    assert np.array_equal(g.row_counts.cpu().numpy(), counts)
    got_rows = g.row_ids.cpu().numpy().view(np.uint32)
    got_grads = g.row_grads.cpu().numpy()
    for tau in range(wl.n_tables):
        c = int(counts[tau])
        assert np.array_equal(got_rows[tau, :c], rows[tau, :c])
        grad_within(got_grads[tau, :c], grads[tau, :c], "table %d rows" % tau)
    del dl
    torch.cuda.empty_cache()


def test_backward_table_rows_three_sort_passes(B):
    """Tables of about 8.4M rows (24 row bits: three radix passes of 8 bits)
    and 4,500 tokens, so each table's items span two full 2,048-item sort
    blocks and a ragged third: rows, counts and row sums against the oracle."""
    say("backward table rows, three sort passes")
    wl = dataclasses.replace(small_wl(batch=3, seqlen=1500), table_target=8_400_000)
    assert all(p >= 1 << 23 for p in wl.primes())
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    n_tok = wl.n_tokens
    idx = torch.zeros((n_tok, wl.n_tables), dtype=torch.int32, device="cuda")
    dl.plan.engram_hash(dev_i32(toks), dl.comp_map, idx)
    rng = np.random.default_rng(11)
    dout = torch.from_numpy(rng.standard_normal((1, n_tok, wl.d_model)).astype(np.float32)).to(torch.bfloat16).cuda()
    dh, g = _backward(dl, idx, dout)
    idx_ref, _, _ = oracle_indices(wl, dl.li, toks, dl.comp_map_host)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), idx_ref)
    L = oracle_layer(wl, dl.li, idx_ref, wl.batch, wl.seqlen)
    ref = L.backward(dout.float().cpu().numpy())
    rows, grads, counts = oracle.table_grad(idx_ref, ref["demb"], wl.head_dim)
    assert np.array_equal(g.row_counts.cpu().numpy(), counts)
    got_rows = g.row_ids.cpu().numpy().view(np.uint32)
    got_grads = g.row_grads.cpu().numpy()
    for tau in range(wl.n_tables):
        c = int(counts[tau])
        assert np.array_equal(got_rows[tau, :c], rows[tau, :c]), tau
        grad_within(got_grads[tau, :c], grads[tau, :c], "table %d rows" % tau)
    del dl
    torch.cuda.empty_cache()


def test_backward_full_size_rows_and_determinism(B):
    """32,768 tokens of the small config: the listed rows of every table are
    exactly the distinct slots the tokens hashed to (ascending), and a second
    call gives the same bits."""
    say("backward full size")
    wl = W.workload("small")
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    n_tok = wl.n_tokens
    idx = torch.zeros((n_tok, wl.n_tables), dtype=torch.int32, device="cuda")
    dl.plan.engram_hash(dev_i32(toks), dl.comp_map, idx)
    dout = (torch.randn((1, n_tok, wl.d_model), generator=torch.Generator().manual_seed(3))
            .to(torch.bfloat16).cuda())
    dh, g = _backward(dl, idx, dout)
    dh2, g2 = _backward(dl, idx, dout)
    assert torch.equal(dh, dh2)
    for name in ("dw", "dgamma_h", "dgamma_k", "dconv_w", "row_ids", "row_grads", "row_counts"):
        assert torch.equal(getattr(g, name), getattr(g2, name)), name
    assert torch.isfinite(dh.float()).all() and torch.isfinite(g.dw).all() and torch.isfinite(g.row_grads).all()
    idx_h = idx.cpu().numpy().view(np.uint32)
    counts = g.row_counts.cpu().numpy()
    rows = g.row_ids.cpu().numpy().view(np.uint32)
    for tau in range(wl.n_tables):
        used = np.unique(idx_h[:, tau])
        assert counts[tau] == len(used)
        assert np.array_equal(rows[tau, :counts[tau]], used)
    del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("in_proj", [False, True])
@pytest.mark.parametrize("batch,seqlen,heads", [(300, 1, 8), (5, 2, 2), (129, 1, 4)])
def test_short_chunks_retrieval_in_projection(B, batch, seqlen, heads, in_proj):
    """Short chunks, retrieval by its own kernel or inside the projection
    launch (E never materialised): out-of-range ids are counted once each and
    hash as PAD, and the result equals the split calls bit for bit and the
    oracle."""
    say("short chunks", batch, seqlen, heads, "retrieval in projection" if in_proj else "")
    wl = small_wl(n_branches=2, batch=batch, seqlen=seqlen, heads=heads, head_dim=32)
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    toks[0, 0] = -5
    toks[-1, -1] = wl.vocab + 3
    if batch > 3:
        toks[3, 0] = 2 ** 31 - 1
    n_bad = int(((toks < 0) | (toks >= wl.vocab)).sum())
    rng = np.random.default_rng(batch)
    prev = rng.integers(0, wl.vocab_comp + 1, (batch, 2)).astype(np.int32)
    state0 = rng.standard_normal((wl.n_branches, batch, wl.conv_kernel - 1, wl.d_model)).astype(np.float32)
    ctx = dev_i32(prev)
    state = to_device(state0, torch.float32, "cuda")
    out, alpha, bad = forward(dl, toks, prev_ctx=ctx, conv_state=state,
                              flags=B.RETRIEVE_IN_PROJECTION if in_proj else 0)
    assert bad == n_bad
    # split calls: hash, gather, gate_fuse on the same inputs
    n_tok = batch * seqlen
    idx = torch.empty((n_tok, wl.n_tables), dtype=torch.int32, device="cuda")
    dl.plan.engram_hash(dev_i32(toks), dl.comp_map, idx, prev_ctx=dev_i32(prev))
    emb = torch.empty((n_tok, wl.emb_dim), dtype=torch.bfloat16, device="cuda")
    dl.plan.engram_gather(idx, dl.tables, emb)
    out2 = torch.empty_like(dl.h)
    state2 = to_device(state0, torch.float32, "cuda")
    dl.plan.engram_gate_fuse(emb, dl.h, dl.weights, out2, dl.plan.workspace(batch, seqlen), batch, seqlen,
                             conv_state=state2)
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy(), out2.view(torch.int16).cpu().numpy())
    assert np.array_equal(state.cpu().numpy(), state2.cpu().numpy())
    ref_idx, _, new_ctx = oracle_indices(wl, dl.li, toks, dl.comp_map_host, prev_ctx=prev)
    assert np.array_equal(idx.cpu().numpy().view(np.uint32), ref_idx)
    assert np.array_equal(ctx.cpu().numpy(), new_ctx)
    L = oracle_layer(wl, dl.li, ref_idx, batch, seqlen, conv_state=state0)
    ref, ref_alpha, _ = L.forward_all()
    assert_within(host(out), ref, "bf16", "short chunks, retrieval in projection")
    assert np.abs(host(alpha) - ref_alpha).max() <= alpha_tol("bf16")


@pytest.mark.parametrize("br,batch,seqlen,heads,head_dim,mode,flags,sdt,with_ctx", [
    (1, 3, 300, 2, 32, oracle.CONV_LINEAR, 0, "f32", True),       # two token tiles, seam rows
    (4, 2, 257, 4, 32, oracle.CONV_SILU_SKIP, 0, "bf16", True),   # four branches, ragged second tile
    (2, 1, 600, 8, 16, oracle.CONV_LINEAR, oracle.OUT_DELTA, "f32", False),  # 16 tables of d_e = 16
    (3, 5, 40, 2, 64, oracle.CONV_SILU_SKIP, oracle.OUT_DELTA, "f32", True),
])
def test_prefill_retrieval_in_projection_bitwise(B, br, batch, seqlen, heads, head_dim, mode, flags, sdt,
                                                 with_ctx):
    """Chunks on the prefill route (W_v launch separate) with retrieval
    inside the W_k and W_v launches: out, gates, carried context, new conv
    state and the out-of-range count equal the separate-retrieval route's
    bit for bit; out against the oracle within the bf16 bound."""
    say("prefill, retrieval in projection", br, batch, seqlen, heads, head_dim, mode, flags, sdt, with_ctx)
    wl = dataclasses.replace(small_wl(n_branches=br, batch=batch, seqlen=seqlen, heads=heads, head_dim=head_dim),
                             decode=with_ctx, state_dtype=sdt)
    dl = make_device_layer(wl, conv_mode=mode)
    toks = W.make_tokens(wl)
    toks[0, 0] = -5
    toks[-1, seqlen // 2] = wl.vocab + 3
    n_bad = int(((toks < 0) | (toks >= wl.vocab)).sum())
    runs = []
    for f in (0, B.RETRIEVE_IN_PROJECTION):
        ctx = dev_i32(dl.li.prev_ctx) if with_ctx else None
        st = to_device(dl.li.conv_state, dl.plan.state_torch_dtype, "cuda") if with_ctx else None
        out, alpha, bad = forward(dl, toks, prev_ctx=ctx, conv_state=st, flags=flags | f)
        runs.append((out, alpha, bad, ctx, st))
    (o1, a1, b1, c1, s1), (o2, a2, b2, c2, s2) = runs
    assert b1 == b2 == n_bad
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(a1, a2)
    idx, _, new_ctx = oracle_indices(wl, dl.li, toks, dl.comp_map_host,
                                     prev_ctx=dl.li.prev_ctx if with_ctx else None)
    if with_ctx:
        assert torch.equal(c1, c2)
        assert np.array_equal(c2.cpu().numpy(), new_ctx)
        assert torch.equal(s1.view(torch.int16) if sdt == "bf16" else s1, s2.view(torch.int16) if sdt == "bf16" else s2)
    L = oracle_layer(wl, dl.li, idx, batch, seqlen, conv_mode=mode, flags=flags,
                     conv_state=dl.li.conv_state if with_ctx else None)
    ref, ref_alpha, _ = L.forward_all()
    assert_within(host(o2), ref, "bf16", "prefill, retrieval in projection")
    assert np.abs(host(a2) - ref_alpha).max() <= alpha_tol("bf16")
    del dl
    torch.cuda.empty_cache()


def test_prefill_retrieval_in_projection_profile(B):
    """With the flag a prefill chunk launches no retrieval kernel: the W_k
    launch, the gate, the W_v launch, the seam rows and the context update."""
    wl = dataclasses.replace(small_wl(n_branches=2, batch=2, seqlen=300), decode=True)
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    ctx = dev_i32(dl.li.prev_ctx)
    dl.plan.engram_profile_begin(64)
    forward(dl, toks, prev_ctx=ctx, flags=B.RETRIEVE_IN_PROJECTION)
    torch.cuda.synchronize()
    prof = dl.plan.engram_profile_end()
    for k, n in (("hash", 0), ("gather", 0), ("gemm", 1), ("gate", 1), ("gemm_v", 1), ("seam", 1), ("aux", 1)):
        assert prof[k]["launches"] == n, (k, prof)


def test_retrieval_in_projection_profile(B):
    """With the flag, a decode step launches no retrieval kernel."""
    wl = small_wl(n_branches=2, batch=64, seqlen=1)
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    dl.plan.engram_profile_begin(64)
    forward(dl, toks, flags=B.RETRIEVE_IN_PROJECTION)
    forward(dl, toks)
    torch.cuda.synchronize()
    prof = dl.plan.engram_profile_end()
    for k, n in (("hash", 0), ("gather", 1), ("gemm", 2), ("fuse", 2)):
        assert prof[k]["launches"] == n, (k, prof)

