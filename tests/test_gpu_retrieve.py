"""engram_retrieve (retrieval on its own, for callers that fetch a later
layer's rows ahead of that layer) against engram_forward.

Retrieval followed by engram_gate_fuse must reproduce engram_forward bit for
bit (output, gates, carried context and conv state, out-of-range count), on
one stream and with E handed from a second stream by an event; the retrieved
E must equal the oracle's rows bit for bit.  Expected rows come only from
``oracle/`` on the same seeded inputs.
"""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from engram_harness import oracle_dtype, oracle_indices
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


def bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def layer_wl(n_branches, batch, seqlen, dtype="bf16", state_dtype="f32", decode=True, d_model=256, heads=2,
             head_dim=32):
    base = W.workload("small")
    return dataclasses.replace(base, name="retrieve_custom", index=60 + n_branches, batch=batch, seqlen=seqlen,
                               d_model=d_model, heads=heads, head_dim=head_dim, table_target=10007,
                               same_prime=False, n_branches=n_branches, conv_kernel=4, dtype=dtype,
                               decode=decode, state_dtype=state_dtype, layers=(2, 6))


def carried(dl):
    """Device copies of the layer's carried context and conv state (or None)."""
    if dl.li.prev_ctx is None:
        return None, None
    return dev_i32(dl.li.prev_ctx), to_device(dl.li.conv_state, dl.plan.state_torch_dtype, "cuda")


def run_forward(dl, toks, ctx, state, out):
    wl = dl.wl
    batch, seqlen = toks.shape
    alpha = torch.full((wl.n_branches, batch * seqlen), -1.0, dtype=torch.float32, device="cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = dl.plan.workspace(batch, seqlen)
    dl.plan.engram_forward(toks, dl.comp_map, dl.tables, dl.h, dl.weights, out, ws, prev_ctx=ctx,
                           conv_state=state, alpha=alpha, bad_tokens=bad)
    return alpha, bad


def run_split(dl, toks, ctx, state, out, emb, ws, side=None):
    """engram_retrieve (on `side` if given, handed over by an event) then
    engram_gate_fuse on the current stream."""
    wl = dl.wl
    batch, seqlen = toks.shape
    alpha = torch.full((wl.n_branches, batch * seqlen), -1.0, dtype=torch.float32, device="cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    main = torch.cuda.current_stream()
    if side is None:
        dl.plan.engram_retrieve(toks, dl.comp_map, dl.tables, emb, prev_ctx=ctx, bad_tokens=bad)
    else:
        side.wait_stream(main)
        dl.plan.engram_retrieve(toks, dl.comp_map, dl.tables, emb, prev_ctx=ctx, bad_tokens=bad, stream=side)
        ev = torch.cuda.Event()
        ev.record(side)
        main.wait_event(ev)
    dl.plan.engram_gate_fuse(emb, dl.h, dl.weights, out, ws, batch, seqlen, conv_state=state, alpha=alpha)
    return alpha, bad


CASES = [
    # branches, batch, seqlen, dtype, state dtype, carried context and state
    (4, 9, 1, "bf16", "bf16", True),     # decode: one token per sequence
    (2, 3, 300, "bf16", "f32", True),    # chunk across two 256-token tiles
    (1, 1, 2, "bf16", "f32", True),      # two tokens: the new context is both of them
    (3, 2, 40, "bf16", "f32", False),    # sequence starts (no carried context)
    (1, 2, 77, "f32", "f32", True),      # fp32 plan
]


@pytest.mark.parametrize("br,batch,seqlen,dt,sdt,with_ctx", CASES)
def test_retrieve_then_gate_fuse_equals_forward(B, br, batch, seqlen, dt, sdt, with_ctx):
    say("retrieve + gate_fuse", br, batch, seqlen, dt, sdt, with_ctx)
    wl = layer_wl(br, batch, seqlen, dtype=dt, state_dtype=sdt, decode=with_ctx)
    dl = make_device_layer(wl)
    toks_h = W.make_tokens(wl)
    toks_h[0, 0] = -5
    toks_h[-1, -1] = wl.vocab + 7
    toks = dev_i32(toks_h)
    n_tok = batch * seqlen

    ctx_a, st_a = carried(dl)
    out_a = torch.empty_like(dl.h)
    alpha_a, bad_a = run_forward(dl, toks, ctx_a, st_a, out_a)

    ctx_b, st_b = carried(dl)
    out_b = torch.empty_like(dl.h)
    emb = torch.empty((n_tok, wl.emb_dim), dtype=dl.plan.torch_dtype, device="cuda")
    ws = dl.plan.workspace(batch, seqlen)
    alpha_b, bad_b = run_split(dl, toks, ctx_b, st_b, out_b, emb, ws)
    torch.cuda.synchronize()

    assert np.array_equal(bits(out_a), bits(out_b))
    assert np.array_equal(bits(alpha_a), bits(alpha_b))
    assert int(bad_a.item()) == int(bad_b.item()) == 2
    if with_ctx:
        assert np.array_equal(ctx_a.cpu().numpy(), ctx_b.cpu().numpy())
        assert np.array_equal(bits(st_a), bits(st_b))
        # the context was rolled: the last two compressed ids of the extended sequence
        comp = dl.comp_map_host
        pad = wl.vocab_comp
        c = lambda x: comp[x] if 0 <= x < wl.vocab else pad
        want = np.empty((batch, 2), np.int32)
        for b in range(batch):
            want[b, 1] = c(int(toks_h[b, -1]))
            want[b, 0] = c(int(toks_h[b, -2])) if seqlen >= 2 else dl.li.prev_ctx[b, 1]
        assert np.array_equal(ctx_b.cpu().numpy(), want)

    # the retrieved rows against the oracle's, bit for bit
    idx_ref, _, _ = oracle_indices(wl, dl.li, toks_h, dl.comp_map_host,
                                   prev_ctx=dl.li.prev_ctx if with_ctx else None)
    emb_ref = oracle.gather_synth(idx_ref, wl.head_dim, dl.li.table_seed, oracle_dtype(wl))
    got = bits(emb)
    assert np.array_equal(got, emb_ref.view(got.dtype))
    del dl
    torch.cuda.empty_cache()


def test_later_layer_retrieved_on_a_side_stream(B):
    """Three decode steps of two layers: layer 2's rows retrieved on a second
    stream while layer 1 runs, E handed over by an event, against both layers
    run one after the other by engram_forward; outputs, contexts and states
    equal bit for bit after every step."""
    say("two layers, side-stream retrieval")
    wl = layer_wl(4, 24, 1, state_dtype="bf16")
    dls = [make_device_layer(wl, layer_slot=s) for s in (0, 1)]
    steps = [dev_i32(W.make_tokens(wl, seed=wl.seed(2) + 17 * i)) for i in range(3)]
    ref = [carried(dl) for dl in dls]
    got = [carried(dl) for dl in dls]
    outs_ref = [torch.empty_like(dl.h) for dl in dls]
    outs_got = [torch.empty_like(dl.h) for dl in dls]
    emb = torch.empty((wl.n_tokens, wl.emb_dim), dtype=dls[1].plan.torch_dtype, device="cuda")
    ws = [dl.plan.workspace(wl.batch, wl.seqlen) for dl in dls]
    side = torch.cuda.Stream()
    for i, toks in enumerate(steps):
        for l, dl in enumerate(dls):
            run_forward(dl, toks, ref[l][0], ref[l][1], outs_ref[l])
        # layer 2 retrieves on the side stream, then layer 1 runs on the main one
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        dls[1].plan.engram_retrieve(toks, dls[1].comp_map, dls[1].tables, emb, prev_ctx=got[1][0], stream=side)
        ready = torch.cuda.Event()
        ready.record(side)
        run_forward(dls[0], toks, got[0][0], got[0][1], outs_got[0])
        main.wait_event(ready)
        dls[1].plan.engram_gate_fuse(emb, dls[1].h, dls[1].weights, outs_got[1], ws[1], wl.batch, wl.seqlen,
                                     conv_state=got[1][1])
        torch.cuda.synchronize()
        for l in range(2):
            assert np.array_equal(bits(outs_ref[l]), bits(outs_got[l])), (i, l)
            assert np.array_equal(ref[l][0].cpu().numpy(), got[l][0].cpu().numpy()), (i, l)
            assert np.array_equal(bits(ref[l][1]), bits(got[l][1])), (i, l)
    del dls
    torch.cuda.empty_cache()
