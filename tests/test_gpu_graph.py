"""The forward path captured into HIP graphs and replayed, against the same
calls made eagerly: every replay (with new token ids and hidden states
copied into the captured buffers between replays, by eager work on the
device) must equal the eager result bit for bit, outputs, gates, carried
context and conv state.  The library's launches hold no memset nodes and
allocate nothing, so one capture serves every later step."""

import dataclasses
import sys

import numpy as np
import pytest
import torch

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


def layer_wl(n_branches, batch, seqlen, state_dtype):
    return dataclasses.replace(W.workload("small"), name="graph_custom", index=70 + n_branches, batch=batch,
                               seqlen=seqlen, d_model=256, heads=2, head_dim=32, table_target=10007,
                               same_prime=False, n_branches=n_branches, conv_kernel=4, dtype="bf16",
                               decode=True, state_dtype=state_dtype, layers=(2, 6))


def carried(dl):
    return dev_i32(dl.li.prev_ctx), to_device(dl.li.conv_state, dl.plan.state_torch_dtype, "cuda")


@pytest.mark.parametrize("br,batch,seqlen,sdt", [(2, 3, 300, "f32"), (4, 16, 1, "bf16")])
def test_forward_graph_replays_equal_eager_calls(B, br, batch, seqlen, sdt):
    say("graph replay, one layer", br, batch, seqlen, sdt)
    wl = layer_wl(br, batch, seqlen, sdt)
    dl = make_device_layer(wl)
    n_tok = batch * seqlen
    toks = dev_i32(W.make_tokens(wl))
    h = dl.h.clone()
    ctx_g, st_g = carried(dl)
    out_g = torch.empty_like(h)
    alpha_g = torch.empty((br, n_tok), dtype=torch.float32, device="cuda")
    ws_g = dl.plan.workspace(batch, seqlen)
    ctx_e, st_e = carried(dl)
    out_e = torch.empty_like(h)
    alpha_e = torch.empty_like(alpha_g)
    ws_e = dl.plan.workspace(batch, seqlen)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        dl.plan.engram_forward(toks, dl.comp_map, dl.tables, h, dl.weights, out_g, ws_g, prev_ctx=ctx_g,
                               conv_state=st_g, alpha=alpha_g)
    for i in range(3):
        new_toks = dev_i32(W.make_tokens(wl, seed=wl.seed(2) + 31 * i))
        toks.copy_(new_toks)
        h.copy_(torch.randn(h.shape, generator=torch.Generator().manual_seed(i)).to(h.dtype).cuda())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        dl.plan.engram_forward(toks, dl.comp_map, dl.tables, h, dl.weights, out_e, ws_e, prev_ctx=ctx_e,
                               conv_state=st_e, alpha=alpha_e)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out_g), bits(out_e)), i
        assert np.array_equal(bits(alpha_g), bits(alpha_e)), i
        assert np.array_equal(ctx_g.cpu().numpy(), ctx_e.cpu().numpy()), i
        assert np.array_equal(bits(st_g), bits(st_e)), i
    del g, dl
    torch.cuda.empty_cache()


def test_two_layer_step_with_side_stream_retrieval_as_a_graph(B):
    """A decode step of two layers, layer 2 retrieved on a second stream
    forked from and joined into the capture, replayed three times against
    engram_forward of both layers one after the other."""
    say("graph replay, two layers with side-stream retrieval")
    wl = layer_wl(4, 24, 1, "bf16")
    dls = [make_device_layer(wl, layer_slot=s) for s in (0, 1)]
    toks = dev_i32(W.make_tokens(wl))
    got = [carried(dl) for dl in dls]
    ref = [carried(dl) for dl in dls]
    outs_g = [torch.empty_like(dl.h) for dl in dls]
    outs_e = [torch.empty_like(dl.h) for dl in dls]
    ws_g = [dl.plan.workspace(wl.batch, wl.seqlen) for dl in dls]
    ws_e = [dl.plan.workspace(wl.batch, wl.seqlen) for dl in dls]
    emb = torch.empty((wl.n_tokens, wl.emb_dim), dtype=dls[1].plan.torch_dtype, device="cuda")
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        dls[1].plan.engram_retrieve(toks, dls[1].comp_map, dls[1].tables, emb, prev_ctx=got[1][0], stream=side)
        ready.record(side)
        dls[0].plan.engram_forward(toks, dls[0].comp_map, dls[0].tables, dls[0].h, dls[0].weights, outs_g[0],
                                   ws_g[0], prev_ctx=got[0][0], conv_state=got[0][1])
        main.wait_event(ready)
        dls[1].plan.engram_gate_fuse(emb, dls[1].h, dls[1].weights, outs_g[1], ws_g[1], wl.batch, wl.seqlen,
                                     conv_state=got[1][1])
    for i in range(3):
        toks.copy_(dev_i32(W.make_tokens(wl, seed=wl.seed(2) + 17 * i)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l, dl in enumerate(dls):
            dl.plan.engram_forward(toks, dl.comp_map, dl.tables, dl.h, dl.weights, outs_e[l], ws_e[l],
                                   prev_ctx=ref[l][0], conv_state=ref[l][1])
        torch.cuda.synchronize()
        for l in range(2):
            assert np.array_equal(bits(outs_g[l]), bits(outs_e[l])), (i, l)
            assert np.array_equal(got[l][0].cpu().numpy(), ref[l][0].cpu().numpy()), (i, l)
            assert np.array_equal(bits(got[l][1]), bits(ref[l][1])), (i, l)
    del g, dls
    torch.cuda.empty_cache()
