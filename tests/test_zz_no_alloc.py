"""engram_forward_noalloc (through the C ABI) against engram_forward.

The no-allocation entry point runs engram_forward's kernels on the library's
per-GPU scratch array instead of a caller workspace, so every output must
equal engram_forward's bit for bit: out, the gates, the carried conv state,
the carried context and the out-of-range count.  Each case makes two calls in
a row, the second with fewer tokens, so a call that read what the previous
call left in the array would show.  A call whose workspace would exceed the
array is rejected before anything is launched.
"""

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


def _run(B, dl, toks, ctx, state, h, noalloc):
    """One forward call; returns (out, alpha, state, ctx, bad) as host arrays."""
    Br = dl.wl.n_branches
    batch, seqlen = toks.shape
    out = torch.full_like(h, 7.0)
    alpha = torch.full((Br, batch * seqlen), -1.0, dtype=torch.float32, device="cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    ctx_d = None if ctx is None else dev_i32(ctx)
    st_d = None if state is None else to_device(state, dl.plan.state_torch_dtype, "cuda")
    tok_d = dev_i32(toks)
    if noalloc:
        dl.plan.engram_forward_noalloc(tok_d, dl.comp_map, dl.tables, h, dl.weights, out, prev_ctx=ctx_d,
                                       conv_state=st_d, alpha=alpha, bad_tokens=bad)
    else:
        ws = dl.plan.workspace(batch, seqlen)
        dl.plan.engram_forward(tok_d, dl.comp_map, dl.tables, h, dl.weights, out, ws, prev_ctx=ctx_d,
                               conv_state=st_d, alpha=alpha, bad_tokens=bad)
    torch.cuda.synchronize()
    bits = out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32)
    return (bits.cpu().numpy(), alpha.view(torch.int32).cpu().numpy(),
            None if st_d is None else st_d.view(torch.int32).cpu().numpy(),
            None if ctx_d is None else ctx_d.cpu().numpy(), int(bad.item()))


def _case(B, wl, shapes, with_state, bad_ids=False):
    dl = make_device_layer(wl, batch=max(b for b, _ in shapes), seqlen=max(s for _, s in shapes))
    rng = np.random.default_rng(9)
    d, Br = wl.d_model, wl.n_branches
    tdt = dl.h.dtype
    for call, (batch, seqlen) in enumerate(shapes):
        say("noalloc", wl.name, "call", call, "batch", batch, "seqlen", seqlen)
        toks = W.make_tokens(wl, batch=batch, seqlen=seqlen, seed=wl.seed(2) + 31 * call)
        if bad_ids:
            toks[0, 0] = -3
            toks[-1, -1] = wl.vocab + 5
        h = torch.from_numpy(rng.standard_normal((Br, batch * seqlen, d)).astype(np.float32)).to(tdt).cuda()
        ctx = state = None
        if with_state:
            ctx = rng.integers(0, wl.vocab_comp + 1, (batch, 2)).astype(np.int32)
            state = rng.standard_normal((Br, batch, wl.conv_kernel - 1, d)).astype(np.float32)
            if wl.state_dtype == "bf16":
                state = W.round_to_bf16(state)
        ref = _run(B, dl, toks, ctx, state, h, noalloc=False)
        got = _run(B, dl, toks, ctx, state, h, noalloc=True)
        names = ("out", "alpha", "conv_state", "prev_ctx")
        for n, a, b in zip(names, ref[:4], got[:4]):
            if a is None:
                assert b is None
            else:
                assert np.array_equal(a, b), "%s differs on call %d" % (n, call)
        assert ref[4] == got[4] == (2 if bad_ids else 0)
    del dl
    torch.cuda.empty_cache()


def test_noalloc_prefill_bf16_two_branches(B):
    wl = dataclasses.replace(W.workload("small"), name="noalloc_prefill", index=71, d_model=512, heads=4,
                             head_dim=32, table_target=20011, n_branches=2)
    _case(B, wl, [(3, 700), (2, 77)], with_state=True, bad_ids=True)


def test_noalloc_prefill_bf16_no_state(B):
    wl = dataclasses.replace(W.workload("layer27b"), name="noalloc_layer", index=72)
    _case(B, wl, [(2, 2048), (1, 300)], with_state=False)


def test_noalloc_decode_four_branches(B):
    wl = W.workload("multibranch_decode")
    _case(B, wl, [(256, 1), (100, 1)], with_state=True)


def test_noalloc_f32(B):
    wl = W.workload("tiny")
    _case(B, wl, [(2, 128), (1, 50)], with_state=True, bad_ids=True)


def test_noalloc_rejects_calls_beyond_the_scratch(B):
    wl = W.workload("small")
    dl = make_device_layer(wl, batch=1, seqlen=8)
    batch, seqlen = 8, 4096
    assert dl.plan.engram_workspace_size(batch, seqlen) > B.NOALLOC_SCRATCH_BYTES
    toks = dev_i32(np.zeros((batch, seqlen), np.int32))
    h = torch.zeros((1, batch * seqlen, wl.d_model), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(h, 3.0)
    with pytest.raises(B.EngramError) as e:
        dl.plan.engram_forward_noalloc(toks, dl.comp_map, dl.tables, h, dl.weights, out)
    assert e.value.status == B.E_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())  # nothing was launched
