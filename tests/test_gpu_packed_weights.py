"""Packed weight matrices (engram_pack_weight, ENGRAM_WEIGHTS_PACKED) through the C ABI.

engram_pack_weight rewrites a [d][D_e] bf16 matrix into the projections'
operand blocks; the forward given the packed W_k and W_v and the flag must
give the bits of the forward on the [d][D_e] matrices, on every route that
reads weights: 256 x 256 and 128 x 128 W_k tiles with the fused W_v launch,
the one-launch W_k + W_v projection of short chunks (decode) with its fusion
kernel, retrieval inside the projection launches, the split retrieval and
fusion calls and the no-allocation entry point.  One small shape is also
checked against the oracle at every position.
"""

import dataclasses
import sys

import numpy as np
import pytest
import torch

from engram_harness import alpha_tol, assert_within, oracle_indices, oracle_layer
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
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def small_wl(n_branches=1, batch=3, seqlen=77, d_model=256, heads=2, head_dim=32, state_dtype="f32"):
    return dataclasses.replace(W.workload("small"), name="packed_w", index=60 + n_branches, batch=batch,
                               seqlen=seqlen, d_model=d_model, heads=heads, head_dim=head_dim,
                               table_target=10007, same_prime=False, n_branches=n_branches,
                               state_dtype=state_dtype)


def swz(r):
    return ((r >> 1) ^ (r >> 2)) & 3


def packed_reference(w: np.ndarray) -> np.ndarray:
    """The layout engram_pack_weight documents, written out with numpy: block
    (n/16, k/32) at 1 KB each, row n%16 of it 64 bytes, piece q of the row at
    position q ^ swz(n%16)."""
    d, K = w.shape
    src = w.reshape(d // 16, 16, K // 32, 4, 8)
    out = np.zeros((d // 16, K // 32, 16, 4, 8), w.dtype)
    for r in range(16):
        for q in range(4):
            out[:, :, r, q ^ swz(r), :] = src[:, r, :, q, :]
    return out.reshape(d, K)


def test_pack_weight_layout(B):
    say("pack layout")
    wl = small_wl(d_model=512, heads=4, head_dim=48)  # D_e = 384
    dl = make_device_layer(wl)
    for w in list(dl.weights.w_k) + [dl.weights.w_v]:
        packed = torch.empty_like(w)
        dl.plan.engram_pack_weight(w, packed)
        torch.cuda.synchronize()
        got = packed.view(torch.int16).cpu().numpy()
        assert np.array_equal(got, packed_reference(w.view(torch.int16).cpu().numpy()))


def _run(dl, toks, weights, flags, ctx0=None, st0=None, route="forward"):
    wl = dl.wl
    batch, seqlen = toks.shape
    n_tok = batch * seqlen
    out = torch.empty_like(dl.h)
    alpha = torch.full((wl.n_branches, n_tok), -1.0, dtype=torch.float32, device="cuda")
    ctx = None if ctx0 is None else dev_i32(ctx0)
    st = None if st0 is None else to_device(st0, dl.plan.state_torch_dtype, "cuda")
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    if route == "split":
        emb = torch.empty((n_tok, wl.emb_dim), dtype=dl.h.dtype, device="cuda")
        dl.plan.engram_retrieve(dev_i32(toks), dl.comp_map, dl.tables, emb, prev_ctx=ctx, bad_tokens=bad)
        ws = dl.plan.workspace(batch, seqlen)
        dl.plan.engram_gate_fuse(emb, dl.h, weights, out, ws, batch, seqlen, conv_state=st, alpha=alpha,
                                 flags=flags)
    elif route == "noalloc":
        dl.plan.engram_forward_noalloc(dev_i32(toks), dl.comp_map, dl.tables, dl.h, weights, out, prev_ctx=ctx,
                                       conv_state=st, alpha=alpha, flags=flags, bad_tokens=bad)
    else:
        ws = dl.plan.workspace(batch, seqlen)
        dl.plan.engram_forward(dev_i32(toks), dl.comp_map, dl.tables, dl.h, weights, out, ws, prev_ctx=ctx,
                               conv_state=st, alpha=alpha, flags=flags, bad_tokens=bad)
    torch.cuda.synchronize()
    return out, alpha, st, ctx, int(bad.item())


CASES = {
    # name: (workload kwargs, route, extra flags, with carried context and state)
    "prefill 256x256 W_k tiles": (dict(n_branches=2, batch=2, seqlen=8200, d_model=512, heads=4, head_dim=64),
                                  "forward", 0, True),
    "prefill 128x128 W_k tiles": (dict(n_branches=1, batch=3, seqlen=300), "forward", 0, True),
    "prefill four branches": (dict(n_branches=4, batch=2, seqlen=130), "forward", 0, False),
    "decode, one launch for W_k and W_v": (dict(n_branches=4, batch=300, seqlen=1, state_dtype="bf16"),
                                           "forward", 0, True),
    "decode, retrieval in projection": (dict(n_branches=4, batch=300, seqlen=1, state_dtype="bf16"),
                                        "forward", "rip", True),
    "prefill, retrieval in projection": (dict(n_branches=1, batch=1, seqlen=70000), "forward", "rip", False),
    "split retrieval and fusion": (dict(n_branches=2, batch=2, seqlen=77), "split", 0, True),
    "no-allocation entry point": (dict(n_branches=1, batch=3, seqlen=300), "noalloc", 0, True),
}


@pytest.mark.parametrize("case", list(CASES))
def test_packed_weights_same_bits(B, case):
    kw, route, extra, carried = CASES[case]
    say("packed weights:", case)
    wl = small_wl(**kw)
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    batch, seqlen = toks.shape
    flags = B.RETRIEVE_IN_PROJECTION if extra == "rip" else 0
    ctx0 = st0 = None
    if carried:
        rng = np.random.default_rng(31)
        ctx0 = rng.integers(0, wl.vocab_comp + 1, (batch, 2)).astype(np.int32)
        st0 = (0.05 * rng.standard_normal((wl.n_branches, batch, wl.conv_kernel - 1, wl.d_model))).astype(np.float32)
    ref = _run(dl, toks, dl.weights, flags, ctx0, st0, route)
    packed = dl.plan.packed_weights(dl.weights)
    got = _run(dl, toks, packed, flags | B.WEIGHTS_PACKED, ctx0, st0, route)
    assert ref[4] == 0 and got[4] == 0
    assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16)), case + ": out"
    assert torch.equal(got[1], ref[1]), case + ": alpha"
    if carried:
        assert torch.equal(got[2].view(torch.int16) if got[2].dtype == torch.bfloat16 else got[2],
                           ref[2].view(torch.int16) if ref[2].dtype == torch.bfloat16 else ref[2]), case + ": state"
        assert torch.equal(got[3], ref[3]), case + ": context"
    del dl
    torch.cuda.empty_cache()


def test_packed_weights_against_oracle(B):
    """Every position of a small two-branch layer, packed weights, against the oracle."""
    say("packed weights vs oracle")
    wl = small_wl(n_branches=2, batch=3, seqlen=130)
    dl = make_device_layer(wl)
    toks = W.make_tokens(wl)
    batch, seqlen = toks.shape
    out, alpha, _, _, bad = _run(dl, toks, dl.plan.packed_weights(dl.weights), B.WEIGHTS_PACKED)
    assert bad == 0
    idx, _, _ = oracle_indices(wl, dl.li, toks, dl.comp_map_host)
    ref, ref_alpha, _ = oracle_layer(wl, dl.li, idx, batch, seqlen).forward_all()
    assert_within(host(out), ref, "bf16", "packed weights out")
    assert np.abs(host(alpha) - ref_alpha).max() <= alpha_tol("bf16")
