"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and its host-side validation rejects bad arguments without touching a GPU."""

import ctypes as C
import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    from hashed_gram_embedding_vocab_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from hashed_gram_embedding_vocab_amd import build
        build.build()
    binding.lib()
    return binding


def declared_symbols():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            names += re.findall(r"ENGRAM_API\s+[\w\s\*]+?\b(engram_\w+)\s*\(", text)
    return names


def test_library_exports_every_declared_symbol(B):
    names = declared_symbols()
    assert len(names) >= 11
    for n in names:
        assert hasattr(B.lib(), n), n


def _cfg(B, **kw):
    c = B.Config()
    c.vocab, c.vocab_comp, c.n_orders = 1000, 770, 2
    c.orders[0], c.orders[1] = 2, 3
    c.heads, c.head_dim = 4, 32
    for i in range(8):
        c.table_rows[i] = 10007
    c.hash_seed = 1
    c.d_model, c.n_branches, c.conv_kernel, c.conv_mode = 256, 1, 4, 0
    c.rms_eps, c.dtype = 1e-6, B.F32
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _create(B, c):
    h = C.c_void_p()
    st = B.lib().engram_plan_create(C.byref(c), C.byref(h))
    if st == 0:
        B.lib().engram_plan_destroy(h)
    return st


def test_plan_validation(B):
    assert _create(B, _cfg(B)) == B.OK
    bad = [dict(vocab_comp=1 << 21), dict(heads=0), dict(heads=17), dict(head_dim=30),
           dict(head_dim=0), dict(d_model=100), dict(n_branches=5), dict(n_branches=0),
           dict(conv_kernel=5), dict(conv_kernel=0), dict(conv_mode=7), dict(n_orders=3),
           dict(dtype=5), dict(rms_eps=-1.0)]
    for kw in bad:
        assert _create(B, _cfg(B, **kw)) == B.E_INVALID_ARG, kw
    c = _cfg(B)
    c.table_rows[3] = 0
    assert _create(B, c) == B.E_INVALID_ARG
    c = _cfg(B)
    c.orders[1] = 4
    assert _create(B, c) == B.E_INVALID_ARG
    # the carried state may be bf16 only on bf16 plans
    assert _create(B, _cfg(B, dtype=B.BF16, state_dtype=B.BF16)) == B.OK
    assert _create(B, _cfg(B, dtype=B.F32, state_dtype=B.BF16)) == B.E_INVALID_ARG
    assert _create(B, _cfg(B, dtype=B.BF16, state_dtype=7)) == B.E_INVALID_ARG
    # bf16 rows of 32 dims are 64 bytes: fine; 4 dims are 8 bytes: rejected
    assert _create(B, _cfg(B, dtype=B.BF16)) == B.OK
    assert _create(B, _cfg(B, dtype=B.BF16, head_dim=4)) == B.E_INVALID_ARG


def test_workspace_size(B):
    p = B.Plan(vocab=1000, vocab_comp=770, heads=4, head_dim=32, table_rows=[10007] * 8, hash_seed=1,
               d_model=256, dtype=B.F32)
    a = p.engram_workspace_size(2, 128)
    b = p.engram_workspace_size(2, 256)
    assert 0 < a < b and a % 256 == 0
    n_tok = 256
    # idx + E + partials + v + k + conv stage, all fp32 here
    assert a >= n_tok * 8 * 4 + n_tok * 256 * 4 + 3 * n_tok * 4 + n_tok * 256 * 4 * 2
    assert p.engram_workspace_size(0, 5) == 0
    assert p.engram_workspace_size(2, -1) == 0


def test_status_strings(B):
    for s in range(5):
        assert B.lib().engram_status_string(s)
    assert B.lib().engram_status_string(99) == b"unknown status"


def _no_gpu():
    # These calls hand the library fake device pointers that only host-side
    # validation stands between and a launch; keep them off machines with a GPU.
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run only where no GPU exists")


def test_entry_points_reject_bad_arguments_before_launching(B):
    _no_gpu()
    L = B.lib()
    p = B.Plan(vocab=1000, vocab_comp=770, heads=4, head_dim=32, table_rows=[10007] * 8, hash_seed=1,
               d_model=256, dtype=B.F32)
    h = p._h
    fake = C.c_void_p(0x10000)       # never dereferenced: validation fails first
    odd = C.c_void_p(0x10004)        # not 16-byte aligned
    assert L.engram_hash(None, fake, 1, 1, fake, None, fake, None, None) == B.E_INVALID_ARG
    assert L.engram_hash(h, None, 1, 1, fake, None, fake, None, None) == B.E_INVALID_ARG
    assert L.engram_hash(h, fake, 0, 1, fake, None, fake, None, None) == B.E_INVALID_ARG
    assert L.engram_hash(h, fake, 1, -3, fake, None, fake, None, None) == B.E_INVALID_ARG
    assert L.engram_hash(h, odd, 1, 1, fake, None, fake, None, None) == B.E_INVALID_ARG
    tabs = (C.c_void_p * 8)(*([0x10000] * 8))
    assert L.engram_gather(h, fake, 0, tabs, fake, None) == B.E_INVALID_ARG
    assert L.engram_gather(h, fake, 4, None, fake, None) == B.E_INVALID_ARG
    tabs_bad = (C.c_void_p * 8)(*([0x10000] * 7 + [0]))
    assert L.engram_gather(h, fake, 4, tabs_bad, fake, None) == B.E_INVALID_ARG
    tabs_odd = (C.c_void_p * 8)(*([0x10000] * 7 + [0x10008]))
    assert L.engram_gather(h, fake, 4, tabs_odd, fake, None) == B.E_INVALID_ARG
    w = B.WeightsC()
    w.w_k[0] = w.w_v = w.gamma_h[0] = w.gamma_k[0] = w.conv_w = 0x10000
    ws_ok = p.engram_workspace_size(1, 4)
    args = [h, fake, fake, 1, 4, C.byref(w), None, fake, None, 0, fake, ws_ok, None]
    # workspace too small, bad flags, missing weight, misaligned workspace
    a = list(args); a[11] = ws_ok - 1
    assert L.engram_gate_fuse(*a) == B.E_INVALID_ARG
    a = list(args); a[9] = 0x8
    assert L.engram_gate_fuse(*a) == B.E_INVALID_ARG
    a = list(args); a[10] = C.c_void_p(0x10010)
    assert L.engram_gate_fuse(*a) == B.E_INVALID_ARG
    w2 = B.WeightsC()
    w2.w_v = w2.gamma_h[0] = w2.gamma_k[0] = w2.conv_w = 0x10000
    a = list(args); a[5] = C.byref(w2)
    assert L.engram_gate_fuse(*a) == B.E_INVALID_ARG
    assert L.engram_forward(h, fake, 1, 4, fake, None, tabs, fake, C.byref(w), None, fake, None, 0,
                            None, 0, None, None) == B.E_INVALID_ARG
    assert L.engram_synth_fill_table(7, 1, 0, 10, 32, fake, None) == B.E_INVALID_ARG
    assert L.engram_synth_fill_table(0, 1, 0, 10, 30, fake, None) == B.E_INVALID_ARG
    assert L.engram_synth_fill_table(0, 1, 0, 10, 32, odd, None) == B.E_INVALID_ARG


def test_bf16_shape_support_is_checked(B):
    _no_gpu()
    L = B.lib()
    # d = 200 is a multiple of 8 but not of 128: the bf16 MFMA path reports UNSUPPORTED
    p = B.Plan(vocab=1000, vocab_comp=770, heads=4, head_dim=32, table_rows=[10007] * 8, hash_seed=1,
               d_model=200, dtype=B.BF16)
    fake = C.c_void_p(0x10000)
    w = B.WeightsC()
    w.w_k[0] = w.w_v = w.gamma_h[0] = w.gamma_k[0] = w.conv_w = 0x10000
    ws = p.engram_workspace_size(1, 4)
    assert L.engram_gate_fuse(p._h, fake, fake, 1, 4, C.byref(w), None, fake, None, 0,
                              C.c_void_p(0x100000), ws, None) == B.E_UNSUPPORTED


def test_pack_weight_argument_checks(B):
    """engram_pack_weight and the packed-weights flag are validated before
    anything is launched: null, misaligned or overlapping buffers, fp32 plans
    and unsupported shapes; the fp32 forward and the backward refuse the flag."""
    _no_gpu()
    L = B.lib()
    src, dst = C.c_void_p(0x1000000), C.c_void_p(0x20000000)
    p = B.Plan(vocab=1000, vocab_comp=770, heads=4, head_dim=32, table_rows=[10007] * 8, hash_seed=1,
               d_model=256, dtype=B.BF16)  # D_e = 256: a [256][256] matrix, 128 KB
    assert L.engram_pack_weight(None, src, dst, None) == B.E_INVALID_ARG
    assert L.engram_pack_weight(p._h, None, dst, None) == B.E_INVALID_ARG
    assert L.engram_pack_weight(p._h, src, None, None) == B.E_INVALID_ARG
    assert L.engram_pack_weight(p._h, C.c_void_p(0x1000004), dst, None) == B.E_INVALID_ARG
    assert L.engram_pack_weight(p._h, src, C.c_void_p(0x20000008), None) == B.E_INVALID_ARG
    for start in (0x1000000, 0x1000000 + 1024, 0x1000000 + 128 * 1024 - 16, 0x1000000 - 128 * 1024 + 16):
        assert L.engram_pack_weight(p._h, src, C.c_void_p(start), None) == B.E_INVALID_ARG, hex(start)
    p32 = B.Plan(vocab=1000, vocab_comp=770, heads=4, head_dim=32, table_rows=[10007] * 8, hash_seed=1,
                 d_model=256, dtype=B.F32)
    assert L.engram_pack_weight(p32._h, src, dst, None) == B.E_UNSUPPORTED
    p200 = B.Plan(vocab=1000, vocab_comp=770, heads=4, head_dim=32, table_rows=[10007] * 8, hash_seed=1,
                  d_model=200, dtype=B.BF16)
    assert L.engram_pack_weight(p200._h, src, dst, None) == B.E_UNSUPPORTED
    # the fp32 projections read [d][D_e] matrices only
    fake = C.c_void_p(0x10000)
    w = B.WeightsC()
    w.w_k[0] = w.w_v = w.gamma_h[0] = w.gamma_k[0] = w.conv_w = 0x10000
    ws = p32.engram_workspace_size(1, 4)
    assert L.engram_gate_fuse(p32._h, fake, fake, 1, 4, C.byref(w), None, fake, None, B.WEIGHTS_PACKED,
                              C.c_void_p(0x100000), ws, None) == B.E_UNSUPPORTED
    # the backward reads W K-major from the [d][D_e] matrices
    g = B.GradsC(*([C.c_void_p(0x10000)] * 7))
    pb = B.Plan(vocab=1000, vocab_comp=770, heads=2, head_dim=32, table_rows=[10007] * 4, hash_seed=1,
                d_model=256, dtype=B.BF16)
    tabs = (C.c_void_p * 4)(*([0x10000] * 4))
    wsb = pb.engram_backward_workspace_size(2, 8)
    assert L.engram_backward(pb._h, fake, tabs, fake, C.byref(w), fake, 2, 8, B.WEIGHTS_PACKED, fake,
                             C.byref(g), C.c_void_p(0x100000), wsb, None) == B.E_INVALID_ARG


def test_backward_argument_checks(B):
    _no_gpu()
    L = B.lib()
    fake = C.c_void_p(0x10000)
    w = B.WeightsC()
    w.w_k[0] = w.w_v = w.gamma_h[0] = w.gamma_k[0] = w.conv_w = 0x10000
    g = B.GradsC(*([C.c_void_p(0x10000)] * 7))
    tabs = (C.c_void_p * 4)(*([0x10000] * 4))
    # the fp32 path has no backward: no workspace size, UNSUPPORTED
    p32 = B.Plan(vocab=1000, vocab_comp=770, heads=2, head_dim=32, table_rows=[10007] * 4, hash_seed=1,
                 d_model=256, dtype=B.F32)
    assert p32.engram_backward_workspace_size(2, 8) == 0
    assert L.engram_backward(p32._h, fake, tabs, fake, C.byref(w), fake, 2, 8, 0, fake, C.byref(g),
                             C.c_void_p(0x100000), 1 << 30, None) == B.E_UNSUPPORTED
    p = B.Plan(vocab=1000, vocab_comp=770, heads=2, head_dim=32, table_rows=[10007] * 4, hash_seed=1,
               d_model=256, dtype=B.BF16)
    ws = p.engram_backward_workspace_size(2, 8)
    assert ws > 0
    assert p.engram_backward_workspace_size(0, 8) == 0
    args = [p._h, fake, tabs, fake, C.byref(w), fake, 2, 8, 0, fake, C.byref(g), C.c_void_p(0x100000), ws, None]
    for i, bad in [(1, None), (3, None), (5, None), (9, None), (10, None), (11, None),
                   (12, ws - 1), (8, 0x4), (5, C.c_void_p(0x10004)), (11, C.c_void_p(0x100010))]:
        a = list(args)
        a[i] = bad
        assert L.engram_backward(*a) == B.E_INVALID_ARG, (i, bad)
    g2 = B.GradsC(*([C.c_void_p(0x10000)] * 6 + [None]))
    a = list(args); a[10] = C.byref(g2)
    assert L.engram_backward(*a) == B.E_INVALID_ARG
    tabs_bad = (C.c_void_p * 4)(*([0x10000] * 3 + [0]))
    a = list(args); a[2] = tabs_bad
    assert L.engram_backward(*a) == B.E_INVALID_ARG


def test_row_cache_argument_checks(B):
    """engram_cache_build / engram_gather_cached reject bad caches before any launch."""
    _no_gpu()
    L = B.lib()
    fake = C.c_void_p(0x10000)
    tabs = (C.c_void_p * 4)(*([0x10000] * 4))
    p = B.Plan(vocab=1000, vocab_comp=770, heads=2, head_dim=32, table_rows=[10007] * 4, hash_seed=1,
               d_model=256, dtype=B.BF16)
    for keys, rows, cap, n_hot in [(0x10000, 0x20000, 0, 1),       # no slots
                                   (0x10000, 0x20000, 6, 1),       # not a power of two
                                   (0x10000, 0x20000, 4, 3),       # load factor above 1/2
                                   (0x10004, 0x20000, 8, 1),       # keys misaligned
                                   (0x10000, None, 8, 1),          # no rows
                                   (0x10000, 0x20000, 1 << 29, 1)]:  # too many slots
        c = B.RowCacheC(keys, rows, cap)
        assert L.engram_cache_build(p._h, fake, n_hot, tabs, C.byref(c), None) == B.E_INVALID_ARG, (keys, rows, cap)
    c = B.RowCacheC(0x10000, 0x20000, 8)
    assert L.engram_cache_build(p._h, None, 1, tabs, C.byref(c), None) == B.E_INVALID_ARG  # no hot rows
    assert L.engram_cache_build(p._h, fake, -1, tabs, C.byref(c), None) == B.E_INVALID_ARG
    assert L.engram_cache_build(p._h, fake, 1, tabs, None, None) == B.E_INVALID_ARG
    bad_tabs = (C.c_void_p * 4)(*([0x10000] * 3 + [0x10008]))
    assert L.engram_cache_build(p._h, fake, 1, bad_tabs, C.byref(c), None) == B.E_INVALID_ARG
    bad = B.RowCacheC(0x10000, 0x20000, 6)
    assert L.engram_gather_cached(p._h, fake, 10, tabs, C.byref(bad), fake, 0, None) == B.E_INVALID_ARG
    assert L.engram_gather_cached(p._h, None, 10, tabs, C.byref(c), fake, 0, None) == B.E_INVALID_ARG
    assert L.engram_gather_cached(p._h, fake, 0, tabs, C.byref(c), fake, 0, None) == B.E_INVALID_ARG
    assert L.engram_gather_cached(p._h, fake, 10, tabs, C.byref(c), fake, -1, None) == B.E_INVALID_ARG
    assert L.engram_host_alloc(1, None) == B.E_INVALID_ARG
    assert L.engram_host_free(None) == B.OK


def test_prefetcher_argument_checks(B):
    """The host-gather prefetcher rejects bad arguments before touching the device."""
    _no_gpu()
    L = B.lib()
    fake = C.c_void_p(0x10000)
    tabs = (C.c_void_p * 4)(*([0x10000] * 4))
    p = B.Plan(vocab=1000, vocab_comp=770, heads=2, head_dim=32, table_rows=[10007] * 4, hash_seed=1,
               d_model=256, dtype=B.BF16)
    out = C.c_void_p()
    assert L.engram_prefetcher_create(p._h, tabs, None, 100, 4, None) == B.E_INVALID_ARG
    assert L.engram_prefetcher_create(None, tabs, None, 100, 4, C.byref(out)) == B.E_INVALID_ARG
    assert L.engram_prefetcher_create(p._h, None, None, 100, 4, C.byref(out)) == B.E_INVALID_ARG
    assert L.engram_prefetcher_create(p._h, tabs, None, 0, 4, C.byref(out)) == B.E_INVALID_ARG
    assert L.engram_prefetcher_create(p._h, tabs, None, 100, 0, C.byref(out)) == B.E_INVALID_ARG
    assert L.engram_prefetcher_create(p._h, tabs, None, 100, 257, C.byref(out)) == B.E_INVALID_ARG
    bad_tabs = (C.c_void_p * 4)(*([0x10000] * 3 + [0x10004]))
    assert L.engram_prefetcher_create(p._h, bad_tabs, None, 100, 4, C.byref(out)) == B.E_INVALID_ARG
    bad_cache = B.RowCacheC(0x10000, 0x20000, 6)
    assert L.engram_prefetcher_create(p._h, tabs, C.byref(bad_cache), 100, 4, C.byref(out)) == B.E_INVALID_ARG
    assert L.engram_prefetcher_create(p._h, tabs, None, 1 << 30, 4, C.byref(out)) == B.E_UNSUPPORTED
    assert out.value is None
    assert L.engram_prefetcher_destroy(None) == B.E_INVALID_ARG
    assert L.engram_prefetch_begin(None, fake, 10, None) == B.E_INVALID_ARG
    assert L.engram_prefetch_finish(None, fake, None, None) == B.E_INVALID_ARG


def test_profiling_argument_checks(B):
    """Profiling control is host-only: a null plan, a non-positive launch
    budget, an unknown kind bit and a sampling period below one are refused;
    the sampling period itself is accepted without a device."""
    L = B.lib()
    p = B.Plan(vocab=1000, vocab_comp=770, heads=4, head_dim=32, table_rows=[10007] * 8, hash_seed=1,
               d_model=256, dtype=B.F32)
    assert L.engram_profile_every(None, 2) == B.E_INVALID_ARG
    assert L.engram_profile_every(p._h, 0) == B.E_INVALID_ARG
    assert L.engram_profile_every(p._h, -4) == B.E_INVALID_ARG
    assert L.engram_profile_every(p._h, 3) == 0
    assert L.engram_profile_every(p._h, 1) == 0
    assert L.engram_profile_begin(None, 8, 0) == B.E_INVALID_ARG
    assert L.engram_profile_begin(p._h, 0, 0) == B.E_INVALID_ARG
    assert L.engram_profile_begin(p._h, 8, 1 << 30) == B.E_INVALID_ARG


def test_probe_stream_rejects_bad_arguments_before_launching(B):
    _no_gpu()
    L = B.lib()
    fake = C.c_void_p(0x10000)
    odd = C.c_void_p(0x10008)
    ok_args = dict(mode=0, flags=0, unroll=8, blocks=2048, src=fake, dst=fake, nbytes=1 << 20)

    def call(**kw):
        a = dict(ok_args, **kw)
        return L.engram_probe_stream(a["mode"], a["flags"], a["unroll"], a["blocks"], a["src"], a["dst"],
                                     a["nbytes"], None)

    for kw in [dict(mode=2), dict(mode=-1), dict(flags=2), dict(unroll=5), dict(unroll=32), dict(blocks=0),
               dict(blocks=(1 << 20) + 1), dict(src=None), dict(dst=None), dict(src=odd), dict(dst=odd),
               dict(nbytes=0), dict(nbytes=-16), dict(nbytes=1000)]:
        assert call(**kw) == B.E_INVALID_ARG, kw


def test_noalloc_forward_rejects_before_touching_a_device(B):
    """engram_forward_noalloc: bad plans and shapes, and calls whose workspace
    would exceed the library's scratch array, return before any device call."""
    _no_gpu()
    L = B.lib()
    p = B.Plan(vocab=32000, vocab_comp=24640, heads=8, head_dim=64, table_rows=[500009] * 16, hash_seed=1,
               d_model=1024, dtype=B.BF16)
    fake = C.c_void_p(0x10000)
    tabs = (C.c_void_p * 16)(*([0x10000] * 16))
    w = B.WeightsC()

    def call(plan, batch, seqlen):
        return L.engram_forward_noalloc(plan, fake, batch, seqlen, fake, None, tabs, fake, C.byref(w), None, fake,
                                        None, 0, None, None)

    assert call(None, 8, 64) == B.E_INVALID_ARG
    assert call(p._h, 0, 64) == B.E_INVALID_ARG
    assert call(p._h, 8, -1) == B.E_INVALID_ARG
    # 8 x 4096 tokens at d = 1024 need about 72 MiB of workspace: beyond the scratch
    assert p.engram_workspace_size(8, 4096) > B.NOALLOC_SCRATCH_BYTES
    assert call(p._h, 8, 4096) == B.E_UNSUPPORTED


def test_retrieve_rejects_bad_arguments_before_launching(B):
    """engram_retrieve: null or misaligned buffers, bad shapes and null tables
    return before any device call."""
    _no_gpu()
    L = B.lib()
    p = B.Plan(vocab=32000, vocab_comp=24640, heads=8, head_dim=64, table_rows=[500009] * 16, hash_seed=1,
               d_model=1024, dtype=B.BF16)
    fake = C.c_void_p(0x10000)
    odd = C.c_void_p(0x10004)
    tabs = (C.c_void_p * 16)(*([0x10000] * 16))
    holey = (C.c_void_p * 16)(*([0x10000] * 15 + [0]))

    def call(plan, tokens=fake, batch=4, seqlen=8, comp=fake, tables=tabs, emb=fake):
        return L.engram_retrieve(plan, tokens, batch, seqlen, comp, None, tables, emb, None, None)

    assert call(None) == B.E_INVALID_ARG
    assert call(p._h, tokens=None) == B.E_INVALID_ARG
    assert call(p._h, comp=None) == B.E_INVALID_ARG
    assert call(p._h, emb=None) == B.E_INVALID_ARG
    assert call(p._h, tables=None) == B.E_INVALID_ARG
    assert call(p._h, batch=0) == B.E_INVALID_ARG
    assert call(p._h, seqlen=-3) == B.E_INVALID_ARG
    assert call(p._h, batch=1 << 16, seqlen=1 << 16) == B.E_UNSUPPORTED
    assert call(p._h, emb=odd) == B.E_INVALID_ARG
    assert call(p._h, tokens=odd) == B.E_INVALID_ARG
    assert call(p._h, tables=holey) == B.E_INVALID_ARG


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 (or a multi-rank launch)
    exits with a message before touching a device."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for extra_env, argv in (({}, ["--gpus", "2"]), ({"WORLD_SIZE": "4"}, [])):
        env = dict(os.environ, **extra_env)
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py")] + argv, capture_output=True, text=True,
                           env=env, timeout=120)
        assert r.returncode == 2, (argv, r.returncode, r.stderr)
        assert "measures one GPU" in r.stderr
        assert r.stdout == ""
