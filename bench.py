#!/usr/bin/env python3
"""Benchmark of the Engram forward pass on one MI355X.

One step = one engram_forward call per Engram layer of the workload over one
batch of synthetic tokens (fused hash + gather, the W_k projections with the
gate partials fused, the W_v projection with gate, gated value, causal conv,
residual and conv state fused into its epilogue).  Inputs are resident in HBM before the
timed region; the token batches and hidden states rotate over several
buffers so gathered rows and activations are not served from the 256 MB
Infinity Cache of a previous step.

Prints one JSON line: whole-job tokens/s, the roofline of the dominant
kernel (the one with the most time per step, timed live with HIP events
recorded by the library around each of its launches on the launch stream),
every kernel's roofline figures and the CPU oracle's tokens/s on a bounded
sample of the same workload.

`--backward` times the training step's backward instead: one engram_backward
call per Engram layer over the workload's tokens (indices computed
beforehand, as the forward pass would have), with its own JSON line in the
same form (metric "Engram bwd tokens/sec").
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
# The largest single-GPU configuration: 16 prime tables of ~78M rows x 80
# bf16 values (100B parameters, 200 GB resident in HBM), d = 2560, 8 x 4096
# Zipf(1.05) tokens per step.
DEFAULT_WORKLOAD = "maxtable_zipf"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rotate", type=int, default=8, help="distinct token/h buffers cycled per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the oracle sample")
    ap.add_argument("--breakdown-steps", type=int, default=20,
                    help="steps of the separate pass that times every kernel")
    ap.add_argument("--timed-every", type=int, default=4,
                    help="in the measured run, time one launch in this many of the dominant kernel (events "
                         "in a dispatch delay the launches around it)")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time only whole steps (no per-launch events; no roofline)")
    ap.add_argument("--unpacked-weights", action="store_true",
                    help="pass W_k and W_v as [d][D_e] matrices (default: packed once by engram_pack_weight at "
                         "set-up, outside the timed region, and read with ENGRAM_WEIGHTS_PACKED)")
    ap.add_argument("--retrieve-in-projection", action="store_true",
                    help="engram_forward flag: retrieval inside the projection launches")
    ap.add_argument("--overlap-retrieval", action="store_true",
                    help="with several layers per step: the later layers' rows are retrieved on a second stream "
                         "while the first layer computes (their slots depend only on the token ids)")
    ap.add_argument("--pipeline-retrieval", action="store_true",
                    help="retrieve the next step's rows on a second stream while this step's projections run "
                         "(engram_retrieve one step ahead, engram_gate_fuse on the main stream; every retrieval "
                         "and fusion of the measured steps lies inside the timed region)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the forward steps replayed from HIP graphs (captured once per rotation slot): "
                         "a `graph_replay` entry of its own, whole-step time only")
    ap.add_argument("--backward", action="store_true",
                    help="time engram_backward (training) instead of the forward: one JSON line of its own")
    ap.add_argument("--offload", action="store_true",
                    help="retrieval from tables in pinned host memory (with and without the hot-row cache in HBM) "
                         "and its overlap with device compute: one JSON line of its own")
    ap.add_argument("--cache-rows", type=int, default=131072, help="hot rows per table cached in HBM (--offload)")
    ap.add_argument("--cal-batches", type=int, default=32, help="calibration batches that pick the hot rows")
    ap.add_argument("--host-threads", type=int, default=16, help="host threads of the prefetcher (--offload)")
    ap.add_argument("--prefetch-wgs", type=int, default=8,
                    help="workgroups of the capped prefetch gather (--offload)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run the library's streaming copy and read over this many MiB, 5 times each "
                         "(counter calibration)")
    ap.add_argument("--no-hbm-probe", action="store_true",
                    help="skip the streaming read/copy ceilings and the extra gather legs")
    ap.add_argument("--probe-gib", type=float, default=4.0, help="buffer size of the streaming ceilings")
    ap.add_argument("--state-dtype", choices=("f32", "bf16"), default=None,
                    help="element type of the carried conv state (default: the workload's; bf16 at decode)")
    return ap.parse_args()


def src_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "hashed_gram_embedding_vocab_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SRC = {"gemm": "proj_bf16.hip", "gemm_v": "proj_bf16.hip", "gather": "gather.hip",
              "gate": "fuse.hip", "seam": "fuse.hip", "fuse": "fuse.hip"}


def load_traffic(workload: str, kind: str):
    """HBM bytes per launch of one kernel from committed rocprofv3 counter
    runs (FETCH_SIZE, WRITE_SIZE scaled by a plain-copy calibration), if they
    were taken on the kernel's current source."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f).get("kernels", {}).get(kind)
    if t is None or t.get("src_sha") != src_digest(KERNEL_SRC[kind]):
        return None
    return t


def cpu_baseline(wl, budget_s: float):
    """The oracle, as it stands, on whole sequences of the workload (as many
    as about budget_s of single-threaded CPU work takes, at least one
    32-token slice), timed end to end: hash, gather, projections, gate, conv."""
    import numpy as np

    import oracle
    from synthetic import workloads as W

    dt = oracle.BF16 if wl.dtype == "bf16" else oracle.F32
    seqlen = wl.seqlen
    comp = W.compression_map(wl.vocab, wl.vocab_comp, wl.seed(1))

    def run(n_seq, n_pos):
        """n_seq sequences, the first n_pos positions of each."""
        li = W.make_layer_inputs(wl, 0, batch=n_seq, seqlen=seqlen)
        toks = W.make_tokens(wl, batch=n_seq, seqlen=seqlen)[:, :n_pos]
        h = li.h.reshape(wl.n_branches, n_seq, seqlen, -1)[:, :, :n_pos].reshape(wl.n_branches, n_seq * n_pos, -1)
        t = time.perf_counter()
        idx, _, _ = oracle.hash_tokens(np.ascontiguousarray(toks), comp, wl.vocab, wl.vocab_comp, wl.heads,
                                       wl.primes(), li.hash_seed, orders=wl.orders)
        emb = oracle.gather_synth(idx, wl.head_dim, li.table_seed, dt)
        L = oracle.Layer(emb, np.ascontiguousarray(h), li.w_k, li.w_v, li.gamma_h, li.gamma_k, li.conv_w, n_seq,
                         n_pos, dt)
        for b in range(n_seq):
            L.forward_range(b, 0, n_pos)
        return time.perf_counter() - t

    n0 = min(32, seqlen)
    t0 = run(1, n0)
    want = max(n0, int(n0 * budget_s / max(t0, 1e-6)))  # tokens for about budget_s
    if want <= seqlen:
        n_seq, n_pos = 1, want
    else:
        n_seq, n_pos = min(wl.batch, -(-want // seqlen)), seqlen
    el = run(n_seq, n_pos)
    n = n_seq * n_pos
    layers = len(wl.layers)
    tok_s = n / el / layers  # a step runs every layer over each token
    return {"value": tok_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "positions 0..%d of %d sequence(s) (%d tokens, 1 layer of the %d per step; "
                      "single-threaded C, fp64), %.1f s" % (n_pos - 1, n_seq, n, layers, el)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the Engram path here is single-GPU (tables fit one "
              "MI355X's 288 GB); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe_mib:
        # Streaming copies and reads of known size: FETCH_SIZE / WRITE_SIZE of
        # these dispatches calibrate the counters against bytes actually moved.
        from hashed_gram_embedding_vocab_amd import binding as B
        n = args.copy_probe_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            B.engram_probe_stream(1, src, dst, n, unroll=8, blocks=2048)
        for _ in range(5):
            B.engram_probe_stream(0, src, dst, n, unroll=8, blocks=2048)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 5, "reads": 5}))
        return

    from hashed_gram_embedding_vocab_amd import binding as B
    from synthetic import workloads as W
    from synthetic.device import make_device_layer, to_device

    B.lib()
    torch.cuda.set_device(0)
    wl = W.workload(args.workload)
    if args.state_dtype is not None:
        import dataclasses
        wl = dataclasses.replace(wl, state_dtype=args.state_dtype)
    if args.backward:
        backward_bench(args, wl)
        return
    if args.offload:
        offload_bench(args, wl)
        return
    n_tok = wl.n_tokens
    R = max(1, args.rotate)
    rip_flag = B.RETRIEVE_IN_PROJECTION if args.retrieve_in_projection else 0
    # weights packed once into the projections' operand layout (bf16 plans)
    packed = not args.unpacked_weights and wl.dtype == "bf16"
    pk_flag = B.WEIGHTS_PACKED if packed else 0
    fwd_flags = rip_flag | pk_flag

    layers = []
    for slot in range(len(wl.layers)):
        dl = make_device_layer(wl, layer_slot=slot)
        hs = [dl.h] + [torch.randn_like(dl.h) for _ in range(R - 1)]
        out = torch.empty_like(dl.h)
        ws = dl.plan.workspace(wl.batch, wl.seqlen)
        ctx = conv = None
        if wl.decode:
            ctx = to_device(dl.li.prev_ctx, torch.int32, "cuda")
            conv = to_device(dl.li.conv_state, dl.plan.state_torch_dtype, "cuda")
        if packed:
            dl.weights = dl.plan.packed_weights(dl.weights)
        layers.append((dl, hs, out, ws, ctx, conv))
    toks = [to_device(W.make_tokens(wl, seed=wl.seed(2) + 17 * r), torch.int32, "cuda") for r in range(R)]
    torch.cuda.synchronize()

    # Later layers' retrieval on a second stream (default priority): engram_retrieve
    # into one of two E buffers per layer, handed to engram_gate_fuse on the main
    # stream by an event; a buffer is refilled only after the fusion two steps
    # earlier has read it.
    overlap = args.overlap_retrieval and len(layers) > 1
    if overlap:
        side = torch.cuda.Stream()
        embs = [[torch.empty((n_tok, wl.emb_dim), dtype=layers[l][0].plan.torch_dtype, device="cuda")
                 for _ in range(2)] for l in range(len(layers))]
        ready = [[torch.cuda.Event() for _ in range(2)] for _ in layers]
        free = [[torch.cuda.Event() for _ in range(2)] for _ in layers]
        used = [[False, False] for _ in layers]

    def enqueue(r, par, captured):
        """One step on token/h buffers r (E buffers `par` when overlapping).
        Under graph capture the side stream forks from the capturing stream
        and joins it again; replays of one graph never overlap, so no buffer
        needs the cross-step wait."""
        if not overlap:
            for dl, hs, out, ws, ctx, conv in layers:
                dl.plan.engram_forward(toks[r], dl.comp_map, dl.tables, hs[r], dl.weights, out, ws,
                                       prev_ctx=ctx, conv_state=conv, flags=fwd_flags)
            return
        main = torch.cuda.current_stream()
        if captured:
            side.wait_stream(main)
        for l in range(1, len(layers)):
            dl, hs, out, ws, ctx, conv = layers[l]
            if not captured and used[l][par]:
                side.wait_event(free[l][par])
            dl.plan.engram_retrieve(toks[r], dl.comp_map, dl.tables, embs[l][par], prev_ctx=ctx, stream=side)
            ready[l][par].record(side)
        dl, hs, out, ws, ctx, conv = layers[0]
        dl.plan.engram_forward(toks[r], dl.comp_map, dl.tables, hs[r], dl.weights, out, ws,
                               prev_ctx=ctx, conv_state=conv, flags=fwd_flags)
        for l in range(1, len(layers)):
            dl, hs, out, ws, ctx, conv = layers[l]
            main.wait_event(ready[l][par])
            dl.plan.engram_gate_fuse(embs[l][par], hs[r], dl.weights, out, ws, wl.batch, wl.seqlen,
                                     conv_state=conv, flags=pk_flag)
            if not captured:
                free[l][par].record(main)
                used[l][par] = True

    # Retrieval one step ahead: step i fuses batch i (E buffers i % 2 of every
    # layer, retrieved on the side stream during step i-1) and retrieves batch
    # i+1 into the other buffers.  Step 0 of a run retrieves its own batch
    # first, and the last step of a run retrieves nothing, so a run of K steps
    # holds exactly K retrievals and K fusions.
    pipeline = args.pipeline_retrieval and not overlap and not rip_flag
    if pipeline:
        pside = torch.cuda.Stream()
        pembs = [[torch.empty((n_tok, wl.emb_dim), dtype=L[0].plan.torch_dtype, device="cuda") for _ in range(2)]
                 for L in layers]
        pready = [[torch.cuda.Event() for _ in range(2)] for _ in layers]
        pfree = [[torch.cuda.Event() for _ in range(2)] for _ in layers]
        pused = [[False, False] for _ in layers]
        prun = {"steps": 0}

    def pipe_retrieve(b, par):
        for l, (dl, hs, out, ws, ctx, conv) in enumerate(layers):
            if pused[l][par]:
                pside.wait_event(pfree[l][par])
            dl.plan.engram_retrieve(toks[b % R], dl.comp_map, dl.tables, pembs[l][par], prev_ctx=ctx, stream=pside)
            pready[l][par].record(pside)

    def pipe_step(i):
        main = torch.cuda.current_stream()
        if i == 0:
            pside.wait_stream(main)
            pipe_retrieve(0, 0)
        if i + 1 < prun["steps"]:
            pipe_retrieve(i + 1, (i + 1) % 2)
        for l, (dl, hs, out, ws, ctx, conv) in enumerate(layers):
            main.wait_event(pready[l][i % 2])
            dl.plan.engram_gate_fuse(pembs[l][i % 2], hs[i % R], dl.weights, out, ws, wl.batch, wl.seqlen,
                                     conv_state=conv, flags=pk_flag)
            pfree[l][i % 2].record(main)
            pused[l][i % 2] = True

    def step(i):
        if pipeline:
            pipe_step(i)
        else:
            enqueue(i % R, i % 2, False)

    def graph_replay():
        """The same steps as HIP graphs (one per rotation slot, captured once),
        replayed: one launch per step from the host.  Whole-step time only."""
        cap = torch.cuda.Stream()
        graphs = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                enqueue(r, r % 2, True)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        for i in range(args.steps):
            graphs[i % R].replay()
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return {"value": n_tok * args.steps / wall, "ms_per_step": round(wall * 1e3 / args.steps, 4),
                "gpu_event_ms_per_step": round(ev0.elapsed_time(ev1) / args.steps, 4), "graphs": R,
                "overlap_retrieval": bool(overlap)}

    if pipeline:
        prun["steps"] = args.warmup
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def timed(steps, kinds, every=1):
        """steps steps between a barrier + synchronize on both sides; launches
        of `kinds` (None: all, []: none) timed by their own dispatch events,
        one launch in `every` of each kind."""
        if kinds != []:
            for dl, *_ in layers:
                dl.plan.engram_profile_every(every)
                dl.plan.engram_profile_begin(8 * steps + 64, kinds)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if pipeline:
            prun["steps"] = steps
        if torch.distributed.is_available() and torch.distributed.is_initialized():
            torch.distributed.barrier()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record()
        for i in range(steps):
            step(i)
        ev1.record()
        torch.cuda.synchronize()
        if torch.distributed.is_available() and torch.distributed.is_initialized():
            torch.distributed.barrier()
        wall = time.perf_counter() - t0
        profs = [dl.plan.engram_profile_end() for dl, *_ in layers] if kinds != [] else None
        return wall, ev0.elapsed_time(ev1), profs

    def kern_of(profs):
        def kern(name):
            tot = sum(p[name]["total_ms"] for p in profs)
            n = sum(p[name]["launches"] for p in profs)
            return tot / max(n, 1), n
        return kern

    if args.no_kernel_events:
        wall, gpu_ms, _ = timed(args.steps, [])
        print(json.dumps({"workload": wl.name, "value": n_tok * args.steps / wall, "ms_per_step": wall * 1e3 / args.steps,
                          "gpu_event_ms_per_step": gpu_ms / args.steps, "kernel_events": False}), flush=True)
        return

    # Breakdown pass (not part of the measured value): every launch timed, to
    # find the kernel that takes the most time per step and give each
    # kernel's figures.  Timing every launch costs whole-step throughput, so
    # the measured run below times only the dominant kernel.
    _, _, profs_all = timed(args.breakdown_steps, None)
    kern = kern_of(profs_all)
    dominant = max(("gather", "gemm", "gate", "gemm_v", "seam", "fuse"), key=lambda k: kern(k)[0] * kern(k)[1])
    wall, gpu_ms, profs = timed(args.steps, [dominant], max(1, args.timed_every))
    kern_dom = kern_of(profs)

    ms_per_step = wall * 1e3 / args.steps
    tokens_per_step = n_tok
    value = tokens_per_step * args.steps / wall

    # Per-kernel algorithmic work per launch.  Projections are MFMA-bound
    # (flops); retrieval and the fusion kernel are HBM-bound (bytes).
    De, d, Br = wl.emb_dim, wl.d_model, wl.n_branches
    eb = 2 if wl.dtype == "bf16" else 4
    state_eb = 2 if wl.state_dtype == "bf16" else 4
    two_launch = kern("gemm_v")[1] > 0
    n_parts = d // 128 if wl.dtype == "bf16" else 1
    # engram_forward retrieves in one kernel (hash + gather): it reads each raw
    # token id, every slot row, and writes E; no index buffer round trip
    fused_retrieval = kern("hash")[1] == 0
    n_w = Br if two_launch else Br + 1
    part_bytes = Br * n_parts * 3 * 4 * n_tok
    models = {
        # W_k e of every branch (and W_v e on the one-launch path)
        "gemm": ("mfma", 2.0 * n_tok * De * n_w * d),
        # W_v e with gate, gated value, conv, residual, state in the epilogue
        "gemm_v": ("mfma", 2.0 * n_tok * De * d),
        "gather": ("hbm", n_tok * ((4 if fused_retrieval else wl.n_tables * 4) + 2 * De * eb)),
        # reads the partial sums, writes one gate per token and branch
        "gate": ("hbm", part_bytes + Br * 4 * n_tok),
        # tile-seam rows: v of 6 rows per tile, h and out of up to 3 rows per tile and branch
        "seam": ("hbm", (n_tok // 256) * (6 * d * 4 + 3 * Br * (2 * d * eb + 16))),
        # reads v (fp32) once, h once per branch and the partial sums (the
        # gate is computed there); writes out per branch; with a carried conv
        # state, reads and rewrites its K_c-1 rows (fp32 or bf16) per sequence
        # and branch
        "fuse": ("hbm", n_tok * (4 * d + Br * 2 * d * eb) + part_bytes
                 + (2 * Br * wl.batch * (wl.conv_kernel - 1) * d * state_eb if wl.decode else 0)),
    }
    # HBM bytes of the projection launches as well (E, weights, h, partials,
    # and v or out): the W_v launch sits close to both roofs
    mem_bytes = {
        "gemm": n_tok * De * eb + n_w * d * De * eb + Br * n_tok * d * eb + part_bytes
                + (0 if two_launch else n_tok * d * 4),
        "gemm_v": n_tok * De * eb + d * De * eb + Br * 4 * n_tok + 2 * Br * n_tok * d * eb,
    }
    kernel_src = {"gemm": "proj_bf16_kernel<0,1>" if wl.dtype == "bf16" else "proj_f32_kernel",
                  "gemm_v": "proj_bf16_kernel<1,%d>" % Br,
                  "gather": "hash_gather_kernel" if fused_retrieval else "gather_kernel",
                  "gate": "gate_kernel",
                  "seam": "seam_kernel<%d,%s>" % (Br, "false"),
                  "fuse": "fuse_kernel<%s,%d>" % ("true" if wl.dtype == "bf16" else "false", Br)}
    per_kernel = {}
    for k, (bound, work) in models.items():
        ms, n = kern(k)
        if n == 0:
            continue
        if bound == "mfma":
            ach, peak, unit = work / (ms * 1e-3) / 1e12, MFMA_PEAK_TFLOPS[wl.dtype], "TFLOP/s"
        else:
            ach, peak, unit = work / (ms * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
        per_kernel[k] = {"kernel": kernel_src[k], "bound": bound, "achieved": round(ach, 2), "peak": peak,
                         "unit": unit, "frac": round(ach / peak, 4), "avg_launch_us": round(ms * 1e3, 2),
                         "launches": n, ("flops_per_launch" if bound == "mfma" else "bytes_per_launch"): work,
                         "ms_per_step": round(ms * n / args.breakdown_steps, 4)}
        if k in mem_bytes:
            gbs = mem_bytes[k] / (ms * 1e-3) / 1e9
            per_kernel[k].update({"hbm_bytes_per_launch": mem_bytes[k], "hbm_GBs": round(gbs, 1),
                                  "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
    dom = dominant
    roofline = dict(per_kernel[dom])
    # the dominant kernel's figures as measured inside the timed run
    ms, n = kern_dom(dom)
    bound, work = models[dom]
    if bound == "mfma":
        ach = work / (ms * 1e-3) / 1e12
    else:
        ach = work / (ms * 1e-3) / 1e9
    per_step = kern(dom)[1] / args.breakdown_steps  # launches of the kernel per step
    roofline.update({"achieved": round(ach, 2), "frac": round(ach / roofline["peak"], 4),
                     "avg_launch_us": round(ms * 1e3, 2), "launches": n, "timed_every": max(1, args.timed_every),
                     "ms_per_step": round(ms * per_step, 4), "timed_in": "measured run"})
    if dom in mem_bytes:
        gbs = mem_bytes[dom] / (ms * 1e-3) / 1e9
        roofline.update({"hbm_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
    tk = load_traffic(wl.name, dom) if wl.dtype == "bf16" or dom not in ("gemm", "gemm_v") else None
    roofline["traffic"] = None if tk is None else tk["bytes_per_launch"]
    roofline["traffic_unit"] = "bytes"
    kernels_us = {k: round(kern(k)[0] * 1e3, 2) for k in B.KERNEL_NAMES}
    # the gate GEMMs together: W_k and W_v flops over the time of every
    # projection launch (breakdown pass)
    proj_ms = sum(kern(k)[0] * kern(k)[1] for k in ("gemm", "gemm_v")) / args.breakdown_steps
    proj_flops = 2.0 * n_tok * De * (Br + 1) * d * len(wl.layers)
    gemm_tf = proj_flops / (proj_ms * 1e-3) / 1e12
    gate_gemm = {"achieved": round(gemm_tf, 2), "peak": MFMA_PEAK_TFLOPS[wl.dtype], "unit": "TFLOP/s",
                 "frac": round(gemm_tf / MFMA_PEAK_TFLOPS[wl.dtype], 4), "ms_per_step": round(proj_ms, 4),
                 "flops_per_step": proj_flops}
    g = per_kernel.get("gather")
    gather = None if g is None else {"kernel": g["kernel"], "achieved_GBs": g["achieved"], "peak_GBs": HBM_PEAK_GBS,
                                     "frac": g["frac"], "bytes_per_launch": g["bytes_per_launch"],
                                     "avg_launch_us": g["avg_launch_us"]}

    hbm = gather_uniform = None
    if not args.no_hbm_probe:
        hbm = hbm_ceiling(args)
        if wl.name.startswith("maxtable"):
            gather_uniform = uniform_gather_legs(wl, layers[0][0], args, R, models["gather"][1], pk_flag)
        if gather is not None and hbm is not None:
            gather["frac_of_stream_read"] = round(gather["achieved_GBs"] / hbm["read"]["GBs"], 4)

    graphed = graph_replay() if args.graph else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds)

    line = {
        "metric": "Engram fwd tokens/sec",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "gpu_event_ms_per_step": round(gpu_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic: Zipf(%s) token ids over V=%d, seeded Philox tables, N(0,1) hidden states"
                % (wl.zipf_s, wl.vocab),
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seqlen,
                   "tokens_per_step": tokens_per_step, "layers": list(wl.layers),
                   "n_branches": Br, "d_model": d, "heads_per_order": wl.heads,
                   "head_dim": wl.head_dim, "emb_dim": De, "table_params": sum(wl.primes()) * wl.head_dim,
                   "rotated_buffers": R, "parallelism": "single GPU",
                   "conv_state_dtype": wl.state_dtype if wl.decode else None,
                   "retrieval_in_projection": bool(rip_flag), "overlap_retrieval": bool(overlap),
                   "packed_weights": bool(packed),
                   "pipeline_retrieval": bool(pipeline)},
        "roofline": roofline,
        "gather": gather,
        "gather_uniform": gather_uniform,
        "hbm_ceiling": hbm,
        "gate_gemm": gate_gemm,
        "kernels": per_kernel,
        "kernel_avg_us": kernels_us,
        "graph_replay": graphed,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def hbm_ceiling(args):
    """The box's streaming ceilings from the library's plain read and copy
    kernels over a buffer far larger than the caches: the best of a small
    sweep of chunks in flight per thread, workgroups and nontemporal access,
    each timed over 5 passes after one untimed pass."""
    import torch

    from hashed_gram_embedding_vocab_amd import binding as B

    n = int(args.probe_gib * (1 << 30)) // 16 * 16
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    best = {}
    for mode, name, moved in ((0, "read", n), (1, "copy", 2 * n)):
        for unroll in (4, 8, 16):
            for blocks in (1024, 2048, 4096):
                for flags in (0, B.PROBE_NONTEMPORAL):
                    B.engram_probe_stream(mode, src, dst, n, unroll=unroll, blocks=blocks, flags=flags)
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(5):
                        B.engram_probe_stream(mode, src, dst, n, unroll=unroll, blocks=blocks, flags=flags)
                    e1.record()
                    torch.cuda.synchronize()
                    gbs = moved * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
                    if gbs > best.get(name, {}).get("GBs", 0):
                        best[name] = {"GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                                      "unroll": unroll, "blocks": blocks, "nontemporal": bool(flags)}
    del src, dst
    torch.cuda.empty_cache()
    best["buffer_bytes"] = n
    best["kernel"] = "stream_read_kernel / stream_copy_kernel (engram_probe_stream)"
    return best


def uniform_gather_legs(wl, dl, args, R, fused_bytes, flags=0):
    """On the same 200 GB of tables: the fused retrieval (hash + gather) of
    uniformly drawn token ids, where the caches cannot help, and the
    index-driven gather of uniformly random slots of every table (engram_gather)."""
    import numpy as np
    import torch

    from synthetic import workloads as W
    from synthetic.device import to_device

    n_tok = wl.n_tokens
    out = {}
    wu = W.workload("maxtable_uniform")
    toks = [to_device(W.make_tokens(wu, seed=wu.seed(2) + 17 * r), torch.int32, "cuda") for r in range(R)]
    ws = dl.plan.workspace(wl.batch, wl.seqlen)
    h_out = torch.empty_like(dl.h)
    steps = max(8, args.breakdown_steps)
    for i in range(4):
        dl.plan.engram_forward(toks[i % R], dl.comp_map, dl.tables, dl.h, dl.weights, h_out, ws, flags=flags)
    torch.cuda.synchronize()
    dl.plan.engram_profile_every(1)
    dl.plan.engram_profile_begin(8 * steps + 64, ["gather"])
    for i in range(steps):
        dl.plan.engram_forward(toks[i % R], dl.comp_map, dl.tables, dl.h, dl.weights, h_out, ws, flags=flags)
    torch.cuda.synchronize()
    p = dl.plan.engram_profile_end()["gather"]
    ms = p["total_ms"] / max(p["launches"], 1)
    gbs = fused_bytes / (ms * 1e-3) / 1e9
    out["tokens_uniform"] = {"kernel": "hash_gather_kernel", "avg_launch_us": round(ms * 1e3, 2),
                             "launches": p["launches"], "bytes_per_launch": fused_bytes,
                             "achieved_GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                             "tokens": "uniform over V=%d (the maxtable_uniform stream)" % wu.vocab}
    del toks, h_out
    # index-driven gather of uniformly random slots: no hashing, no token reuse
    eb = 2 if wl.dtype == "bf16" else 4
    primes = np.array(wl.primes(), np.int64)
    rng = np.random.default_rng(wl.seed(7))
    idxs = []
    for r in range(R):
        x = (rng.random((n_tok, wl.n_tables)) * primes).astype(np.int64).astype(np.int32)
        idxs.append(to_device(x, torch.int32, "cuda"))
    emb = torch.empty((n_tok, wl.emb_dim), dtype=dl.h.dtype, device="cuda")
    for i in range(4):
        dl.plan.engram_gather(idxs[i % R], dl.tables, emb)
    torch.cuda.synchronize()
    dl.plan.engram_profile_begin(8 * steps + 64, ["gather"])
    for i in range(steps):
        dl.plan.engram_gather(idxs[i % R], dl.tables, emb)
    torch.cuda.synchronize()
    p = dl.plan.engram_profile_end()["gather"]
    ms = p["total_ms"] / max(p["launches"], 1)
    idx_bytes = n_tok * (wl.n_tables * 4 + 2 * wl.emb_dim * eb)
    gbs = idx_bytes / (ms * 1e-3) / 1e9
    out["slots_uniform"] = {"kernel": "gather_kernel", "avg_launch_us": round(ms * 1e3, 2),
                            "launches": p["launches"], "bytes_per_launch": idx_bytes,
                            "achieved_GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    del idxs, emb, ws
    torch.cuda.empty_cache()
    return out


def backward_cpu_baseline(wl, budget_s: float):
    """The backward oracle, as it stands, on one sequence prefix of the
    workload's widths (hash, gather and the chain rule; about budget_s of
    single-threaded CPU work), in tokens per second."""
    import numpy as np

    import oracle
    from synthetic import workloads as W

    def run(n_pos):
        toks = np.ascontiguousarray(W.make_tokens(wl)[:1, :n_pos])
        li = W.make_layer_inputs(wl, 0, batch=1, seqlen=n_pos)
        comp = W.compression_map(wl.vocab, wl.vocab_comp, wl.seed(1))
        dt = oracle.BF16 if wl.dtype == "bf16" else oracle.F32
        dout = np.random.default_rng(1).standard_normal((wl.n_branches, n_pos, wl.d_model)).astype(np.float32)
        t0 = time.perf_counter()
        idx, _, _ = oracle.hash_tokens(toks, comp, wl.vocab, wl.vocab_comp, wl.heads, wl.primes(), li.hash_seed,
                                       orders=wl.orders)
        emb = oracle.gather_synth(idx, wl.head_dim, li.table_seed, dt)
        L = oracle.Layer(emb, li.h, li.w_k, li.w_v, li.gamma_h, li.gamma_k, li.conv_w, 1, n_pos, dt)
        g = L.backward(dout)
        oracle.table_grad(idx, g["demb"], wl.head_dim)
        return time.perf_counter() - t0

    n = 16
    dt = run(n)
    while dt < budget_s / 8 and n < wl.seqlen:
        n = min(wl.seqlen, n * 4)
        dt = run(n)
    if n < wl.seqlen:
        n = min(wl.seqlen, max(n, int(n * budget_s / dt)))
        dt = run(n)
    return {"value": n / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "positions 0..%d of one sequence (%d tokens, 1 layer; single-threaded C, fp64), %.1f s"
                      % (n - 1, n, dt)}


def backward_bench(args, wl):
    """engram_backward over the workload's tokens (every layer of a step), the
    retrieval indices computed beforehand as the forward pass would have."""
    import numpy as np
    import torch

    from hashed_gram_embedding_vocab_amd import binding as B
    from synthetic import workloads as W
    from synthetic.device import make_device_layer, to_device

    if wl.dtype != "bf16" or wl.decode:
        print("the backward covers bf16 whole sequences", file=sys.stderr)
        sys.exit(2)
    n_tok = wl.n_tokens
    R = max(1, args.rotate)
    gen = torch.Generator().manual_seed(11)
    layers = []
    for slot in range(len(wl.layers)):
        dl = make_device_layer(wl, layer_slot=slot)
        toks = [to_device(W.make_tokens(wl, seed=wl.seed(2) + 17 * r), torch.int32, "cuda") for r in range(R)]
        idx = []
        for r in range(R):
            x = torch.empty((n_tok, wl.n_tables), dtype=torch.int32, device="cuda")
            dl.plan.engram_hash(toks[r], dl.comp_map, x)
            idx.append(x)
        hs = [dl.h] + [torch.randn(dl.h.shape, generator=gen).to(dl.h.dtype).cuda() for _ in range(R - 1)]
        douts = [torch.randn(dl.h.shape, generator=gen).to(dl.h.dtype).cuda() for _ in range(R)]
        dh = torch.empty_like(dl.h)
        grads = B.Grads(wl.n_branches, wl.d_model, wl.emb_dim, wl.conv_kernel, wl.n_tables, n_tok, wl.head_dim)
        ws = dl.plan.backward_workspace(wl.batch, wl.seqlen)
        layers.append((dl, idx, hs, douts, dh, grads, ws))
    torch.cuda.synchronize()

    def step(i):
        r = i % R
        for dl, idx, hs, douts, dh, grads, ws in layers:
            dl.plan.engram_backward(idx[r], dl.tables, hs[r], dl.weights, douts[r], dh, grads, ws,
                                    wl.batch, wl.seqlen)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def timed(steps, kinds):
        if kinds != []:
            for dl, *_ in layers:
                dl.plan.engram_profile_begin(8 * steps + 64, kinds)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        profs = [dl.plan.engram_profile_end() for dl, *_ in layers] if kinds != [] else None
        return wall, profs

    # breakdown pass: every kind timed by its own dispatch events; the
    # measured run below times only the kind with the most time per step
    _, profs = timed(args.breakdown_steps, None)
    kinds = ("gather", "bwd_gemm", "bwd_fuse", "bwd_table")
    calls = args.breakdown_steps * len(layers)
    per_call = {k: sum(p[k]["total_ms"] for p in profs) / calls * 1e3 for k in kinds}  # us per engram_backward call
    dominant = max(kinds, key=lambda k: per_call[k])
    wall, profs_m = timed(args.steps, [dominant])
    dom_us = sum(p[dominant]["total_ms"] for p in profs_m) / (args.steps * len(layers)) * 1e3
    De, d, Br = wl.emb_dim, wl.d_model, wl.n_branches
    N = (Br + 1) * d
    n_pad = (n_tok + 127) // 128 * 128
    eb = 2
    # work per engram_backward call.  Contractions: k and v again, dE and dW,
    # each 2 (B_r + 1) d D_e flop per token.  HBM kinds: the bytes their
    # kernels move in this design (gate partials, fp32 k and v read back,
    # bf16 dk/dv; table rows: dE slices read, row gradients written).
    models = {
        "bwd_gemm": ("mfma", 2.0 * De * N * (2 * n_tok + n_pad)),
        "gather": ("hbm", n_tok * (wl.n_tables * 4 + 2 * De * eb)),
        "bwd_fuse": ("hbm", Br * n_tok * (3 * 4 * (d // 128) + 16)          # gate statistics: partials; rh, rk, s, alpha
                     + n_tok * d * (4 + 2) + Br * n_tok * d * eb            # conv: v, dout; dv
                     + Br * n_tok * d * (eb + 4 + eb + eb + 2)),            # gate: h, k, dout; dh, dk
        "bwd_table": ("hbm", wl.n_tables * n_tok * (wl.head_dim * 4 * 2 + 4 * 8)),
    }

    def figures(kind, us):
        bound, work = models[kind]
        if bound == "mfma":
            ach, peak, unit = work / (us * 1e-6) / 1e12, MFMA_PEAK_TFLOPS["bf16"], "TFLOP/s"
        else:
            ach, peak, unit = work / (us * 1e-6) / 1e9, HBM_PEAK_GBS, "GB/s"
        return {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
                ("flops_per_call" if bound == "mfma" else "bytes_per_call"): work, "us_per_call": round(us, 2)}

    kernel_of = {"bwd_gemm": "proj_bf16_kernel<5> (k and v, gate partials), <6> (dE, W read K-major), <4> (dW from "
                             "token-major operands, with its split-K sum)",
                 "bwd_fuse": "bwd_gate_stats, bwd_conv, bwd_gate, ordered sums",
                 "bwd_table": "table-row gradients (keys, segmented radix sort, run-head scan, segmented sums)",
                 "gather": "gather_kernel"}
    per_kind = {k: dict(figures(k, per_call[k]), kernel=kernel_of[k]) for k in kinds}
    roofline = dict(figures(dominant, dom_us), kernel=kernel_of[dominant], timed_in="measured run", traffic=None)
    cpu = None if args.no_cpu_baseline else backward_cpu_baseline(wl, args.cpu_seconds)
    line = {
        "metric": "Engram bwd tokens/sec",
        "value": round(n_tok * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic: Zipf(%s) token ids, seeded Philox tables, N(0,1) hidden states and output gradients"
                % wl.zipf_s,
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seqlen, "tokens_per_step": n_tok,
                   "layers": list(wl.layers), "n_branches": Br, "d_model": d, "emb_dim": De,
                   "rotated_buffers": R, "parallelism": "single GPU"},
        "roofline": roofline,
        "kinds": per_kind,
        "us_per_call": {k: round(v, 2) for k, v in per_call.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def offload_bench(args, wl):
    """Retrieval with the tables in pinned host memory (the GPU reads the rows
    over the host link), without and with the hot rows cached in HBM, next to
    the same gather from HBM-resident tables; then the cached host gather of
    the next batch on a second stream while a stand-in for the backbone's
    earlier layers (bf16 matrix products) runs on the first."""
    import numpy as np
    import torch

    from hashed_gram_embedding_vocab_amd import binding as B
    from synthetic import workloads as W
    from synthetic.device import make_device_layer, to_device

    if wl.decode:
        print("--offload measures whole prefill batches", file=sys.stderr)
        sys.exit(2)
    n_tok = wl.n_tokens
    R = max(1, args.rotate)
    dl_dev = make_device_layer(wl)
    dl_host = make_device_layer(wl, host_tables=True)
    plan = dl_dev.plan
    tdt = dl_dev.h.dtype
    # every batch draws from one rank->token permutation: the same tokens
    # (hence n-grams, hence rows) are frequent in all of them
    perm_seed = wl.seed(2) + 1
    idx = []
    for r in range(R):
        toks = to_device(W.make_tokens(wl, seed=wl.seed(2) + 17 * r, perm_seed=perm_seed), torch.int32, "cuda")
        x = torch.empty((n_tok, wl.n_tables), dtype=torch.int32, device="cuda")
        plan.engram_hash(toks, dl_dev.comp_map, x)
        idx.append(x)
    # hot rows: the most frequent slots of separate calibration traffic
    # (args.cal_batches batches, none of them a measured one)
    cal_h = []
    for c in range(args.cal_batches):
        cal_t = to_device(W.make_tokens(wl, seed=wl.seed(2) + 1000 + 17 * c, perm_seed=perm_seed), torch.int32,
                          "cuda")
        cal = torch.empty((n_tok, wl.n_tables), dtype=torch.int32, device="cuda")
        plan.engram_hash(cal_t, dl_dev.comp_map, cal)
        cal_h.append(cal.cpu().numpy().view(np.uint32))
    cal_h = np.concatenate(cal_h)
    n_hot = args.cache_rows
    hot = np.zeros((wl.n_tables, n_hot), np.uint32)
    for tau in range(wl.n_tables):
        u, c = np.unique(cal_h[:, tau], return_counts=True)
        top = u[np.argsort(-c, kind="stable")][:n_hot]
        hot[tau, :len(top)] = top
        hot[tau, len(top):] = 0xFFFFFFFF  # past every table: skipped
    cap = 1
    while cap < 2 * n_hot:
        cap *= 2
    cache = B.RowCache(wl.n_tables, cap, wl.head_dim, tdt)
    plan.engram_cache_build(to_device(hot.view(np.int32), torch.int32, "cuda"), dl_host.tables, cache)
    # hit rate of the measured batches (host side, from the indices)
    hits = 0
    for r in range(R):
        ih = idx[r].cpu().numpy().view(np.uint32)
        hits += sum(int(np.isin(ih[:, tau], hot[tau]).sum()) for tau in range(wl.n_tables))
    hit_rate = hits / (R * n_tok * wl.n_tables)
    emb = [torch.empty((n_tok, wl.emb_dim), dtype=tdt, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()

    def time_gather(fn, steps):
        for i in range(3):
            fn(i, emb[0], None)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i, emb[i & 1], None)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps  # ms per gather

    g_dev = lambda i, e, s: plan.engram_gather(idx[i % R], dl_dev.tables, e, stream=s)
    g_host = lambda i, e, s: plan.engram_gather(idx[i % R], dl_host.tables, e, stream=s)
    g_cached = lambda i, e, s, wg=0: plan.engram_gather_cached(idx[i % R], dl_host.tables, cache, e,
                                                               max_workgroups=wg, stream=s)
    steps = max(4, args.steps // 5)
    ms_dev = time_gather(g_dev, steps)
    ms_host = time_gather(g_host, steps)
    ms_cached = time_gather(g_cached, steps)
    row_b = wl.head_dim * (2 if wl.dtype == "bf16" else 4)
    link_bytes = n_tok * wl.n_tables * row_b  # every row over the link
    # whole forward with host tables (retrieval inside engram_forward reads them)
    out = torch.empty_like(dl_host.h)
    ws = plan.workspace(wl.batch, wl.seqlen)
    toks0 = to_device(W.make_tokens(wl, seed=wl.seed(2)), torch.int32, "cuda")
    fwd = lambda dl: dl.plan.engram_forward(toks0, dl.comp_map, dl.tables, dl.h, dl.weights, out, ws)

    def time_fwd(dl, k=10):
        for _ in range(3):
            fwd(dl)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(k):
            fwd(dl)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / k

    fwd_dev_ms, fwd_host_ms = time_fwd(dl_dev), time_fwd(dl_host)

    # overlap: cached host gathers of later batches on a second stream under
    # a stand-in for the backbone's earlier layers: bf16 products of
    # 16384 x 4096 by 4096 x 16384 (4096 tiles of 256 x 256, sixteen rounds
    # on 256 CUs, so a few CUs taken by the prefetch cost a few percent, not
    # a whole round), as many as take about twice the prefetch alone.  First
    # one workgroup per token group, then capped at args.prefetch_wgs
    # workgroups that keep their CU slots for the whole gather.
    Mb, Kb = 16384, 4096
    x = torch.randn((Mb, Kb), device="cuda").to(torch.bfloat16)
    y = torch.randn((Kb, Mb), device="cuda").to(torch.bfloat16)
    z = torch.empty((Mb, Mb), device="cuda", dtype=torch.bfloat16)
    n_g = 4

    def wall(fns):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for f in fns:
            f()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3

    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()

    def backbone_of(n_mm):
        def backbone():
            with torch.cuda.stream(sa):
                for _ in range(n_mm):
                    torch.mm(x, y, out=z)
        return backbone

    def prefetch_of(wg):
        def prefetch():
            for i in range(n_g):
                g_cached(i, emb[i & 1], sb, wg)
        return prefetch

    one = backbone_of(1)
    for _ in range(2):
        wall([one])
    mm_ms = min(wall([one]) for _ in range(3))
    pf0 = prefetch_of(0)
    wall([pf0])
    pf_est = min(wall([pf0]) for _ in range(2))
    n_mm = max(2, int(np.ceil(2.0 * pf_est / mm_ms)))
    backbone = backbone_of(n_mm)

    def overlap(wg):
        # the prefetch is issued first: a step's indices are known before its
        # layers run, so its gathers are queued ahead of them
        prefetch = prefetch_of(wg)
        for _ in range(2):
            wall([prefetch, backbone])
        bb = min(wall([backbone]) for _ in range(3))
        pf = min(wall([prefetch]) for _ in range(3))
        both = min(wall([prefetch, backbone]) for _ in range(3))
        return bb, pf, both

    bb_full, pf_full, both_full = overlap(0)
    bb_cap, pf_cap, both_cap = overlap(args.prefetch_wgs)
    mm_flops = 2.0 * Mb * Mb * Kb * n_mm

    # host-gather prefetcher: host threads copy the missed rows, a DMA
    # engine stages them, one assembly kernel builds E; begin before the
    # backbone, finish after it
    pfr = B.Prefetcher(plan, dl_host.tables, cache, max_tokens=n_tok, n_threads=args.host_threads)

    def host_job(i):
        pfr.begin(idx[i % R], stream=sb)
        return pfr.finish(emb[i & 1], stream=sb)

    for i in range(3):
        host_job(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    misses = 0
    for i in range(n_g):
        misses += host_job(i)
    torch.cuda.synchronize()
    hg_ms = (time.perf_counter() - t0) * 1e3 / n_g

    # each job under its share of the backbone: begin, that many products
    # on the other stream, finish (the pipeline of one layer per job)
    slice_fn = backbone_of(max(1, n_mm // n_g))

    def host_overlap():
        for i in range(n_g):
            pfr.begin(idx[i % R], stream=sb)
            slice_fn()
            pfr.finish(emb[i & 1], stream=sb)

    def slices():
        for _ in range(n_g):
            slice_fn()

    for _ in range(2):
        wall([host_overlap])
    both_host = min(wall([host_overlap]) for _ in range(3))
    bb_host = min(wall([slices]) for _ in range(3))
    pfr.close()
    line = {
        "metric": "Engram host-table gather tokens/sec",
        "value": round(n_tok / (ms_cached * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": 3,
        "ms_per_step": round(ms_cached, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic: Zipf(%s) token ids, seeded Philox tables in pinned host memory" % wl.zipf_s,
        "config": {"workload": wl.name, "tokens_per_step": n_tok, "n_tables": wl.n_tables, "head_dim": wl.head_dim,
                   "table_bytes": sum(wl.primes()) * row_b, "cache_rows_per_table": n_hot,
                   "cache_slots_per_table": cap, "cache_bytes": wl.n_tables * cap * (row_b + 4),
                   "rotated_batches": R, "parallelism": "single GPU"},
        "gather_ms": {"hbm_tables": round(ms_dev, 4), "host_tables": round(ms_host, 4),
                      "host_tables_cached": round(ms_cached, 4)},
        "host_link_GBs_uncached": round(link_bytes / (ms_host * 1e-3) / 1e9, 2),
        "host_link_GBs_cached": round(link_bytes * (1 - hit_rate) / (ms_cached * 1e-3) / 1e9, 2),
        "cache_hit_rate": round(hit_rate, 4),
        "forward_ms": {"hbm_tables": round(fwd_dev_ms, 4), "host_tables": round(fwd_host_ms, 4)},
        # overhead_frac: extra time of backbone + prefetch over the backbone
        # alone on the whole chip
        "overlap": {"backbone_matmuls": "%d x bf16 %dx%d by %dx%d" % (n_mm, Mb, Kb, Kb, Mb), "prefetch_gathers": n_g,
                    "uncapped": {"backbone_ms": round(bb_full, 3),
                                 "backbone_TFLOPs": round(mm_flops / (bb_full * 1e-3) / 1e12, 1),
                                 "prefetch_ms": round(pf_full, 3), "together_ms": round(both_full, 3),
                                 "overhead_frac": round((both_full - bb_full) / bb_full, 4)},
                    "capped": {"prefetch_workgroups": args.prefetch_wgs, "backbone_ms": round(bb_cap, 3),
                               "prefetch_ms": round(pf_cap, 3), "together_ms": round(both_cap, 3),
                               "overhead_frac": round((both_cap - bb_cap) / bb_cap, 4)},
                    # n_g jobs, each begun before its share of the backbone and finished after it
                    "host_gather": {"backbone_matmuls": "%d x %d" % (n_g, max(1, n_mm // n_g)),
                                    "host_threads": args.host_threads, "backbone_ms": round(bb_host, 3),
                                    "prefetch_ms": round(hg_ms * n_g, 3), "together_ms": round(both_host, 3),
                                    "overhead_frac": round((both_host - bb_host) / bb_host, 4)}},
        "host_gather_ms": round(hg_ms, 4),
        "host_gather_miss_frac": round(misses / (n_g * n_tok * wl.n_tables), 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
