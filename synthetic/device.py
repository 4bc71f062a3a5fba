"""Device-resident inputs of a workload (harness for tests and benchmarks).

Allocates the caller-owned buffers one Engram layer needs on the GPU and
fills them: dense inputs come from ``synthetic.workloads`` (host, seeded);
embedding tables are generated on the device by the library's synthetic-table
entry point so that even 200 GB of tables need no host copy.  Nothing here
computes a step of the method.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

from . import workloads as W


@dataclasses.dataclass
class DeviceLayer:
    wl: W.Workload
    li: W.LayerInputs
    plan: object
    tables: List[torch.Tensor]
    h: torch.Tensor
    weights: object
    comp_map_host: np.ndarray
    comp_map: torch.Tensor

    def free_tables(self):
        self.tables = []


def to_device(x: np.ndarray, dtype: torch.dtype, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).to(device)


def make_device_layer(wl: W.Workload, layer_slot: int = 0, device="cuda", batch: Optional[int] = None,
                      seqlen: Optional[int] = None, with_tables: bool = True,
                      conv_mode: int = 0, rms_eps: float = 1e-6, host_tables: bool = False) -> DeviceLayer:
    """host_tables: the tables go to pinned host memory (HostBuffer objects,
    read by the GPU over the host link), generated on the device one at a time
    and copied there."""
    from hashed_gram_embedding_vocab_amd import binding as B

    li = W.make_layer_inputs(wl, layer_slot, batch=batch, seqlen=seqlen)
    dt = B.BF16 if wl.dtype == "bf16" else B.F32
    tdt = torch.bfloat16 if dt == B.BF16 else torch.float32
    primes = wl.primes()
    plan = B.Plan(vocab=wl.vocab, vocab_comp=wl.vocab_comp, heads=wl.heads, head_dim=wl.head_dim,
                  table_rows=primes, hash_seed=li.hash_seed, d_model=wl.d_model,
                  n_branches=wl.n_branches, conv_kernel=wl.conv_kernel, conv_mode=conv_mode,
                  rms_eps=rms_eps, dtype=dt, orders=wl.orders,
                  state_dtype=B.BF16 if wl.state_dtype == "bf16" else B.F32)
    tables = []
    if with_tables:
        for tau, p in enumerate(primes):
            t = torch.empty((p, wl.head_dim), dtype=tdt, device=device)
            B.engram_synth_fill_table(t, li.table_seed, tau, dt)
            if host_tables:
                hb = B.HostBuffer(t.numel() * t.element_size())
                hb.view(tdt, t.shape).copy_(t.cpu())
                del t
                tables.append(hb)
            else:
                tables.append(t)
    h = to_device(li.h, tdt, device)
    weights = B.Weights(
        w_k=[to_device(li.w_k[m], tdt, device) for m in range(wl.n_branches)],
        w_v=to_device(li.w_v, tdt, device),
        gamma_h=[to_device(li.gamma_h[m], torch.float32, device) for m in range(wl.n_branches)],
        gamma_k=[to_device(li.gamma_k[m], torch.float32, device) for m in range(wl.n_branches)],
        conv_w=to_device(li.conv_w, torch.float32, device))
    comp = W.compression_map(wl.vocab, wl.vocab_comp, wl.seed(1))
    return DeviceLayer(wl=wl, li=li, plan=plan, tables=tables, h=h, weights=weights,
                       comp_map_host=comp, comp_map=to_device(comp, torch.int32, device))
