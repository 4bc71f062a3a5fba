"""Seeded synthetic inputs for the Engram forward pass.

This package produces the *inputs* that both the CPU oracle and the HIP
library consume: workload shapes, compression maps, Zipf token streams,
dense activations and weights.  It holds none of the method's arithmetic
(no hashing, no gathering, no gate, no convolution).  Embedding-table
contents are not produced here: each side regenerates them from the
published Philox4x64-10 counter-based generator (Salmon et al., SC'11),
with the counter layout documented in ``synthetic.workloads.TABLE_RECIPE``.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    LayerInputs,
    TABLE_RECIPE,
    compression_map,
    largest_primes_at_most,
    make_layer_inputs,
    make_tokens,
    workload,
)
