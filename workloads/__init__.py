"""Seeded synthetic inputs for paged-KV decode.

This module only draws inputs: sequence lengths, the initial order of the
free-block list, which sequences share which prefix blocks, token keys /
values and queries.  It holds none of the method's arithmetic: it does not
compute slots, place tokens into blocks, quantise or attend.  Both the HIP path
(through its binding) and the CPU oracle consume what it returns, each with its
own code.

Integer structure comes from ``numpy.random.default_rng(seed)``; floating-point
data from ``torch.Generator`` on the requested device (so a GPU run draws its
large tensors on the GPU; CPU and GPU draws of the same seed differ, and every
test compares two sides fed from one draw).

Draw order: lengths, free-list permutation, outlier channels, prompt K/V,
queries, new-token K/V.
"""

from .synth import (  # noqa: F401
    WORKLOADS,
    Workload,
    draw_tensors,
    get_workload,
    plan_ops,
)
