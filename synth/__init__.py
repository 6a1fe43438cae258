"""Seeded synthetic inputs for the compressed-KV decode path.

This module draws inputs only: query vectors, orthonormal bases, rank tables,
cache lengths and the bulk key/value rows. It holds none of the method's
arithmetic (no projection, no attention, no softmax). Both the GPU path and
the float64 oracle consume what it produces.

Bulk key/value rows come from a counter-based generator (see ``host.py``)
that is implemented twice, once in numpy and once as a HIP kernel
(``csrc/synth_gen.hip``), so that any slice of a multi-GiB workload can be
regenerated bit for bit on the host without copying it back from the GPU.
"""
from .configs import (CONFIGS, LLAMA3_32_LAYERS, LLAMA3_LAYER_32K, LONG_CONTEXT_128K,  # noqa: F401
                      PER_HEAD_RAGGED, SINGLE_HEAD_F32, WORKLOADS, Config)
