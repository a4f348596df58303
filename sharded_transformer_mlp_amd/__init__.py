"""MI355X-native hot path of one rank's TSP gated-MLP block.

The compute runs in hand-written gfx950 HIP kernels behind the C-ABI library
``libtsp_mlp.so`` (declared in ``include/tsp_mlp.h``); ``binding`` is a thin
ctypes layer over it. ``inputs`` holds the seeded synthetic workloads.
"""
from .inputs import WORKLOADS, ALIASES, Workload, workload, make_inputs  # noqa: F401
