"""fp64 CPU oracle (test infrastructure only; never on the product path)."""
from .tsp_oracle import (f64, silu, gelu_tanh, ring_order, shard_hidden, shard_partial,
                         mlp_forward, tsp_simulate, flops)

__all__ = ["f64", "silu", "gelu_tanh", "ring_order", "shard_hidden", "shard_partial",
           "mlp_forward", "tsp_simulate", "flops"]
