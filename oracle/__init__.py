"""fp64 CPU oracle (test infrastructure only; never on the product path)."""
from .tsp_oracle import (f64, silu, gelu_tanh, ring_order, shard_hidden, shard_partial,
                         mlp_forward, tsp_simulate, flops, silu_grad, gelu_tanh_grad, shard_backward,
                         mlp_backward, mlp_backward_columns, backward_flops)

__all__ = ["f64", "silu", "gelu_tanh", "ring_order", "shard_hidden", "shard_partial",
           "mlp_forward", "tsp_simulate", "flops", "silu_grad", "gelu_tanh_grad", "shard_backward",
           "mlp_backward", "mlp_backward_columns", "backward_flops"]
