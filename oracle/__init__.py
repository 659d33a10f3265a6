"""fp64 CPU oracle (test infrastructure only; see hla_oracle's header)."""
from .hla_oracle import (  # noqa: F401
    LINEAR, SOFTMAX, as_f64, relu, sigmoid, linear_state, linear_readout, gated_linear, gated_linear_write,
    softmax_probs, gated_softmax, hybrid_kinds, layer, hybrid_stack, max_rel_error,
    ATTNRES_BLOCK, block_summary, attnres_route,
)
