"""fp64 CPU oracle of the DECO MoE feed-forward layer (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  The product path (the HIP library and its binding) never imports
it, and it imports nothing from the product path.
"""
from .deco_oracle import (router, router_topk, mean_up, normsilu, silu, expert_mlp, expert_mlp_gated, shared_expert,
                          forward, forward_dense_bruteforce, OracleResult)
from .deco_backward import (backward, objective, router_entropy, sparsity_coef_update, dsilu, Grads)

__all__ = ["router", "router_topk", "mean_up", "normsilu", "silu", "expert_mlp", "expert_mlp_gated", "shared_expert",
           "forward", "forward_dense_bruteforce", "OracleResult",
           "backward", "objective", "router_entropy", "sparsity_coef_update", "dsilu", "Grads"]
