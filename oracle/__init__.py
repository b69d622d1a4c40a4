"""CPU oracle of the fused MoE layer (test infrastructure only; see
moe_oracle.py).  Nothing on the product path imports this package."""
