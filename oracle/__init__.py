"""CPU oracle of the MoE layer (test infrastructure only; see moe_oracle.py)."""
