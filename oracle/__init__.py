"""fp64 CPU oracle of the MoE expert layer: test infrastructure only (see moe_oracle)."""
