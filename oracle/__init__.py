"""CPU FP64 oracle (test infrastructure only; see moe_oracle)."""
