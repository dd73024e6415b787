"""CPU oracle of the batch-invariant MoE layer forward (test infrastructure only)."""
