"""Float64 CPU oracle of the sparse-MoE layer (test infrastructure only)."""
