"""Float64 CPU oracle of the DyRA layer forward (test infrastructure only)."""
