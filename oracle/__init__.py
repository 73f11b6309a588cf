"""fp64 CPU oracle for the MoE layer forward (test infrastructure only)."""
