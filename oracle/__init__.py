"""fp64 CPU oracle for selective decode attention (test infrastructure only)."""
