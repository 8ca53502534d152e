"""CPU fp64 oracle for LCSA (test infrastructure only; never imported by the product path)."""
