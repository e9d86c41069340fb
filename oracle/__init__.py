"""CPU oracle for the transposable 2:4 FFN path (test infrastructure only)."""
