"""CPU decode oracle (test infrastructure only)."""
