"""CPU fp64 attention oracle (test infrastructure only; see ref_attention)."""
