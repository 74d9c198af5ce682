"""fp64 CPU oracle for SQuad-Attention (test infrastructure only; see squad_oracle)."""
