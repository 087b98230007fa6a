"""CPU oracle (test infrastructure only; never imported by the GPU library or its binding)."""
