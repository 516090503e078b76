"""CPU oracle (test infrastructure only): see mx_oracle's module docstring."""
