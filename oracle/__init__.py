"""CPU oracle (test infrastructure only; see polestar_oracle.py)."""
