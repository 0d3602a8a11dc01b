"""CPU oracle (test infrastructure only; see wan_oracle.py)."""
