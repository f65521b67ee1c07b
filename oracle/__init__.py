"""CPU oracle package (test infrastructure only; see qsa_oracle.py)."""
