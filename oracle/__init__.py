"""CPU oracle of the DF-SSM hot path (test infrastructure only; see dfssm_oracle.py)."""
