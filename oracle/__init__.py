"""CPU oracle (test infrastructure only; see oracle.py and indexer_oracle.c)."""
