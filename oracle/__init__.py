"""CPU oracle package (test infrastructure; see oracle/oracle.py)."""
