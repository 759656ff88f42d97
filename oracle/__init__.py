"""fp64 CPU oracle for the SSD layer (test infrastructure; see oracle.py)."""
